"""accumulate = 1 on every 16-bit backward path: each epilogue reads the output element, adds
its fp32 gradient and rounds once.  A second call with accumulate = 1 into the outputs of a
first (plain) call must therefore give RNE(g1 + x) for the same unrounded gradient x, with
g1 = RNE(x): within one bf16 unit in the last place of 2 g1 (doubling is exact), element by
element.  Paths: the fused small-grid launch (MHA), its GQA halves, the two-launch backward
(dense D64, THD D128), the kernels with 64-bit addressing (a dK output whose rows are not
16-byte aligned), and a block-sparse mask."""
import numpy as np
import pytest
import torch

import scaled_dot_product_05_amd as S
import synth
from gpu_util import DEV, cu_dev, gpu_backward, gpu_forward, say, to_dev

pytestmark = pytest.mark.gpu


def _case(name):
    if name == "fused_mha_d64":
        return synth.dense(40, 1400, "bf16", "bshd", 2, 640, 640, 4, 4, 64, 0.125, (-1, 0), with_grad=True)
    if name == "gqa_halves_d128":
        return synth.target(b=1, s=1024, h=16, hk=4, d=128, with_grad=True)
    if name == "wide_d64":
        return synth.dense(41, 1401, "bf16", "bshd", 8, 2048, 2048, 8, 8, 64, 0.125, (-1, 0), with_grad=True)
    if name == "wide_thd_d128":
        return synth.c4(2)
    return synth.dense(42, 1402, "bf16", "bshd", 1, 300, 300, 4, 2, 128, 128 ** -0.5, (64, 0), with_grad=True)


def _assert_doubled(g1, g2, what):
    a = g1.float() * 2
    b = g2.float()
    bound = a.abs() * 2.0 ** -7 + 1e-30
    bad = (b - a).abs() > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements off, e.g. {a[bad][:3].tolist()} vs {b[bad][:3].tolist()}"


@pytest.mark.parametrize("name", ["fused_mha_d64", "gqa_halves_d128", "wide_d64", "wide_thd_d128",
                                  "unaligned_dk", "block_mask"])
def test_accumulate_adds_once_rounded(name):
    w = _case(name)
    say(f"case accumulate {name}")
    q, k, v = to_dev(w)
    cq, ck = cu_dev(w)
    g = w.dout.to(DEV)
    kw = {}
    if name == "block_mask":
        mask = synth.flex_mask("sliding_window_causal", w.seqlen_q, w.seqlen_k, band=100)
        bits = np.ascontiguousarray(synth.pack_mask(mask[None, None])).view(np.int64)
        kw["block_mask"] = S.BlockMask(torch.from_numpy(bits).to(DEV), w.seqlen_q, w.seqlen_k)
    if w.is_thd:
        o, lse = gpu_forward(w, q, k, v, cq, ck)
    else:
        o, lse = S.forward(q, k, v, w.layout, w.scale, w.window, w.diag_align, **kw)
    dk_buf = None
    if name == "unaligned_dk":
        dk_buf = torch.zeros(k.shape[:-1] + (k.shape[-1] + 1,), dtype=k.dtype, device=DEV)[..., 1:]
    outs = []
    for acc in (False, True):
        if acc:
            dq, dk, dv = (t.clone() for t in outs[0])
            if dk_buf is not None:
                dk_buf.copy_(outs[0][1])
                dk = dk_buf
        else:
            dq = dk = dv = None
            dk = dk_buf
        if w.is_thd:
            r = gpu_backward(w, q, k, v, o, lse, g, None, cq, ck, dq=dq, dk=dk, dv=dv, accumulate=acc)
        else:
            r = S.backward(q, k, v, o, lse, g, w.layout, w.scale, w.window, w.diag_align, dq=dq, dk=dk,
                           dv=dv, accumulate=acc, **kw)
        torch.cuda.synchronize()
        outs.append(tuple(t.clone() for t in r))
    for n, a, b in zip(("dq", "dk", "dv"), outs[0], outs[1]):
        _assert_doubled(a, b, f"{name} {n}")
