"""GPU parity of the short-sequence forward against the fp64 oracle.

Calls whose sequences hold at most 32 queries run a forward in which every wave is a work
unit of its own (32 query rows of one (sequence, q head)); these cases cover it across
dtypes, head dims, key lengths with ragged tails, windows, both diagonal alignments, GQA,
packed views, THD (plain and padded), fully masked rows and a large batch checked on
sampled (batch, head) pairs.  The backward that follows runs on the O and LSE it wrote.
"""
import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_05_amd as S
import synth
from gpu_util import (DEV, check_forward, check_grads, cu_dev, gpu_backward, gpu_bhsd,
                      gpu_forward, oracle_backward, oracle_forward, say, to_dev)

pytestmark = pytest.mark.gpu


def kernels_of(fn):
    """Names of the kernels the library launched inside fn()."""
    torch.cuda.synchronize()
    S.sdpa_profile_enable(True)
    try:
        fn()
        torch.cuda.synchronize()
    finally:
        S.sdpa_profile_enable(False)
    return set(S.sdpa_profile_read())


def run_case(w, backward=True):
    say(f"case {w.name} {w.dtype} {w.layout} B={w.batch} Sq={w.seqlen_q} Sk={w.seqlen_k} "
        f"Hq={w.heads_q} Hk={w.heads_kv} D={w.head_dim} win={w.window} al={w.diag_align}")
    q, k, v = to_dev(w)
    cq, ck = cu_dev(w)
    res = {}
    names = kernels_of(lambda: res.update(ol=gpu_forward(w, q, k, v, cq, ck)))
    assert "attn_fwd_short" in names, names
    o, lse = res["ol"]
    o_ref, lse_ref = oracle_forward(w)
    check_forward(gpu_bhsd(o, w), synth.f64(lse), o_ref, lse_ref, w.dtype, "fwd")
    if backward:
        dq, dk, dv = gpu_backward(w, q, k, v, o, lse, w.dout.to(DEV), None, cq, ck)
        torch.cuda.synchronize()
        check_grads([gpu_bhsd(t, w) for t in (dq, dk, dv)], oracle_backward(w), w.dtype, "bwd")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_dtype_headdim_causal(dtype, d):
    w = synth.dense(31, 900 + d, dtype, "bshd", 3, 32, 32, 4, 2, d, d ** -0.5, (-1, 0),
                    with_grad=True, name="short")
    run_case(w)


@pytest.mark.parametrize("sq,sk", [(1, 1), (7, 300), (32, 33), (17, 64), (25, 1000)])
@pytest.mark.parametrize("window,align", [((-1, -1), 0), ((-1, 0), 1), ((5, 3), 0),
                                          ((40, 0), 1)])
def test_key_lengths_and_windows(sq, sk, window, align):
    w = synth.dense(32, 910 + sq + sk, "bf16", "bhsd", 2, sq, sk, 4, 4, 64, 0.3, window, align,
                    with_grad=True, name="short_win")
    run_case(w)


def test_fully_masked_rows_and_negative_scale():
    # window (-1, -5): the first 5 queries see no key -> O = 0, LSE = -inf
    w = synth.dense(33, 920, "f16", "sbhd", 2, 30, 30, 2, 1, 64, -0.4, (-1, -5),
                    with_grad=True, name="short_empty_rows")
    run_case(w)


def test_packed_qkv_views():
    buf, q, k, v = synth.packed_qkv(34, 930, "f16", 32, 3, 16, 1, 64)
    w = synth.Workload("short_packed", "f16", "sbhd", 3, 32, 32, 16, 1, 64, 0.1, (-1, 0), 0,
                       q, k, v)
    w.extra["packed"] = buf
    run_case(w, backward=False)


def test_thd_short_sequences():
    w = synth.thd(35, 940, "bf16", [1, 0, 32, 17, 5, 31], 8, 2, 128, 0.125, (-1, 0),
                  with_grad=True, name="short_thd")
    run_case(w)


def test_thd_padded_short_sequences():
    lengths = [3, 32, 0, 19]
    w = synth.thd(36, 950, "bf16", lengths, 4, 4, 64, 0.125, (-1, 0), name="short_thd_pad")
    # each sequence starts at a multiple of 40 rows; the gaps hold other values
    starts = np.arange(len(lengths) + 1, dtype=np.int32) * 40
    tot = int(starts[-1])
    q, k, v = (torch.full((tot, t.shape[1], 64), 7.0, dtype=torch.bfloat16, device=DEV)
               for t in (w.q, w.k, w.v))
    cu = w.cu_seqlens_q
    for i, L in enumerate(lengths):
        for dst, src in zip((q, k, v), (w.q, w.k, w.v)):
            dst[starts[i]:starts[i] + L] = src[cu[i]:cu[i] + L].to(DEV)
    cqd = torch.from_numpy(cu).to(DEV)
    pad = torch.from_numpy(starts).to(DEV)
    res = {}
    names = kernels_of(lambda: res.update(ol=S.forward(
        q, k, v, "thd", w.scale, w.window, cu_seqlens_q=cqd, cu_seqlens_k=cqd,
        max_seqlen_q=32, max_seqlen_k=32, cu_seqlens_q_padded=pad, cu_seqlens_k_padded=pad)))
    assert "attn_fwd_short" in names, names
    o, lse = res["ol"]
    o_ref, lse_ref = oracle_forward(w)
    rows = np.concatenate([np.arange(starts[i], starts[i] + L) for i, L in enumerate(lengths)])
    check_forward(synth.f64(o)[rows], synth.f64(lse)[:, rows], o_ref, lse_ref, "bf16",
                  "padded thd fwd")


def test_longer_sequences_take_the_tiled_kernel():
    w = synth.dense(37, 960, "bf16", "bshd", 1, 33, 33, 2, 2, 64, 0.125, (-1, 0))
    q, k, v = to_dev(w)
    names = kernels_of(lambda: gpu_forward(w, q, k, v))
    assert "attn_fwd" in names and "attn_fwd_short" not in names, names


def test_large_batch_sampled():
    # S = 32, B = 512, H = 16, D = 64 (as in the short-sequence bandwidth measurement, at a
    # quarter of its batch): oracle on 12 sampled batch entries, every head
    b, s, h, d = 512, 32, 16, 64
    w = synth.dense(38, 970, "bf16", "bshd", b, s, s, h, h, d, 0.125, (-1, -1), name="short_big")
    q, k, v = to_dev(w)
    names = kernels_of(lambda: gpu_forward(w, q, k, v))
    assert "attn_fwd_short" in names, names
    o, lse = gpu_forward(w, q, k, v)
    torch.cuda.synchronize()
    pick = np.random.default_rng(970).choice(b, size=12, replace=False)
    pick = np.concatenate([[0, b - 1], pick])
    qs, ks, vs = (synth.f64(synth.to_bhsd(t[pick].cpu(), "bshd")) for t in (w.q, w.k, w.v))
    o_ref, lse_ref = oracle.windowed_forward(qs, ks, vs, w.scale, w.window, 0)
    og = synth.f64(synth.to_bhsd(o[pick].cpu(), "bshd"))
    check_forward(og, synth.f64(lse[pick]), o_ref, lse_ref, "bf16", "sampled fwd")
