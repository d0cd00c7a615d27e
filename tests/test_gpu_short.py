"""GPU parity of the short-sequence kernels against the fp64 oracle.

Calls whose sequences hold at most 32 queries run a forward in which every wave is a work
unit of its own (32 query rows of one (sequence, q head)); with at most 32 keys as well and
head_dim <= 64 the backward does the same per (sequence, kv head).  These cases cover both
across dtypes, head dims, key lengths with ragged tails, windows, both diagonal alignments,
GQA, dLSE, accumulation, packed views, THD (plain and padded), fully masked rows and a
large batch checked on sampled (batch, head) pairs; each asserts which kernels ran.
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
        dl = w.dlse.to(DEV) if w.dlse is not None else None
        names = kernels_of(lambda: res.update(g=gpu_backward(w, q, k, v, o, lse, w.dout.to(DEV),
                                                             dl, cq, ck)))
        short_bwd = w.seqlen_q <= 32 and w.seqlen_k <= 32 and w.head_dim <= 64
        assert ("bwd_short" in names) == short_bwd, names
        refs = oracle_backward(w, synth.f64(w.dlse) if dl is not None else None)
        check_grads([gpu_bhsd(t, w) for t in res["g"]], refs, w.dtype, "bwd")


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


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_backward_groups_dlse_bottom_right(dtype):
    w = synth.dense(39, 980, dtype, "bshd", 3, 20, 29, 8, 2, 64, 0.2, (-1, 0), 1,
                    with_grad=True, with_dlse=True, name="short_bwd_gqa")
    run_case(w)


def test_backward_accumulates():
    w = synth.dense(40, 990, "bf16", "sbhd", 2, 32, 32, 4, 4, 64, 0.125, (7, 0),
                    with_grad=True, name="short_bwd_acc")
    q, k, v = to_dev(w)
    o, lse = gpu_forward(w, q, k, v)
    g = w.dout.to(DEV)
    dq, dk, dv = gpu_backward(w, q, k, v, o, lse, g)
    names = kernels_of(lambda: gpu_backward(w, q, k, v, o, lse, g, dq=dq, dk=dk, dv=dv,
                                            accumulate=True))
    assert "bwd_short" in names, names
    refs = [2 * r for r in oracle_backward(w)]
    check_grads([gpu_bhsd(t, w) for t in (dq, dk, dv)], refs, "bf16", "bwd accumulated twice")


@pytest.mark.parametrize("d", [32, 64])
def test_backward_thd_short_sequences(d):
    w = synth.thd(41, 1000 + d, "bf16", [1, 0, 32, 17, 5, 31], 8, 2, d, d ** -0.5, (-1, 0),
                  with_grad=True, with_dlse=True, name="short_bwd_thd")
    run_case(w)


def test_backward_thd_cross_lengths():
    w = synth.thd(42, 1010, "f16", [3, 32, 9, 0], 4, 4, 64, 0.3, (-1, 0), with_grad=True,
                  lengths_k=[30, 7, 32, 5], diag_align=1, name="short_bwd_thd_cross")
    run_case(w)
