"""sdpa_bwd_noalloc (the backward for callers that cannot allocate: its workspace is the
library's static scratch buffer) against sdpa_bwd with a caller workspace, through the C ABI.

Two calls in a row share the buffer, the second on a smaller problem, and each must give
exactly sdpa_bwd's bits (same kernels; the buffer keeps the previous call's contents, which
no kernel may rely on).  The cases cover the dense path, the GQA dK/dV split (its arrival
counters live in the buffer) and THD (its work lists live in the buffer)."""
import numpy as np
import pytest
import torch

import scaled_dot_product_05_amd as S
import synth
from gpu_util import DEV, check_grads, gpu_bhsd, oracle_backward, say


def _setup(w):
    q, k, v = (t.to(DEV) for t in (w.q, w.k, w.v))
    g = w.dout.to(DEV)
    kw = {}
    if w.is_thd:
        cu = torch.from_numpy(w.cu_seqlens_q).to(DEV)
        kw = dict(cu_seqlens_q=cu, max_seqlen_q=int(np.diff(w.cu_seqlens_q).max()))
    o, lse = S.forward(q, k, v, w.layout, w.scale, w.window, **kw)
    pr = S.Problem(q, k, w.layout, w.scale, w.window, **kw)
    return pr, (q, k, v, o, lse, g)


def _noalloc(pr, t):
    q, k, v, o, lse, g = t
    dq, dk, dv = torch.full_like(q, float("nan")), torch.full_like(k, float("nan")), \
        torch.full_like(v, float("nan"))
    S.sdpa_bwd_noalloc(pr.desc, q, k, v, o, lse, g, None, dq, dk, dv)
    return dq, dk, dv


def _reference(pr, t):
    q, k, v, o, lse, g = t
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(S.sdpa_bwd_workspace_size(pr.desc), 1), dtype=torch.uint8, device=DEV)
    S.sdpa_bwd(pr.desc, q, k, v, o, lse, g, None, dq, dk, dv, False, ws)
    return dq, dk, dv


CASES = {
    "dense_mha": (lambda: synth.dense(60, 1100, "bf16", "bshd", 2, 1024, 1024, 8, 8, 64, 0.125,
                                      (-1, 0), with_grad=True, name="na_big"),
                  lambda: synth.dense(61, 1101, "bf16", "bshd", 1, 300, 300, 4, 4, 64, 0.125,
                                      (-1, 0), with_grad=True, name="na_small")),
    "gqa_split": (lambda: synth.dense(62, 1102, "bf16", "bshd", 1, 1024, 1024, 16, 4, 128,
                                      128 ** -0.5, (-1, 0), with_grad=True, name="na_gqa_big"),
                  lambda: synth.dense(63, 1103, "bf16", "bshd", 1, 200, 200, 8, 2, 128, 0.1,
                                      (-1, 0), with_grad=True, name="na_gqa_small")),
    "thd": (lambda: synth.thd(64, 1104, "f16", [700, 0, 1300, 65], 8, 2, 64, 0.125, (-1, 0),
                              with_grad=True),
            lambda: synth.thd(65, 1105, "f16", [129, 3], 4, 2, 64, 0.125, (-1, 0),
                              with_grad=True)),
}


@pytest.mark.gpu
@pytest.mark.parametrize("case", list(CASES))
def test_noalloc_equals_sdpa_bwd_twice_in_a_row(case):
    big, small = (f() for f in CASES[case])
    for w in (big, small):
        say(f"case noalloc {case} {w.name} {w.dtype} {w.layout} B={w.batch} Sq={w.seqlen_q} "
            f"Hq={w.heads_q} Hk={w.heads_kv} D={w.head_dim}")
        pr, t = _setup(w)
        need = S.sdpa_bwd_workspace_size(pr.desc)
        assert need <= S.sdpa_bwd_noalloc_max_workspace()
        got = _noalloc(pr, t)
        torch.cuda.synchronize()
        ref = _reference(pr, t)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
        check_grads([gpu_bhsd(x, w) for x in got], oracle_backward(w), w.dtype, "noalloc bwd")


def test_noalloc_rejects_a_problem_beyond_its_buffer():
    # a host-side check before anything runs (no GPU needed): 16 q heads x 600k queries,
    # whose Delta and LSE log2(e) alone need ~77 MB, more than the 64 MiB buffer
    desc = S.make_desc("bshd", "bf16", 1, 600000, 600000, 16, 16, 64, 0.125, (-1, 0))
    need = S.sdpa_bwd_workspace_size(desc)
    assert need > S.sdpa_bwd_noalloc_max_workspace()
    null = S.tensor(None)
    rc = S.lib().sdpa_bwd_noalloc(desc, null, null, null, null, S.rowstat(None), null,
                                  S.rowstat(None), null, null, null, 0, None)
    assert S.STATUS[rc] == "ERR_WORKSPACE"
    assert b"static scratch buffer" in S.lib().sdpa_last_error()
