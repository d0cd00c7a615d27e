"""Seeded random problems large enough for the two-launch backward (more than 12 fused-launch
blocks per compute unit): dtype, layout (BSHD, SBHD, BHSD, THD with cross lengths), head_dim,
GQA grouping, window kind and diagonal alignment, softmax scale (including negative) and dLSE
are drawn per case.  Outputs are checked on sampled query rows and key columns against the
fp64 oracle's row functions: O, LSE and dQ of the sampled rows of a few (batch, q head)
pairs, dK and dV of sampled key rows of a few (batch, kv head) pairs."""
import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_05_amd as S
import synth
from gpu_util import (DEV, G_TOL, LSE_TOL, O_TOL, cu_dev, gpu_backward, gpu_forward, rel_err, say,
                      to_dev)

pytestmark = pytest.mark.gpu

N_CASES = 16
WIDE_BLOCKS = 3300  # 64-row dQ plus 64-key dK/dV blocks; the two launches start above 12 per CU


def _window(rng):
    kind = int(rng.integers(0, 4))
    return [(-1, 0), (-1, -1), (int(rng.integers(64, 1500)), int(rng.integers(0, 300))),
            (-1, int(rng.integers(0, 200)))][kind]


def _case(i):
    rng = np.random.default_rng([2025, i])
    dtype = ("bf16", "f16")[int(rng.integers(0, 2))]
    layout = ("bshd", "sbhd", "bhsd", "thd")[int(rng.integers(0, 4))]
    d = (64, 128)[int(rng.integers(0, 2))]
    hk = (1, 2, 4, 8)[int(rng.integers(0, 4))]
    hq = hk * (1, 2, 4)[int(rng.integers(0, 3))]
    scale = float(d ** -0.5 * (1.0, 0.7, -1.0)[int(rng.integers(0, 3))])
    window = _window(rng)
    align = int(rng.integers(0, 2))
    dlse = bool(rng.integers(0, 2))
    if layout == "thd":
        n = int(rng.integers(4, 17))
        lengths = rng.integers(200, 4001, n)
        while (hq + hk) * (lengths.sum() / 64 + n) < WIDE_BLOCKS:
            lengths = np.concatenate([lengths, rng.integers(200, 4001, 4)])
        lengths_k = np.maximum(1, lengths + rng.integers(-150, 151, len(lengths)))
        w = synth.thd(300 + i, 3000 + i, dtype, lengths.tolist(), hq, hk, d, scale, window,
                      with_grad=True, with_dlse=dlse, lengths_k=lengths_k.tolist(), diag_align=align,
                      name=f"wide{i}")
    else:
        sq, sk = int(rng.integers(1024, 3073)), int(rng.integers(1024, 3073))
        b = int(np.ceil(WIDE_BLOCKS * 64 / (hq * sq + hk * sk)))
        w = synth.dense(300 + i, 3000 + i, dtype, layout, b, sq, sk, hq, hk, d, scale, window, align,
                        with_grad=True, with_dlse=dlse, name=f"wide{i}")
    return w, dlse, rng


def _pairs(w, rng, n):
    """(sequence or batch, q head) pairs to sample, with each pair's row extents."""
    nb = len(w.cu_seqlens_q) - 1 if w.is_thd else w.batch
    return [(int(rng.integers(0, nb)), int(rng.integers(0, w.heads_q))) for _ in range(n)]


@pytest.mark.parametrize("i", range(N_CASES))
def test_wide_random_problem_sampled(i):
    w, dlse, rng = _case(i)
    say(f"case wide{i} {w.dtype} {w.layout} B={w.batch} Sq={w.seqlen_q} Sk={w.seqlen_k} "
        f"Hq={w.heads_q} Hk={w.heads_kv} D={w.head_dim} scale={w.scale:.3f} win={w.window} "
        f"al={w.diag_align} dlse={dlse}")
    q, k, v = to_dev(w)
    cq, ck = cu_dev(w)
    o, lse = gpu_forward(w, q, k, v, cq, ck)
    dl = w.dlse.to(DEV) if dlse else None
    torch.cuda.synchronize()
    S.sdpa_profile_enable(True)
    dq, dk, dv = gpu_backward(w, q, k, v, o, lse, w.dout.to(DEV), dl, cq, ck)
    torch.cuda.synchronize()
    S.sdpa_profile_enable(False)
    names = set(S.sdpa_profile_read())
    # the two launches: dQ (which forms Delta, so no pre-pass), then dK/dV
    assert {"bwd_dq", "bwd_dkdv"} <= names and not names & {"bwd_pre", "bwd_main"}, names
    o, lse, dq, dk, dv = (t.cpu() for t in (o, lse, dq, dk, dv))
    g = w.heads_q // w.heads_kv
    if w.is_thd:
        cu, cuk = w.cu_seqlens_q, w.cu_seqlens_k
        rows_of = lambda t, s, h, c: synth.f64(t[c[s]:c[s + 1], h])  # [L, D]
        stat_of = lambda t, s, h: synth.f64(t[h, cu[s]:cu[s + 1]])
        dlse_of = lambda s, h: synth.f64(w.dlse[h, cu[s]:cu[s + 1]]) if dlse else None
        src = lambda t, s, h, c: rows_of(t, s, h, c)
    else:
        cu = cuk = None
        bh = {n: synth.to_bhsd(t, w.layout) for n, t in (("q", w.q), ("k", w.k), ("v", w.v),
                                                          ("g", w.dout), ("o", o), ("dq", dq),
                                                          ("dk", dk), ("dv", dv))}
        rows_of = lambda name, s, h, _c: synth.f64(bh[name][s, h])
        stat_of = lambda t, s, h: synth.f64(t[s, h])
        dlse_of = lambda s, h: synth.f64(w.dlse[s, h]) if dlse else None
        src = rows_of
    pick = (lambda t, name: t) if w.is_thd else (lambda t, name: name)
    worst_o = worst_l = 0.0
    got = {"dq": [], "dk": [], "dv": []}
    ref = {"dq": [], "dk": [], "dv": []}
    for s, h in _pairs(w, rng, 3):
        hk = h // g
        qs = src(pick(w.q, "q"), s, h, cu)
        gs = src(pick(w.dout, "g"), s, h, cu)
        ks = src(pick(w.k, "k"), s, hk, cuk)
        vs = src(pick(w.v, "v"), s, hk, cuk)
        if len(qs) == 0 or len(ks) == 0:
            continue
        rows = np.unique(np.concatenate([[0, len(qs) - 1], rng.integers(0, len(qs), 12)]))
        ro, rl = oracle.forward_rows(qs, ks, vs, w.scale, rows, w.window, w.diag_align)
        go = src(pick(o, "o"), s, h, cu)[rows]
        gl = stat_of(lse, s, h)[rows]
        fin = np.isfinite(rl)
        assert (np.isneginf(gl) == ~fin).all(), f"-inf rows differ at ({s}, {h})"
        assert (go[~fin] == 0).all()
        worst_o = max(worst_o, float(np.abs(go - ro).max()))
        if fin.any():
            worst_l = max(worst_l, float(np.abs(gl[fin] - rl[fin]).max()))
        got["dq"].append(src(pick(dq, "dq"), s, h, cu)[rows])
        ref["dq"].append(oracle.dq_rows(qs, ks, vs, gs, w.scale, rows, w.window, w.diag_align,
                                        dlse_of(s, h)))
        # dK, dV of sampled key rows: every q head of the kv head's group
        qh = np.stack([src(pick(w.q, "q"), s, hk * g + j, cu) for j in range(g)])
        gh = np.stack([src(pick(w.dout, "g"), s, hk * g + j, cu) for j in range(g)])
        dlh = np.stack([dlse_of(s, hk * g + j) for j in range(g)]) if dlse else None
        cols = np.unique(np.concatenate([[0, len(ks) - 1], rng.integers(0, len(ks), 6)]))
        rk, rv = oracle.dkdv_cols(qh, ks, vs, gh, w.scale, cols, w.window, w.diag_align, dlh)
        got["dk"].append(src(pick(dk, "dk"), s, hk, cuk)[cols])
        got["dv"].append(src(pick(dv, "dv"), s, hk, cuk)[cols])
        ref["dk"].append(rk)
        ref["dv"].append(rv)
    errs = {n: rel_err(np.concatenate(got[n]), np.concatenate(ref[n])) for n in got}
    say(f"  sampled: max |O err| {worst_o:.2e}, max |LSE err| {worst_l:.2e}, " +
        ", ".join(f"{n} rel err {e:.2e}" for n, e in errs.items()))
    assert worst_o <= O_TOL[w.dtype] and worst_l <= LSE_TOL
    for n, e in errs.items():
        assert e <= G_TOL[w.dtype], f"{n}: {e}"
