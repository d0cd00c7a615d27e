"""The long-sequence causal cases at full size (bf16, BSHD, scale 1/sqrt(D)): every shape the
benchmark times, (B, S) = (8, 4096), (4, 8192), (2, 16384) at H8 D64 and B8 S4096 at H16 D128
with 16 or 4 kv heads, in the launch configuration the benchmark uses: the full O and LSE (and dQ, dK, dV) come from the
HIP path, and sampled rows (tile edges, first and last rows, random rows of several heads)
are checked against the fp64 oracle one row at a time; sampled dK/dV rows (key rows) are
checked against the oracle's sums over every query row of the kv head's group."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, G_TOL, LSE_TOL, O_TOL, gpu_backward, gpu_forward, rel_err, say

pytestmark = pytest.mark.gpu


def _rows(s, rng):
    edge = [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 257, 511, 512, s // 2, s - 257, s - 256,
            s - 129, s - 128, s - 2, s - 1]
    return np.unique(np.concatenate([edge, rng.integers(0, s, 12)]))


SHAPES = [(8, 4096, 8, 8, 64), (4, 8192, 8, 8, 64), (2, 16384, 8, 8, 64), (8, 4096, 16, 16, 128),
          (8, 4096, 16, 4, 128)]


@pytest.mark.parametrize("b,s,h,hk,d", SHAPES)
def test_target_causal_sampled_rows(b, s, h, hk, d):
    w = synth.target(seed=3, b=b, s=s, h=h, hk=hk, d=d)
    say(f"case target B{w.batch} S{w.seqlen_q} H{h}/{hk} D{d}")
    q, k, v = (t.to(DEV) for t in (w.q, w.k, w.v))
    o, lse = gpu_forward(w, q, k, v)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    rng = np.random.default_rng(11)
    group = h // hk
    worst_o = worst_l = 0.0
    for b, hh in [(0, 0), (min(3, w.batch - 1), h - 1), (w.batch - 1, h // 2 + 1)]:
        rows = _rows(w.seqlen_q, rng)
        qb = synth.f64(w.q[b, :, hh])
        kg, vg = synth.f64(w.k[b, :, hh // group]), synth.f64(w.v[b, :, hh // group])
        ro, rl = oracle.forward_rows(qb, kg, vg, w.scale, rows, w.window)
        worst_o = max(worst_o, float(np.abs(synth.f64(o[b, rows, hh]) - ro).max()))
        worst_l = max(worst_l, float(np.abs(synth.f64(lse[b, hh, rows]) - rl).max()))
    say(f"  sampled rows: max |O err| {worst_o:.2e}, max |LSE err| {worst_l:.2e}")
    assert worst_o <= O_TOL["bf16"] and worst_l <= LSE_TOL


@pytest.mark.parametrize("b,s,h,hk,d", SHAPES)
def test_target_backward_sampled(b, s, h, hk, d):
    w = synth.target(seed=4, b=b, s=s, h=h, hk=hk, d=d, with_grad=True)
    say(f"case target backward B{w.batch} S{w.seqlen_q} H{h}/{hk} D{d}")
    q, k, v, g = (t.to(DEV) for t in (w.q, w.k, w.v, w.dout))
    o, lse = gpu_forward(w, q, k, v)
    dq, dk, dv = gpu_backward(w, q, k, v, o, lse, g)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    rng = np.random.default_rng(12)
    group = h // hk
    got = {"dq": [], "dk": [], "dv": []}
    ref = {"dq": [], "dk": [], "dv": []}
    for b, kh in [(min(1, w.batch - 1), 0), (max(w.batch - 2, 0), hk - 1)]:
        heads = list(range(kh * group, (kh + 1) * group))
        kg, vg = synth.f64(w.k[b, :, kh]), synth.f64(w.v[b, :, kh])
        qh = np.stack([synth.f64(w.q[b, :, hh]) for hh in heads])
        gh = np.stack([synth.f64(w.dout[b, :, hh]) for hh in heads])
        rows = _rows(w.seqlen_q, rng)
        for i, hh in enumerate(heads[:2]):
            got["dq"].append(synth.f64(dq[b, rows, hh]))
            ref["dq"].append(oracle.dq_rows(qh[i], kg, vg, gh[i], w.scale, rows, w.window))
        cols = _rows(w.seqlen_k, rng)
        rk, rv = oracle.dkdv_cols(qh, kg, vg, gh, w.scale, cols, w.window)
        got["dk"].append(synth.f64(dk[b, cols, kh]))
        got["dv"].append(synth.f64(dv[b, cols, kh]))
        ref["dk"].append(rk)
        ref["dv"].append(rv)
    errs = {n: rel_err(np.concatenate(got[n]), np.concatenate(ref[n])) for n in got}
    say("  sampled: " + ", ".join(f"{n} rel err {e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= G_TOL["bf16"], f"{n}: {e}"


# Grids above 12 fused-launch blocks per CU (of 256) take the two four-wave launches (dQ,
# which also forms Delta from dLSE, then dK/dV); ragged S, windows and a given dLSE.
TWO_LAUNCH = [(5, 3000, 8, 8, 64, (512, 0)), (4, 3000, 16, 4, 128, (-1, 0)),
              (3, 3000, 16, 16, 128, (300, 20))]


@pytest.mark.parametrize("b,s,h,hk,d,window", TWO_LAUNCH)
def test_two_launch_backward_sampled(b, s, h, hk, d, window):
    import scaled_dot_product_05_amd as S
    w = synth.dense(5, 960, "bf16", "bshd", b, s, s, h, hk, d, d ** -0.5, window, 0,
                    with_grad=True, with_dlse=True, name="two_launch")
    say(f"case two-launch backward B{b} S{s} H{h}/{hk} D{d} window {window}")
    q, k, v, g, dl = (t.to(DEV) for t in (w.q, w.k, w.v, w.dout, w.dlse))
    o, lse = gpu_forward(w, q, k, v)
    torch.cuda.synchronize()
    S.sdpa_profile_enable(True)
    dq, dk, dv = gpu_backward(w, q, k, v, o, lse, g, dlse=dl)
    torch.cuda.synchronize()
    S.sdpa_profile_enable(False)
    launched = set(S.sdpa_profile_read())
    assert {"bwd_dq", "bwd_dkdv"} <= launched and "bwd_pre" not in launched, launched
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    rng = np.random.default_rng(13)
    group = h // hk
    got = {"dq": [], "dk": [], "dv": []}
    ref = {"dq": [], "dk": [], "dv": []}
    for bb, kh in [(0, 0), (b - 1, hk - 1)]:
        heads = list(range(kh * group, (kh + 1) * group))
        kg, vg = synth.f64(w.k[bb, :, kh]), synth.f64(w.v[bb, :, kh])
        qh = np.stack([synth.f64(w.q[bb, :, hh]) for hh in heads])
        gh = np.stack([synth.f64(w.dout[bb, :, hh]) for hh in heads])
        dlh = np.stack([synth.f64(w.dlse[bb, hh]) for hh in heads])
        rows = _rows(s, rng)
        for i, hh in enumerate(heads[:2]):
            got["dq"].append(synth.f64(dq[bb, rows, hh]))
            ref["dq"].append(oracle.dq_rows(qh[i], kg, vg, gh[i], w.scale, rows, window, 0, dlh[i]))
        cols = _rows(s, rng)
        rk, rv = oracle.dkdv_cols(qh, kg, vg, gh, w.scale, cols, window, 0, dlh)
        got["dk"].append(synth.f64(dk[bb, cols, kh]))
        got["dv"].append(synth.f64(dv[bb, cols, kh]))
        ref["dk"].append(rk)
        ref["dv"].append(rv)
    errs = {n: rel_err(np.concatenate(got[n]), np.concatenate(ref[n])) for n in got}
    say("  sampled: " + ", ".join(f"{n} rel err {e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= G_TOL["bf16"], f"{n}: {e}"
