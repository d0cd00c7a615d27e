"""GPU parity of the FP8 (E4M3) forward against the fp64 oracle (exact attention on the
dequantised inputs, code * descale).

Tolerance, derived from the arithmetic.  The kernel rounds P * 256 to E4M3 for the P V
product (P taken against the running row max, so P <= 1): within 2^-4 of P relatively in
E4M3's normal range and within 2^-18 absolutely below it.  The row sum uses the unrounded
fp32 P and is at least 1, and a later rescale only shrinks an error.  So, with the
oracle's normalised weights p_j and the dequantised values v_j, every element obeys

    |O_d - O_ref_d| <= 2^-4 sum_j p_j |v_jd| + 2^-18 sum_j |v_jd| + 2^-8 |O_d|

(the last term: the bf16 output rounding; sums over the row's visible keys).  A bound that
large still admits an all-zero O on long rows, so the error's size is also checked against
the rounding model: RNE to 3 mantissa bits leaves a relative error with E[e^2] <= 2^-8 / 3,
independent between keys, so E[(O_d - O_ref_d)^2] <= sum_j (2^-8/3 p_j^2 + 2^-36/3) v_jd^2
+ 2^-16/3 O_ref_d^2.  The measured mean square over a case must stay within 1.5^2 of the
predicted one.  LSE uses no rounded value: |LSE - LSE_ref| <= 1e-3.  Rows without a
visible key must give O = 0 and LSE = -inf exactly.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_05_amd as S
import synth
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def fp8_inputs(seed, b, sq, sk, hq, hk, d, layout="bshd"):
    shp = {"bshd": lambda s, h: (b, s, h, d), "sbhd": lambda s, h: (s, b, h, d),
           "bhsd": lambda s, h: (b, h, s, d)}[layout]
    out = []
    for i, (s, h) in enumerate(((sq, hq), (sk, hk), (sk, hk))):
        codes, descale = synth.e4m3_codes(synth.normal(seed, 90, i, shp(s, h)))
        out.append((codes, descale))
    return out


def _expand_heads(v, hq):
    return np.repeat(v, hq // v.shape[1], axis=1)


def check_fp8(o_gpu, lse_gpu, o_ref, lse_ref, p_ref, v_deq, what):
    """o [B,Hq,Sq,D], lse [B,Hq,Sq], p_ref [B,Hq,Sq,Sk] (the oracle's weights), v_deq
    [B,Hk,Sk,D] dequantised values."""
    fin = np.isfinite(lse_ref)
    assert (np.isneginf(lse_gpu) == ~fin).all(), f"{what}: -inf rows differ"
    assert (o_gpu[~fin] == 0).all(), f"{what}: O of an empty row is not 0"
    va = _expand_heads(np.abs(v_deq), o_ref.shape[1])
    vis = p_ref > 0
    wsum = p_ref @ va                      # sum_j p_j |v_jd|
    asum = vis.astype(np.float64) @ va     # sum_j |v_jd| over keys with p_j > 0
    err = np.abs(o_gpu - o_ref)
    tol = 2.0 ** -4 * wsum + 2.0 ** -18 * asum + 2.0 ** -8 * np.abs(o_gpu) + 1e-7
    pred_ms = ((2.0 ** -8 / 3) * (p_ref ** 2) @ (va ** 2) + (2.0 ** -36 / 3) * (vis @ (va ** 2))
               + (2.0 ** -16 / 3) * o_ref ** 2).mean()
    meas_ms = (err ** 2).mean()
    lse_err = np.abs(lse_gpu[fin] - lse_ref[fin]).max() if fin.any() else 0.0
    say(f"  {what}: max|dO|={err.max():.3e} rms|dO|={math.sqrt(meas_ms):.3e} "
        f"(model {math.sqrt(pred_ms):.3e}) worst err/tol={np.max(err / tol):.3f} "
        f"max|dLSE|={lse_err:.3e}")
    assert (err <= tol).all(), f"{what}: O beyond the per-element E4M3 bound"
    assert meas_ms <= 1.5 ** 2 * pred_ms + 1e-30, f"{what}: O error above the rounding model"
    assert lse_err <= 1e-3, f"{what}: LSE error {lse_err}"


def dequant(codes, descale):
    return oracle.e4m3_decode(codes) * descale


def run_fp8(seed, b, sq, sk, hq, hk, d, scale, window=(-1, -1), align=0, layout="bshd", what=""):
    say(f"case fp8 {what} {layout} B={b} Sq={sq} Sk={sk} Hq={hq} Hk={hk} D={d} scale={scale} "
        f"win={window} al={align}")
    (q8, dq), (k8, dk), (v8, dv) = fp8_inputs(seed, b, sq, sk, hq, hk, d, layout)
    q, k, v = (t.to(DEV) for t in (q8, k8, v8))
    ds = [torch.tensor([x], dtype=torch.float32, device=DEV) for x in (dq, dk, dv)]
    o, lse = S.forward_fp8(q, k, v, layout, scale, *ds, window=window,
                           diag_align="bottom_right" if align else "top_left")
    torch.cuda.synchronize()
    to_b = lambda t: synth.to_bhsd(t, layout).numpy()
    mask = oracle.window_mask(sq, sk, window[0], window[1], align)
    o_ref, lse_ref, p_ref = oracle.fp8_forward(to_b(q8), to_b(k8), to_b(v8), dq, dk, dv, scale,
                                               mask, return_p=True)
    og = synth.f64(synth.to_bhsd(o.cpu(), layout))
    check_fp8(og, synth.f64(lse), o_ref, lse_ref, p_ref, dequant(to_b(v8), dv), "fwd")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("window,align", [((-1, 0), 0), ((-1, -1), 0), ((3, 2), 0), ((-1, 0), 1),
                                          ((40, 0), 1), ((-1, -129), 0)])
def test_windows_ragged_gqa(d, window, align):
    run_fp8(1, 2, 300, 333, 4, 2, d, d ** -0.5, window, align)


@pytest.mark.parametrize("layout", ["bshd", "sbhd", "bhsd"])
def test_layouts(layout):
    run_fp8(2, 2, 257, 257, 8, 1, 64, 0.125, (-1, 0), 0, layout)


@pytest.mark.parametrize("scale", [1.0, 0.1, -0.125])
def test_scales_including_negative(scale):
    run_fp8(3, 1, 200, 200, 2, 2, 64, scale, (-1, 0))


def test_fully_masked_rows():
    # window (-1, -129): the first 129 rows see no key
    run_fp8(4, 1, 300, 300, 2, 2, 64, 0.125, (-1, -129))


def test_packed_qkv_views_issue_1195_shape():
    # TransformerEngine issue 1195's [2048, 1, 18, 64] tensor, here as E4M3 codes: q, k, v are
    # views (strides 1152, 1152, 64, 1) of one buffer with one descale each
    say("case fp8 packed sbhd [2048,1,18,64]")
    x = synth.normal(5, 91, 0, (2048, 1, 18, 64))
    parts = [x[:, :, :16], x[:, :, 16:17], x[:, :, 17:18]]
    coded = [synth.e4m3_codes(t) for t in parts]
    buf = torch.cat([c for c, _ in coded], dim=2).to(DEV)
    q, k, v = buf.split([16, 1, 1], dim=2)
    assert q.stride() == (1152, 1152, 64, 1)
    ds = [torch.tensor([s], dtype=torch.float32, device=DEV) for _, s in coded]
    o, lse = S.forward_fp8(q, k, v, "sbhd", 0.1, *ds, window=(-1, 0))
    torch.cuda.synchronize()
    to_b = lambda t: synth.to_bhsd(t, "sbhd").numpy()
    mask = oracle.window_mask(2048, 2048, -1, 0)
    o_ref, lse_ref, p_ref = oracle.fp8_forward(to_b(coded[0][0]), to_b(coded[1][0]),
                                               to_b(coded[2][0]), coded[0][1], coded[1][1],
                                               coded[2][1], 0.1, mask, return_p=True)
    check_fp8(synth.f64(synth.to_bhsd(o.cpu(), "sbhd")), synth.f64(lse), o_ref, lse_ref, p_ref,
              dequant(to_b(coded[2][0]), coded[2][1]), "packed")


def test_thd_varlen():
    lens = [0, 1, 130, 257, 64]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    t, h, d = int(cu[-1]), 4, 128
    say(f"case fp8 thd lengths {lens}")
    coded = [synth.e4m3_codes(synth.normal(6, 92, i, (t, h, d))) for i in range(3)]
    q, k, v = (c.to(DEV) for c, _ in coded)
    ds = [torch.tensor([s], dtype=torch.float32, device=DEV) for _, s in coded]
    cud = torch.from_numpy(cu).to(DEV)
    o, lse = S.forward_fp8(q, k, v, "thd", d ** -0.5, *ds, window=(-1, 0), cu_seqlens_q=cud,
                           max_seqlen_q=max(lens))
    torch.cuda.synchronize()
    og, lg = synth.f64(o.cpu()), synth.f64(lse.cpu())
    for si, L in enumerate(lens):
        if L == 0:
            continue
        a = cu[si]
        sl = lambda c: c.numpy()[a:a + L].transpose(1, 0, 2)[None]
        mask = oracle.window_mask(L, L, -1, 0)
        o_ref, l_ref, p_ref = oracle.fp8_forward(sl(coded[0][0]), sl(coded[1][0]),
                                                 sl(coded[2][0]), coded[0][1], coded[1][1],
                                                 coded[2][1], d ** -0.5, mask, return_p=True)
        check_fp8(og[a:a + L].transpose(1, 0, 2)[None], lg[:, a:a + L][None], o_ref, l_ref,
                  p_ref, dequant(sl(coded[2][0]), coded[2][1]), f"seq {si} len {L}")


def long_rows_case(seed, b, s, h, d, heads, what):
    say(f"case fp8 long {what} B={b} S={s} H={h} D={d}")
    (q8, dq), (k8, dk), (v8, dv) = fp8_inputs(seed, b, s, s, h, h, d)
    q, k, v = (t.to(DEV) for t in (q8, k8, v8))
    ds = [torch.tensor([x], dtype=torch.float32, device=DEV) for x in (dq, dk, dv)]
    o, lse = S.forward_fp8(q, k, v, "bshd", d ** -0.5, *ds, window=(-1, 0))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, s // 2 - 1, s // 2, s - 129, s - 2,
                                      s - 1], np.random.default_rng(seed).integers(0, s, 24)]))
    for bi, hi in heads:
        qq = q8.numpy()[bi, rows, hi][None, None]
        kk = k8.numpy()[bi, :, hi][None, None]
        vv = v8.numpy()[bi, :, hi][None, None]
        mask = oracle.window_mask(s, s, -1, 0)[rows]
        o_ref, l_ref, p_ref = oracle.fp8_forward(qq, kk, vv, dq, dk, dv, d ** -0.5, mask,
                                                 return_p=True)
        og = synth.f64(o[bi, rows, hi].cpu())[None, None]
        lg = synth.f64(lse[bi, hi, rows].cpu())[None, None]
        check_fp8(og, lg, o_ref, l_ref, p_ref, dequant(vv, dv), f"rows b={bi} h={hi}")


def test_long_sequence_sampled_rows():
    long_rows_case(7, 2, 4096, 8, 64, ((0, 0), (1, 5)), "S4096")


@pytest.mark.parametrize("b,s,h,d", [(2, 16384, 8, 64), (8, 4096, 16, 128)])
def test_benchmarked_shapes_sampled_rows(b, s, h, d):
    # the causal FP8 shapes the benchmark times, in its launch configuration (BSHD
    # contiguous, scale 1/sqrt(D)); sampled rows of the first and last (batch, head)
    long_rows_case(8, b, s, h, d, ((0, 0), (b - 1, h - 1)), "bench shape")
