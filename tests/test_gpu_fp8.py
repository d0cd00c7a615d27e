"""GPU parity of the FP8 (E4M3) forward against the fp64 oracle (exact attention on the
dequantised inputs, code * descale).

Tolerance, derived from the arithmetic: the kernel rounds P * 256 to E4M3 for the P V
product, within 2^-4 of P relatively in E4M3's normal range and within 2^-18 absolutely
below it, while the row sum uses the unrounded fp32 P and is at least 1 (the row's maximum
has P = 1 exactly).  So per row |O - O_ref| <= max|v| (2^-4 + 2^-18 n) + 2^-8 |O_ref| (the
last term: bf16 output rounding), n = visible keys of the row.  LSE uses no rounded value:
|LSE - LSE_ref| <= 1e-3.  Rows without a visible key must give O = 0 and LSE = -inf exactly.
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


def check_fp8(o_gpu, lse_gpu, o_ref, lse_ref, vmax, nvis, what):
    fin = np.isfinite(lse_ref)
    assert (np.isneginf(lse_gpu) == ~fin).all(), f"{what}: -inf rows differ"
    assert (o_gpu[~fin] == 0).all(), f"{what}: O of an empty row is not 0"
    err = np.abs(o_gpu - o_ref).max(axis=-1)
    tol = vmax * (2.0 ** -4 + 2.0 ** -18 * nvis) + 2.0 ** -8 * np.abs(o_ref).max(axis=-1) + 1e-6
    lse_err = np.abs(lse_gpu[fin] - lse_ref[fin]).max() if fin.any() else 0.0
    say(f"  {what}: max|dO|={err.max():.3e} mean|dO|={np.abs(o_gpu - o_ref).mean():.3e} "
        f"worst err/tol={np.max(err / tol):.3f} max|dLSE|={lse_err:.3e}")
    assert (err <= tol).all(), f"{what}: O beyond the E4M3 bound"
    assert lse_err <= 1e-3, f"{what}: LSE error {lse_err}"


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
    o_ref, lse_ref = oracle.fp8_forward(to_b(q8), to_b(k8), to_b(v8), dq, dk, dv, scale, mask)
    og = synth.f64(synth.to_bhsd(o.cpu(), layout))
    vmax = np.abs(oracle.e4m3_decode(v8.numpy()) * dv).max()
    nvis = np.broadcast_to(mask.sum(axis=1), lse_ref.shape)
    check_fp8(og, synth.f64(lse), o_ref, lse_ref, vmax, nvis, "fwd")


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
    o_ref, lse_ref = oracle.fp8_forward(to_b(coded[0][0]), to_b(coded[1][0]), to_b(coded[2][0]),
                                        coded[0][1], coded[1][1], coded[2][1], 0.1, mask)
    vmax = np.abs(oracle.e4m3_decode(coded[2][0].numpy()) * coded[2][1]).max()
    nvis = np.broadcast_to(mask.sum(axis=1), lse_ref.shape)
    check_fp8(synth.f64(synth.to_bhsd(o.cpu(), "sbhd")), synth.f64(lse), o_ref, lse_ref, vmax, nvis,
              "packed")


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
    vmax = max(np.abs(oracle.e4m3_decode(coded[2][0].numpy()) * coded[2][1]).max(), 1e-30)
    for si, L in enumerate(lens):
        if L == 0:
            continue
        a = cu[si]
        sl = lambda c: c.numpy()[a:a + L].transpose(1, 0, 2)[None]
        mask = oracle.window_mask(L, L, -1, 0)
        o_ref, l_ref = oracle.fp8_forward(sl(coded[0][0]), sl(coded[1][0]), sl(coded[2][0]),
                                          coded[0][1], coded[1][1], coded[2][1], d ** -0.5, mask)
        nvis = np.broadcast_to(mask.sum(axis=1), l_ref.shape)
        check_fp8(og[a:a + L].transpose(1, 0, 2)[None], lg[:, a:a + L][None], o_ref, l_ref, vmax,
                  nvis, f"seq {si} len {L}")


def test_long_sequence_sampled_rows():
    b, s, h, d = 2, 4096, 8, 64
    say(f"case fp8 long B={b} S={s} H={h} D={d}")
    (q8, dq), (k8, dk), (v8, dv) = fp8_inputs(7, b, s, s, h, h, d)
    q, k, v = (t.to(DEV) for t in (q8, k8, v8))
    ds = [torch.tensor([x], dtype=torch.float32, device=DEV) for x in (dq, dk, dv)]
    o, lse = S.forward_fp8(q, k, v, "bshd", 0.125, *ds, window=(-1, 0))
    torch.cuda.synchronize()
    rows = np.array([0, 1, 63, 64, 1000, 2047, 2048, 4000, 4095])
    vmax = np.abs(oracle.e4m3_decode(v8.numpy()) * dv).max()
    for bi, hi in ((0, 0), (1, 5)):
        qq = q8.numpy()[bi, rows, hi][None, None]
        kk = k8.numpy()[bi, :, hi][None, None]
        vv = v8.numpy()[bi, :, hi][None, None]
        mask = oracle.window_mask(s, s, -1, 0)[rows]
        o_ref, l_ref = oracle.fp8_forward(qq, kk, vv, dq, dk, dv, 0.125, mask)
        og = synth.f64(o[bi, rows, hi].cpu())[None, None]
        lg = synth.f64(lse[bi, hi, rows].cpu())[None, None]
        check_fp8(og, lg, o_ref, l_ref, vmax, mask.sum(axis=1)[None, None], f"rows b={bi} h={hi}")
