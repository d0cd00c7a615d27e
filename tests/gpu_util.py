"""Helpers for the GPU parity tests: move seeded inputs to the device, call the HIP path
through the C-ABI binding, and compare with the fp64 oracle.

Tolerances (stated for this method): forward max |O - O_ref| <= 4e-3 (fp16), 3e-2 (bf16),
1e-5 (fp32); |LSE - LSE_ref| <= 1e-3 on rows with a visible key, and rows without one must
be exactly (O = 0, LSE = -inf); gradients max |g - g_ref| / max |g_ref| <= 1e-2 (16-bit)
and 1e-4 (fp32).
"""
import sys

import numpy as np
import torch

import oracle
import scaled_dot_product_05_amd as S
import synth

O_TOL = {"f16": 4e-3, "bf16": 3e-2, "f32": 1e-5}
LSE_TOL = 1e-3
G_TOL = {"f16": 1e-2, "bf16": 1e-2, "f32": 1e-4}

DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(w: synth.Workload):
    """Device copies of q, k, v (packed views stay views of one device buffer)."""
    if "packed" in w.extra:
        buf = w.extra["packed"].to(DEV)
        q, k, v = buf.split([w.heads_q, w.heads_kv, w.heads_kv], dim=2)
        return q, k, v
    return w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)


def cu_dev(w):
    if not w.is_thd:
        return None, None
    cq = torch.from_numpy(w.cu_seqlens_q).to(DEV)
    ck = cq if w.cu_seqlens_k is w.cu_seqlens_q else torch.from_numpy(w.cu_seqlens_k).to(DEV)
    return cq, ck


def gpu_forward(w, q, k, v, cq=None, ck=None, out=None, lse=None):
    return S.forward(q, k, v, w.layout, w.scale, w.window, w.diag_align, cq, ck,
                     w.seqlen_q if w.is_thd else None, w.seqlen_k if w.is_thd else None,
                     out=out, lse=lse)


def gpu_backward(w, q, k, v, o, lse, dout, dlse=None, cq=None, ck=None, **kw):
    return S.backward(q, k, v, o, lse, dout, w.layout, w.scale, w.window, w.diag_align, dlse, cq,
                      ck, w.seqlen_q if w.is_thd else None, w.seqlen_k if w.is_thd else None, **kw)


def bhsd64(t, layout):
    return synth.f64(synth.to_bhsd(t.cpu(), layout))


def oracle_forward(w):
    if w.is_thd:
        return oracle.thd_forward(synth.f64(w.q), synth.f64(w.k), synth.f64(w.v), w.cu_seqlens_q,
                                  w.cu_seqlens_k, w.scale, w.window, w.diag_align)
    q, k, v = (bhsd64(t, w.layout) for t in (w.q, w.k, w.v))
    return oracle.windowed_forward(q, k, v, w.scale, w.window, w.diag_align)


def oracle_backward(w, dlse=None):
    if w.is_thd:
        return oracle.thd_backward(synth.f64(w.q), synth.f64(w.k), synth.f64(w.v),
                                   synth.f64(w.dout), w.cu_seqlens_q, w.cu_seqlens_k, w.scale,
                                   w.window, w.diag_align, dlse)
    q, k, v, g = (bhsd64(t, w.layout) for t in (w.q, w.k, w.v, w.dout))
    return oracle.windowed_backward(q, k, v, g, w.scale, w.window, w.diag_align, dlse)


def gpu_bhsd(t, w):
    """GPU result (in w's layout) as fp64 [B,H,S,D] (or [T,H,D] for THD)."""
    if w.is_thd:
        return synth.f64(t)
    return synth.f64(synth.to_bhsd(t.cpu(), w.layout))


def check_forward(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    o_err = np.abs(o_gpu - o_ref).max() if o_ref.size else 0.0
    fin = np.isfinite(lse_ref)
    assert (np.isneginf(lse_gpu) == ~fin).all(), f"{what}: -inf rows differ"
    lse_err = np.abs(lse_gpu[fin] - lse_ref[fin]).max() if fin.any() else 0.0
    empty = ~fin
    if empty.any():
        # rows without a visible key: O must be exactly zero
        if o_gpu.ndim == 4:  # [B,H,S,D], lse [B,H,S]
            assert (o_gpu[empty] == 0).all(), f"{what}: O of an empty row is not 0"
        else:  # THD: O [T,H,D], lse [H,T]
            assert (o_gpu.transpose(1, 0, 2)[empty] == 0).all(), f"{what}: O of an empty row is not 0"
    say(f"  {what}: max|dO|={o_err:.3e} (tol {O_TOL[dtype]:.0e}) max|dLSE|={lse_err:.3e}")
    assert o_err <= O_TOL[dtype], f"{what}: O error {o_err}"
    assert lse_err <= LSE_TOL, f"{what}: LSE error {lse_err}"


def rel_err(g, r, floor=0.0):
    m = max(np.abs(r).max() if r.size else 0.0, floor)
    return np.abs(g - r).max() / (m if m > 0 else 1.0) if r.size else 0.0


GRAD_NAMES = ("dq", "dk", "dv")


def check_grads(grads, refs, dtype, what="", zero_exact=()):
    """max |g - g_ref| / max |g_ref| <= G_TOL for each of dQ, dK, dV, each normalised by its
    own max.  ``zero_exact`` names the gradients a test declares zero in exact arithmetic
    (e.g. dQ and dK with a single key: P = 1 and dP = Delta, so dS = 0); only rounding
    noise is left there, and only those are normalised by 1e-2 of the largest of the
    three instead."""
    big = max(np.abs(r).max() if r.size else 0.0 for r in refs)
    errs = [rel_err(g, r, 1e-2 * big if n in zero_exact else 0.0)
            for n, g, r in zip(GRAD_NAMES, grads, refs)]
    say(f"  {what}: rel err dq={errs[0]:.3e} dk={errs[1]:.3e} dv={errs[2]:.3e} (tol {G_TOL[dtype]:.0e})"
        + (f" zero in exact arithmetic: {','.join(zero_exact)}" if zero_exact else ""))
    for name, e in zip(GRAD_NAMES, errs):
        assert e <= G_TOL[dtype], f"{what}: {name} error {e}"
