"""FP8 (E4M3) forward: exact attention on the dequantised inputs.  TEST INFRASTRUCTURE
ONLY (see the package docstring).

"[PyTorch] fused CUDNN attention kernel not properly handling strides" (TransformerEngine
issue 1195) passes an FP8 recipe, ``DelayedScaling``, to its fused attention call.  In that
recipe a tensor is stored as 8-bit codes with one fp32 scale per tensor; its value is
code * descale.  The pages give no more (R22 in the design notes takes per-tensor descales
and the OCP E4M3 format); what the method computes on such inputs is plain attention on
the dequantised values, which this module writes out.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_forward


def e4m3_decode(codes) -> np.ndarray:
    """fp64 values of E4M3 codes: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
    exponent 0 holds subnormals m * 2^-9; S.1111.111 is NaN; there is no infinity."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.power(2.0, e - 7)
    sub = m * 2.0 ** -9
    val = sign * np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def fp8_forward(q8, k8, v8, descale_q, descale_k, descale_v, scale, mask=None,
                return_p=False):
    """O, LSE of attention on q8 * descale_q, k8 * descale_k, v8 * descale_v (E4M3 codes,
    [B,H,S,D]); ``mask`` as in attention_forward; with ``return_p`` also the softmax
    weights P [B,Hq,Sq,Sk]."""
    q = e4m3_decode(q8) * float(descale_q)
    k = e4m3_decode(k8) * float(descale_k)
    v = e4m3_decode(v8) * float(descale_v)
    return attention_forward(q, k, v, scale, mask, return_p=return_p)
