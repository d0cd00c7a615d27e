"""fp64 CPU oracle: the plain definition of scaled-dot-product attention, its backward
and the LSE merge, used to check the HIP path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or run anything under
``oracle/``.  The product path never reaches it, and it never reaches the product path.

Parity status: every function here is pinned by CPU tests in
``tests/test_oracle_pins.py`` against closed forms, invariants, finite differences and
PyTorch's float64 CPU attention and autograd.  None is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

from .attention import (NEG_INF, attention_backward, attention_forward, dkdv_cols,
                        dq_rows, forward_rows, merge_backward, merge_forward, window_mask)
from .block_mask import block_kinds, block_lists
from .fp8 import e4m3_decode, fp8_forward

__all__ = [
    "NEG_INF", "window_mask", "attention_forward", "attention_backward", "forward_rows",
    "dq_rows", "dkdv_cols", "merge_forward", "merge_backward", "thd_forward",
    "thd_backward", "windowed_forward", "windowed_backward", "block_kinds", "block_lists",
    "masked_forward", "masked_backward", "e4m3_decode", "fp8_forward",
]


def windowed_forward(q, k, v, scale, window=(-1, -1), diag_align=0):
    """Forward over dense [B,H,S,D] arrays with a (left, right) window mask."""
    mask = window_mask(q.shape[2], k.shape[2], window[0], window[1], diag_align)
    return attention_forward(q, k, v, scale, mask)


def windowed_backward(q, k, v, dout, scale, window=(-1, -1), diag_align=0, dlse=None):
    mask = window_mask(q.shape[2], k.shape[2], window[0], window[1], diag_align)
    return attention_backward(q, k, v, dout, scale, mask, dlse)


def _seq(t, lo, hi):
    """[T,H,D] rows lo..hi -> [1,H,L,D]."""
    return np.asarray(t[lo:hi], np.float64).transpose(1, 0, 2)[None]


def _rows(cu, pad, s):
    """Packed rows of sequence s: [pad[s], pad[s] + len) with len from cu (pad None: cu)."""
    lo = int(cu[s]) if pad is None else int(pad[s])
    return lo, lo + int(cu[s + 1]) - int(cu[s])


def thd_forward(q, k, v, cu_q, cu_k, scale, window=(-1, -1), diag_align=0, pad_q=None,
                pad_k=None):
    """Packed varlen forward: every sequence is its own B=1 problem.

    q [T,Hq,D], k,v [Tk,Hk,D]; returns O [T,Hq,D] and LSE [Hq,T].  With pad_q / pad_k
    ("Add support for cuDNN FusedAttention + THD + CP", TransformerEngine issue 885:
    cu_seqlens_padded) sequence s starts at packed row pad[s] and the rows after its end are
    padding: they are not keys, and their O / LSE entries are NaN here (never written).
    """
    q = np.asarray(q, np.float64)
    padded = pad_q is not None or pad_k is not None
    o = np.full(q.shape, np.nan) if padded else np.zeros(q.shape)
    lse = np.full((q.shape[1], q.shape[0]), np.nan if padded else NEG_INF)
    for s in range(len(cu_q) - 1):
        q0, q1 = _rows(cu_q, pad_q, s)
        k0, k1 = _rows(cu_k, pad_k, s)
        if q1 == q0:
            continue
        os_, ls = windowed_forward(_seq(q, q0, q1), _seq(k, k0, k1), _seq(v, k0, k1), scale,
                                   window, diag_align)
        o[q0:q1] = os_[0].transpose(1, 0, 2)
        lse[:, q0:q1] = ls[0]
    return o, lse


def thd_backward(q, k, v, dout, cu_q, cu_k, scale, window=(-1, -1), diag_align=0, dlse=None,
                 pad_q=None, pad_k=None):
    """Packed varlen backward; dlse [Hq,T] or None.  Returns dQ [T,Hq,D], dK, dV [Tk,Hk,D]
    (padding rows NaN when pad_q / pad_k are given)."""
    q, k, v, dout = (np.asarray(t, np.float64) for t in (q, k, v, dout))
    padded = pad_q is not None or pad_k is not None
    fill = np.nan if padded else 0.0
    dq, dk, dv = np.full(q.shape, fill), np.full(k.shape, fill), np.full(v.shape, fill)
    for s in range(len(cu_q) - 1):
        q0, q1 = _rows(cu_q, pad_q, s)
        k0, k1 = _rows(cu_k, pad_k, s)
        if padded:
            dq[q0:q1], dk[k0:k1], dv[k0:k1] = 0.0, 0.0, 0.0
        if q1 == q0 or k1 == k0:
            continue
        dl = None if dlse is None else np.asarray(dlse, np.float64)[:, q0:q1][None]
        a, b, c = windowed_backward(_seq(q, q0, q1), _seq(k, k0, k1), _seq(v, k0, k1),
                                    _seq(dout, q0, q1), scale, window, diag_align, dl)
        dq[q0:q1] = a[0].transpose(1, 0, 2)
        dk[k0:k1] = b[0].transpose(1, 0, 2)
        dv[k0:k1] = c[0].transpose(1, 0, 2)
    return dq, dk, dv


def masked_forward(q, k, v, scale, mask, window=(-1, -1), diag_align=0):
    """Forward with an element mask (boolean, broadcastable to [B,Hq,Sq,Sk]) ANDed with the
    (left, right) window: the block-sparse path's result (the block table only decides
    which blocks need the element test, never which pairs are visible)."""
    wm = window_mask(q.shape[2], k.shape[2], window[0], window[1], diag_align)
    return attention_forward(q, k, v, scale, np.asarray(mask, bool) & wm)


def masked_backward(q, k, v, dout, scale, mask, window=(-1, -1), diag_align=0, dlse=None):
    wm = window_mask(q.shape[2], k.shape[2], window[0], window[1], diag_align)
    return attention_backward(q, k, v, dout, scale, np.asarray(mask, bool) & wm, dlse)
