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

__all__ = [
    "NEG_INF", "window_mask", "attention_forward", "attention_backward", "forward_rows",
    "dq_rows", "dkdv_cols", "merge_forward", "merge_backward", "thd_forward",
    "thd_backward", "windowed_forward", "windowed_backward",
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


def thd_forward(q, k, v, cu_q, cu_k, scale, window=(-1, -1), diag_align=0):
    """Packed varlen forward: every sequence is its own B=1 problem.

    q [T,Hq,D], k,v [Tk,Hk,D]; returns O [T,Hq,D] and LSE [Hq,T].
    """
    q = np.asarray(q, np.float64)
    o = np.zeros(q.shape)
    lse = np.full((q.shape[1], q.shape[0]), NEG_INF)
    for s in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[s]), int(cu_q[s + 1]), int(cu_k[s]), int(cu_k[s + 1])
        if q1 == q0:
            continue
        os_, ls = windowed_forward(_seq(q, q0, q1), _seq(k, k0, k1), _seq(v, k0, k1), scale,
                                   window, diag_align)
        o[q0:q1] = os_[0].transpose(1, 0, 2)
        lse[:, q0:q1] = ls[0]
    return o, lse


def thd_backward(q, k, v, dout, cu_q, cu_k, scale, window=(-1, -1), diag_align=0, dlse=None):
    """Packed varlen backward; dlse [Hq,T] or None.  Returns dQ [T,Hq,D], dK, dV [Tk,Hk,D]."""
    q, k, v, dout = (np.asarray(t, np.float64) for t in (q, k, v, dout))
    dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for s in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[s]), int(cu_q[s + 1]), int(cu_k[s]), int(cu_k[s + 1])
        if q1 == q0 or k1 == k0:
            continue
        dl = None if dlse is None else np.asarray(dlse, np.float64)[:, q0:q1][None]
        a, b, c = windowed_backward(_seq(q, q0, q1), _seq(k, k0, k1), _seq(v, k0, k1),
                                    _seq(dout, q0, q1), scale, window, diag_align, dl)
        dq[q0:q1] = a[0].transpose(1, 0, 2)
        dk[k0:k1] = b[0].transpose(1, 0, 2)
        dv[k0:k1] = c[0].transpose(1, 0, 2)
    return dq, dk, dv
