"""fp64 CPU oracle for fused scaled-dot-product attention, its backward and the LSE merge.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  It shares no code
with the HIP path and imports nothing from it.

Everything here is the plain definition, in float64, with the full score matrix
materialised for each (batch, q-head).  numpy's matmul is the only library primitive;
there is no tiling, no online softmax, no fusion.

Definitions followed (page titles as printed on the pages):

* Forward: O = softmax(scale * Q K^T + mask) V and the per-row log-sum-exp
  LSE_i = log sum_j exp(s_ij) over the visible keys (natural log, scores include the
  scale) - "Significant Accuracy Difference between Compiled and Eager Flex Attention"
  (PyTorch issue 135161), the ``return_lse=True`` calls of its second repro and the
  ``merge_attn`` helper, which only agrees with a natural-log LSE.
* Masks: window (left, right) with -1 = unbounded; key j is visible to query i iff
  -left <= j - (i + off) <= right, off = 0 (top-left) or Sk - Sq (bottom-right);
  (-1, 0) is causal - TransformerEngine issue 1195 ("fused CUDNN attention kernel not
  properly handling strides"), first repro ``window_size=(-1, 0)``; the sliding-window
  predicate of issue 135161 (q >= kv and q - kv <= 128) is window (128, 0).
* Rows with no visible key: O = 0, LSE = -inf, no gradient.  Issue 135161's table of
  exact zeros for attn_v1 vs attn_v2 (eager) only holds when such a partial merges as
  the identity.
* GQA/MQA: q head h reads kv head floor(h / G), G = Hq / Hk (issue 1195, second repro,
  ``num_gqa_groups``).
* Backward (gradient of a loss through O and LSE):
  Delta_i = sum_d dO_id O_id;  dP = dO V^T;  dS_ij = P_ij (dP_ij - Delta_i + dLSE_i);
  dQ = scale dS K;  dK = scale dS^T Q;  dV = P^T dO;  dK, dV summed over the q heads of
  a group.  (d LSE_i / d s_ij = P_ij gives the dLSE term.)
* Merge (issue 135161, ``merge_attn``): m = max(lse_a, lse_b); w = exp(lse - m);
  x = (x_a w_a + x_b w_b) / (w_a + w_b); lse = m + log(w_a + w_b).  Two -inf rows give
  (0, -inf).  Its backward with alpha = exp(lse_a - lse), beta = exp(lse_b - lse):
  dx_a = alpha g, dx_b = beta g, dlse_a = alpha (sum_d g (x_a - x) + g_lse),
  dlse_b = beta (sum_d g (x_b - x) + g_lse).  The max is gradient-neutral.

Arrays are dense fp64: q [B,Hq,Sq,D], k and v [B,Hk,Sk,D], LSE [B,Hq,Sq].
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------------------------------
# masks
# ---------------------------------------------------------------------------------------

def window_mask(sq: int, sk: int, window_left: int = -1, window_right: int = -1,
                diag_align: int = 0, rows=None) -> np.ndarray:
    """Boolean [Sq,Sk] (or [len(rows),Sk]) visibility of key j to query i."""
    i = np.arange(sq) if rows is None else np.asarray(rows)
    off = 0 if diag_align == 0 else sk - sq
    rel = np.arange(sk)[None, :] - (i[:, None] + off)
    vis = np.ones(rel.shape, dtype=bool)
    if window_left != -1:
        vis &= rel >= -window_left
    if window_right != -1:
        vis &= rel <= window_right
    return vis


# ---------------------------------------------------------------------------------------
# attention forward / backward for one (batch, q-head)
# ---------------------------------------------------------------------------------------

def _rows_forward(q_rows, k, v, scale, vis, bias=None):
    """Forward for a set of query rows against all keys of one kv head.

    q_rows [n,D], k,v [Sk,D], vis bool [n,Sk], bias optional additive fp64 [n,Sk].
    Returns O [n,D], LSE [n], P [n,Sk].
    """
    s = scale * (q_rows @ k.T)
    if bias is not None:
        s = s + bias
    s = np.where(vis, s, NEG_INF)
    any_visible = vis.any(axis=1)
    m = np.where(any_visible, s.max(axis=1, initial=NEG_INF), 0.0)
    e = np.where(vis, np.exp(s - m[:, None]), 0.0)
    l = e.sum(axis=1)
    p = np.where(any_visible[:, None], e / np.where(any_visible, l, 1.0)[:, None], 0.0)
    o = p @ v
    lse = np.where(any_visible, m + np.log(np.where(any_visible, l, 1.0)), NEG_INF)
    return o, lse, p


def _group(hq: int, hk: int) -> int:
    if hk <= 0 or hq % hk:
        raise ValueError(f"heads_q={hq} is not a multiple of heads_kv={hk}")
    return hq // hk


def attention_forward(q, k, v, scale, mask=None, bias=None, return_p=False):
    """O [B,Hq,Sq,D], LSE [B,Hq,Sq] (and P [B,Hq,Sq,Sk] if asked).

    ``mask`` is a boolean array broadcastable to [B,Hq,Sq,Sk] (None = all visible);
    ``bias`` an optional additive score term of the same broadcast shape.
    """
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    b, hq, sq, d = q.shape
    hk, sk = k.shape[1], k.shape[2]
    g = _group(hq, hk)
    vis_all = np.broadcast_to(np.ones((1, 1, 1, 1), bool) if mask is None else mask,
                              (b, hq, sq, sk))
    bias_all = None if bias is None else np.broadcast_to(bias, (b, hq, sq, sk))
    o = np.zeros((b, hq, sq, d))
    lse = np.zeros((b, hq, sq))
    p_all = np.zeros((b, hq, sq, sk)) if return_p else None
    for bi in range(b):
        for h in range(hq):
            kv = h // g
            o[bi, h], lse[bi, h], p = _rows_forward(
                q[bi, h], k[bi, kv], v[bi, kv], scale, vis_all[bi, h],
                None if bias_all is None else bias_all[bi, h])
            if return_p:
                p_all[bi, h] = p
    return (o, lse, p_all) if return_p else (o, lse)


def attention_backward(q, k, v, dout, scale, mask=None, dlse=None, bias=None):
    """dQ, dK, dV of a loss L with dL/dO = dout and dL/dLSE = dlse (None = 0)."""
    q, k, v, dout = (np.asarray(t, dtype=np.float64) for t in (q, k, v, dout))
    b, hq, sq, d = q.shape
    hk, sk = k.shape[1], k.shape[2]
    g = _group(hq, hk)
    vis_all = np.broadcast_to(np.ones((1, 1, 1, 1), bool) if mask is None else mask,
                              (b, hq, sq, sk))
    bias_all = None if bias is None else np.broadcast_to(bias, (b, hq, sq, sk))
    dlse = np.zeros((b, hq, sq)) if dlse is None else np.asarray(dlse, dtype=np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for bi in range(b):
        for h in range(hq):
            kv = h // g
            o, _, p = _rows_forward(q[bi, h], k[bi, kv], v[bi, kv], scale, vis_all[bi, h],
                                    None if bias_all is None else bias_all[bi, h])
            delta = (dout[bi, h] * o).sum(axis=1)
            dp = dout[bi, h] @ v[bi, kv].T
            ds = p * (dp - delta[:, None] + dlse[bi, h][:, None])
            dq[bi, h] = scale * (ds @ k[bi, kv])
            dk[bi, kv] += scale * (ds.T @ q[bi, h])
            dv[bi, kv] += p.T @ dout[bi, h]
    return dq, dk, dv


# ---------------------------------------------------------------------------------------
# large problems: selected query rows / selected key columns, same definition
# ---------------------------------------------------------------------------------------

def forward_rows(q_bh, k_g, v_g, scale, rows, window=(-1, -1), diag_align=0):
    """O and LSE of the given query rows of one (batch, q-head); q_bh [Sq,D], k_g,v_g [Sk,D]."""
    q_bh, k_g, v_g = (np.asarray(t, dtype=np.float64) for t in (q_bh, k_g, v_g))
    rows = np.asarray(rows)
    vis = window_mask(q_bh.shape[0], k_g.shape[0], window[0], window[1], diag_align, rows)
    o, lse, _ = _rows_forward(q_bh[rows], k_g, v_g, scale, vis)
    return o, lse


def dq_rows(q_bh, k_g, v_g, dout_bh, scale, rows, window=(-1, -1), diag_align=0,
            dlse_bh=None):
    """dQ of the given query rows of one (batch, q-head)."""
    q_bh, k_g, v_g, dout_bh = (np.asarray(t, dtype=np.float64)
                               for t in (q_bh, k_g, v_g, dout_bh))
    rows = np.asarray(rows)
    vis = window_mask(q_bh.shape[0], k_g.shape[0], window[0], window[1], diag_align, rows)
    o, _, p = _rows_forward(q_bh[rows], k_g, v_g, scale, vis)
    delta = (dout_bh[rows] * o).sum(axis=1)
    dl = np.zeros(len(rows)) if dlse_bh is None else np.asarray(dlse_bh, np.float64)[rows]
    ds = p * (dout_bh[rows] @ v_g.T - delta[:, None] + dl[:, None])
    return scale * (ds @ k_g)


def dkdv_cols(q_heads, k_g, v_g, dout_heads, scale, cols, window=(-1, -1), diag_align=0,
              dlse_heads=None, chunk=1024):
    """dK and dV of the given key rows of one kv head, summed over its q heads.

    q_heads, dout_heads [G,Sq,D] are the group's q heads.  Every query row's P is
    needed, so the rows are visited in chunks of ``chunk`` (memory only).
    """
    q_heads, k_g, v_g, dout_heads = (np.asarray(t, dtype=np.float64)
                                     for t in (q_heads, k_g, v_g, dout_heads))
    cols = np.asarray(cols)
    ng, sq, d = q_heads.shape
    dk = np.zeros((len(cols), d))
    dv = np.zeros((len(cols), d))
    for hh in range(ng):
        for r0 in range(0, sq, chunk):
            rows = np.arange(r0, min(sq, r0 + chunk))
            vis = window_mask(sq, k_g.shape[0], window[0], window[1], diag_align, rows)
            o, _, p = _rows_forward(q_heads[hh, rows], k_g, v_g, scale, vis)
            dof = dout_heads[hh, rows]
            delta = (dof * o).sum(axis=1)
            dl = (np.zeros(len(rows)) if dlse_heads is None
                  else np.asarray(dlse_heads[hh], np.float64)[rows])
            ds = p[:, cols] * (dof @ v_g[cols].T - delta[:, None] + dl[:, None])
            dk += scale * (ds.T @ q_heads[hh, rows])
            dv += p[:, cols].T @ dof
    return dk, dv


# ---------------------------------------------------------------------------------------
# LSE merge of two partial results
# ---------------------------------------------------------------------------------------

def merge_forward(x_a, lse_a, x_b, lse_b):
    """Merged (x, lse) of two partial attentions; x [...,D], lse [...]."""
    x_a, lse_a, x_b, lse_b = (np.asarray(t, dtype=np.float64) for t in (x_a, lse_a, x_b, lse_b))
    m = np.maximum(lse_a, lse_b)
    both_empty = np.isneginf(m)
    m_safe = np.where(both_empty, 0.0, m)
    wa = np.where(both_empty, 0.0, np.exp(lse_a - m_safe))
    wb = np.where(both_empty, 0.0, np.exp(lse_b - m_safe))
    den = np.where(both_empty, 1.0, wa + wb)
    x = (x_a * wa[..., None] + x_b * wb[..., None]) / den[..., None]
    lse = np.where(both_empty, NEG_INF, m_safe + np.log(den))
    return x, lse


def merge_backward(x_a, lse_a, x_b, lse_b, g, g_lse=None):
    """dx_a, dlse_a, dx_b, dlse_b given g = dL/dx and g_lse = dL/dlse (None = 0)."""
    x_a, lse_a, x_b, lse_b, g = (np.asarray(t, dtype=np.float64)
                                 for t in (x_a, lse_a, x_b, lse_b, g))
    g_lse = np.zeros(lse_a.shape) if g_lse is None else np.asarray(g_lse, np.float64)
    x, lse = merge_forward(x_a, lse_a, x_b, lse_b)
    empty = np.isneginf(lse)
    lse_safe = np.where(empty, 0.0, lse)
    alpha = np.where(empty, 0.0, np.exp(lse_a - lse_safe))
    beta = np.where(empty, 0.0, np.exp(lse_b - lse_safe))
    dx_a = alpha[..., None] * g
    dx_b = beta[..., None] * g
    dlse_a = alpha * ((g * (x_a - x)).sum(axis=-1) + g_lse)
    dlse_b = beta * ((g * (x_b - x)).sum(axis=-1) + g_lse)
    return dx_a, dlse_a, dx_b, dlse_b
