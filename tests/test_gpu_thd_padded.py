"""Padded THD ("Add support for cuDNN FusedAttention + THD + CP", TransformerEngine issue
885: cu_seqlens_padded, unused rows between packed sequences).  The padding rows of q, k, v, dO
hold NaN: if any kernel read them as keys or queries the results would show it.  Outputs
start as a sentinel, and padding rows must keep it.  Valid rows are checked against the fp64
oracle and must equal, bit for bit, the same sequences packed without padding."""
import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_05_amd as S
import synth
from gpu_util import DEV, check_forward, check_grads, say

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


def _padded(t, rows, total):
    out = torch.full((total,) + tuple(t.shape[1:]), float("nan"), dtype=t.dtype)
    out[torch.from_numpy(rows)] = t
    return out


@pytest.mark.parametrize("dtype,hq,hk,d,window", [
    ("bf16", 8, 2, 128, (-1, 0)),
    ("bf16", 4, 4, 64, (-1, -1)),
    ("f16", 4, 2, 64, (64, 0)),
    ("f32", 2, 2, 64, (-1, 0)),
])
def test_padded_thd_matches_oracle_and_packed(dtype, hq, hk, d, window):
    run_padded(dtype, hq, hk, d, window, [300, 1, 0, 129, 64], [5, 0, 3, 17, 2])


@pytest.mark.parametrize("hq,hk", [(4, 2), (4, 4)])
def test_padded_thd_short_sequences(hq, hk):
    # at most 32 rows per sequence: the short-sequence forward and backward kernels
    names = run_padded("bf16", hq, hk, 64, (-1, 0), [30, 1, 0, 17, 32], [5, 0, 3, 17, 2])
    assert {"attn_fwd_short", "bwd_short"} <= names, names


def run_padded(dtype, hq, hk, d, window, lengths, gaps):
    """Returns the names of the kernels the padded calls launched."""
    w = synth.thd(4, 41, dtype, lengths, hq, hk, d, d ** -0.5, window, with_grad=True)
    cu = w.cu_seqlens_q
    pad = np.concatenate([[0], np.cumsum(np.add(lengths, gaps))]).astype(np.int32)
    total = int(pad[-1])
    rows = np.concatenate([np.arange(pad[s], pad[s] + lengths[s]) for s in range(len(lengths))])
    gap = np.setdiff1d(np.arange(total), rows)
    say(f"case padded thd {dtype} H{hq}/{hk} D{d} window={window} total {total} (valid {len(rows)})")
    qp, kp, vp, gp = (_padded(t, rows, total).to(DEV) for t in (w.q, w.k, w.v, w.dout))
    cq = torch.from_numpy(cu).to(DEV)
    cp = torch.from_numpy(pad).to(DEV)
    smax = max(lengths)
    tdt = qp.dtype
    o = torch.full_like(qp, SENTINEL)
    lse = torch.full((hq, total), SENTINEL, dtype=torch.float32, device=DEV)
    dq, dk, dv = (torch.full_like(t, SENTINEL) for t in (qp, kp, vp))
    torch.cuda.synchronize()
    S.sdpa_profile_enable(True)
    S.forward(qp, kp, vp, "thd", w.scale, window, "top_left", cq, cq, smax, smax, out=o, lse=lse,
              cu_seqlens_q_padded=cp, cu_seqlens_k_padded=cp)
    S.backward(qp, kp, vp, o, lse, gp, "thd", w.scale, window, "top_left", None, cq, cq, smax, smax,
               dq=dq, dk=dk, dv=dv, cu_seqlens_q_padded=cp, cu_seqlens_k_padded=cp)
    torch.cuda.synchronize()
    S.sdpa_profile_enable(False)
    names = set(S.sdpa_profile_read())
    # padding rows untouched
    gi = torch.from_numpy(gap).to(DEV)
    for t in (o, dq, dk, dv):
        assert (t[gi] == SENTINEL).all()
    assert (lse[:, gi] == SENTINEL).all()
    # valid rows against the oracle (its padding rows are NaN; compare valid rows)
    ro, rl = oracle.thd_forward(synth.f64(w.q), synth.f64(w.k), synth.f64(w.v), cu, cu, w.scale, window)
    ri = torch.from_numpy(rows).to(DEV)
    check_forward(synth.f64(o[ri]), synth.f64(lse[:, ri]), ro, rl, dtype, "padded fwd")
    rg = oracle.thd_backward(synth.f64(w.q), synth.f64(w.k), synth.f64(w.v), synth.f64(w.dout), cu,
                             cu, w.scale, window)
    check_grads([synth.f64(t[ri]) for t in (dq, dk, dv)], rg, dtype, "padded bwd")
    # the same sequences packed back to back: identical bits
    q, k, v, g = (t.to(DEV) for t in (w.q, w.k, w.v, w.dout))
    o2, l2 = S.forward(q, k, v, "thd", w.scale, window, "top_left", cq, cq, smax, smax)
    d2 = S.backward(q, k, v, o2, l2, g, "thd", w.scale, window, "top_left", None, cq, cq, smax, smax)
    assert torch.equal(o[ri], o2) and torch.equal(lse[:, ri], l2)
    for a, b in zip((dq, dk, dv), d2):
        assert torch.equal(a[ri], b)
    return names
