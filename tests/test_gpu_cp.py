"""Context-parallel ring attention emulated on one GPU ("Add support for cuDNN FusedAttention
+ THD + CP", TransformerEngine issue 885): 2*cp load-balanced chunks, per-hop forward and
backward over (q chunk, kv chunk) pairs, folded with the LSE merge.  The pages' claims
checked here: the result is attention over the whole sequence (fp64 oracle), and the ring
does not depend on the order of its hops (two hop orders agree within rounding)."""
import numpy as np
import pytest
import torch

import scaled_dot_product_05_amd as S
import synth
from gpu_util import (DEV, G_TOL, check_forward, check_grads, gpu_bhsd, oracle_backward,
                      oracle_forward, rel_err, say)

pytestmark = pytest.mark.gpu


def _case(seed, dtype, layout, b, s, h, hk, d, window):
    return synth.dense(seed, 31, dtype, layout, b, s, s, h, hk, d, d ** -0.5, window, with_grad=True)


@pytest.mark.parametrize("cp,dtype,layout,h,hk,d,window", [
    (2, "bf16", "bshd", 4, 4, 64, (-1, 0)),
    (4, "bf16", "bshd", 4, 2, 64, (-1, 0)),
    (4, "f16", "sbhd", 4, 4, 128, (-1, 0)),
    (2, "bf16", "bhsd", 2, 2, 64, (-1, -1)),
    (3, "f32", "bshd", 2, 2, 64, (-1, 0)),
])
def test_cp_ring_equals_full_attention(cp, dtype, layout, h, hk, d, window):
    s = 2 * cp * 96
    w = _case(cp, dtype, layout, 2, s, h, hk, d, window)
    say(f"case cp={cp} {dtype} {layout} S{s} H{h}/{hk} D{d} window={window}")
    q, k, v, g = (t.to(DEV) for t in (w.q, w.k, w.v, w.dout))
    o, lse = S.cp_forward(q, k, v, layout, w.scale, window, cp)
    check_forward(gpu_bhsd(o, w), synth.f64(lse), *oracle_forward(w), dtype, f"cp{cp} fwd")
    dq, dk, dv = S.cp_backward(q, k, v, o, lse, g, layout, w.scale, window, cp)
    check_grads([gpu_bhsd(t, w) for t in (dq, dk, dv)], oracle_backward(w), dtype, f"cp{cp} bwd")


def test_cp_hop_order_does_not_matter():
    cp = 4
    w = _case(9, "bf16", "bshd", 2, 2 * cp * 64, 4, 4, 64, (-1, 0))
    q, k, v, g = (t.to(DEV) for t in (w.q, w.k, w.v, w.dout))
    ref_o, ref_l = oracle_forward(w)
    ref_g = oracle_backward(w)
    outs = []
    for order in ([0, 1, 2, 3], [3, 1, 0, 2]):
        o, lse = S.cp_forward(q, k, v, "bshd", w.scale, (-1, 0), cp, hop_order=order)
        grads = S.cp_backward(q, k, v, o, lse, g, "bshd", w.scale, (-1, 0), cp, hop_order=order)
        check_forward(gpu_bhsd(o, w), synth.f64(lse), ref_o, ref_l, "bf16", f"order {order}")
        check_grads([gpu_bhsd(t, w) for t in grads], ref_g, "bf16", f"order {order}")
        outs.append((synth.f64(o), synth.f64(lse), [synth.f64(t) for t in grads]))
    (o0, l0, g0), (o1, l1, g1) = outs
    assert np.abs(o0 - o1).max() <= 2 ** -7 and np.abs(l0 - l1).max() <= 1e-5
    for a, b in zip(g0, g1):
        assert rel_err(a, b) <= G_TOL["bf16"]


def test_cp_single_rank_is_plain_attention():
    # cp = 1: two chunks on one rank; the fold of (chunk 1 over chunk 0, causal diagonal)
    w = _case(5, "bf16", "bshd", 1, 256, 2, 2, 64, (-1, 0))
    q, k, v = (t.to(DEV) for t in (w.q, w.k, w.v))
    o, lse = S.cp_forward(q, k, v, "bshd", w.scale, (-1, 0), 1)
    fo, fl = S.forward(q, k, v, "bshd", w.scale, (-1, 0))
    # chunk 0 is one plain causal call on the same rows: identical bits
    assert torch.equal(o[:, :128], fo[:, :128]) and torch.equal(lse[:, :, :128], fl[:, :, :128])
    check_forward(gpu_bhsd(o, w), synth.f64(lse), *oracle_forward(w), "bf16", "cp1")


# ---------------------------------------------------------------------------------------
# THD (the page's own case): every sequence of the packed batch cut into 2 cp chunks, of
# any length (chunk lengths then differ by at most one), with or without padding rows
# ---------------------------------------------------------------------------------------

import oracle  # noqa: E402

SENTINEL = 7.0


@pytest.mark.parametrize("cp,dtype,hq,hk,d,window", [
    (2, "bf16", 4, 2, 64, (-1, 0)),
    (3, "bf16", 8, 2, 128, (-1, 0)),
    (2, "f16", 4, 4, 64, (-1, -1)),
    (4, "f32", 2, 2, 64, (-1, 0)),
])
def test_cp_thd_equals_varlen_attention(cp, dtype, hq, hk, d, window):
    lengths = [0, 1, 37, 130, 257, 64, 5]
    w = synth.thd(11, 33, dtype, lengths, hq, hk, d, d ** -0.5, window, with_grad=True)
    say(f"case cp thd cp={cp} {dtype} H{hq}/{hk} D{d} window={window} lengths {lengths}")
    q, k, v, g = (t.to(DEV) for t in (w.q, w.k, w.v, w.dout))
    cu = torch.from_numpy(w.cu_seqlens_q).to(DEV)
    o, lse = S.cp_forward(q, k, v, "thd", w.scale, window, cp, cu_seqlens=cu, max_seqlen=max(lengths))
    torch.cuda.synchronize()
    check_forward(synth.f64(o), synth.f64(lse), *oracle_forward(w), dtype, f"cp{cp} thd fwd")
    dq, dk, dv = S.cp_backward(q, k, v, o, lse, g, "thd", w.scale, window, cp, cu_seqlens=cu,
                               max_seqlen=max(lengths))
    torch.cuda.synchronize()
    check_grads([synth.f64(t) for t in (dq, dk, dv)], oracle_backward(w), dtype, f"cp{cp} thd bwd")


def test_cp_thd_padded_rows_untouched_and_hop_order():
    # padding rows between sequences hold NaN in the inputs and a sentinel in the outputs
    lengths, gaps = [200, 3, 0, 96], [4, 0, 7, 9]
    cp, hq, hk, d = 2, 4, 2, 64
    w = synth.thd(12, 34, "bf16", lengths, hq, hk, d, 0.125, (-1, 0), with_grad=True)
    pad = np.concatenate([[0], np.cumsum(np.add(lengths, gaps))]).astype(np.int32)
    total = int(pad[-1])
    rows = np.concatenate([np.arange(pad[s], pad[s] + lengths[s]) for s in range(len(lengths))])
    gap = torch.from_numpy(np.setdiff1d(np.arange(total), rows)).to(DEV)

    def padded(t):
        out = torch.full((total,) + tuple(t.shape[1:]), float("nan"), dtype=t.dtype)
        out[torch.from_numpy(rows)] = t
        return out.to(DEV)

    q, k, v, g = (padded(t) for t in (w.q, w.k, w.v, w.dout))
    cu = torch.from_numpy(w.cu_seqlens_q).to(DEV)
    cpad = torch.from_numpy(pad).to(DEV)
    say(f"case cp thd padded cp={cp} total {total} valid {len(rows)}")
    ro, rl = oracle_forward(w)
    rg = oracle_backward(w)
    ri = torch.from_numpy(rows).to(DEV)
    results = []
    for order in ([0, 1], [1, 0]):
        o = torch.full_like(q, SENTINEL)
        lse = torch.full((hq, total), SENTINEL, dtype=torch.float32, device=DEV)
        S.cp_forward(q, k, v, "thd", w.scale, (-1, 0), cp, hop_order=order, cu_seqlens=cu,
                     max_seqlen=max(lengths), cu_seqlens_padded=cpad, out=o)
        # the LSE comes back in the call's own buffer: copy the forward's LSE rows
        o2, lse2 = S.cp_forward(q, k, v, "thd", w.scale, (-1, 0), cp, hop_order=order,
                                cu_seqlens=cu, max_seqlen=max(lengths), cu_seqlens_padded=cpad)
        dq, dk, dv = (torch.full_like(t, SENTINEL) for t in (q, k, v))
        S.cp_backward(q, k, v, o2, lse2, g, "thd", w.scale, (-1, 0), cp, hop_order=order,
                      cu_seqlens=cu, max_seqlen=max(lengths), cu_seqlens_padded=cpad, dq=dq, dk=dk, dv=dv)
        torch.cuda.synchronize()
        for t in (o, dq, dk, dv):
            assert (t[gap] == SENTINEL).all()
        check_forward(synth.f64(o[ri]), synth.f64(lse2[:, ri]), ro, rl, "bf16", f"order {order}")
        check_grads([synth.f64(t[ri]) for t in (dq, dk, dv)], rg, "bf16", f"order {order}")
        results.append(synth.f64(o[ri]))
    assert np.abs(results[0] - results[1]).max() <= 2 ** -7


def test_merge_with_sequence_map_touches_only_those_rows():
    # sdpa_merge_fwd on THD with cu_seqlens / cu_seqlens_padded: listed rows merged, others kept
    lengths, starts = [5, 0, 9, 3], [2, 10, 12, 30]
    total, h, d = 40, 2, 64
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    pad = np.array(starts + [total], np.int32)
    rows = np.concatenate([np.arange(starts[s], starts[s] + lengths[s]) for s in range(4)])
    rng = np.random.default_rng(3)
    xa, xb = (torch.from_numpy(rng.standard_normal((total, h, d))).float().to(DEV) for _ in range(2))
    la, lb = (torch.from_numpy(rng.standard_normal((h, total))).float().to(DEV) for _ in range(2))
    x = torch.full_like(xa, SENTINEL)
    lse = torch.full_like(la, SENTINEL)
    md = S.make_merge_desc("thd", "f32", 4, 0, h, d, total, torch.from_numpy(cu).to(DEV),
                           torch.from_numpy(pad).to(DEV))
    S.sdpa_merge_fwd(md, xa, la, xb, lb, x, lse)
    torch.cuda.synchronize()
    keep = np.setdiff1d(np.arange(total), rows)
    assert (x[torch.from_numpy(keep).to(DEV)] == SENTINEL).all()
    assert (lse[:, torch.from_numpy(keep).to(DEV)] == SENTINEL).all()
    A, B = synth.f64(xa).transpose(1, 0, 2), synth.f64(xb).transpose(1, 0, 2)
    mo, ml = oracle.merge_forward(A, synth.f64(la), B, synth.f64(lb))
    got = synth.f64(x).transpose(1, 0, 2)
    assert np.abs(got[:, rows] - mo[:, rows]).max() < 1e-5
    assert np.abs(synth.f64(lse)[:, rows] - ml[:, rows]).max() < 1e-5
