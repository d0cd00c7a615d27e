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
