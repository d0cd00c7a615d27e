"""GPU parity on grids large enough for every XCD block order of the forward and backward:
(batch, head) pairs per XCD taken in groups (causal, more than 4 pairs per XCD), pair after
pair (every query sees every key), contiguous head ranges under GQA and for THD.  Each case
compares O, LSE, dQ, dK and dV with the fp64 oracle over the whole problem, so a block
order that missed or repeated a tile would show."""
import pytest

import synth
from gpu_util import (DEV, check_forward, check_grads, cu_dev, gpu_backward, gpu_bhsd,
                      gpu_forward, oracle_backward, oracle_forward, say, to_dev)

pytestmark = pytest.mark.gpu


def run_case(w):
    say(f"case {w.name} {w.dtype} {w.layout} B={w.batch} Sq={w.seqlen_q} Sk={w.seqlen_k} "
        f"Hq={w.heads_q} Hk={w.heads_kv} D={w.head_dim} win={w.window}")
    q, k, v = to_dev(w)
    cq, ck = cu_dev(w)
    o, lse = gpu_forward(w, q, k, v, cq, ck)
    if w.is_thd:
        check_forward(synth.f64(o), synth.f64(lse), *oracle_forward(w), w.dtype, "fwd")
        grads = gpu_backward(w, q, k, v, o, lse, w.dout.to(DEV), None, cq, ck)
        check_grads([synth.f64(t) for t in grads], oracle_backward(w), w.dtype, "bwd")
        return
    check_forward(gpu_bhsd(o, w), synth.f64(lse), *oracle_forward(w), w.dtype, "fwd")
    grads = gpu_backward(w, q, k, v, o, lse, w.dout.to(DEV))
    check_grads([gpu_bhsd(t, w) for t in grads], oracle_backward(w), w.dtype, "bwd")


@pytest.mark.parametrize("d", [64, 128])
def test_causal_grouped_pairs(d):
    # 64 (batch, head) pairs: 8 per XCD, taken in groups of 4 (forward; backward at D128)
    w = synth.dense(61, 1200 + d, "bf16", "bshd", 4, 384, 384, 16, 16, d, d ** -0.5, (-1, 0),
                    with_grad=True, name="order_grouped")
    run_case(w)


@pytest.mark.parametrize("d", [64, 128])
def test_full_attention_pair_after_pair(d):
    # every query sees every key: each XCD walks its 8 pairs one after the other
    w = synth.dense(62, 1210 + d, "f16", "bshd", 8, 300, 257, 8, 8, d, 0.1, (-1, -1),
                    with_grad=True, name="order_uniform")
    run_case(w)


def test_gqa_window_contiguous_heads():
    # GQA with a sliding window: contiguous pair ranges, tiles longest first
    w = synth.dense(63, 1220, "bf16", "sbhd", 2, 320, 320, 32, 8, 128, 0.09, (100, 0),
                    with_grad=True, name="order_gqa_window")
    run_case(w)


def test_thd_sixteen_kv_heads():
    # THD with 16 q and 16 kv heads: contiguous head ranges per XCD (D128 backward too)
    w = synth.thd(64, 1230, "bf16", [200, 0, 129, 64, 257, 1], 16, 16, 128, 128 ** -0.5,
                  (-1, 0), with_grad=True, name="order_thd")
    run_case(w)
