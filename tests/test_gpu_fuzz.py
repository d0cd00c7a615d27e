"""Seeded random small problems through the C ABI against the fp64 oracle: dtype, layout
(BSHD, SBHD, BHSD, THD with empty sequences and cross lengths), head_dim, GQA/MQA grouping,
window kind and diagonal alignment, softmax scale (including negative) and dLSE are drawn
per case, forward and backward.  Windows of width one ((0, 0)) and single-key problems are
left out: there dQ and dK vanish in exact arithmetic and only rounding noise is left."""
import numpy as np
import pytest

import synth
from gpu_util import (DEV, check_forward, check_grads, cu_dev, gpu_backward, gpu_bhsd, gpu_forward,
                      oracle_backward, oracle_forward, say, to_dev)

pytestmark = pytest.mark.gpu

N_CASES = 120


def _window(rng):
    kind = int(rng.integers(0, 5))
    if kind == 0:
        return (-1, -1)
    if kind == 1:
        return (-1, 0)
    if kind == 2:
        return (int(rng.integers(1, 101)), int(rng.integers(0, 51)))
    if kind == 3:
        return (-1, int(rng.integers(0, 21)))
    return (int(rng.integers(1, 61)), -1)


def _case(i):
    rng = np.random.default_rng([2024, i])
    dtype = ("bf16", "f16", "f32")[int(rng.integers(0, 3))]
    layout = ("bshd", "sbhd", "bhsd", "thd")[int(rng.integers(0, 4))]
    d = (32, 64, 128)[int(rng.integers(0, 3))]
    hk = (1, 2, 4)[int(rng.integers(0, 3))]
    hq = hk * (1, 2, 4)[int(rng.integers(0, 3))]
    scale = float(d ** -0.5 * (1.0, 0.5, 2.0, -1.0)[int(rng.integers(0, 4))])
    window = _window(rng)
    align = int(rng.integers(0, 2))
    dlse = bool(rng.integers(0, 2))
    if layout == "thd":
        n = int(rng.integers(1, 7))
        lengths = rng.integers(0, 201, n).tolist()
        lengths[int(rng.integers(0, n))] = int(rng.integers(2, 201))  # at least one real sequence
        lengths_k = None
        if rng.integers(0, 2):
            lengths_k = [max(2, x + int(rng.integers(-40, 41))) if x else 0 for x in lengths]
        w = synth.thd(100 + i, 2000 + i, dtype, lengths, hq, hk, d, scale, window, with_grad=True,
                      with_dlse=dlse, lengths_k=lengths_k, diag_align=align, name=f"fuzz{i}")
    else:
        b = int(rng.integers(1, 4))
        sq, sk = int(rng.integers(2, 301)), int(rng.integers(2, 301))
        w = synth.dense(100 + i, 2000 + i, dtype, layout, b, sq, sk, hq, hk, d, scale, window, align,
                        with_grad=True, with_dlse=dlse, name=f"fuzz{i}")
    return w, dlse


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_problem_matches_oracle(i):
    w, dlse = _case(i)
    say(f"case fuzz{i} {w.dtype} {w.layout} B={w.batch} Sq={w.seqlen_q} Sk={w.seqlen_k} Hq={w.heads_q} "
        f"Hk={w.heads_kv} D={w.head_dim} scale={w.scale:.3f} win={w.window} al={w.diag_align} dlse={dlse}")
    q, k, v = to_dev(w)
    cq, ck = cu_dev(w)
    o, lse = gpu_forward(w, q, k, v, cq, ck)
    check_forward(gpu_bhsd(o, w), synth.f64(lse), *oracle_forward(w), w.dtype, "fwd")
    dl = w.dlse.to(DEV) if dlse else None
    grads = gpu_backward(w, q, k, v, o, lse, w.dout.to(DEV), dl, cq, ck)
    refs = oracle_backward(w, synth.f64(w.dlse) if dlse else None)
    check_grads([gpu_bhsd(t, w) for t in grads], refs, w.dtype, "bwd")
