"""The C-ABI calls under HIP graph capture.  Every call only launches kernels on the caller's
stream (no allocation, no host synchronisation, no device-to-host read, no memset), so a
caller can capture a forward + backward step once and replay it.  Each case runs the calls
eagerly, captures the same calls into a graph, and replays it three times with eager work
in between (the outputs overwritten with NaN (or -7) by a fill kernel, then a device
synchronisation); every replay must reproduce the eager outputs bit for bit.  Then new
input values are written in place and one more replay must match a fresh eager call on
them: the graph reads the live buffers, not values of the capture.

Covered: the THD scheduler and the two-launch backward (C4), the split key tiles with their
combine launch (C4 with one dominant sequence), the small-grid GQA halves with their
arrival counters (zeroed by the pre-pass kernel on every call), a window with dLSE, fp32,
the backward that allocates nothing (its static scratch buffer), the FP8 forward, the LSE
merge, the block-mask build with the masked forward and backward, and the
context-parallel ring emulation."""
import numpy as np
import pytest
import torch

import scaled_dot_product_05_amd as S
import synth
from gpu_util import DEV, cu_dev, say, to_dev

pytestmark = pytest.mark.gpu

_INT = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}


def _bits(t):
    return t.contiguous().view(_INT[t.element_size()])


def _poison(t):
    t.fill_(float("nan") if t.is_floating_point() else -7)


def _ws(n):
    return torch.empty(max(n, 1), dtype=torch.uint8, device=DEV) if n else None


def _replays_match_eager(run, inputs, outputs, name):
    """run() issues the calls on the current stream; inputs are refilled in place."""
    run()
    torch.cuda.synchronize()
    ref = [_bits(t).clone() for t in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for r in range(3):
        for t in outputs:
            _poison(t)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, e) in enumerate(zip(outputs, ref)):
            assert torch.equal(_bits(t), e), f"{name}: replay {r}, output {i} differs from eager"
    gen = torch.Generator(device=DEV).manual_seed(7)
    for t in inputs:
        if t.dtype == torch.uint8:  # E4M3 codes: finite ones only (0x7f / 0xff are NaN)
            t.copy_(torch.randint(0, 0x7f, t.shape, generator=gen, device=DEV, dtype=torch.int32).to(t.dtype) |
                    (torch.randint(0, 2, t.shape, generator=gen, device=DEV, dtype=torch.int32) << 7).to(t.dtype))
        else:
            t.copy_(torch.randn(t.shape, generator=gen, device=DEV, dtype=torch.float32).to(t.dtype))
    run()
    torch.cuda.synchronize()
    ref = [_bits(t).clone() for t in outputs]
    for t in outputs:
        _poison(t)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    for i, (t, e) in enumerate(zip(outputs, ref)):
        assert torch.equal(_bits(t), e), f"{name}: replay on new inputs, output {i} differs"
    del g


def _attention_case(w, dlse=False, block_mask=None, noalloc=False):
    q, k, v = to_dev(w)
    cq, ck = cu_dev(w)
    dout = w.dout.to(DEV)
    dl = w.dlse.to(DEV) if dlse else None
    pr = S.Problem(q, k, w.layout, w.scale, w.window, w.diag_align, cq, ck,
                   w.seqlen_q if w.is_thd else None, w.seqlen_k if w.is_thd else None,
                   block_mask=block_mask)
    o = torch.empty_like(q)
    lse = torch.empty(pr.lse_shape, dtype=torch.float32, device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    wsf = _ws(S.sdpa_fwd_workspace_size(pr.desc))
    wsb = _ws(S.sdpa_bwd_workspace_size(pr.desc))

    def run():
        S.sdpa_fwd(pr.desc, q, k, v, o, lse, wsf)
        if noalloc:
            S.sdpa_bwd_noalloc(pr.desc, q, k, v, o, lse, dout, dl, dq, dk, dv)
        else:
            S.sdpa_bwd(pr.desc, q, k, v, o, lse, dout, dl, dq, dk, dv, False, wsb)

    inputs = [q, k, v, dout] + ([dl] if dlse else [])
    return run, inputs, [o, lse, dq, dk, dv], pr


@pytest.mark.parametrize("name", ["c4", "c4_seed3", "gqa_halves", "window_dlse", "f32",
                                  "noalloc_c2", "noalloc_c4"])
def test_graph_replays_attention(name):
    say(f"case graph {name}")
    dlse = name == "window_dlse"
    if name == "c4":
        w = synth.c4(0)
    elif name == "c4_seed3":
        w = synth.c4(3)
    elif name == "gqa_halves":
        w = synth.target(b=1, s=1024, h=16, hk=4, d=128, with_grad=True)
    elif name == "noalloc_c2":
        w = synth.c2()
    elif name == "noalloc_c4":
        w = synth.c4(1)
    elif name == "window_dlse":
        w = synth.dense(5, 41, "bf16", "bshd", 2, 700, 700, 8, 2, 64, 0.125, (128, 0), 0,
                        with_grad=True, with_dlse=True, name="graph_window")
    else:
        w = synth.dense(6, 42, "f32", "bshd", 2, 300, 300, 4, 2, 64, 0.125, (-1, 0), 0,
                        with_grad=True, name="graph_f32")
    run, inputs, outputs, _ = _attention_case(w, dlse, noalloc=name.startswith("noalloc"))
    _replays_match_eager(run, inputs, outputs, name)


def test_graph_replays_fp8_forward():
    say("case graph fp8 forward")
    b, s, hq, hk, d = 2, 640, 4, 2, 128
    coded = [synth.e4m3_codes(synth.normal(10, 45, i, (b, s, h, d))) for i, h in enumerate((hq, hk, hk))]
    q, k, v = (c.to(DEV) for c, _ in coded)
    ds = [torch.tensor([x], dtype=torch.float32, device=DEV) for _, x in coded]
    o = torch.empty((b, s, hq, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((b, hq, s), dtype=torch.float32, device=DEV)

    def run():
        S.forward_fp8(q, k, v, "bshd", d ** -0.5, *ds, window=(-1, 0), out=o, lse=lse)

    _replays_match_eager(run, [q, k, v], [o, lse], "fp8 forward")


def test_graph_replays_merge():
    say("case graph merge")
    gen = torch.Generator(device=DEV).manual_seed(3)
    b, s, h, d = 2, 777, 4, 64
    rnd = lambda *shape: torch.randn(*shape, generator=gen, device=DEV)
    xa, xb, g = (rnd(b, s, h, d) for _ in range(3))
    la, lb, gl = (rnd(b, h, s) for _ in range(3))
    la[0, 0, :5] = float("-inf")
    lb[0, 0, :3] = float("-inf")
    md = S.make_merge_desc("bshd", "f32", b, s, h, d)
    x, lse = torch.empty_like(xa), torch.empty_like(la)
    dxa, dxb, dla, dlb = torch.empty_like(xa), torch.empty_like(xb), torch.empty_like(la), torch.empty_like(lb)

    def run():
        S.sdpa_merge_fwd(md, xa, la, xb, lb, x, lse)
        S.sdpa_merge_bwd(md, xa, la, xb, lb, g, gl, dxa, dla, dxb, dlb)

    _replays_match_eager(run, [xa, xb, g, gl], [x, lse, dxa, dla, dxb, dlb], "merge")


def test_graph_replays_block_mask():
    say("case graph block mask")
    w = synth.dense(8, 43, "bf16", "bshd", 1, 640, 640, 4, 4, 64, 0.125, (-1, -1), 0,
                    with_grad=True, name="graph_mask")
    mask = synth.flex_mask("sliding_window_causal", 640, 640, band=200)
    bits = torch.from_numpy(np.ascontiguousarray(synth.pack_mask(mask[None, None])).view(np.int64)).to(DEV)
    bm = S.BlockMask(bits, 640, 640)
    run_attn, inputs, outputs, _ = _attention_case(w, block_mask=bm)

    def run():
        S.sdpa_block_mask_build(bm.desc, 640, 640)
        run_attn()

    _replays_match_eager(run, inputs, outputs + [bm.kv_count, bm.q_count], "block mask")


def test_graph_replays_cp_ring():
    say("case graph cp ring")
    cp = 2
    w = synth.dense(9, 44, "bf16", "bshd", 2, 4 * cp * 64, 4 * cp * 64, 4, 2, 64, 0.125, (-1, 0), 0,
                    with_grad=True, name="graph_cp")
    q, k, v, dout = (t.to(DEV) for t in (w.q, w.k, w.v, w.dout))
    pr = S.Problem(q, k, "bshd", w.scale, (-1, 0))
    o = torch.empty_like(q)
    lse = torch.empty(pr.lse_shape, dtype=torch.float32, device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = _ws(S.sdpa_cp_workspace_size(pr.desc, cp))

    def run():
        S.sdpa_cp_fwd(pr.desc, cp, [1, 0], q, k, v, o, lse, ws)
        S.sdpa_cp_bwd(pr.desc, cp, [1, 0], q, k, v, o, lse, dout, None, dq, dk, dv, ws)

    _replays_match_eager(run, [q, k, v, dout], [o, lse, dq, dk, dv], "cp ring")
