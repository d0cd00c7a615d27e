"""The pages' workloads at full size on the GPU, checked against the fp64 oracle, plus the
properties that tie them to the pages: packed views read exactly like contiguous copies
(TransformerEngine issue 1195), THD sequences equal their dense counterparts, results are
bitwise reproducible, and the local/global LSE merge of issue 135161 holds end to end.
"""
import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_05_amd as S
import synth
from gpu_util import (DEV, G_TOL, O_TOL, check_forward, check_grads, cu_dev, gpu_backward,
                      gpu_bhsd, gpu_forward, oracle_backward, oracle_forward, rel_err, say, to_dev)

pytestmark = pytest.mark.gpu

SEEDS = [0, 1, 2]  # the pages' five workloads at the default seed and two more


@pytest.mark.parametrize("seed", SEEDS)
def test_c1_fp32_noncausal_bhsd(seed):
    w = synth.c1(seed)
    say(f"case c1 seed={seed}")
    q, k, v = to_dev(w)
    o, lse = gpu_forward(w, q, k, v)
    check_forward(gpu_bhsd(o, w), synth.f64(lse), *oracle_forward(w), "f32", "c1")


@pytest.mark.parametrize("seed", SEEDS)
def test_c2_bf16_causal_fwd_bwd(seed):
    w = synth.c2(seed)
    say(f"case c2 seed={seed}")
    q, k, v = to_dev(w)
    o, lse = gpu_forward(w, q, k, v)
    check_forward(gpu_bhsd(o, w), synth.f64(lse), *oracle_forward(w), "bf16", "c2 fwd")
    dq, dk, dv = gpu_backward(w, q, k, v, o, lse, w.dout.to(DEV))
    check_grads([gpu_bhsd(t, w) for t in (dq, dk, dv)], oracle_backward(w), "bf16", "c2 bwd")


@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("scale", [1.0, 0.1])
def test_c3_fp16_packed_mqa_views(scale, seed):
    w = synth.c3(seed, scale=scale)
    say(f"case c3 scale={scale} seed={seed}")
    q, k, v = to_dev(w)
    assert not q.is_contiguous() and q.stride() == (1152, 1152, 64, 1)
    o, lse = gpu_forward(w, q, k, v)
    check_forward(gpu_bhsd(o, w), synth.f64(lse), *oracle_forward(w), "f16", "c3 views")
    # issue 1195: the same data as contiguous copies must give the same bits
    oc, lc = gpu_forward(w, q.contiguous(), k.contiguous(), v.contiguous())
    assert torch.equal(o, oc) and torch.equal(lse, lc)
    # and as a BHSD permutation of those copies (strides only)
    wb = synth.Workload("c3b", "f16", "bhsd", 1, w.seqlen_q, w.seqlen_k, 16, 1, 64, scale, (-1, 0))
    ob, lb = gpu_forward(wb, *(t.permute(1, 2, 0, 3) for t in (q, k, v)))
    assert torch.equal(ob.permute(2, 0, 1, 3), o) and torch.equal(lb, lse)


@pytest.mark.parametrize("seed", SEEDS)
def test_c4_thd_gqa_fwd_full_and_bwd(seed):
    w = synth.c4(seed)
    say(f"case c4 seed={seed} lengths={np.diff(w.cu_seqlens_q).tolist()}")
    q, k, v = to_dev(w)
    cq, ck = cu_dev(w)
    o, lse = gpu_forward(w, q, k, v, cq, ck)
    check_forward(synth.f64(o), synth.f64(lse), *oracle_forward(w), "bf16", "c4 fwd")
    dq, dk, dv = gpu_backward(w, q, k, v, o, lse, w.dout.to(DEV), None, cq, ck)
    refs = oracle_backward(w)
    check_grads([synth.f64(t) for t in (dq, dk, dv)], refs, "bf16", "c4 bwd")


def test_thd_sequence_equals_dense_bitwise():
    w = synth.thd(21, 900, "bf16", [300, 77, 512], 8, 2, 128, 0.09, (-1, 0), with_grad=True)
    say("case thd-vs-dense")
    q, k, v = to_dev(w)
    cq, ck = cu_dev(w)
    o, lse = gpu_forward(w, q, k, v, cq, ck)
    dq, dk, dv = gpu_backward(w, q, k, v, o, lse, w.dout.to(DEV), None, cq, ck)
    cu = w.cu_seqlens_q
    for s in range(3):
        a, b = int(cu[s]), int(cu[s + 1])
        ws = synth.Workload("one", "bf16", "bshd", 1, b - a, b - a, 8, 2, 128, 0.09, (-1, 0))
        qs, ks, vs, gs = (t[a:b].unsqueeze(0) for t in (q, k, v, w.dout.to(DEV)))
        os_, ls = gpu_forward(ws, qs, ks, vs)
        assert torch.equal(os_[0], o[a:b]) and torch.equal(ls[0], lse[:, a:b])
        g3 = gpu_backward(ws, qs, ks, vs, os_, ls, gs)
        for x, y in zip(g3, (dq, dk, dv)):
            assert torch.equal(x[0], y[a:b])


def test_bitwise_determinism():
    w = synth.c2(seed=3)
    q, k, v = to_dev(w)
    g = w.dout.to(DEV)
    runs = []
    for _ in range(2):
        o, lse = gpu_forward(w, q, k, v)
        runs.append((o, lse) + tuple(gpu_backward(w, q, k, v, o, lse, g)))
    for a, b in zip(*runs):
        assert torch.equal(a, b)


def test_strided_output_guard_bands():
    # outputs written into every other head of a NaN-filled buffer: the gaps stay NaN
    w = synth.dense(22, 950, "bf16", "bshd", 2, 200, 200, 4, 4, 64, 0.125, (-1, 0), with_grad=True)
    q, k, v = to_dev(w)
    obuf = torch.full((2, 200, 8, 64), float("nan"), dtype=torch.bfloat16, device=DEV)
    lbuf = torch.full((2, 8, 200), float("nan"), device=DEV)
    o, lse = gpu_forward(w, q, k, v, out=obuf[:, :, ::2], lse=lbuf[:, ::2])
    assert torch.isnan(obuf[:, :, 1::2]).all() and torch.isnan(lbuf[:, 1::2]).all()
    check_forward(gpu_bhsd(o, w), synth.f64(lse), *oracle_forward(w), "bf16", "guarded fwd")
    # packed gradient buffer with unused heads 4, 9, 14, 15 between and after the views
    gbuf = torch.full((2, 200, 16, 64), float("nan"), dtype=torch.bfloat16, device=DEV)
    dq, dk, dv = gbuf[:, :, 0:4], gbuf[:, :, 5:9], gbuf[:, :, 10:14]
    gpu_backward(w, q, k, v, o, lse, w.dout.to(DEV), dq=dq, dk=dk, dv=dv)
    for hh in (4, 9, 14, 15):
        assert torch.isnan(gbuf[:, :, hh]).all()
    check_grads([gpu_bhsd(t, w) for t in (dq, dk, dv)], oracle_backward(w), "bf16", "guarded bwd")


# ---------------------------------------------------------------------------------------
# merge
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_merge_kernels(dtype, d):
    rng = np.random.default_rng([23, d])
    b, h, s = 2, 3, 129
    xa, xb = (synth.cast(rng.standard_normal((b, s, h, d)), dtype) for _ in range(2))
    la = torch.from_numpy((3 * rng.standard_normal((b, h, s))).astype(np.float32))
    lb = torch.from_numpy((3 * rng.standard_normal((b, h, s))).astype(np.float32))
    la[0, 0, :5] = -float("inf")  # one side empty
    lb[0, 0, 3:8] = -float("inf")  # both empty on rows 3, 4
    g = synth.cast(rng.standard_normal((b, s, h, d)), dtype)
    gl = torch.from_numpy(rng.standard_normal((b, h, s)).astype(np.float32))
    say(f"case merge {dtype} d={d}")
    dev = [t.to(DEV) for t in (xa, la, xb, lb, g, gl)]
    x, l = S.merge(dev[0], dev[1], dev[2], dev[3], "bshd")
    bh = lambda t: synth.f64(t).transpose(0, 2, 1, 3)
    x_ref, l_ref = oracle.merge_forward(bh(xa), synth.f64(la), bh(xb), synth.f64(lb))
    check_forward(bh(x.cpu()), synth.f64(l), x_ref, l_ref, dtype, "merge fwd")
    grads = S.merge_backward(dev[0], dev[1], dev[2], dev[3], dev[4], dev[5], "bshd")
    refs = oracle.merge_backward(bh(xa), synth.f64(la), bh(xb), synth.f64(lb), bh(g),
                                 synth.f64(gl))
    got = [bh(grads[0].cpu()), synth.f64(grads[1]), bh(grads[2].cpu()), synth.f64(grads[3])]
    for name, a, r in zip(("dx_a", "dlse_a", "dx_b", "dlse_b"), got, refs):
        e = rel_err(a, r)
        say(f"  {name}: rel err {e:.3e}")
        assert e <= G_TOL[dtype]
    assert (got[1][0, 0, 3:5] == 0).all() and (got[3][0, 0, 3:5] == 0).all()


def _c5_device(seed=0):
    c = synth.c5(seed)
    qkv = c["qkv"].to(DEV)
    da = c["heads"] * c["d"]
    q = qkv[:, :, :da].unflatten(2, (c["heads"], c["d"]))
    k = qkv[:, :, da:2 * da].unflatten(2, (c["heads"], c["d"]))
    v = qkv[:, :, 2 * da:].unflatten(2, (c["heads"], c["d"]))
    return c, q, k, v


@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("upstream", ["ones", "random"])
def test_c5_local_global_merge_fwd_bwd(upstream, seed):
    c, q, k, v = _c5_device(seed)
    say(f"case c5 upstream={upstream} seed={seed}")
    sc, ng = c["scale"], c["global_keys"]
    ol, ll = S.forward(q, k, v, "bshd", sc, c["local_window"])
    og, lg = S.forward(q, k[:, :ng], v[:, :ng], "bshd", sc, (-1, 0))
    x, lse = S.merge(ol, ll, og, lg, "bshd")
    g = (c["g_ones"] if upstream == "ones" else c["g_rand"]).to(DEV)
    gl = (c["glse_zero"] if upstream == "ones" else c["glse_rand"]).to(DEV)
    dxa, dla, dxb, dlb = S.merge_backward(ol, ll, og, lg, g, gl, "bshd")
    dqkv = torch.zeros_like(c["qkv"], device=DEV)
    da = c["heads"] * c["d"]
    dq = dqkv[:, :, :da].unflatten(2, (c["heads"], c["d"]))
    dk = dqkv[:, :, da:2 * da].unflatten(2, (c["heads"], c["d"]))
    dv = dqkv[:, :, 2 * da:].unflatten(2, (c["heads"], c["d"]))
    S.backward(q, k, v, ol, ll, dxa, "bshd", sc, c["local_window"], dlse=dla, dq=dq, dk=dk, dv=dv)
    S.backward(q, k[:, :ng], v[:, :ng], og, lg, dxb, "bshd", sc, (-1, 0), dlse=dlb, dq=dq,
               dk=dk[:, :ng], dv=dv[:, :ng], accumulate=True)
    torch.cuda.synchronize()
    # oracle chain in fp64 from the same fp32 inputs
    qo, ko, vo = (synth.f64(t.cpu()).transpose(0, 2, 1, 3) for t in (q, k, v))
    s_ = qo.shape[2]
    loc = oracle.window_mask(s_, s_, 128, 0)
    glb = oracle.window_mask(s_, ng, -1, 0)
    xl, l1 = oracle.attention_forward(qo, ko, vo, sc, loc)
    xg, l2 = oracle.attention_forward(qo, ko[:, :, :ng], vo[:, :, :ng], sc, glb)
    xr, lr = oracle.merge_forward(xl, l1, xg, l2)
    check_forward(synth.f64(x.cpu()).transpose(0, 2, 1, 3), synth.f64(lse), xr, lr, "f32", "c5 merged")
    gg = synth.f64(g.cpu()).transpose(0, 2, 1, 3)
    a1, b1, a2, b2 = oracle.merge_backward(xl, l1, xg, l2, gg, synth.f64(gl.cpu()))
    r1 = oracle.attention_backward(qo, ko, vo, a1, sc, loc, b1)
    r2 = oracle.attention_backward(qo, ko[:, :, :ng], vo[:, :, :ng], a2, sc, glb, b2)
    rdq = r1[0] + r2[0]
    rdk = r1[1].copy()
    rdk[:, :, :ng] += r2[1]
    rdv = r1[2].copy()
    rdv[:, :, :ng] += r2[2]
    got = [synth.f64(t.cpu()).transpose(0, 2, 1, 3) for t in (dq, dk, dv)]
    check_grads(got, [rdq, rdk, rdv], "f32", "c5 grads")


@pytest.mark.parametrize("version", [1, 2])
def test_p3_partition_merge_equals_causal(version):
    # issue 135161's split: local band 128 plus the global remainder is causal attention
    w = synth.dense(24, 1000, "f32", "bhsd", 2, 512, 512, 4, 4, 32, 32 ** -0.5, (-1, 0),
                    with_grad=True, name="p3")
    say(f"case p3 v{version}")
    q, k, v = to_dev(w)
    oc, lc = gpu_forward(w, q, k, v)
    xl, ll = S.forward(q, k, v, "bhsd", w.scale, (128, 0))
    if version == 2:
        xg, lg = S.forward(q, k, v, "bhsd", w.scale, (-1, -129))
        x, lse = S.merge(xl, ll, xg, lg, "bhsd")
    else:
        qs = q[:, :, 128:]
        xg, lg = S.forward(qs, k, v, "bhsd", w.scale, (-1, -129), diag_align="bottom_right")
        xm, lm = S.merge(xl[:, :, 128:], ll[:, :, 128:], xg, lg, "bhsd")
        x = torch.cat([xl[:, :, :128], xm], 2)
        lse = torch.cat([ll[:, :, :128], lm], 2)
    o_ref, l_ref = oracle_forward(w)
    check_forward(synth.f64(x), synth.f64(lse), o_ref, l_ref, "f32", "p3 merged")
    assert (x - oc).abs().max().item() <= 2 * O_TOL["f32"]
