"""Tensors whose elements lie more than 4 GiB past their base pointer.  The descriptor carries
64-bit element strides ("[PyTorch] fused CUDNN attention kernel not properly handling
strides", TransformerEngine issue 1195: strides are read, never assumed), and the kernels'
16-byte buffer loads take 32-bit offsets from a per-(sequence, head) base.  Each case places
a batch, a sequence or every row beyond 2^32 bytes:

- a batch stride of 2^31 + 8192 elements (bf16, batch 1 starts 4 GiB in), on a grid large
  enough for the two-launch backward, against the same call on contiguous tensors, bit for
  bit;
- padded THD whose sequences start up to 4.6 GB into q ("Add support for cuDNN
  FusedAttention + THD + CP", TransformerEngine issue 885: cu_seqlens_padded), against the
  packed call, bit for bit;
- fp32 with a batch stride of 2^30 + 4096 elements (4 GiB), against the contiguous call, bit
  for bit;
- a row stride of 2^21 + 64 elements, so that a sequence spans more than 2^31 bytes and the
  host routes the call to the kernels with 64-bit row addressing, against the fp64 oracle;
- row statistics (LSE log2(e) and Delta, one fp32 per q head and row) past 2^31 bytes, which
  the host routes away from the dK/dV kernel that reads them through one 32-bit resource,
  with a backward pre-pass over 537M rows (a dispatch counts work-items in 32 bits, so that
  kernel loops over a capped grid);
- an LSE merge over more rows than its capped grid covers in one pass.

Up to about 70 GB of device memory per case; the gaps between the used elements are
allocated and never touched."""
import numpy as np
import pytest
import torch

import scaled_dot_product_05_amd as S
import synth
import oracle
from gpu_util import (DEV, G_TOL, check_forward, check_grads, gpu_bhsd, oracle_backward, oracle_forward,
                      rel_err, say)

pytestmark = pytest.mark.gpu

_INT = {2: torch.int16, 4: torch.int32}


def _bits(t):
    return t.contiguous().view(_INT[t.element_size()])


def _strided(shape, strides, dtype):
    n = 1 + sum((a - 1) * b for a, b in zip(shape, strides))
    return torch.empty(n, dtype=dtype, device=DEV).as_strided(shape, strides)


def _like(t, strides, src=None):
    out = _strided(tuple(t.shape), strides, t.dtype)
    if src is not None:
        out.copy_(src)
    return out


def _dense_call(w, q, k, v, g):
    o, lse = S.forward(q, k, v, w.layout, w.scale, w.window, w.diag_align)
    return (o, lse) + tuple(S.backward(q, k, v, o, lse, g, w.layout, w.scale, w.window, w.diag_align))


def _dense_far(w, stride_of):
    """Run w on device copies laid out with the strides stride_of(shape) gives, outputs too."""
    q, k, v, g = (_like(t, stride_of(t.shape), t.to(DEV)) for t in (w.q, w.k, w.v, w.dout))
    o = _like(q, stride_of(q.shape))
    dq, dk, dv = _like(q, stride_of(q.shape)), _like(k, stride_of(k.shape)), _like(v, stride_of(v.shape))
    lse = torch.empty((w.batch, w.heads_q, w.seqlen_q), dtype=torch.float32, device=DEV)
    S.forward(q, k, v, w.layout, w.scale, w.window, w.diag_align, out=o, lse=lse)
    S.backward(q, k, v, o, lse, g, w.layout, w.scale, w.window, w.diag_align, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def _assert_bitwise(got, ref, name):
    for i, (a, b) in enumerate(zip(got, ref)):
        assert a.shape == b.shape
        assert torch.equal(_bits(a), _bits(b)), f"{name}: output {i} differs"


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,sb", [("bf16", 2 ** 31 + 8192), ("f32", 2 ** 30 + 4096)])
def test_batch_beyond_4gib_matches_contiguous(dtype, sb):
    if dtype == "bf16":
        w = synth.dense(3, 51, "bf16", "bshd", 2, 8192, 8192, 16, 4, 128, 128 ** -0.5, (-1, 0),
                        with_grad=True, name="far_batch")
    else:
        w = synth.dense(3, 52, "f32", "bshd", 2, 512, 512, 4, 4, 64, 0.125, (-1, 0),
                        with_grad=True, name="far_batch_f32")
    say(f"case far batch {dtype} batch stride {sb} elements")
    ref = [t.clone() for t in _dense_call(w, *(t.to(DEV) for t in (w.q, w.k, w.v, w.dout)))]
    torch.cuda.synchronize()
    got = _dense_far(w, lambda shp: (sb, shp[2] * shp[3], shp[3], 1))
    _assert_bitwise(got, ref, f"far batch {dtype}")
    del got, ref
    _free()


def test_padded_thd_beyond_4gib_matches_packed():
    lengths = [4096, 6000, 5000]
    starts = [0, 600_000, 1_120_000]
    hq, hk, d = 16, 4, 128
    w = synth.thd(5, 53, "bf16", lengths, hq, hk, d, d ** -0.5, (-1, 0), with_grad=True, name="far_thd")
    total = starts[-1] + lengths[-1] + 3
    say(f"case far padded thd: starts {starts}, {total} rows, q {total * hq * d * 2 / 2 ** 30:.1f} GiB")
    cu = torch.from_numpy(w.cu_seqlens_q).to(DEV)
    smax = max(lengths)
    q, k, v, g = (t.to(DEV) for t in (w.q, w.k, w.v, w.dout))
    o, lse = S.forward(q, k, v, "thd", w.scale, (-1, 0), "top_left", cu, cu, smax, smax)
    ref = [o, lse] + list(S.backward(q, k, v, o, lse, g, "thd", w.scale, (-1, 0), "top_left", None,
                                     cu, cu, smax, smax))
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(s, s + n) for s, n in zip(starts, lengths)])
    ri = torch.from_numpy(rows).to(DEV)
    pad = torch.tensor(starts + [total], dtype=torch.int32, device=DEV)

    def far(t):
        out = torch.empty((total,) + tuple(t.shape[1:]), dtype=t.dtype, device=DEV)
        out[ri] = t
        return out

    qp, kp, vp, gp = far(q), far(k), far(v), far(g)
    op, dqp = torch.empty_like(qp), torch.empty_like(qp)
    dkp, dvp = torch.empty_like(kp), torch.empty_like(vp)
    lsep = torch.empty((hq, total), dtype=torch.float32, device=DEV)
    S.forward(qp, kp, vp, "thd", w.scale, (-1, 0), "top_left", cu, cu, smax, smax, out=op, lse=lsep,
              cu_seqlens_q_padded=pad, cu_seqlens_k_padded=pad)
    S.backward(qp, kp, vp, op, lsep, gp, "thd", w.scale, (-1, 0), "top_left", None, cu, cu, smax,
               smax, dq=dqp, dk=dkp, dv=dvp, cu_seqlens_q_padded=pad, cu_seqlens_k_padded=pad)
    torch.cuda.synchronize()
    got = [op[ri], lsep[:, ri], dqp[ri], dkp[ri], dvp[ri]]
    _assert_bitwise(got, ref, "far padded thd")
    del got, ref, qp, kp, vp, gp, op, dqp, dkp, dvp, lsep
    _free()


def test_rows_beyond_2gib_take_the_64bit_kernels():
    # a sequence spans (600 rows) x (2^21 + 64 elements) x 2 bytes > 2^31: no 32-bit offsets
    w = synth.dense(6, 54, "bf16", "bshd", 1, 600, 600, 2, 2, 64, 0.125, (-1, 0),
                    with_grad=True, name="far_rows")
    ss = 2 ** 21 + 64
    say(f"case far rows: row stride {ss} elements")
    got = _dense_far(w, lambda shp: (shp[1] * ss, ss, shp[3], 1))
    o, lse, dq, dk, dv = got
    check_forward(gpu_bhsd(o, w), synth.f64(lse), *oracle_forward(w), "bf16", "far rows fwd")
    check_grads([gpu_bhsd(t, w) for t in (dq, dk, dv)], oracle_backward(w), "bf16", "far rows bwd")
    del got, o, lse, dq, dk, dv
    _free()


def test_stat_rows_beyond_2gib():
    # 64 q heads x (2^23 + 64) rows of fp32 LSE and Delta: the backward's row statistics pass
    # 2^31 bytes.  Bottom-right causal over 256 keys: only each head's last 256 rows see keys,
    # and head 63's lie past that boundary, so its dK and dV come from them alone.  Heads are
    # broadcast (stride 0) in q, k, v, dO, O and LSE, so every head's gradients equal those of
    # one head; only dQ (64 GiB) is stored in full.
    hq, d, sk = 64, 64, 256
    sq = 2 ** 23 + 64
    say(f"case stat rows beyond 2 GiB: H{hq} Sq {sq} Sk {sk} D{d}")
    scale = 0.125
    gen = torch.Generator(device=DEV).manual_seed(11)
    rnd = lambda n: torch.randn((1, n, 1, d), generator=gen, device=DEV).to(torch.bfloat16)
    q1, g1, k1, v1 = rnd(sq), rnd(sq), rnd(sk), rnd(sk)
    o1, lse1 = S.forward(q1, k1, v1, "bshd", scale, (-1, 0), "bottom_right")
    heads = lambda t, n: t.as_strided((1, n, hq, d), (0, d, 0, 1))
    q, g, o, k, v = heads(q1, sq), heads(g1, sq), heads(o1, sq), heads(k1, sk), heads(v1, sk)
    lse = lse1.as_strided((1, hq, sq), (0, 0, 1))
    dq = torch.empty((1, sq, hq, d), dtype=torch.bfloat16, device=DEV)
    dk = torch.empty((1, sk, hq, d), dtype=torch.bfloat16, device=DEV)
    dv = torch.empty_like(dk)
    S.backward(q, k, v, o, lse, g, "bshd", scale, (-1, 0), "bottom_right", dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    # every head equals head 0 bit for bit (identical inputs), and head 0 equals one head's
    # attention over the last 256 rows (causal, fp64 oracle)
    for t in (dk, dv, dq[:, sq - sk:]):
        ref = t[:, :, :1]
        assert torch.equal(_bits(t), _bits(ref.expand_as(t))), "heads differ"
    w = synth.Workload("stat_rows", "bf16", "bhsd", 1, sk, sk, 1, 1, d, scale, (-1, 0), 0)
    w.q, w.k, w.v, w.dout = (t[:, -sk:].permute(0, 2, 1, 3).cpu() for t in (q1, k1, v1, g1))
    last = lambda t: synth.f64(t[:, :, 63:64].permute(0, 2, 1, 3).cpu())
    check_grads([last(dq[:, sq - sk:]), last(dk), last(dv)], oracle_backward(w), "bf16", "head 63")
    # rows that see no key have zero gradients
    for r0 in range(0, sq - sk, 2 ** 18):
        r1 = min(r0 + 2 ** 18, sq - sk)
        assert dq[:, r0:r1].abs().max().item() == 0, f"rows {r0}..{r1}"
    del q1, g1, k1, v1, o1, lse1, dq, dk, dv
    _free()


def test_merge_rows_beyond_one_grid():
    # fp32, head_dim 32: 32 rows per workgroup, and the grid is capped at 2^20 workgroups, so
    # 2^25 + 2^23 + 5 rows take a second pass; rows of that pass (including both-empty and
    # one-empty rows) and of the first are sampled against the fp64 oracle
    s, d = 2 ** 25 + 2 ** 23 + 5, 32
    say(f"case merge beyond one grid: {s} rows, D{d}")
    gen = torch.Generator(device=DEV).manual_seed(13)
    rnd = lambda *shape: torch.randn(*shape, generator=gen, device=DEV)
    xa, xb, g = (rnd(1, s, 1, d) for _ in range(3))
    la, lb, gl = (3 * rnd(1, 1, s) for _ in range(3))
    la[0, 0, -9:-5] = float("-inf")
    lb[0, 0, -7:-3] = float("-inf")  # rows -7, -6 empty on both sides
    x, lse = S.merge(xa, la, xb, lb, "bshd")
    dxa, dla, dxb, dlb = S.merge_backward(xa, la, xb, lb, g, gl, "bshd")
    torch.cuda.synchronize()
    rng = np.random.default_rng(13)
    split = 2 ** 25  # first row of the second pass
    rows = np.unique(np.concatenate([rng.integers(0, split, 2048), rng.integers(split, s, 4096),
                                     np.arange(split - 3, split + 3), np.arange(s - 64, s)]))
    ri = torch.from_numpy(rows).to(DEV)
    xr = lambda t: synth.f64(t[0, ri, 0].cpu())[None, None]  # [1, 1, rows, D]
    lr = lambda t: synth.f64(t[0, 0, ri].cpu())[None, None]  # [1, 1, rows]
    x_ref, l_ref = oracle.merge_forward(xr(xa), lr(la), xr(xb), lr(lb))
    check_forward(xr(x), lr(lse), x_ref, l_ref, "f32", "merge fwd")
    refs = oracle.merge_backward(xr(xa), lr(la), xr(xb), lr(lb), xr(g), lr(gl))
    for name, a, r in zip(("dx_a", "dlse_a", "dx_b", "dlse_b"), (xr(dxa), lr(dla), xr(dxb), lr(dlb)), refs):
        assert rel_err(a, r) <= G_TOL["f32"], name
    assert (lr(dla)[..., -7:-5] == 0).all() and (lr(dlb)[..., -7:-5] == 0).all()
    del xa, xb, g, la, lb, gl, x, lse, dxa, dla, dxb, dlb
    _free()
