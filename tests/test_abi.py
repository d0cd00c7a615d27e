"""C-ABI boundary on the CPU: the library loads, exports every declared symbol, and its
host-only validation accepts the pages' layouts and rejects the failure classes.

No compute call is made here (no GPU): the *_validate entry points run exactly the checks
that sdpa_fwd / sdpa_bwd / sdpa_merge_* run before any launch.  Host tensors serve as
stand-ins for device buffers: validation never dereferences them.
"""
import os
import re

import numpy as np
import pytest
import torch

import scaled_dot_product_05_amd as S
from oracle import window_mask

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "sdpa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(sdpa_\w+)\(", text, re.M)))


def test_every_declared_symbol_is_exported_and_bound():
    lib = S.lib()
    names = header_functions()
    assert len(names) == 20
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(S.exported_symbols())
    assert S.sdpa_version() == 5


def status_of(fn, *args):
    try:
        fn(*args)
        return "OK"
    except S.SdpaError as e:
        assert S.lib().sdpa_last_error().decode()  # a message is always left
        return e.name


def p1_views(hq=16, hk=1, s=2048, d=64, dtype=torch.float16):
    """TransformerEngine issue 1195: one [s,1,hq+2hk,d] tensor split on the head dim."""
    buf = torch.zeros(s, 1, hq + 2 * hk, d, dtype=dtype)
    q, k, v = buf.split([hq, hk, hk], dim=2)
    return buf, q, k, v


def fwd_status(desc, q, k, v, o, lse, ws=0):
    return status_of(S.sdpa_fwd_validate, desc, q, k, v, o, lse, ws)


def test_packed_views_are_accepted_with_their_own_strides():
    buf, q, k, v = p1_views()
    assert q.stride() == (1152, 1152, 64, 1) and k.stride() == (1152, 1152, 64, 1)
    assert k.data_ptr() - q.data_ptr() == 1024 * 2 and v.data_ptr() - q.data_ptr() == 1088 * 2
    desc = S.make_desc("sbhd", "f16", 1, 2048, 2048, 16, 1, 64, 0.1, (-1, 0))
    o = torch.empty(2048, 1, 16, 64, dtype=torch.float16)
    lse = torch.empty(1, 16, 2048)
    assert fwd_status(desc, q, k, v, o, lse) == "OK"


def test_rejections():
    buf, q, k, v = p1_views()
    o = torch.empty(2048, 1, 16, 64, dtype=torch.float16)
    lse = torch.empty(1, 16, 2048)
    good = lambda **kw: S.make_desc(**{**dict(layout="sbhd", dtype="f16", batch=1, seqlen_q=2048,
                                              seqlen_k=2048, heads_q=16, heads_kv=1, head_dim=64,
                                              softmax_scale=1.0, window=(-1, 0)), **kw})
    # last stride must be 1 (a d-strided view)
    wide = torch.empty(2048, 1, 16, 128, dtype=torch.float16)[..., ::2]
    assert fwd_status(good(), wide, k, v, o, lse) == "ERR_STRIDE"
    # output aliasing an input, or overlapping itself, or the LSE overlapping O
    assert fwd_status(good(), q, k, v, q, lse) == "ERR_ALIAS"
    assert fwd_status(good(), q, k, v, buf[:, :, 2:, :], lse) == "ERR_ALIAS"
    bcast = torch.empty(1, 1, 16, 64, dtype=torch.float16).expand(2048, 1, 16, 64)
    assert fwd_status(good(), q, k, v, bcast, lse) == "ERR_STRIDE"
    o32 = torch.empty(2048 * 16 * 64 // 2)
    o_in = o32.view(torch.float16).view(2048, 1, 16, 64)
    assert fwd_status(good(), q, k, v, o_in, o32[:16 * 2048].view(1, 16, 2048)) == "ERR_ALIAS"
    # shapes and options
    k3 = torch.empty(2048, 1, 3, 64, dtype=torch.float16)
    assert fwd_status(good(heads_kv=3), q, k3, k3, o, lse) == "ERR_SHAPE"
    assert fwd_status(good(head_dim=96), q, k, v, o, lse) == "ERR_UNSUPPORTED"
    assert fwd_status(good(layout="bshd", dtype="f16", softmax_scale=float("nan")), q, k, v, o,
                      lse) == "ERR_ARG"
    bad = good()
    bad.layout = 7
    assert fwd_status(bad, q, k, v, o, lse) == "ERR_ARG"
    assert fwd_status(good(), q, k, v, o, lse) == "OK"
    # a NULL data pointer
    rc = S.lib().sdpa_fwd_validate(good(), S.tensor(None), S.tensor(k), S.tensor(v), S.tensor(o),
                                   S.rowstat(lse), 0)
    assert S.STATUS[rc] == "ERR_NULL" and b"NULL" in S.lib().sdpa_last_error()
    # THD without cu_seqlens
    t = torch.empty(100, 4, 64, dtype=torch.bfloat16)
    thd = S.make_desc("thd", "bf16", 2, 60, 60, 4, 4, 64, 0.125, (-1, 0), total_q=100, total_k=100)
    assert fwd_status(thd, t, t, t, torch.empty_like(t), torch.empty(4, 100)) == "ERR_NULL"


def test_workspace_sizes_and_checks():
    cu = torch.tensor([0, 40, 100], dtype=torch.int32)
    t = torch.empty(100, 4, 64, dtype=torch.bfloat16)
    thd = S.make_desc("thd", "bf16", 2, 60, 60, 4, 4, 64, 0.125, (-1, 0), cu_seqlens_q=cu,
                      total_q=100, total_k=100)
    n = S.sdpa_fwd_workspace_size(thd)
    assert n > 0
    o, lse = torch.empty_like(t), torch.empty(4, 100)
    assert fwd_status(thd, t, t, t, o, lse, n) == "OK"
    assert fwd_status(thd, t, t, t, o, lse, n - 1) == "ERR_WORKSPACE"
    dense = S.make_desc("bshd", "bf16", 2, 50, 50, 4, 4, 64, 0.125)
    assert S.sdpa_fwd_workspace_size(dense) == 0
    assert S.sdpa_bwd_workspace_size(dense) >= 2 * 4 * 50 * 4


def test_grids_beyond_32bit_work_items_are_refused():
    # A dispatch counts its work-items in 32 bits and the tile kernels launch at most 4 per
    # query and per key row (rows padded to 128 per sequence and head): with 64 heads, 2^23
    # query and key rows each is the first size refused, dense and THD alike.
    ok = S.make_desc("bshd", "bf16", 1, 2 ** 23 - 128, 2 ** 23 - 128, 64, 64, 64, 0.125)
    assert S.sdpa_bwd_workspace_size(ok) >= 2 * 4 * 64 * (2 ** 23 - 128)
    assert S.sdpa_fwd_workspace_size(ok) == 0
    for fn in (S.sdpa_fwd_workspace_size, S.sdpa_bwd_workspace_size):
        with pytest.raises(S.SdpaError) as e:
            fn(S.make_desc("bshd", "bf16", 1, 2 ** 23, 2 ** 23, 64, 64, 64, 0.125))
        assert e.value.name == "ERR_UNSUPPORTED" and "too large" in str(e.value)
    cu = torch.tensor([0, 40, 100], dtype=torch.int32)
    rows = 2 ** 23 - 2 * 128 - 1  # THD: each of 2 sequences may add a partial tile
    thd_ok = S.make_desc("thd", "bf16", 2, 60, 60, 64, 64, 64, 0.125, cu_seqlens_q=cu,
                         total_q=rows, total_k=rows)
    assert S.sdpa_fwd_workspace_size(thd_ok) > 0
    with pytest.raises(S.SdpaError) as e:
        S.sdpa_fwd_workspace_size(S.make_desc("thd", "bf16", 2, 60, 60, 64, 64, 64, 0.125,
                                              cu_seqlens_q=cu, total_q=rows + 1, total_k=rows + 1))
    assert e.value.name == "ERR_UNSUPPORTED"


def bwd_status(desc, q, k, v, o, lse, do, dlse, dq, dk, dv, ws):
    return status_of(S.sdpa_bwd_validate, desc, q, k, v, o, lse, do, dlse, dq, dk, dv, ws)


def test_backward_outputs_as_packed_views_are_accepted():
    # gradients written into one packed [s,1,hq+2hk,d] buffer: disjoint head ranges
    _, q, k, v = p1_views(hq=8, hk=2, s=256)
    gbuf, dq, dk, dv = p1_views(hq=8, hk=2, s=256)
    o = torch.empty(256, 1, 8, 64, dtype=torch.float16)
    do = torch.empty_like(o)
    lse = torch.empty(1, 8, 256)
    desc = S.make_desc("sbhd", "f16", 1, 256, 256, 8, 2, 64, 0.125, (-1, 0))
    ws = S.sdpa_bwd_workspace_size(desc)
    assert bwd_status(desc, q, k, v, o, lse, do, None, dq, dk, dv, ws) == "OK"
    assert bwd_status(desc, q, k, v, o, lse, do, None, dq, dk, dv, ws - 4) == "ERR_WORKSPACE"
    # dk and dv pointing at the same heads overlap
    assert bwd_status(desc, q, k, v, o, lse, do, None, dq, dk, dk, ws) == "ERR_ALIAS"
    # dq overlapping an input (dO)
    assert bwd_status(desc, q, k, v, o, lse, do, None, do, dk, dv, ws) == "ERR_ALIAS"


def test_row_sliced_views_of_one_buffer_are_accepted():
    # the local+global split: dq over all 512 rows, dk/dv over rows 0..63 of one [1,512,768]
    g = torch.empty(1, 512, 768)
    dq = g[:, :, :256].unflatten(2, (4, 64))
    dk = g[:, :64, 256:512].unflatten(2, (4, 64))
    dv = g[:, :64, 512:].unflatten(2, (4, 64))
    x = torch.empty(1, 512, 768)
    q = x[:, :, :256].unflatten(2, (4, 64))
    k = x[:, :64, 256:512].unflatten(2, (4, 64))
    v = x[:, :64, 512:].unflatten(2, (4, 64))
    o, do = torch.empty(1, 512, 4, 64), torch.empty(1, 512, 4, 64)
    lse = torch.empty(1, 4, 512)
    desc = S.make_desc("bshd", "f32", 1, 512, 64, 4, 4, 64, 0.125, (-1, 0))
    ws = S.sdpa_bwd_workspace_size(desc)
    assert bwd_status(desc, q, k, v, o, lse, do, lse, dq, dk, dv, ws) == "OK"
    # rows 0..63 of dk against rows 32..95 of the same columns overlap
    dv_bad = g[:, 32:96, 256:512].unflatten(2, (4, 64))
    assert bwd_status(desc, q, k, v, o, lse, do, lse, dq, dk, dv_bad, ws) == "ERR_ALIAS"


def test_merge_validation():
    xa, xb, x = (torch.empty(1, 512, 4, 64) for _ in range(3))
    la, lb, l = (torch.empty(1, 4, 512) for _ in range(3))
    md = S.make_merge_desc("bshd", "f32", 1, 512, 4, 64)
    assert status_of(S.sdpa_merge_fwd_validate, md, xa, la, xb, lb, x, l) == "OK"
    assert status_of(S.sdpa_merge_fwd_validate, md, xa, la, xb, lb, xa, l) == "ERR_ALIAS"
    assert status_of(S.sdpa_merge_fwd_validate, md, xa, la, xb, lb, x, la) == "ERR_ALIAS"
    g, dxa, dxb = (torch.empty(1, 512, 4, 64) for _ in range(3))
    dla, dlb = torch.empty(1, 4, 512), torch.empty(1, 4, 512)
    assert status_of(S.sdpa_merge_bwd_validate, md, xa, la, xb, lb, g, None, dxa, dla, dxb,
                     dlb) == "OK"
    assert status_of(S.sdpa_merge_bwd_validate, md, xa, la, xb, lb, g, None, dxa, dla, dxa,
                     dlb) == "ERR_ALIAS"
    md96 = S.make_merge_desc("bshd", "f32", 1, 512, 4, 96)
    x96 = torch.empty(1, 512, 4, 96)
    assert status_of(S.sdpa_merge_fwd_validate, md96, x96, la, x96, lb, torch.empty_like(x96),
                     l) == "ERR_UNSUPPORTED"


@pytest.mark.parametrize("sq,sk,window,align", [(100, 100, (-1, 0), 0), (64, 200, (-1, 0), 1),
                                                (300, 300, (128, 0), 0), (50, 70, (3, -2), 1),
                                                (40, 40, (-1, -129), 0), (33, 17, (-1, -1), 0)])
def test_visible_pair_count_matches_the_mask(sq, sk, window, align):
    assert S.n_visible(sq, sk, window, align) == int(window_mask(sq, sk, *window, align).sum())


def test_cp_validation_on_host():
    import torch
    q = torch.empty(2, 192, 4, 64, dtype=torch.bfloat16)
    pr = S.Problem(q, q, "bshd", 0.125, (-1, 0))
    assert S.sdpa_cp_workspace_size(pr.desc, 2) > 0
    # seqlen 192 is not a multiple of 2 * 5
    with pytest.raises(S.SdpaError) as e:
        S.sdpa_cp_workspace_size(pr.desc, 5)
    assert e.value.args[0] == "SDPA_ERR_SHAPE" or "SHAPE" in str(e.value)
    # a sliding window is not a ring-decomposable mask here
    pw = S.Problem(q, q, "bshd", 0.125, (128, 0))
    with pytest.raises(S.SdpaError):
        S.sdpa_cp_workspace_size(pw.desc, 2)
    # THD: self-attention with q and k sharing cu_seqlens; any sequence lengths
    cu = torch.tensor([0, 96, 192], dtype=torch.int32)
    pt = S.Problem(q[0], q[0], "thd", 0.125, (-1, 0), cu_seqlens_q=cu, max_seqlen_q=96)
    assert S.sdpa_cp_workspace_size(pt.desc, 5) > 0
    cu2 = torch.tensor([0, 96, 192], dtype=torch.int32)
    px = S.Problem(q[0], q[0], "thd", 0.125, (-1, 0), cu_seqlens_q=cu, cu_seqlens_k=cu2,
                   max_seqlen_q=96)
    with pytest.raises(S.SdpaError) as e:
        S.sdpa_cp_workspace_size(px.desc, 2)
    assert e.value.name == "ERR_UNSUPPORTED"
    # hop_order must be a permutation
    o = torch.empty_like(q)
    lse = torch.empty(2, 4, 192)
    ws = torch.empty(S.sdpa_cp_workspace_size(pr.desc, 2), dtype=torch.uint8)
    with pytest.raises(S.SdpaError):
        S.sdpa_cp_fwd(pr.desc, 2, [0, 0], q, q, q, o, lse, ws)


class _FakeMask:
    """Host stand-in for a device BlockMask: validation never reads the arrays."""

    def __init__(self, batch, heads):
        self.buf = torch.zeros(64, dtype=torch.int64)
        p = self.buf.data_ptr()
        self.desc = S.BlockMaskDesc(batch, heads, p, p, p, p, p)


def _bm_problem(dtype, d=64, sq=512, sk=512, hq=4, hk=4, b=2, mask=None, layout="bshd",
                aligned=True):
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    q = torch.zeros(b, sq, hq, d, dtype=tdt)
    k = torch.zeros(b, sk, hk, d, dtype=tdt)
    v = torch.zeros(b, sk, hk, d, dtype=tdt)
    if not aligned:  # rows that start 2 elements past a 16-byte boundary
        big = torch.zeros(b, sq, hq, d + 2, dtype=tdt)
        q = big[..., 2:]
    o = torch.zeros(b, sq, hq, d, dtype=tdt)
    lse = torch.zeros(b, hq, sq, dtype=torch.float32)
    desc = S.make_desc(layout, dtype, b, sq, sk, hq, hk, d, 0.125, (-1, 0), block_mask=mask)
    return desc, q, k, v, o, lse


def test_block_mask_validation_on_host():
    m = _FakeMask(1, 1)
    for dt in ("bf16", "f16", "f32"):
        desc, q, k, v, o, lse = _bm_problem(dt, mask=m)
        assert fwd_status(desc, q, k, v, o, lse) == "OK"
        dq, dk, dv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)
        ws = S.sdpa_bwd_workspace_size(desc)
        assert status_of(S.sdpa_bwd_validate, desc, q, k, v, o, lse, o.clone(), None, dq, dk, dv,
                         ws) == "OK"
    # extents: 1 or the problem's batch / q heads
    assert fwd_status(*_bm_problem("bf16", mask=_FakeMask(2, 4))) == "OK"
    assert fwd_status(*_bm_problem("bf16", mask=_FakeMask(3, 1))) == "ERR_SHAPE"
    assert fwd_status(*_bm_problem("bf16", mask=_FakeMask(1, 2))) == "ERR_SHAPE"
    # NULL arrays
    bad = _FakeMask(1, 1)
    bad.desc.q_list = None
    assert fwd_status(*_bm_problem("bf16", mask=bad)) == "ERR_NULL"
    # keys above the staged list length
    assert fwd_status(*_bm_problem("bf16", sk=512 * 128 + 1, mask=m)) == "ERR_UNSUPPORTED"
    # 16-bit rows the pipelined kernels cannot take
    assert fwd_status(*_bm_problem("bf16", mask=m, aligned=False)) == "ERR_UNSUPPORTED"
    assert fwd_status(*_bm_problem("f32", mask=m, aligned=False)) == "OK"
    # 16-bit backward at head_dim 32
    desc, q, k, v, o, lse = _bm_problem("bf16", d=32, mask=m)
    assert fwd_status(desc, q, k, v, o, lse) == "OK"
    dq, dk, dv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)
    ws = S.sdpa_bwd_workspace_size(desc)
    assert status_of(S.sdpa_bwd_validate, desc, q, k, v, o, lse, o.clone(), None, dq, dk, dv,
                     ws) == "ERR_UNSUPPORTED"
    # per-head masks: the group's column lists must fit the staged list
    desc, q, k, v, o, lse = _bm_problem("bf16", sq=128 * 200, sk=256, hq=4, hk=1, b=1,
                                        mask=_FakeMask(1, 4))
    dq, dk, dv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)
    ws = S.sdpa_bwd_workspace_size(desc)
    assert status_of(S.sdpa_bwd_validate, desc, q, k, v, o, lse, o.clone(), None, dq, dk, dv,
                     ws) == "ERR_UNSUPPORTED"
    # THD takes no block mask
    t = torch.zeros(64, 2, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 64], dtype=torch.int32)
    desc = S.make_desc("thd", "bf16", 1, 64, 64, 2, 2, 64, 0.1, (-1, 0), cu_seqlens_q=cu,
                       total_q=64, total_k=64, block_mask=m)
    assert status_of(S.sdpa_fwd_validate, desc, t, t.clone(), t.clone(), t.clone(),
                     torch.zeros(2, 64), 1 << 20) == "ERR_UNSUPPORTED"


def test_block_mask_build_rejects_bad_arguments():
    m = _FakeMask(1, 1)
    assert status_of(S.sdpa_block_mask_build, m.desc, 0, 64) == "ERR_SHAPE"
    assert status_of(S.sdpa_block_mask_build, m.desc, 64, (1 << 28)) == "ERR_SHAPE"
    bad = _FakeMask(0, 1)
    assert status_of(S.sdpa_block_mask_build, bad.desc, 64, 64) == "ERR_SHAPE"
    bad = _FakeMask(1, 1)
    bad.desc.bits = None
    assert status_of(S.sdpa_block_mask_build, bad.desc, 64, 64) == "ERR_NULL"


def test_fp8_validation_on_host():
    b, s_, h, d = 1, 256, 4, 64
    q = torch.zeros(b, s_, h, d, dtype=torch.uint8)
    k, v = q.clone(), q.clone()
    o = torch.zeros(b, s_, h, d, dtype=torch.bfloat16)
    lse = torch.zeros(b, h, s_, dtype=torch.float32)
    desc = S.make_desc("bshd", "e4m3", b, s_, s_, h, h, d, 0.125, (-1, 0))
    assert status_of(S.sdpa_fwd_fp8_validate, desc, q, k, v, o, lse) == "OK"
    # the other entry points take no FP8
    assert fwd_status(desc, q, k, v, o, lse) == "ERR_UNSUPPORTED"
    ws = S.sdpa_bwd_workspace_size(desc)
    assert status_of(S.sdpa_bwd_validate, desc, q, k, v, o, lse, o, None, q.clone(), k.clone(),
                     v.clone(), ws) == "ERR_UNSUPPORTED"
    # fp16 / bf16 / fp32 descriptors do not take the FP8 call
    d16 = S.make_desc("bshd", "bf16", b, s_, s_, h, h, d, 0.125, (-1, 0))
    assert status_of(S.sdpa_fwd_fp8_validate, d16, q, k, v, o, lse) == "ERR_UNSUPPORTED"
    # head_dim 32, unaligned rows
    d32 = S.make_desc("bshd", "e4m3", b, s_, s_, h, h, 32, 0.125, (-1, 0))
    q32 = torch.zeros(b, s_, h, 32, dtype=torch.uint8)
    o32 = torch.zeros(b, s_, h, 32, dtype=torch.bfloat16)
    assert status_of(S.sdpa_fwd_fp8_validate, d32, q32, q32.clone(), q32.clone(), o32,
                     lse) == "ERR_UNSUPPORTED"
    big = torch.zeros(b, s_, h, d + 8, dtype=torch.uint8)
    assert status_of(S.sdpa_fwd_fp8_validate, desc, big[..., 8:], k, v, o, lse) == "ERR_UNSUPPORTED"
    # O (bf16) over the bytes of an input
    buf = torch.zeros(b, s_, h, 2 * d, dtype=torch.uint8)
    qa = buf[..., :d]
    oa = buf.view(torch.bfloat16)
    assert status_of(S.sdpa_fwd_fp8_validate, desc, qa, k, v, oa, lse) == "ERR_ALIAS"
