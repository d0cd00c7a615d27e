"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each test names what fixes the expected value: a closed form, an invariant of the
mathematics, finite differences, PyTorch's float64 CPU attention / autograd (library
routines that share nothing with the oracle), or a value printed on the pages
(fixtures under tests/golden/).  A dropped term, a wrong sign, a wrong index or a
transposed operand anywhere in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import (attention_backward, attention_forward, merge_backward, merge_forward,
                    window_mask)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def torch_sdpa(q, k, v, scale, mask=None, bias=None):
    """PyTorch float64 CPU attention (math path) with K/V expanded to the q heads."""
    g = q.shape[1] // k.shape[1]
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64) for a in (q, k, v))
    tk = tk.repeat_interleave(g, dim=1)
    tv = tv.repeat_interleave(g, dim=1)
    attn_mask = None
    if mask is not None or bias is not None:
        m = torch.zeros(q.shape[0], q.shape[1], q.shape[2], k.shape[2], dtype=torch.float64)
        if bias is not None:
            m = m + torch.tensor(np.broadcast_to(bias, m.shape).copy())
        if mask is not None:
            m = m.masked_fill(~torch.tensor(np.broadcast_to(mask, m.shape).copy()), -math.inf)
        attn_mask = m
    return F.scaled_dot_product_attention(tq, tk, tv, attn_mask=attn_mask, scale=scale)


# ---------------------------------------------------------------------------------------
# masks
# ---------------------------------------------------------------------------------------

def test_causal_window_is_lower_triangle():
    # window (-1, 0) is causal: key j visible to query i iff j <= i
    vis = window_mask(7, 7, -1, 0)
    assert (vis == np.tril(np.ones((7, 7), bool))).all()


def test_sliding_window_matches_flex_predicate():
    # issue 135161: (q_idx >= kv_idx) & (q_idx - kv_idx <= n_local_band) is window (band, 0)
    band, n = 5, 17
    vis = window_mask(n, n, band, 0)
    for qi in range(n):
        for kj in range(n):
            assert vis[qi, kj] == ((qi >= kj) and (qi - kj <= band))
    # every row past the band sees band + 1 keys
    assert (vis.sum(1)[band:] == band + 1).all()


def test_global_v2_predicate_is_negative_right_window():
    # issue 135161 global_causal_v2: (q >= kv) & (q - kv > band) == window (-1, -(band+1))
    band, n = 4, 13
    vis = window_mask(n, n, -1, -(band + 1))
    for qi in range(n):
        for kj in range(n):
            assert vis[qi, kj] == ((qi >= kj) and (qi - kj > band))


def test_bottom_right_alignment():
    # Sq < Sk, bottom-right: the last query sees every key, query i sees keys j <= i + Sk - Sq
    vis = window_mask(3, 8, -1, 0, diag_align=1)
    assert vis.sum(1).tolist() == [6, 7, 8]
    vis_tl = window_mask(3, 8, -1, 0, diag_align=0)
    assert vis_tl.sum(1).tolist() == [1, 2, 3]


def test_global_v1_sliced_rows_equal_v2_rows():
    # v1 applies q_idx > kv_idx to query rows sliced from `band` on (local index), v2 applies
    # (q >= kv) & (q - kv > band) to all rows: same absolute predicate on rows >= band.
    band, n = 4, 13
    v1 = window_mask(n - band, n, -1, -(band + 1), diag_align=1)
    for ql in range(n - band):
        for kj in range(n):
            assert v1[ql, kj] == (ql > kj)
    v2 = window_mask(n, n, -1, -(band + 1))
    assert (v1 == v2[band:]).all()


# ---------------------------------------------------------------------------------------
# forward: closed forms
# ---------------------------------------------------------------------------------------

def test_uniform_v_gives_that_value():
    q, k = rnd(1, 2, 3, 9, 4), rnd(2, 2, 3, 11, 4)
    v = np.broadcast_to(np.array([0.5, -2.0, 3.0, 7.0]), (2, 3, 11, 4)).copy()
    o, lse = oracle.windowed_forward(q, k, v, 0.7, (3, 2))
    has_key = np.isfinite(lse)
    assert has_key.all()
    assert np.allclose(o, v[:, :, :9], atol=1e-14)


def test_single_key():
    q, k, v = rnd(3, 1, 2, 5, 4), rnd(4, 1, 2, 1, 4), rnd(5, 1, 2, 1, 4)
    o, lse = oracle.windowed_forward(q, k, v, 0.3)
    assert np.allclose(o, np.broadcast_to(v, o.shape), atol=1e-14)
    s = 0.3 * np.einsum("bhid,bhjd->bhij", q, k)[..., 0]
    assert np.allclose(lse, s, atol=1e-14)


def test_diagonal_window_selects_own_key():
    q, k, v = rnd(6, 1, 2, 6, 4), rnd(7, 1, 2, 6, 4), rnd(8, 1, 2, 6, 4)
    o, lse = oracle.windowed_forward(q, k, v, 0.5, (0, 0))
    assert np.allclose(o, v, atol=1e-14)
    assert np.allclose(lse, 0.5 * (q * k).sum(-1), atol=1e-14)


@pytest.mark.parametrize("window,count", [((-1, 0), lambda i: i + 1),
                                          ((128, 0), lambda i: min(i, 128) + 1)])
def test_zero_q_gives_mean_and_log_count(window, count):
    s = 300
    q = np.zeros((1, 1, s, 8))
    k, v = rnd(9, 1, 1, s, 8), rnd(10, 1, 1, s, 8)
    o, lse = oracle.windowed_forward(q, k, v, 0.125, window)
    for i in (0, 1, 5, 127, 128, 129, 200, s - 1):
        n = count(i)
        assert lse[0, 0, i] == pytest.approx(math.log(n), abs=1e-13)
        lo = i - n + 1
        assert np.allclose(o[0, 0, i], v[0, 0, lo:i + 1].mean(0), atol=1e-13)


def test_rows_sum_to_one_and_lse_by_fsum():
    q, k, v = rnd(11, 1, 2, 4, 3), rnd(12, 1, 2, 5, 3), rnd(13, 1, 2, 5, 3)
    o, lse, p = attention_forward(q, k, v, 0.9, window_mask(4, 5, 1, 1), return_p=True)
    vis = window_mask(4, 5, 1, 1)
    for h in range(2):
        for i in range(4):
            assert math.fsum(p[0, h, i]) == pytest.approx(1.0, abs=1e-15)
            terms = [math.exp(0.9 * sum(q[0, h, i, d] * k[0, h, j, d] for d in range(3)))
                     for j in range(5) if vis[i, j]]
            assert lse[0, h, i] == pytest.approx(math.log(math.fsum(terms)), abs=1e-14)
            out = [math.fsum(p[0, h, i, j] * v[0, h, j, d] for j in range(5)) for d in range(3)]
            assert np.allclose(o[0, h, i], out, atol=1e-15)
            assert all(p[0, h, i, j] == 0.0 for j in range(5) if not vis[i, j])


# ---------------------------------------------------------------------------------------
# forward: PyTorch float64 attention (a library routine)
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("hq,hk", [(4, 4), (4, 2), (6, 1)])
@pytest.mark.parametrize("window,align", [((-1, -1), 0), ((-1, 0), 0), ((3, 2), 0),
                                          ((-1, 0), 1), ((5, 0), 1)])
def test_forward_matches_torch_sdpa(hq, hk, window, align):
    sq, sk = 9, 13
    q, k, v = rnd(20, 2, hq, sq, 8), rnd(21, 2, hk, sk, 8), rnd(22, 2, hk, sk, 8)
    mask = window_mask(sq, sk, window[0], window[1], align)
    assert mask.any(1).all()
    o, lse = attention_forward(q, k, v, 0.37, mask)
    ref = torch_sdpa(q, k, v, 0.37, mask).numpy()
    assert np.abs(o - ref).max() < 1e-13
    # LSE: PyTorch logsumexp of the masked, scaled scores (K expanded to the q heads)
    g = hq // hk
    tk = torch.tensor(k).repeat_interleave(g, 1)
    s = 0.37 * torch.tensor(q) @ tk.transpose(-1, -2)
    s = s.masked_fill(~torch.tensor(mask), -math.inf)
    assert np.abs(lse - torch.logsumexp(s, -1).numpy()).max() < 1e-13


def test_gqa_equals_mha_with_repeated_kv():
    q, k, v = rnd(30, 1, 8, 7, 4), rnd(31, 1, 2, 7, 4), rnd(32, 1, 2, 7, 4)
    mask = window_mask(7, 7, -1, 0)
    o, lse = attention_forward(q, k, v, 0.5, mask)
    o2, lse2 = attention_forward(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 0.5, mask)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_fully_masked_row_is_zero_and_neg_inf():
    # window (-1, -3): rows 0..2 see no key
    q, k, v = rnd(33, 1, 2, 6, 4), rnd(34, 1, 2, 6, 4), rnd(35, 1, 2, 6, 4)
    o, lse = oracle.windowed_forward(q, k, v, 1.0, (-1, -3))
    assert (o[:, :, :3] == 0).all() and np.isneginf(lse[:, :, :3]).all()
    assert np.isfinite(lse[:, :, 3:]).all()
    dout = rnd(36, 1, 2, 6, 4)
    dq, dk, dv = oracle.windowed_backward(q, k, v, dout, 1.0, (-1, -3), dlse=rnd(37, 1, 2, 6))
    assert (dq[:, :, :3] == 0).all()
    # keys 4, 5 are never visible (query i sees j <= i - 3 <= 2)
    assert (dk[:, :, 3:] == 0).all() and (dv[:, :, 3:] == 0).all()


# ---------------------------------------------------------------------------------------
# backward: finite differences, PyTorch autograd, identities
# ---------------------------------------------------------------------------------------

def _loss(q, k, v, scale, mask, g, gl):
    o, lse = attention_forward(q, k, v, scale, mask)
    fin = np.isfinite(lse)
    return (o * g).sum() + (np.where(fin, lse, 0.0) * gl).sum()


@pytest.mark.parametrize("hq,hk,window", [(2, 2, (-1, -1)), (4, 2, (-1, 0)), (3, 1, (2, 1))])
def test_backward_finite_differences(hq, hk, window):
    sq, sk, d, scale = 5, 6, 3, 0.8
    q, k, v = rnd(40, 1, hq, sq, d), rnd(41, 1, hk, sk, d), rnd(42, 1, hk, sk, d)
    g, gl = rnd(43, 1, hq, sq, d), rnd(44, 1, hq, sq)
    mask = window_mask(sq, sk, window[0], window[1])
    dq, dk, dv = attention_backward(q, k, v, g, scale, mask, dlse=gl)
    h = 1e-6
    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = _loss(q, k, v, scale, mask, g, gl)
            arr[idx] = old - h
            lm = _loss(q, k, v, scale, mask, g, gl)
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        assert np.abs(num - grad).max() < 1e-7 * max(1.0, np.abs(grad).max())


@pytest.mark.parametrize("hq,hk,window,align", [(4, 4, (-1, 0), 0), (4, 1, (3, 0), 0),
                                                (6, 2, (-1, -1), 0), (2, 2, (-1, 0), 1)])
def test_backward_matches_torch_autograd(hq, hk, window, align):
    sq, sk, d, scale = 10, 12, 8, 0.3
    q, k, v = rnd(50, 2, hq, sq, d), rnd(51, 2, hk, sk, d), rnd(52, 2, hk, sk, d)
    g = rnd(53, 2, hq, sq, d)
    mask = window_mask(sq, sk, window[0], window[1], align)
    dq, dk, dv = attention_backward(q, k, v, g, scale, mask)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    gg = hq // hk
    am = torch.zeros(sq, sk, dtype=torch.float64).masked_fill(~torch.tensor(mask), -math.inf)
    out = F.scaled_dot_product_attention(tq, tk.repeat_interleave(gg, 1),
                                         tv.repeat_interleave(gg, 1), attn_mask=am, scale=scale)
    (out * torch.tensor(g)).sum().backward()
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.abs(mine - ref.numpy()).max() < 1e-12


def test_backward_dlse_term_matches_torch_autograd():
    # gradient through LSE alone: L = sum(LSE * gl), PyTorch autograd of logsumexp
    q, k, v = rnd(60, 1, 2, 6, 4), rnd(61, 1, 2, 7, 4), rnd(62, 1, 2, 7, 4)
    gl = rnd(63, 1, 2, 6)
    mask = window_mask(6, 7, 2, 1)
    dq, dk, dv = attention_backward(q, k, v, np.zeros((1, 2, 6, 4)), 0.6, mask, dlse=gl)
    tq, tk = torch.tensor(q, requires_grad=True), torch.tensor(k, requires_grad=True)
    s = (0.6 * tq @ tk.transpose(-1, -2)).masked_fill(~torch.tensor(mask), -math.inf)
    (torch.logsumexp(s, -1) * torch.tensor(gl)).sum().backward()
    assert np.abs(dq - tq.grad.numpy()).max() < 1e-13
    assert np.abs(dk - tk.grad.numpy()).max() < 1e-13
    assert np.abs(dv).max() == 0.0


def test_backward_identities():
    # K translation invariance, sum of dV, and the Q<->K scaling invariance
    hq, hk, s, d, scale = 4, 2, 16, 5, 0.45
    q, k, v = rnd(70, 1, hq, s, d), rnd(71, 1, hk, s, d), rnd(72, 1, hk, s, d)
    g, gl = rnd(73, 1, hq, s, d), rnd(74, 1, hq, s)
    dq, dk, dv = oracle.windowed_backward(q, k, v, g, scale, (4, 0), dlse=gl)
    grp = hq // hk
    for kv in range(hk):
        heads = range(kv * grp, (kv + 1) * grp)
        lhs = dk[0, kv].sum(0)
        rhs = scale * sum((gl[0, h][:, None] * q[0, h]).sum(0) for h in heads)
        assert np.allclose(lhs, rhs, atol=1e-12)
        assert np.allclose(dv[0, kv].sum(0), sum(g[0, h].sum(0) for h in heads), atol=1e-12)
    lhs = (q * dq).sum()
    rhs = sum((k[0, kv] * dk[0, kv]).sum() for kv in range(hk))
    assert lhs == pytest.approx(rhs, abs=1e-11)


def _torch_attention_with_lse(q, k, v, scale, vis):
    """PyTorch float64 SDPA (boolean mask, K/V expanded to the q heads) plus the LSE as
    torch.logsumexp of the masked scores; every row of ``vis`` must see a key.  Returns
    the leaf tensors too, for autograd."""
    g = q.shape[1] // k.shape[1]
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    tm = torch.tensor(np.broadcast_to(vis, (q.shape[0], q.shape[1], q.shape[2], k.shape[2])).copy())
    ke, ve = tk.repeat_interleave(g, 1), tv.repeat_interleave(g, 1)
    out = F.scaled_dot_product_attention(tq, ke, ve, attn_mask=tm, scale=scale)
    sc = (scale * tq @ ke.transpose(-1, -2)).masked_fill(~tm, -math.inf)
    return out, torch.logsumexp(sc, -1), (tq, tk, tv)


def _random_element_mask(seed, shape, window, align, density=0.6):
    """Random boolean element bits [B,H,Sq,Sk]; each row keeps one key that the window admits
    (so every row of mask AND window sees a key and PyTorch's SDPA is defined)."""
    rng = np.random.default_rng(seed)
    m = rng.random(shape) < density
    wm = window_mask(shape[2], shape[3], window[0], window[1], align)
    assert wm.any(1).all()
    first = wm.argmax(1)
    m[..., np.arange(shape[2]), first] = True
    return m


@pytest.mark.parametrize("window,align,sq,sk", [((3, 2), 0, 11, 13), ((-1, 0), 1, 9, 14),
                                                ((-1, -129), 1, 7, 140), ((-1, -1), 0, 8, 10)])
def test_masked_forward_backward_match_torch(window, align, sq, sk):
    # the block-sparse path's result: element bits AND the window, against PyTorch float64
    # SDPA and autograd under (bits & window); dropping either side of the AND fails here
    hq, hk, d, scale = 4, 2, 6, 0.45
    q, k, v = rnd(160, 2, hq, sq, d), rnd(161, 2, hk, sk, d), rnd(162, 2, hk, sk, d)
    g, gl = rnd(163, 2, hq, sq, d), rnd(164, 2, hq, sq)
    bits = _random_element_mask(165, (2, hq, sq, sk), window, align)
    vis = bits & window_mask(sq, sk, window[0], window[1], align)
    assert not (vis == bits).all() or window == (-1, -1)
    o, lse = oracle.masked_forward(q, k, v, scale, bits, window, align)
    out, tl, (tq, tk, tv) = _torch_attention_with_lse(q, k, v, scale, vis)
    assert np.abs(o - out.detach().numpy()).max() < 1e-13
    assert np.abs(lse - tl.detach().numpy()).max() < 1e-13
    dq, dk, dv = oracle.masked_backward(q, k, v, g, scale, bits, window, align, dlse=gl)
    ((out * torch.tensor(g)).sum() + (tl * torch.tensor(gl)).sum()).backward()
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.abs(mine - ref.numpy()).max() < 1e-12


def test_masked_rows_without_keys_are_zero():
    # element bits that leave rows 1 and 4 empty (and key 2 never visible): O = 0,
    # LSE = -inf, no gradient on those rows, none into the invisible key
    q, k, v = rnd(170, 1, 2, 6, 4), rnd(171, 1, 2, 7, 4), rnd(172, 1, 2, 7, 4)
    bits = np.ones((6, 7), bool)
    bits[[1, 4]] = False
    bits[:, 2] = False
    o, lse = oracle.masked_forward(q, k, v, 0.8, bits, (-1, -1))
    assert (o[:, :, [1, 4]] == 0).all() and np.isneginf(lse[:, :, [1, 4]]).all()
    assert np.isfinite(lse[:, :, [0, 2, 3, 5]]).all()
    dq, dk, dv = oracle.masked_backward(q, k, v, rnd(173, 1, 2, 6, 4), 0.8, bits, (-1, -1),
                                        dlse=rnd(174, 1, 2, 6))
    assert (dq[:, :, [1, 4]] == 0).all() and (dk[:, :, 2] == 0).all() and (dv[:, :, 2] == 0).all()


def test_backward_random_mask_finite_differences():
    # attention_backward with an arbitrary boolean mask (one row fully masked), against
    # central differences of L = sum(O g) + sum(LSE gl) over rows with a visible key
    hq, hk, sq, sk, d, scale = 2, 1, 5, 6, 3, 0.9
    q, k, v = rnd(175, 1, hq, sq, d), rnd(176, 1, hk, sk, d), rnd(177, 1, hk, sk, d)
    g, gl = rnd(178, 1, hq, sq, d), rnd(179, 1, hq, sq)
    mask = np.random.default_rng(180).random((1, hq, sq, sk)) < 0.5
    mask[0, 0, 2] = False
    mask[0, 1, 3] = False
    mask[0, 1, 3, 4] = True
    dq, dk, dv = attention_backward(q, k, v, g, scale, mask, dlse=gl)
    h = 1e-6
    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = _loss(q, k, v, scale, mask, g, gl)
            arr[idx] = old - h
            lm = _loss(q, k, v, scale, mask, g, gl)
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        assert np.abs(num - grad).max() < 1e-7 * max(1.0, np.abs(grad).max())
    assert (dq[0, 0, 2] == 0).all()


def test_backward_random_mask_matches_torch_autograd():
    hq, hk, sq, sk, d, scale = 4, 2, 12, 9, 5, 0.35
    q, k, v = rnd(181, 2, hq, sq, d), rnd(182, 2, hk, sk, d), rnd(183, 2, hk, sk, d)
    g, gl = rnd(184, 2, hq, sq, d), rnd(185, 2, hq, sq)
    mask = _random_element_mask(186, (2, hq, sq, sk), (-1, -1), 0, density=0.4)
    dq, dk, dv = attention_backward(q, k, v, g, scale, mask, dlse=gl)
    out, tl, (tq, tk, tv) = _torch_attention_with_lse(q, k, v, scale, mask)
    ((out * torch.tensor(g)).sum() + (tl * torch.tensor(gl)).sum()).backward()
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.abs(mine - ref.numpy()).max() < 1e-12


@pytest.mark.parametrize("align", [1, 0])
def test_thd_cross_lengths_match_torch_per_sequence(align):
    # packed varlen with cu_seqlens_k != cu_seqlens_q: sequence s is its own problem of
    # Lq_s queries and Lk_s keys; causal aligned bottom-right (query i sees key j iff
    # j <= i + Lk - Lq) or top-left (j <= i).  Reference: PyTorch float64 SDPA per sequence
    # with the mask built by torch.tril; a sequence with no keys gives O = 0, LSE = -inf.
    lq, lk = [4, 7, 3, 5, 2], [6, 3, 3, 0, 9]
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    hq, hk, d, scale = 4, 2, 5, 0.55
    rng = np.random.default_rng(187)
    q, g = rng.standard_normal((cq[-1], hq, d)), rng.standard_normal((cq[-1], hq, d))
    k, v = rng.standard_normal((ck[-1], hk, d)), rng.standard_normal((ck[-1], hk, d))
    gl = rng.standard_normal((hq, cq[-1]))
    o, lse = oracle.thd_forward(q, k, v, cq, ck, scale, (-1, 0), align)
    dq, dk, dv = oracle.thd_backward(q, k, v, g, cq, ck, scale, (-1, 0), align, dlse=gl)
    for s_ in range(len(lq)):
        a, b = cq[s_], cq[s_ + 1]
        c, e = ck[s_], ck[s_ + 1]
        diag = (lk[s_] - lq[s_]) if align else 0
        vis = torch.ones(lq[s_], lk[s_], dtype=torch.bool).tril(diagonal=diag).numpy()
        rows = vis.any(1)
        assert (o[a:b][~rows] == 0).all() and np.isneginf(lse[:, a:b][:, ~rows]).all()
        assert (dq[a:b][~rows] == 0).all()
        if not rows.any():
            continue
        sel = np.flatnonzero(rows)
        bh = lambda t, lo, hi: t[lo:hi].transpose(1, 0, 2)[None]
        out, tl, (tq, tk, tv) = _torch_attention_with_lse(bh(q, a, b)[:, :, sel], bh(k, c, e),
                                                          bh(v, c, e), scale, vis[sel])
        assert np.abs(o[a:b][sel] - out.detach().numpy()[0].transpose(1, 0, 2)).max() < 1e-13
        assert np.abs(lse[:, a:b][:, sel] - tl.detach().numpy()[0]).max() < 1e-13
        loss = (out * torch.tensor(bh(g, a, b)[:, :, sel])).sum() + \
            (tl * torch.tensor(gl[:, a:b][:, sel][None])).sum()
        loss.backward()
        assert np.abs(dq[a:b][sel] - tq.grad.numpy()[0].transpose(1, 0, 2)).max() < 1e-12
        assert np.abs(dk[c:e] - tk.grad.numpy()[0].transpose(1, 0, 2)).max() < 1e-12
        assert np.abs(dv[c:e] - tv.grad.numpy()[0].transpose(1, 0, 2)).max() < 1e-12


# ---------------------------------------------------------------------------------------
# restricted forms used at full size: rows / columns of the same definition
# ---------------------------------------------------------------------------------------

def test_rows_and_columns_agree_with_full():
    hq, hk, s, d, scale, win = 4, 2, 40, 6, 0.4, (9, 0)
    q, k, v = rnd(80, 1, hq, s, d), rnd(81, 1, hk, s, d), rnd(82, 1, hk, s, d)
    g, gl = rnd(83, 1, hq, s, d), rnd(84, 1, hq, s)
    o, lse = oracle.windowed_forward(q, k, v, scale, win)
    dq, dk, dv = oracle.windowed_backward(q, k, v, g, scale, win, dlse=gl)
    rows = [0, 3, 17, 39]
    for h in range(hq):
        orow, lrow = oracle.forward_rows(q[0, h], k[0, h // 2], v[0, h // 2], scale, rows, win)
        assert np.allclose(orow, o[0, h, rows], atol=1e-14)
        assert np.allclose(lrow, lse[0, h, rows], atol=1e-14)
        dqr = oracle.dq_rows(q[0, h], k[0, h // 2], v[0, h // 2], g[0, h], scale, rows, win,
                             dlse_bh=gl[0, h])
        assert np.allclose(dqr, dq[0, h, rows], atol=1e-13)
    cols = [0, 5, 21, 39]
    for kv in range(hk):
        sl = slice(2 * kv, 2 * kv + 2)
        dkc, dvc = oracle.dkdv_cols(q[0, sl], k[0, kv], v[0, kv], g[0, sl], scale, cols, win,
                                    dlse_heads=gl[0, sl], chunk=7)
        assert np.allclose(dkc, dk[0, kv, cols], atol=1e-13)
        assert np.allclose(dvc, dv[0, kv, cols], atol=1e-13)


def test_thd_equal_lengths_equals_batched_dense():
    b, s, hq, hk, d = 3, 9, 4, 2, 5
    q, k, v, g = rnd(90, b, hq, s, d), rnd(91, b, hk, s, d), rnd(92, b, hk, s, d), rnd(93, b, hq, s, d)
    o, lse = oracle.windowed_forward(q, k, v, 0.6, (-1, 0))
    dq, dk, dv = oracle.windowed_backward(q, k, v, g, 0.6, (-1, 0))
    pack = lambda a: a.transpose(0, 2, 1, 3).reshape(b * s, a.shape[1], d)
    cu = np.arange(0, (b + 1) * s, s)
    ot, lt = oracle.thd_forward(pack(q), pack(k), pack(v), cu, cu, 0.6, (-1, 0))
    assert np.allclose(ot, pack(o), atol=1e-15)
    assert np.allclose(lt, lse.transpose(1, 0, 2).reshape(hq, b * s), atol=1e-15)
    a, bb, c = oracle.thd_backward(pack(q), pack(k), pack(v), pack(g), cu, cu, 0.6, (-1, 0))
    assert np.allclose(a, pack(dq)) and np.allclose(bb, pack(dk)) and np.allclose(c, pack(dv))
    # a zero-length sequence contributes no rows and leaves its neighbours unchanged
    cu0 = np.array([0, s, s, 2 * s, 3 * s])
    ot0, _ = oracle.thd_forward(pack(q), pack(k), pack(v), cu0, cu0, 0.6, (-1, 0))
    assert np.allclose(ot0, pack(o), atol=1e-15)


# ---------------------------------------------------------------------------------------
# merge
# ---------------------------------------------------------------------------------------

def _merge_torch(xa, la, xb, lb):
    """The merge as written on issue 135161 (max detached), in PyTorch float64."""
    m = torch.maximum(la, lb).detach()
    ea, eb = torch.exp(la - m), torch.exp(lb - m)
    x = (xa * ea[..., None] + xb * eb[..., None]) / (ea[..., None] + eb[..., None])
    return x, m + torch.log(ea + eb)


def test_merge_forward_and_backward_match_torch_formula_and_autograd():
    xa, xb = rnd(100, 2, 3, 5, 4), rnd(101, 2, 3, 5, 4)
    la, lb = 3 * rnd(102, 2, 3, 5), 3 * rnd(103, 2, 3, 5)
    g, gl = rnd(104, 2, 3, 5, 4), rnd(105, 2, 3, 5)
    x, lse = merge_forward(xa, la, xb, lb)
    t = [torch.tensor(a, requires_grad=True) for a in (xa, la, xb, lb)]
    tx, tl = _merge_torch(*t)
    assert np.abs(x - tx.detach().numpy()).max() < 1e-14
    assert np.abs(lse - tl.detach().numpy()).max() < 1e-14
    ((tx * torch.tensor(g)).sum() + (tl * torch.tensor(gl)).sum()).backward()
    mine = merge_backward(xa, la, xb, lb, g, gl)
    for a, ref in zip(mine, (t[0].grad, t[1].grad, t[2].grad, t[3].grad)):
        assert np.abs(a - ref.numpy()).max() < 1e-13


def test_merge_identity_commutative_associative():
    xa, xb, xc = rnd(110, 3, 6, 4), rnd(111, 3, 6, 4), rnd(112, 3, 6, 4)
    la, lb, lc = rnd(113, 3, 6), rnd(114, 3, 6), rnd(115, 3, 6)
    x, l = merge_forward(xa, la, np.zeros_like(xa), np.full(la.shape, -np.inf))
    assert np.array_equal(x, xa) and np.array_equal(l, la)
    x1, l1 = merge_forward(xa, la, xb, lb)
    x2, l2 = merge_forward(xb, lb, xa, la)
    assert np.allclose(x1, x2, atol=1e-15) and np.allclose(l1, l2, atol=1e-15)
    y1, m1 = merge_forward(*merge_forward(xa, la, xb, lb), xc, lc)
    y2, m2 = merge_forward(xa, la, *merge_forward(xb, lb, xc, lc))
    assert np.allclose(y1, y2, atol=1e-14) and np.allclose(m1, m2, atol=1e-14)
    # two empty partials merge to (0, -inf) with zero gradients
    e = np.full((3, 6), -np.inf)
    x0, l0 = merge_forward(xa, e, xb, e)
    assert (x0 == 0).all() and np.isneginf(l0).all()
    grads = merge_backward(xa, e, xb, e, rnd(116, 3, 6, 4), rnd(117, 3, 6))
    assert all((gr == 0).all() for gr in grads)


def test_merge_backward_finite_differences():
    xa, xb = rnd(120, 1, 2, 3, 4), rnd(121, 1, 2, 3, 4)
    la, lb = rnd(122, 1, 2, 3), rnd(123, 1, 2, 3)
    g, gl = rnd(124, 1, 2, 3, 4), rnd(125, 1, 2, 3)
    grads = merge_backward(xa, la, xb, lb, g, gl)
    loss = lambda: (lambda x, l: (x * g).sum() + (l * gl).sum())(*merge_forward(xa, la, xb, lb))
    for arr, grad in zip((xa, la, xb, lb), grads):
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + 1e-6
            lp = loss()
            arr[idx] = old - 1e-6
            lm = loss()
            arr[idx] = old
            assert (lp - lm) / 2e-6 == pytest.approx(grad[idx], abs=1e-8)


def _p3_split(q, k, v, scale, band, version):
    """Causal attention as local (band,0) + global partial merged by LSE (issue 135161)."""
    s = q.shape[2]
    loc = window_mask(s, s, band, 0)
    xl, ll = attention_forward(q, k, v, scale, loc)
    if version == 2:
        xg, lg = attention_forward(q, k, v, scale, window_mask(s, s, -1, -(band + 1)))
        return merge_forward(xl, ll, xg, lg)
    # v1: global over query rows band.. only, keys absolute, q_idx > kv_idx on local index
    qs = q[:, :, band:]
    xg, lg = attention_forward(qs, k, v, scale, window_mask(s - band, s, -1, -(band + 1), 1))
    xm, lm = merge_forward(xl[:, :, band:], ll[:, :, band:], xg, lg)
    return (np.concatenate([xl[:, :, :band], xm], 2), np.concatenate([ll[:, :, :band], lm], 2))


def test_p3_partition_merges_to_causal_attention():
    # issue 135161 second repro: attn_v1 and attn_v2 agree exactly (eager) and both equal
    # causal attention; the golden fixture holds the page's printed eager differences.
    with open(os.path.join(GOLDEN, "p3_merge_partition.json")) as f:
        gold = json.load(f)
    q, k, v = rnd(130, 1, 2, 40, 8), rnd(131, 1, 2, 40, 8), rnd(132, 1, 2, 40, 8)
    band, scale = 8, 0.35
    causal_o, causal_l = oracle.windowed_forward(q, k, v, scale, (-1, 0))
    for version in (1, 2):
        x, l = _p3_split(q, k, v, scale, band, version)
        assert np.abs(x - causal_o).max() <= gold["eager_max_abs_diff"]["output"] + 1e-14
        assert np.abs(l - causal_l).max() < 1e-13
    # gradients of a sum loss through the v2 split equal causal attention's gradients
    g = np.ones(q.shape)
    s = q.shape[2]
    loc, glb = window_mask(s, s, band, 0), window_mask(s, s, -1, -(band + 1))
    xl, ll = attention_forward(q, k, v, scale, loc)
    xg, lg = attention_forward(q, k, v, scale, glb)
    dxa, dla, dxb, dlb = merge_backward(xl, ll, xg, lg, g)
    ga = attention_backward(q, k, v, dxa, scale, loc, np.where(np.isfinite(ll), dla, 0))
    gb = attention_backward(q, k, v, dxb, scale, glb, np.where(np.isfinite(lg), dlb, 0))
    ref = oracle.windowed_backward(q, k, v, g, scale, (-1, 0))
    for name, a, b, r in zip(("query", "key", "value"), ga, gb, ref):
        assert np.abs(a + b - r).max() <= gold["eager_max_abs_diff"][name] + 1e-13


def test_c5_overlap_merge_is_union_with_log_count_bias():
    # local (128,0) and "first 64 keys, causal" overlap; merging counts shared keys twice,
    # i.e. attention over the union with +ln 2 on each doubly covered score (PyTorch SDPA
    # with an additive float mask is the independent side).
    s, band, nglob, d = 200, 128, 64, 8
    q, k, v = rnd(140, 1, 2, s, d), rnd(141, 1, 2, s, d), rnd(142, 1, 2, s, d)
    loc = window_mask(s, s, band, 0)
    xl, ll = attention_forward(q, k, v, 0.2, loc)
    glob = window_mask(s, nglob, -1, 0)
    xg, lg = attention_forward(q, k[:, :, :nglob], v[:, :, :nglob], 0.2, glob)
    x, l = merge_forward(xl, ll, xg, lg)
    cover = loc.astype(float)
    cover[:, :nglob] += glob
    ref = torch_sdpa(q, k, v, 0.2, mask=cover > 0, bias=np.log(np.maximum(cover, 1))).numpy()
    assert np.abs(x - ref).max() < 1e-13


def test_pages_tolerance_context():
    # the pages' cross-implementation differences sit inside the stated tolerances
    with open(os.path.join(GOLDEN, "p1_fp16_diffs.json")) as f:
        gold = json.load(f)
    assert gold["contiguous_copies"] <= 4e-3 and gold["fixed_scale_0p1"] <= 4e-3
    assert gold["strided_views_wrong"] > 1.0  # the signature of strides read wrongly


def test_cp_load_balanced_ring_fold_equals_causal_attention():
    """"Add support for cuDNN FusedAttention + THD + CP" (TransformerEngine issue 885): a
    sequence cut into 2*cp chunks, rank r holding chunks r and 2*cp-1-r, K/V chunks visited
    in any hop order, each (q chunk, kv chunk) pair attended fully (earlier kv chunk),
    causally (same chunk) or not at all (later chunk), and the partials folded with the LSE
    merge, is causal attention over the whole sequence, and the fold order does not matter.
    Gradients: each pair's backward with the final O and LSE sums to the full backward."""
    rng = np.random.default_rng(885)
    cp, L, d = 3, 5, 4
    s = 2 * cp * L
    q, k, v, g = (rng.standard_normal((1, 2, s, d)) for _ in range(4))
    scale = 0.7
    full_o, full_l = oracle.attention_forward(q, k, v, scale, oracle.window_mask(s, s, -1, 0))
    dq_f, dk_f, dv_f = oracle.attention_backward(q, k, v, g, scale, oracle.window_mask(s, s, -1, 0))
    sl = lambda c: slice(c * L, (c + 1) * L)
    for order in ([0, 1, 2], [2, 0, 1]):
        o = np.zeros_like(full_o)
        l = np.zeros_like(full_l)
        for r in range(cp):
            for i in (r, 2 * cp - 1 - r):
                acc = None
                for h in order:
                    src = (r - h) % cp
                    for c in sorted((src, 2 * cp - 1 - src)):
                        if c > i:
                            continue
                        m = np.ones((L, L), bool) if c < i else np.tril(np.ones((L, L), bool))
                        part = oracle.attention_forward(q[:, :, sl(i)], k[:, :, sl(c)], v[:, :, sl(c)], scale, m)
                        acc = part if acc is None else oracle.merge_forward(*acc, *part)
                o[:, :, sl(i)], l[:, :, sl(i)] = acc
        assert np.abs(o - full_o).max() < 1e-12 and np.abs(l - full_l).max() < 1e-12
    # per-pair backward with the final statistics: P and Delta of full attention
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for i in range(2 * cp):
        for c in range(i + 1):
            m = np.ones((L, L), bool) if c < i else np.tril(np.ones((L, L), bool))
            qi, kc, vc, gi = q[:, :, sl(i)], k[:, :, sl(c)], v[:, :, sl(c)], g[:, :, sl(i)]
            sc = scale * qi[0] @ kc[0].transpose(0, 2, 1)
            p = np.where(m, np.exp(sc - full_l[0, :, sl(i), None]), 0.0)
            delta = (gi[0] * full_o[0, :, sl(i)]).sum(-1)
            dp = gi[0] @ vc[0].transpose(0, 2, 1)
            ds = p * (dp - delta[..., None])
            dq[0, :, sl(i)] += scale * ds @ kc[0]
            dk[0, :, sl(c)] += scale * ds.transpose(0, 2, 1) @ qi[0]
            dv[0, :, sl(c)] += p.transpose(0, 2, 1) @ gi[0]
    for a, b in ((dq, dq_f), (dk, dk_f), (dv, dv_f)):
        assert np.abs(a - b).max() < 1e-12


def test_thd_padded_rows_equal_compact_rows():
    """Padded THD ("Add support for cuDNN FusedAttention + THD + CP", TransformerEngine issue
    885: cu_seqlens_padded): sequence s lives at packed rows [pad[s], pad[s] + len_s); on the
    compacted tensor the same sequence gives the same rows, and padding rows are never
    written (NaN in the oracle's outputs), whatever the padding rows of q/k/v hold."""
    rng = np.random.default_rng(7)
    lengths, gaps = [5, 0, 3, 7], [2, 1, 0, 3]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    pad = np.concatenate([[0], np.cumsum(np.add(lengths, gaps))]).astype(np.int32)
    hq, hk, d = 4, 2, 8
    T, Tp = int(cu[-1]), int(pad[-1])
    q, k, v, g = (rng.standard_normal((T, h, d)) for h in (hq, hk, hk, hq))
    rows = np.concatenate([np.arange(pad[s], pad[s] + lengths[s]) for s in range(len(lengths))])
    def padded(t):
        out = np.full((Tp,) + t.shape[1:], np.nan)
        out[rows] = t
        return out
    o, l = oracle.thd_forward(q, k, v, cu, cu, 0.5, (-1, 0))
    op, lp = oracle.thd_forward(padded(q), padded(k), padded(v), cu, cu, 0.5, (-1, 0), pad_q=pad, pad_k=pad)
    assert np.array_equal(op[rows], o) and np.array_equal(lp[:, rows], l)
    gap_rows = np.setdiff1d(np.arange(Tp), rows)
    assert np.isnan(op[gap_rows]).all() and np.isnan(lp[:, gap_rows]).all()
    grads = oracle.thd_backward(q, k, v, g, cu, cu, 0.5, (-1, 0))
    gradsp = oracle.thd_backward(padded(q), padded(k), padded(v), padded(g), cu, cu, 0.5, (-1, 0),
                                 pad_q=pad, pad_k=pad)
    for a, b in zip(gradsp, grads):
        assert np.array_equal(a[rows], b) and np.isnan(a[gap_rows]).all()


# ---------------------------------------------------------------------------------------
# block-sparse masks (FlexAttention BlockMask model, issue 135161's create_block_mask)
# ---------------------------------------------------------------------------------------

import synth  # noqa: E402  (input generators; no attention arithmetic)
from oracle import block_kinds, block_lists  # noqa: E402
from oracle.block_mask import EMPTY, FULL, PARTIAL  # noqa: E402


@pytest.mark.parametrize("s", [512, 300])
def test_block_kinds_causal_closed_form(s):
    # q >= kv: a block row qb sees every key of earlier block columns, its own diagonal
    # block in part, and nothing after it (also with a ragged last block).
    k = block_kinds(synth.flex_mask("causal", s, s))
    n = -(-s // 128)
    want = np.array([[FULL if kb < qb else PARTIAL if kb == qb else EMPTY for kb in range(n)]
                     for qb in range(n)])
    assert (k == want).all()


@pytest.mark.parametrize("band", [128, 256])
def test_block_kinds_sliding_window_closed_form(band):
    # (q >= kv) & (q - kv <= band): over blocks qb, kb the differences q - kv span
    # 128 (qb - kb) + [-127, 127]; the block is full when that span lies in [0, band], empty
    # when it misses [0, band], partial otherwise.
    s = 768
    k = block_kinds(synth.flex_mask("sliding_window_causal", s, s, band=band))
    n = s // 128
    for qb in range(n):
        for kb in range(n):
            lo, hi = 128 * (qb - kb) - 127, 128 * (qb - kb) + 127
            want = FULL if lo >= 0 and hi <= band else EMPTY if hi < 0 or lo > band else PARTIAL
            assert k[qb, kb] == want, (qb, kb)


@pytest.mark.parametrize("name,sq,sk", [("random_blocks", 640, 520), ("random", 200, 330),
                                        ("document", 700, 700), ("prefix", 300, 600)])
def test_block_table_covers_the_mask(name, sq, sk):
    # every visible pair lies in a listed block; a full block has every pair visible, an
    # empty one none; rows and columns list the same blocks, in increasing order
    m = synth.flex_mask(name, sq, sk, band=200, doc_lengths=[100, 250, 350], seed=3)
    kinds = block_kinds(m)
    kvc, kvl, qc, ql = block_lists(kinds)
    nqb, nkb = kinds.shape
    listed = np.zeros((nqb, nkb), np.int32) - 1
    for qb in range(nqb):
        ent = kvl[qb, :kvc[qb]]
        assert (np.diff(ent // 2) > 0).all()
        for e in ent:
            listed[qb, e // 2] = e % 2
        assert (kvl[qb, kvc[qb]:] == -1).all()
    for kb in range(nkb):
        ent = ql[kb, :qc[kb]]
        assert (np.diff(ent // 2) > 0).all()
        for e in ent:
            assert listed[e // 2, kb] == e % 2
    assert qc.sum() == kvc.sum()
    for qb in range(nqb):
        for kb in range(nkb):
            t = m[qb * 128:(qb + 1) * 128, kb * 128:(kb + 1) * 128]
            if listed[qb, kb] == -1:
                assert not t.any()
            elif listed[qb, kb] == 0:
                assert t.all()
            else:
                assert t.any() and not t.all()


def _blockwise_forward(q, k, v, scale, mask):
    """Attention that visits only the listed blocks of each block row, testing the element
    mask only in partial blocks, with an online (running max / sum) softmax in fp64."""
    kinds = block_kinds(mask)
    kvc, kvl, _, _ = block_lists(kinds)
    sq, d = q.shape
    o = np.zeros((sq, d))
    lse = np.full(sq, -np.inf)
    for qb in range(kinds.shape[0]):
        rows = slice(qb * 128, min((qb + 1) * 128, sq))
        m = np.full(rows.stop - rows.start, -np.inf)
        l = np.zeros_like(m)
        acc = np.zeros((rows.stop - rows.start, d))
        for e in kvl[qb, :kvc[qb]]:
            cols = slice((e // 2) * 128, min((e // 2 + 1) * 128, k.shape[0]))
            s = scale * q[rows] @ k[cols].T
            if e % 2:
                s = np.where(mask[rows, cols], s, -np.inf)
            mn = np.maximum(m, s.max(axis=1))
            safe = np.where(np.isfinite(mn), mn, 0.0)
            a = np.exp(m - safe)
            p = np.exp(s - safe[:, None])
            l = l * a + p.sum(axis=1)
            acc = acc * a[:, None] + p @ v[cols]
            m = mn
        ok = l > 0
        o[rows] = np.where(ok[:, None], acc / np.where(ok, l, 1.0)[:, None], 0.0)
        lse[rows] = np.where(ok, m + np.log(np.where(ok, l, 1.0)), -np.inf)
    return o, lse


@pytest.mark.parametrize("name", ["random_blocks", "document", "global_causal_v2"])
def test_blockwise_traversal_equals_masked_attention(name):
    # skipping empty blocks and not testing full ones changes nothing: the block-sparse
    # result is the plain masked attention (PyTorch float64 SDPA with the boolean mask)
    sq, sk, d = 300, 400, 8
    m = synth.flex_mask(name, sq, sk, band=100, doc_lengths=[90, 150, 160], seed=5)
    q, k, v = rnd(140, sq, d), rnd(141, sk, d), rnd(142, sk, d)
    o, lse = _blockwise_forward(q, k, v, 0.3, m)
    ref = torch_sdpa(q[None, None], k[None, None], v[None, None], 0.3, m[None, None]).numpy()[0, 0]
    rows = m.any(axis=1)
    assert np.abs(o[rows] - ref[rows]).max() < 1e-12
    assert (o[~rows] == 0).all() and np.isneginf(lse[~rows]).all()
    oo, ol = oracle.masked_forward(q[None, None], k[None, None], v[None, None], 0.3, m)
    assert np.abs(oo[0, 0] - o).max() < 1e-12
    assert np.abs(ol[0, 0][rows] - lse[rows]).max() < 1e-12


def test_flex_predicates_equal_their_windows():
    # issue 135161's predicates as element masks: sliding_window_causal = window (band, 0),
    # global_causal_v2 = window (-1, -(band + 1)); v1 on rows sliced from `band` on
    # (local index, keys absolute) = v2's rows from `band` on
    s, band = 512, 128
    assert (synth.flex_mask("sliding_window_causal", s, s, band) == window_mask(s, s, band, 0)).all()
    assert (synth.flex_mask("global_causal_v2", s, s, band) == window_mask(s, s, -1, -(band + 1))).all()
    v1 = synth.flex_mask("global_causal_v1", s - band, s)
    assert (v1 == window_mask(s - band, s, -1, -(band + 1), diag_align=1)).all()


def test_pack_mask_bit_order():
    m = np.zeros((3, 130), bool)
    m[0, 0] = m[1, 63] = m[1, 64] = m[2, 129] = True
    b = synth.pack_mask(m)
    assert b.shape == (3, 3) and b.dtype == np.uint64
    assert int(b[0, 0]) == 1 and int(b[1, 0]) == 1 << 63 and int(b[1, 1]) == 1
    assert int(b[2, 2]) == 2 and int(b[2, 0]) == 0


# ---------------------------------------------------------------------------------------
# FP8 E4M3 decode (the FP8 forward's oracle is exact attention on decoded inputs)
# ---------------------------------------------------------------------------------------

def test_e4m3_decode_closed_forms():
    from oracle import e4m3_decode
    # 1.0 = 0.0111.000, 448 = 0.1111.110 (largest finite), 2^-9 = 0.0000.001 (smallest
    # subnormal), 2^-6 = 0.0001.000 (smallest normal), -1.5 = 1.0111.100
    codes = np.array([0x38, 0x7E, 0x01, 0x08, 0xBC, 0x00, 0x80, 0x07, 0x7F, 0xFF], np.uint8)
    v = e4m3_decode(codes)
    assert list(v[:8]) == [1.0, 448.0, 2.0 ** -9, 2.0 ** -6, -1.5, 0.0, -0.0, 7 * 2.0 ** -9]
    assert np.isnan(v[8]) and np.isnan(v[9])


def test_e4m3_decode_equals_torch_float8():
    from oracle import e4m3_decode
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    got = e4m3_decode(codes)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()


def test_fp8_forward_is_attention_on_dequantised_inputs():
    # the codes' values times their descales, through PyTorch float64 SDPA
    import synth as sy
    from oracle import e4m3_decode, fp8_forward
    x = [rnd(150 + i, 1, 2, 40, 16) for i in range(3)]
    (q8, dq), (k8, dk), (v8, dv) = (sy.e4m3_codes(t) for t in x)
    o, lse = fp8_forward(q8.numpy(), k8.numpy(), v8.numpy(), dq, dk, dv, 0.25,
                         window_mask(40, 40, -1, 0))
    qd, kd, vd = (e4m3_decode(c.numpy()) * s for c, s in ((q8, dq), (k8, dk), (v8, dv)))
    ref = torch_sdpa(qd, kd, vd, 0.25, window_mask(40, 40, -1, 0)).numpy()
    assert np.abs(o - ref).max() < 1e-12
    # quantisation: every code is within half an E4M3 step of its scaled value
    for t, (c, s) in zip(x, ((q8, dq), (k8, dk), (v8, dv))):
        d = e4m3_decode(c.numpy())
        assert (np.abs(d - t / s) <= np.maximum(np.abs(d) * 2.0 ** -4, 2.0 ** -10) + 1e-12).all()
