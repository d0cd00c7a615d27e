"""THD work lists past the scheduler's one-pass sizes: more sequences than its workgroup has
waves (16), more items in one list than it has threads (1024) and thousands of sequences of
mixed lengths, through the C ABI against the fp64 oracle (TE 885's packed THD layout with
int32 cu_seqlens)."""
import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_05_amd as S
import synth
from gpu_util import (DEV, G_TOL, LSE_TOL, O_TOL, check_forward, check_grads, cu_dev, gpu_backward,
                      gpu_bhsd, gpu_forward, oracle_backward, oracle_forward, rel_err, say, to_dev)

pytestmark = pytest.mark.gpu


def test_thd_more_than_64_sequences():
    rng = np.random.default_rng(70)
    lengths = rng.integers(0, 90, 70).tolist()
    lengths[5] = 0
    lengths[40] = 200
    w = synth.thd(31, 1100, "bf16", lengths, 4, 2, 64, 0.125, (-1, 0), with_grad=True,
                  with_dlse=True)
    say(f"case thd 70 sequences total {sum(lengths)}")
    q, k, v = to_dev(w)
    cq, ck = cu_dev(w)
    o, lse = gpu_forward(w, q, k, v, cq, ck)
    torch.cuda.synchronize()
    check_forward(gpu_bhsd(o, w), synth.f64(lse), *oracle_forward(w), "bf16", "fwd")
    dl = w.dlse.to(DEV)
    dq, dk, dv = gpu_backward(w, q, k, v, o, lse, w.dout.to(DEV), dl, cq, ck)
    torch.cuda.synchronize()
    refs = oracle_backward(w, synth.f64(w.dlse))
    check_grads([gpu_bhsd(t, w) for t in (dq, dk, dv)], refs, "bf16", "bwd")


def test_thd_more_than_1024_tiles_sampled():
    # 64 sequences of 2050-2200 rows: at least 17 query tiles of 128 rows each (and twice as
    # many of 64), over 1024 items in one list; GQA 2/1
    rng = np.random.default_rng(71)
    lengths = rng.integers(2050, 2201, 64).tolist()
    w = synth.thd(32, 1200, "bf16", lengths, 2, 1, 64, 0.125, (-1, 0), with_grad=True)
    say("case thd 64 x 2050-2200 rows")
    q, k, v = to_dev(w)
    cq, ck = cu_dev(w)
    o, lse = gpu_forward(w, q, k, v, cq, ck)
    dq, dk, dv = gpu_backward(w, q, k, v, o, lse, w.dout.to(DEV), None, cq, ck)
    torch.cuda.synchronize()
    o, lse, dq, dk, dv = (t.cpu() for t in (o, lse, dq, dk, dv))
    cu = w.cu_seqlens_q
    worst_o = worst_l = 0.0
    got = {"dq": [], "dk": [], "dv": []}
    ref = {"dq": [], "dk": [], "dv": []}
    for s in range(len(lengths)):
        a, b = int(cu[s]), int(cu[s + 1])
        n = b - a
        rows = np.unique(np.concatenate([[0, 127, 128, n - 1], rng.integers(0, n, 2)]))
        hh = s % 2
        qs, gs = (synth.f64(t[a:b, hh]) for t in (w.q, w.dout))
        ks, vs = (synth.f64(t[a:b, 0]) for t in (w.k, w.v))
        ro, rl = oracle.forward_rows(qs, ks, vs, w.scale, rows, w.window)
        worst_o = max(worst_o, float(np.abs(synth.f64(o[a + rows, hh]) - ro).max()))
        worst_l = max(worst_l, float(np.abs(synth.f64(lse[hh, a + rows]) - rl).max()))
        got["dq"].append(synth.f64(dq[a + rows, hh]))
        ref["dq"].append(oracle.dq_rows(qs, ks, vs, gs, w.scale, rows, w.window))
        if s % 21 == 0:  # dK, dV sum over every query row of both q heads: four sequences
            qh = np.stack([synth.f64(w.q[a:b, i]) for i in range(2)])
            gh = np.stack([synth.f64(w.dout[a:b, i]) for i in range(2)])
            rk, rv = oracle.dkdv_cols(qh, ks, vs, gh, w.scale, rows, w.window)
            got["dk"].append(synth.f64(dk[a + rows, 0]))
            got["dv"].append(synth.f64(dv[a + rows, 0]))
            ref["dk"].append(rk)
            ref["dv"].append(rv)
    errs = {n: rel_err(np.concatenate(got[n]), np.concatenate(ref[n])) for n in got}
    say(f"  sampled: max |O err| {worst_o:.2e}, max |LSE err| {worst_l:.2e}, " +
        ", ".join(f"{n} rel err {e:.2e}" for n, e in errs.items()))
    assert worst_o <= O_TOL["bf16"] and worst_l <= LSE_TOL
    for n, e in errs.items():
        assert e <= G_TOL["bf16"], f"{n}: {e}"


def test_thd_long_dkdv_items_run_in_halves():
    # seed 3 of the varlen GQA D128 workload: one 3706-token sequence among shorter ones, so
    # the first key tiles' chains of (q head, q tile) steps exceed the mean per workgroup
    # slot and run as two half blocks plus a combine; results against the oracle on the
    # split tiles and elsewhere, and bitwise repeatable
    w = synth.c4(3)
    lengths = np.diff(w.cu_seqlens_q).tolist()
    say(f"case c4 seed 3 lengths {lengths}")
    q, k, v = to_dev(w)
    cq, ck = cu_dev(w)
    g = w.dout.to(DEV)
    o, lse = gpu_forward(w, q, k, v, cq, ck)
    torch.cuda.synchronize()
    S.sdpa_profile_enable(True)
    runs = [gpu_backward(w, q, k, v, o, lse, g, None, cq, ck) for _ in range(2)]
    torch.cuda.synchronize()
    S.sdpa_profile_enable(False)
    launched = set(S.sdpa_profile_read())
    assert {"bwd_dq", "bwd_dkdv", "bwd_dkdv_combine"} <= launched, launched
    for x, y in zip(*runs):
        assert torch.equal(x, y)
    dq, dk, dv = (t.cpu() for t in runs[0])
    cu = w.cu_seqlens_q
    s_long = int(np.argmax(lengths))
    got = {"dq": [], "dk": [], "dv": []}
    ref = {"dq": [], "dk": [], "dv": []}
    rng = np.random.default_rng(72)
    for s, kh in [(s_long, 0), (s_long, 3), (int(np.argsort(lengths)[-2]), 1)]:
        a, b = int(cu[s]), int(cu[s + 1])
        n = b - a
        heads = list(range(kh * 4, kh * 4 + 4))
        ks, vs = (synth.f64(t[a:b, kh]) for t in (w.k, w.v))
        qh = np.stack([synth.f64(w.q[a:b, h]) for h in heads])
        gh = np.stack([synth.f64(w.dout[a:b, h]) for h in heads])
        cols = np.unique(np.concatenate([[0, 1, 127, 128, 255, 256, 383, 511, n // 2, n - 1],
                                         rng.integers(0, n, 4)]))
        rk, rv = oracle.dkdv_cols(qh, ks, vs, gh, w.scale, cols, w.window)
        got["dk"].append(synth.f64(dk[a + cols, kh]))
        got["dv"].append(synth.f64(dv[a + cols, kh]))
        ref["dk"].append(rk)
        ref["dv"].append(rv)
        rows = np.unique(np.concatenate([[0, 127, n - 1], rng.integers(0, n, 3)]))
        got["dq"].append(synth.f64(dq[a + rows, heads[1]]))
        ref["dq"].append(oracle.dq_rows(qh[1], ks, vs, gh[1], w.scale, rows, w.window))
    errs = {n: rel_err(np.concatenate(got[n]), np.concatenate(ref[n])) for n in got}
    say("  sampled: " + ", ".join(f"{n} rel err {e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= G_TOL["bf16"], f"{n}: {e}"


def test_thd_long_dkdv_items_run_in_halves_d64():
    # head_dim 64 (two dK/dV workgroups per CU): one 6000-token sequence among 120 short
    # ones, GQA 4/2; its first key tiles run as halves, and the list has over 64 sequences
    rng = np.random.default_rng(73)
    lengths = [6000] + rng.integers(100, 301, 120).tolist()
    w = synth.thd(33, 1300, "bf16", lengths, 4, 2, 64, 0.125, (-1, 0), with_grad=True)
    say(f"case thd D64 6000 + 120 short, total {sum(lengths)}")
    q, k, v = to_dev(w)
    cq, ck = cu_dev(w)
    g = w.dout.to(DEV)
    o, lse = gpu_forward(w, q, k, v, cq, ck)
    torch.cuda.synchronize()
    S.sdpa_profile_enable(True)
    runs = [gpu_backward(w, q, k, v, o, lse, g, None, cq, ck) for _ in range(2)]
    torch.cuda.synchronize()
    S.sdpa_profile_enable(False)
    launched = set(S.sdpa_profile_read())
    assert {"bwd_dq", "bwd_dkdv", "bwd_dkdv_combine"} <= launched, launched
    for x, y in zip(*runs):
        assert torch.equal(x, y)
    dq, dk, dv = (t.cpu() for t in runs[0])
    cu = w.cu_seqlens_q
    got = {"dq": [], "dk": [], "dv": []}
    ref = {"dq": [], "dk": [], "dv": []}
    for s, kh in [(0, 0), (0, 1), (7, 1)]:
        a, b = int(cu[s]), int(cu[s + 1])
        n = b - a
        heads = [2 * kh, 2 * kh + 1]
        ks, vs = (synth.f64(t[a:b, kh]) for t in (w.k, w.v))
        qh = np.stack([synth.f64(w.q[a:b, h]) for h in heads])
        gh = np.stack([synth.f64(w.dout[a:b, h]) for h in heads])
        cols = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 129, 255, 256, n // 2, n - 1],
                                         rng.integers(0, n, 3)]))
        cols = cols[cols < n]
        rk, rv = oracle.dkdv_cols(qh, ks, vs, gh, w.scale, cols, w.window)
        got["dk"].append(synth.f64(dk[a + cols, kh]))
        got["dv"].append(synth.f64(dv[a + cols, kh]))
        ref["dk"].append(rk)
        ref["dv"].append(rv)
        rows = np.unique(np.concatenate([[0, 127, n - 1], rng.integers(0, n, 3)]))
        got["dq"].append(synth.f64(dq[a + rows, heads[0]]))
        ref["dq"].append(oracle.dq_rows(qh[0], ks, vs, gh[0], w.scale, rows, w.window))
    errs = {n: rel_err(np.concatenate(got[n]), np.concatenate(ref[n])) for n in got}
    say("  sampled: " + ", ".join(f"{n} rel err {e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= G_TOL["bf16"], f"{n}: {e}"


def test_thd_split_items_accumulate_f16_dlse():
    # the split path's combine with accumulate=1, fp16 and dLSE: dK, dV added to nonzero
    # buffers equal the buffers plus the plain result within one fp16 rounding of the sum,
    # and the plain result matches the oracle on the split key tiles
    lengths = [290, 3706, 2500, 2006, 1179, 706, 2958, 651]
    w = synth.thd(34, 1400, "f16", lengths, 16, 4, 128, 128 ** -0.5, (-1, 0), with_grad=True,
                  with_dlse=True)
    say("case thd split f16 dLSE accumulate")
    q, k, v = to_dev(w)
    cq, ck = cu_dev(w)
    g, dl = w.dout.to(DEV), w.dlse.to(DEV)
    o, lse = gpu_forward(w, q, k, v, cq, ck)
    torch.cuda.synchronize()
    S.sdpa_profile_enable(True)
    dq, dk, dv = gpu_backward(w, q, k, v, o, lse, g, dl, cq, ck)
    torch.cuda.synchronize()
    S.sdpa_profile_enable(False)
    assert "bwd_dkdv_combine" in set(S.sdpa_profile_read())
    base_k = (torch.randn(dk.shape, generator=torch.Generator().manual_seed(5)) * 0.01).half().to(DEV)
    base_v = (torch.randn(dv.shape, generator=torch.Generator().manual_seed(6)) * 0.01).half().to(DEV)
    base_q = torch.zeros_like(dq)
    aq, ak, av = gpu_backward(w, q, k, v, o, lse, g, dl, cq, ck, dq=base_q.clone(), dk=base_k.clone(),
                              dv=base_v.clone(), accumulate=True)
    torch.cuda.synchronize()
    for acc, base, plain in ((ak, base_k, dk), (av, base_v, dv), (aq, base_q, dq)):
        want = base.double() + plain.double()
        err = float((acc.double() - want).abs().max())
        assert err <= 2.0 ** -10 * float(want.abs().max()) + 1e-6, err
    dk, dv = dk.cpu(), dv.cpu()
    cu = w.cu_seqlens_q
    s, kh = 1, 2
    a, b = int(cu[s]), int(cu[s + 1])
    n = b - a
    heads = list(range(kh * 4, kh * 4 + 4))
    ks, vs = (synth.f64(t[a:b, kh]) for t in (w.k, w.v))
    qh = np.stack([synth.f64(w.q[a:b, h]) for h in heads])
    gh = np.stack([synth.f64(w.dout[a:b, h]) for h in heads])
    dlh = np.stack([synth.f64(w.dlse[h, a:b]) for h in heads])
    cols = np.array([0, 1, 127, 128, 300, 511, 700, n - 1])
    rk, rv = oracle.dkdv_cols(qh, ks, vs, gh, w.scale, cols, w.window, 0, dlh)
    ek = rel_err(synth.f64(dk[a + cols, kh]), rk)
    ev = rel_err(synth.f64(dv[a + cols, kh]), rv)
    say(f"  sampled: dk rel err {ek:.2e}, dv rel err {ev:.2e}")
    assert ek <= G_TOL["f16"] and ev <= G_TOL["f16"]


def test_thd_split_room_in_the_workspace_is_optional():
    # a workspace one byte short of sdpa_bwd_workspace_size lacks the room for split items:
    # the same call then splits nothing (no combine launch), dQ is bitwise the same and dK, dV
    # differ only by the order of their fp32 sums
    w = synth.c4(3)
    q, k, v = to_dev(w)
    g = w.dout.to(DEV)
    kw = dict(cu_seqlens_q=torch.from_numpy(w.cu_seqlens_q).to(DEV),
              max_seqlen_q=int(np.diff(w.cu_seqlens_q).max()))
    o, lse = S.forward(q, k, v, w.layout, w.scale, w.window, **kw)
    pr = S.Problem(q, k, w.layout, w.scale, w.window, **kw)
    full = S.sdpa_bwd_workspace_size(pr.desc)
    say(f"case c4 seed 3 workspace {full} and {full - 1} bytes")

    def run(nbytes):
        grads = tuple(torch.empty_like(t) for t in (q, k, v))
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        torch.cuda.synchronize()
        S.sdpa_profile_enable(True)
        S.sdpa_bwd(pr.desc, q, k, v, o, lse, g, None, *grads, False, ws)
        torch.cuda.synchronize()
        S.sdpa_profile_enable(False)
        return grads, set(S.sdpa_profile_read())

    (dq1, dk1, dv1), l1 = run(full)
    (dq2, dk2, dv2), l2 = run(full - 1)
    assert "bwd_dkdv_combine" in l1 and "bwd_dkdv_combine" not in l2, (l1, l2)
    assert torch.equal(dq1, dq2)
    for a, b in ((dk1, dk2), (dv1, dv2)):
        a, b = a.double(), b.double()
        assert float((a - b).abs().max()) <= 2.0 ** -7 * float(b.abs().max())


@pytest.mark.parametrize("seed,hq,hk,d", [(80, 16, 4, 128), (81, 8, 2, 64), (82, 16, 16, 128),
                                          (83, 8, 1, 64)])
def test_thd_split_equals_unsplit_on_skewed_mixes(seed, hq, hk, d):
    # seeded length mixes with one long sequence: the backward with the split room (items
    # above the mean may run as halves) against the same call without it (no split); dQ is
    # bitwise the same, dK and dV differ only by the order of their fp32 sums
    rng = np.random.default_rng(seed)
    lengths = [int(rng.integers(3000, 6001))] + rng.integers(1, 1500, int(rng.integers(30, 60))).tolist()
    w = synth.thd(seed, 1500, "bf16", lengths, hq, hk, d, d ** -0.5, (-1, 0), with_grad=True)
    q, k, v = to_dev(w)
    g = w.dout.to(DEV)
    kw = dict(cu_seqlens_q=torch.from_numpy(w.cu_seqlens_q).to(DEV), max_seqlen_q=max(lengths))
    o, lse = S.forward(q, k, v, w.layout, w.scale, w.window, **kw)
    pr = S.Problem(q, k, w.layout, w.scale, w.window, **kw)
    full = S.sdpa_bwd_workspace_size(pr.desc)
    out = []
    for nbytes in (full, full - 1):
        grads = tuple(torch.empty_like(t) for t in (q, k, v))
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        S.sdpa_profile_enable(True)
        S.sdpa_bwd(pr.desc, q, k, v, o, lse, g, None, *grads, False, ws)
        torch.cuda.synchronize()
        S.sdpa_profile_enable(False)
        out.append((grads, set(S.sdpa_profile_read())))
    (dq1, dk1, dv1), l1 = out[0]
    (dq2, dk2, dv2), l2 = out[1]
    say(f"case seed {seed} H{hq}/{hk} D{d} {len(lengths)} sequences, total {sum(lengths)}: "
        f"combine {'bwd_dkdv_combine' in l1}")
    assert "bwd_dkdv_combine" not in l2
    assert torch.equal(dq1, dq2)
    for a, b in ((dk1, dk2), (dv1, dv2)):
        a, b = a.double(), b.double()
        assert float((a - b).abs().max()) <= 2.0 ** -7 * float(b.abs().max())


def test_thd_thousands_of_sequences_sampled():
    # 3000 sequences, mostly short with a long tail (and empty ones), GQA 4/2, bottom-right
    # causal over cross lengths: one list of ~6000 query tiles and ~3000 key tiles, each
    # sequence against its own dense attention (fp64 oracle) on a sample of 48 sequences
    rng = np.random.default_rng(72)
    n = 3000
    kind = rng.random(n)
    lengths = np.where(kind < 0.85, rng.integers(0, 49, n),
                       np.where(kind < 0.95, rng.integers(49, 301, n), rng.integers(301, 1501, n)))
    lengths[[7, 1234]] = 0
    lengths_k = np.where(lengths > 0, np.maximum(1, lengths + rng.integers(-20, 21, n)), 0)
    w = synth.thd(33, 1300, "bf16", lengths.tolist(), 4, 2, 64, 0.125, (-1, 0), with_grad=True,
                  lengths_k=lengths_k.tolist(), diag_align=1)
    say(f"case thd {n} sequences, {int(lengths.sum())} query and {int(lengths_k.sum())} key rows")
    q, k, v = to_dev(w)
    cq, ck = cu_dev(w)
    o, lse = gpu_forward(w, q, k, v, cq, ck)
    dq, dk, dv = gpu_backward(w, q, k, v, o, lse, w.dout.to(DEV), None, cq, ck)
    torch.cuda.synchronize()
    o, lse, dq, dk, dv = (t.cpu() for t in (o, lse, dq, dk, dv))
    cu, cuk = w.cu_seqlens_q, w.cu_seqlens_k
    sample = np.unique(np.concatenate([rng.choice(np.flatnonzero(lengths > 0), 45, replace=False),
                                       [int(np.argmax(lengths)), 7, 1234]]))
    worst_o = worst_l = 0.0
    got = {"dq": [], "dk": [], "dv": []}
    ref = {"dq": [], "dk": [], "dv": []}
    bhsd = lambda t, a, b: synth.f64(t[a:b]).transpose(1, 0, 2)[None]  # [T,H,D] rows -> [1,H,L,D]
    for s in sample:
        a, b, c, e = int(cu[s]), int(cu[s + 1]), int(cuk[s]), int(cuk[s + 1])
        if b == a:
            continue
        qs, gs = bhsd(w.q, a, b), bhsd(w.dout, a, b)
        ks, vs = bhsd(w.k, c, e), bhsd(w.v, c, e)
        ro, rl = oracle.windowed_forward(qs, ks, vs, w.scale, w.window, 1)
        go, gl = bhsd(o, a, b), synth.f64(lse[:, a:b])[None]
        fin = np.isfinite(rl)
        assert (np.isneginf(gl) == ~fin).all(), f"sequence {s}: -inf rows differ"
        worst_o = max(worst_o, float(np.abs(go - ro).max()))
        worst_l = max(worst_l, float(np.abs(gl[fin] - rl[fin]).max()) if fin.any() else 0.0)
        rq, rk, rv = oracle.windowed_backward(qs, ks, vs, gs, w.scale, w.window, 1)
        for name, t, r, lo, hi in (("dq", dq, rq, a, b), ("dk", dk, rk, c, e), ("dv", dv, rv, c, e)):
            got[name].append(bhsd(t, lo, hi).ravel())
            ref[name].append(r.ravel())
    errs = {m: rel_err(np.concatenate(got[m]), np.concatenate(ref[m])) for m in got}
    say(f"  {len(sample)} sequences: max |O err| {worst_o:.2e}, max |LSE err| {worst_l:.2e}, " +
        ", ".join(f"{m} rel err {x:.2e}" for m, x in errs.items()))
    assert worst_o <= O_TOL["bf16"] and worst_l <= LSE_TOL
    for m, x in errs.items():
        assert x <= G_TOL["bf16"], f"{m}: {x}"
