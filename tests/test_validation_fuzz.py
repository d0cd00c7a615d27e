"""Seeded fuzz of the C-ABI validation layer (host only, no device needed), checked against an
independent model of element addresses.

"[PyTorch] fused CUDNN attention kernel not properly handling strides" (TransformerEngine
issue 1195) is the failure this layer exists for: strided views of one packed buffer were
read as if contiguous, and the checks that would have caught it sat above the callable
modules.  Here tiny problems get random layouts, random physical dimension orders, padded
strides, stride-0 inputs, views of one packed buffer and outputs that overlap or interleave
with other tensors, and ``sdpa_fwd_validate`` / ``sdpa_bwd_validate`` must agree with a
model that enumerates every byte each tensor addresses:

* d stride != 1, or a negative stride on a dimension of extent > 1: ERR_STRIDE;
* a pointer not aligned to its element: ERR_ALIGN;
* an output whose elements share bytes (stride 0 included): ERR_STRIDE;
* an output sharing a byte with another output or an input: ERR_ALIAS;
* otherwise the call is valid.  The library may reject a valid call it cannot prove
  disjoint (ERR_ALIAS), but never when the tensors are disjoint boxes of one packed
  parent with equal strides, the case it claims to decide exactly.  Every OK must be
  valid in the model.

The same fuzz runs a second time on a host build of the entry points made with
AddressSanitizer and UndefinedBehaviorSanitizer (g++, kernel launchers stubbed), in a child
process with the sanitizer runtimes preloaded.
"""
import ctypes
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import scaled_dot_product_05_amd as S  # noqa: E402

OK, ERR_STRIDE, ERR_ALIGN, ERR_ALIAS = 0, 3, 4, 5
ESIZE = {"f16": 2, "bf16": 2, "f32": 4}
ORDER = {"bshd": "bshd", "sbhd": "sbhd", "bhsd": "bhsd", "thd": "thd"}  # logical dim order
ARENA = 1 << 40  # fake device addresses: validation never dereferences


class T:
    """A tensor handle: byte address, logical extents and element strides, element size."""

    def __init__(self, addr, ext, st, esize):
        self.addr, self.ext, self.st, self.esize = int(addr), list(ext), list(st), esize

    def offsets(self):
        """Byte offsets of every element's first byte."""
        off = np.zeros(1, np.int64)
        for n, s in zip(self.ext, self.st):
            off = (off[:, None] + np.arange(n, dtype=np.int64)[None, :] * s).ravel()
        return self.addr + off * self.esize

    def bytes(self):
        o = self.offsets()
        return (o[:, None] + np.arange(self.esize)[None, :]).ravel()

    def numel(self):
        return int(np.prod(self.ext))

    def handle(self):
        st = self.st + [0] * (4 - len(self.st))
        return S.Tensor(ctypes.c_void_p(self.addr), (ctypes.c_int64 * 4)(*st[:4]))

    def rowstat(self):
        st = self.st + [0] * (3 - len(self.st))
        return S.RowStat(ctypes.c_void_p(self.addr), (ctypes.c_int64 * 3)(*st[:3]))


# ---------------------------------------------------------------------------------------
# the model
# ---------------------------------------------------------------------------------------

def model_status(tensors, outputs, inputs, rowstats=()):
    """Expected status: per-tensor defects in call order, then output self-overlap, then
    aliasing.  ``tensors`` lists (name, T) in the library's checking order."""
    for name, t in tensors:
        if t.numel() == 0:
            continue
        is_stat = name in rowstats
        if not is_stat and t.st[-1] != 1:
            return ERR_STRIDE
        if any(n > 1 and s < 0 for n, s in zip(t.ext, t.st)):
            return ERR_STRIDE
        if t.addr % t.esize:
            return ERR_ALIGN
        if name in outputs:
            b = t.offsets()
            if len(np.unique(b)) != len(b):
                return ERR_STRIDE
    for i, (na, a) in enumerate((n, t) for n, t in tensors if n in outputs):
        ba = set(a.bytes().tolist())
        for nb, b in tensors:
            if nb == na or (nb in outputs and outputs.index(nb) < outputs.index(na)):
                continue
            if nb not in outputs and nb not in inputs:
                continue
            if ba.intersection(b.bytes().tolist()):
                return ERR_ALIAS
    return OK


# ---------------------------------------------------------------------------------------
# random problems
# ---------------------------------------------------------------------------------------

def logical_dims(layout, b, s, h, d):
    return {"bshd": [b, s, h, d], "sbhd": [s, b, h, d], "bhsd": [b, h, s, d],
            "thd": [s, h, d]}[layout]


def place(rng, ext, esize, cursor, pad_max=3, perm=True):
    """A fresh region: the logical dims laid out in a random physical order (d innermost),
    each with random padding.  Returns (T, new cursor)."""
    nd = len(ext)
    order = list(range(nd - 1))
    if perm:
        rng.shuffle(order)
    st = [0] * nd
    st[-1] = 1
    span = ext[-1] + int(rng.integers(0, pad_max + 1)) * 8
    for i in reversed(order):  # innermost last in `order`
        st[i] = span
        span *= ext[i] + int(rng.integers(0, 2))
    t = T(cursor, ext, st, esize)
    return t, cursor + (span + 64) * esize


def parent_views(rng, layout, dims, heads, esize, cursor):
    """Views of one packed parent [.., h_total, ..] (TransformerEngine's sb(h+2h_g)d): each
    tensor takes a head range; the parent's other dims are laid out in a random order with
    padding.  Returns the views (same strides) and the new cursor."""
    htot = sum(heads) + int(rng.integers(0, 3))
    pdims = list(dims)
    hpos = ORDER[layout].index("h")
    pdims[hpos] = htot
    parent, cursor = place(rng, pdims, esize, cursor)
    out, h0 = [], 0
    for h in heads:
        ext = list(dims)
        ext[hpos] = h
        out.append(T(parent.addr + h0 * parent.st[hpos] * esize, ext, parent.st, esize))
        h0 += h
    return out, cursor


def make_problem(rng):
    layout = ["bshd", "sbhd", "bhsd", "thd"][int(rng.integers(0, 4))]
    dtype = ["f16", "bf16", "f32"][int(rng.integers(0, 3))]
    hk = int(rng.integers(1, 3))
    hq = hk * int(rng.integers(1, 3))
    b = int(rng.integers(1, 3))
    sq, sk = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    d = 32
    if layout == "thd":
        sk = sq  # self-attention packing: rows = total tokens
        tot = b * sq
        qd, kd = logical_dims(layout, 1, tot, hq, d), logical_dims(layout, 1, tot, hk, d)
    else:
        qd, kd = logical_dims(layout, b, sq, hq, d), logical_dims(layout, b, sk, hk, d)
    return layout, dtype, b, sq, sk, hq, hk, d, qd, kd


def desc_of(layout, dtype, b, sq, sk, hq, hk, d):
    if layout == "thd":
        fake = ctypes.c_void_p(ARENA - 4096)
        return S.Desc(S.LAYOUTS[layout], S.DTYPES[dtype], b, sq, sq, hq, hk, d, fake, fake,
                      b * sq, b * sq, 0.125, -1, 0, 0, None, None, None)
    return S.Desc(S.LAYOUTS[layout], S.DTYPES[dtype], b, sq, sk, hq, hk, d, None, None, 0, 0,
                  0.125, -1, 0, 0, None, None, None)


def stat_tensor(rng, layout, b, hq, sq, cursor):
    """LSE-like fp32 [B,H,S] (THD [H,T]), contiguous or with padded strides."""
    ext = [hq, b * sq] if layout == "thd" else [b, hq, sq]
    t, cursor = place(rng, ext + [1], 4, cursor, pad_max=1)
    return T(t.addr, ext, t.st[:-1], 4), cursor


DEFECTS = ["none"] * 6 + ["dstride", "negative", "misalign", "out_stride0", "in_stride0",
                          "overlap_parent", "overlap_region", "interleave"]


def inject(rng, kind, tensors, outputs, inputs, layout):
    """Mutates one tensor per the defect kind (in place)."""
    names = [n for n, _ in tensors]
    tmap = dict(tensors)
    if kind == "dstride":
        t = tmap[names[int(rng.integers(0, len(names)))]]
        if len(t.ext) == len(ORDER[layout]):
            t.st[-1] = 2
    elif kind == "negative":
        t = tmap[names[int(rng.integers(0, len(names)))]]
        dims = [i for i, n in enumerate(t.ext[:-1]) if n > 1]
        if dims:
            i = dims[int(rng.integers(0, len(dims)))]
            t.addr += (t.ext[i] - 1) * t.st[i] * t.esize
            t.st[i] = -t.st[i]
    elif kind == "misalign":
        t = tmap[names[int(rng.integers(0, len(names)))]]
        if t.esize > 1:
            t.addr += 1
    elif kind in ("out_stride0", "in_stride0"):
        pool = outputs if kind == "out_stride0" else inputs
        t = tmap[pool[int(rng.integers(0, len(pool)))]]
        dims = [i for i, n in enumerate(t.ext[:-1]) if n > 1]
        if dims:
            t.st[dims[int(rng.integers(0, len(dims)))]] = 0
    elif kind == "overlap_region":
        # an output moved to start inside another tensor's span
        o = tmap[outputs[int(rng.integers(0, len(outputs)))]]
        other = tmap[names[int(rng.integers(0, len(names)))]]
        if other is not o:
            span = int(other.offsets().max() - other.addr) // other.esize
            o.addr = other.addr + int(rng.integers(0, span + 1)) * other.esize
    elif kind == "interleave":
        # an output offset by one element inside another's padded rows (disjoint or not)
        o = tmap[outputs[int(rng.integers(0, len(outputs)))]]
        other = tmap[names[int(rng.integers(0, len(names)))]]
        if other is not o and o.esize == other.esize and len(o.ext) == len(other.ext):
            o.st = list(other.st)
            o.addr = other.addr + int(rng.integers(1, 40)) * o.esize


def fuzz_forward(lib, rng):
    layout, dtype, b, sq, sk, hq, hk, d, qd, kd = make_problem(rng)
    es = ESIZE[dtype]
    cursor = ARENA
    box = (sq == sk or layout == "thd") and bool(rng.integers(0, 2))
    if box:  # q, k, v and o as head ranges of one parent (o after them, or over them)
        (q, k, v, o), cursor = parent_views(rng, layout, list(qd), [hq, hk, hk, hq], es, cursor)
    else:
        q, cursor = place(rng, qd, es, cursor)
        k, cursor = place(rng, kd, es, cursor)
        v, cursor = place(rng, kd, es, cursor)
        o, cursor = place(rng, qd, es, cursor)
    lse, cursor = stat_tensor(rng, layout, b, hq, sq, cursor)
    tensors = [("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse)]
    outputs, inputs = ["o", "lse"], ["q", "k", "v"]
    kind = DEFECTS[int(rng.integers(0, len(DEFECTS)))]
    if kind == "overlap_parent" and box:
        # o's head range slides back over v's (same strides: decidable exactly)
        hpos = ORDER[layout].index("h")
        o.addr -= int(rng.integers(1, hk + 1)) * o.st[hpos] * es
    else:
        inject(rng, kind, tensors, outputs, inputs, layout)
    want = model_status(tensors, outputs, inputs, rowstats=("lse",))
    desc = desc_of(layout, dtype, b, sq, sk, hq, hk, d)
    got = lib.sdpa_fwd_validate(ctypes.byref(desc), q.handle(), k.handle(), v.handle(),
                                o.handle(), lse.rowstat(), 1 << 40)
    exact = box and kind in ("none", "overlap_parent", "in_stride0")
    return want, got, exact, (layout, dtype, kind, box)


def fuzz_backward(lib, rng):
    layout, dtype, b, sq, sk, hq, hk, d, qd, kd = make_problem(rng)
    es = ESIZE[dtype]
    cursor = ARENA
    box = (sq == sk or layout == "thd") and bool(rng.integers(0, 2))
    if box:  # inputs from one parent, the gradients as head ranges of another (C5's dqkv)
        (q, k, v), cursor = parent_views(rng, layout, list(qd), [hq, hk, hk], es, cursor)
        (dq, dk, dv), cursor = parent_views(rng, layout, list(qd), [hq, hk, hk], es, cursor)
    else:
        q, cursor = place(rng, qd, es, cursor)
        k, cursor = place(rng, kd, es, cursor)
        v, cursor = place(rng, kd, es, cursor)
        dq, cursor = place(rng, qd, es, cursor)
        dk, cursor = place(rng, kd, es, cursor)
        dv, cursor = place(rng, kd, es, cursor)
    o, cursor = place(rng, qd, es, cursor)
    do, cursor = place(rng, qd, es, cursor)
    lse, cursor = stat_tensor(rng, layout, b, hq, sq, cursor)
    dlse, cursor = stat_tensor(rng, layout, b, hq, sq, cursor)
    tensors = [("q", q), ("k", k), ("v", v), ("o", o), ("dout", do), ("lse", lse),
               ("dq", dq), ("dk", dk), ("dv", dv), ("dlse", dlse)]
    outputs, inputs = ["dq", "dk", "dv"], ["q", "k", "v", "o", "dout", "lse", "dlse"]
    kind = DEFECTS[int(rng.integers(0, len(DEFECTS)))]
    if kind == "overlap_parent" and box:
        hpos = ORDER[layout].index("h")
        dv.addr -= int(rng.integers(1, hk + 1)) * dv.st[hpos] * es  # dv over dk's heads
    else:
        inject(rng, kind, tensors, outputs, inputs, layout)
    want = model_status(tensors, outputs, inputs, rowstats=("lse", "dlse"))
    desc = desc_of(layout, dtype, b, sq, sk, hq, hk, d)
    got = lib.sdpa_bwd_validate(ctypes.byref(desc), q.handle(), k.handle(), v.handle(),
                                o.handle(), lse.rowstat(), do.handle(), dlse.rowstat(),
                                dq.handle(), dk.handle(), dv.handle(), 1 << 40)
    exact = box and kind in ("none", "overlap_parent", "in_stride0")
    return want, got, exact, (layout, dtype, kind, box)


def run_fuzz(lib, n, seed):
    """n forward and n backward cases; returns counts, raises on a disagreement."""
    rng = np.random.default_rng(seed)
    stats = {"ok": 0, "rejected": 0, "conservative": 0}
    for i in range(n):
        for fn in (fuzz_forward, fuzz_backward):
            want, got, exact, info = fn(lib, rng)
            msg = f"case {i} {fn.__name__} {info}: model {want}, library {got} " \
                  f"({lib.sdpa_last_error().decode()})"
            if got == OK:
                assert want == OK, msg  # soundness: every accepted call is valid
                stats["ok"] += 1
            elif want == OK:
                # valid but unproven: only ERR_ALIAS, and never for boxes of one parent
                assert got == ERR_ALIAS and not exact, msg
                stats["conservative"] += 1
            else:
                assert got == want, msg
                stats["rejected"] += 1
    return stats


def run_size_extremes(lib, n, seed):
    """Workspace sizing at extreme descriptor values (batch up to 2^31 - 1, heads up to
    65535, sequence lengths up to the 2^28 - 1 limit, THD totals up to 2^31 - 1): each call
    returns an error or a size, and every size returned covers at least the fp32 Delta and
    LSE log2(e) rows of the backward."""
    rng = np.random.default_rng(seed)
    big = lambda lo, hi: int(np.exp(rng.uniform(np.log(lo), np.log(hi))))
    sizes = 0
    for _ in range(n):
        layout = ["bshd", "sbhd", "bhsd", "thd"][int(rng.integers(0, 4))]
        dtype = ["f16", "bf16", "f32"][int(rng.integers(0, 3))]
        hk = big(1, 65535)
        hq = hk * big(1, max(1, 65535 // hk))
        b, sq, sk = big(1, 2 ** 31 - 1), big(1, 2 ** 28 - 1), big(1, 2 ** 28 - 1)
        d = [32, 64, 128][int(rng.integers(0, 3))]
        if layout == "thd":
            fake = ctypes.c_void_p(ARENA - 4096)
            tq, tk = big(1, 2 ** 31 - 1), big(1, 2 ** 31 - 1)
            desc = S.Desc(S.LAYOUTS[layout], S.DTYPES[dtype], b, sq, sk, hq, hk, d, fake, fake,
                          tq, tk, 0.125, -1, 0, 0, None, None, None)
            rows = hq * tq
        else:
            desc = S.Desc(S.LAYOUTS[layout], S.DTYPES[dtype], b, sq, sk, hq, hk, d, None, None,
                          0, 0, 0.125, -1, 0, 0, None, None, None)
            rows = b * hq * sq
        for fn in ("sdpa_fwd_workspace_size", "sdpa_bwd_workspace_size"):
            out = ctypes.c_size_t(0)
            rc = getattr(lib, fn)(ctypes.byref(desc), ctypes.byref(out))
            if rc == OK:
                sizes += 1
                if fn == "sdpa_bwd_workspace_size":
                    assert out.value >= 8 * rows, (fn, layout, b, hq, sq, out.value)
        out = ctypes.c_size_t(0)
        lib.sdpa_cp_workspace_size(ctypes.byref(desc), int(rng.integers(1, 9)), ctypes.byref(out))
    return sizes


def _bound_lib(path):
    h = ctypes.CDLL(path)
    for name in ("sdpa_fwd_validate", "sdpa_bwd_validate", "sdpa_last_error",
                 "sdpa_fwd_workspace_size", "sdpa_bwd_workspace_size", "sdpa_cp_workspace_size"):
        args, res = S._SIGNATURES[name]
        getattr(h, name).argtypes = args
        getattr(h, name).restype = res
    return h


def test_validation_fuzz_against_address_model():
    stats = run_fuzz(S.lib(), 800, seed=1195)
    print(stats)
    assert stats["ok"] > 300 and stats["rejected"] > 300


def test_workspace_sizes_at_extreme_shapes():
    print(run_size_extremes(S.lib(), 2000, seed=7))


# ---------------------------------------------------------------------------------------
# the same fuzz on a host build with AddressSanitizer + UndefinedBehaviorSanitizer
# ---------------------------------------------------------------------------------------

SAN_LIB = os.path.join(ROOT, "_build", "libsdpa_host_asan_ubsan.so")
CSRC = os.path.join(ROOT, "scaled_dot_product_05_amd", "csrc")


def build_sanitized():
    os.makedirs(os.path.dirname(SAN_LIB), exist_ok=True)
    flags = ["-std=c++17", "-O1", "-g", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
             "-I" + os.path.join(ROOT, "include"), "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    srcs = [os.path.join(CSRC, f) for f in ("api.cpp", "cp.cpp", "profile.cpp")] + \
        [os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp")]
    cmd = ["g++", *flags, "-shared", "-o", SAN_LIB, *srcs, "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,--no-undefined"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, "sanitized host build failed:\n" + res.stderr[-4000:]


@pytest.mark.slow
def test_validation_fuzz_under_asan_ubsan():
    try:
        build_sanitized()
    except FileNotFoundError as e:  # pragma: no cover
        pytest.skip(f"no g++ on this host: {e}")
    rt = [subprocess.run(["g++", f"-print-file-name={n}"], capture_output=True,
                         text=True).stdout.strip() for n in ("libasan.so", "libubsan.so")]
    env = dict(os.environ, LD_PRELOAD=":".join(rt),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = ("import sys; sys.path.insert(0, %r); sys.path.insert(0, %r); "
            "import test_validation_fuzz as F; "
            "L = F._bound_lib(%r); print(F.run_fuzz(L, 300, seed=885)); "
            "print(F.run_size_extremes(L, 1000, seed=8))" %
            (ROOT, os.path.join(ROOT, "tests"), SAN_LIB))
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                         timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, res.stderr
    print(res.stdout.strip())
