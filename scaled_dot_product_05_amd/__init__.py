"""Python binding of the MI355X fused scaled-dot-product attention library (libsdpa.so).

Argument marshalling only: torch tensors (device memory) become the C ABI's
(pointer, element strides) handles, and every step of the computation runs in the HIP
kernels behind ``include/sdpa.h``.  There is no fallback: if the library is missing or a
call fails, an exception is raised.

The names mirror the C entry points (``sdpa_fwd``, ``sdpa_bwd``, ``sdpa_merge_fwd`` ...).
Tensor conventions: a tensor's torch dimensions are the layout's logical order --
BSHD [B,S,H,D], SBHD [S,B,H,D], BHSD [B,H,S,D], THD [T,H,D]; LSE-like row statistics
are fp32 [B,H,S] (THD: [H,T]).  Any strides are accepted as long as the last is 1.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libsdpa.so")

LAYOUTS = {"bshd": 0, "sbhd": 1, "bhsd": 2, "thd": 3}
DTYPES = {"f16": 0, "bf16": 1, "f32": 2, "e4m3": 3}
ALIGN = {"top_left": 0, "bottom_right": 1}

STATUS = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_STRIDE", 4: "ERR_ALIGN",
          5: "ERR_ALIAS", 6: "ERR_UNSUPPORTED", 7: "ERR_WORKSPACE", 8: "ERR_HIP", 9: "ERR_ARG"}


class SdpaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride", ctypes.c_int64 * 4)]


class RowStat(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride", ctypes.c_int64 * 3)]


class BlockMaskDesc(ctypes.Structure):
    """sdpa_block_mask_t: element bits and the block table built from them (device arrays)."""
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("bits", ctypes.c_void_p),
                ("kv_count", ctypes.c_void_p), ("kv_list", ctypes.c_void_p),
                ("q_count", ctypes.c_void_p), ("q_list", ctypes.c_void_p)]


class Desc(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("dtype", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("seqlen_q", ctypes.c_int32), ("seqlen_k", ctypes.c_int32),
                ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("cu_seqlens_q", ctypes.c_void_p),
                ("cu_seqlens_k", ctypes.c_void_p), ("total_q", ctypes.c_int64),
                ("total_k", ctypes.c_int64), ("softmax_scale", ctypes.c_float),
                ("window_left", ctypes.c_int32), ("window_right", ctypes.c_int32),
                ("diag_align", ctypes.c_int32), ("cu_seqlens_q_padded", ctypes.c_void_p),
                ("cu_seqlens_k_padded", ctypes.c_void_p), ("block_mask", ctypes.c_void_p)]


class MergeDesc(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("dtype", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("seqlen", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("total", ctypes.c_int64),
                ("cu_seqlens", ctypes.c_void_p), ("cu_seqlens_padded", ctypes.c_void_p)]


_P = ctypes.POINTER
_SIGNATURES = {
    "sdpa_version": ([], ctypes.c_int),
    "sdpa_last_error": ([], ctypes.c_char_p),
    "sdpa_fwd_workspace_size": ([_P(Desc), _P(ctypes.c_size_t)], ctypes.c_int),
    "sdpa_fwd_validate": ([_P(Desc)] + [_P(Tensor)] * 4 + [_P(RowStat), ctypes.c_size_t],
                          ctypes.c_int),
    "sdpa_fwd": ([_P(Desc)] + [_P(Tensor)] * 4 + [_P(RowStat), ctypes.c_void_p, ctypes.c_size_t,
                                                   ctypes.c_void_p], ctypes.c_int),
    "sdpa_fwd_fp8_validate": ([_P(Desc)] + [_P(Tensor)] * 4 + [_P(RowStat), ctypes.c_size_t],
                              ctypes.c_int),
    "sdpa_fwd_fp8": ([_P(Desc)] + [_P(Tensor)] * 3 + [ctypes.c_void_p] * 3
                     + [_P(Tensor), _P(RowStat), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p],
                     ctypes.c_int),
    "sdpa_bwd_workspace_size": ([_P(Desc), _P(ctypes.c_size_t)], ctypes.c_int),
    "sdpa_bwd_validate": ([_P(Desc)] + [_P(Tensor)] * 4 + [_P(RowStat), _P(Tensor), _P(RowStat)]
                          + [_P(Tensor)] * 3 + [ctypes.c_size_t], ctypes.c_int),
    "sdpa_bwd": ([_P(Desc)] + [_P(Tensor)] * 4 + [_P(RowStat), _P(Tensor), _P(RowStat)]
                 + [_P(Tensor)] * 3 + [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p], ctypes.c_int),
    "sdpa_merge_fwd_validate": ([_P(MergeDesc), _P(Tensor), _P(RowStat), _P(Tensor), _P(RowStat),
                                 _P(Tensor), _P(RowStat)], ctypes.c_int),
    "sdpa_merge_bwd_validate": ([_P(MergeDesc), _P(Tensor), _P(RowStat), _P(Tensor), _P(RowStat),
                                 _P(Tensor), _P(RowStat), _P(Tensor), _P(RowStat), _P(Tensor),
                                 _P(RowStat)], ctypes.c_int),
    "sdpa_merge_fwd": ([_P(MergeDesc), _P(Tensor), _P(RowStat), _P(Tensor), _P(RowStat),
                        _P(Tensor), _P(RowStat), ctypes.c_void_p], ctypes.c_int),
    "sdpa_merge_bwd": ([_P(MergeDesc), _P(Tensor), _P(RowStat), _P(Tensor), _P(RowStat),
                        _P(Tensor), _P(RowStat), _P(Tensor), _P(RowStat), _P(Tensor),
                        _P(RowStat), ctypes.c_void_p], ctypes.c_int),
    "sdpa_bwd_noalloc_max_workspace": ([], ctypes.c_size_t),
    "sdpa_bwd_noalloc": ([_P(Desc)] + [_P(Tensor)] * 4 + [_P(RowStat), _P(Tensor), _P(RowStat)]
                         + [_P(Tensor)] * 3 + [ctypes.c_int, ctypes.c_void_p], ctypes.c_int),
    "sdpa_block_mask_build": ([_P(BlockMaskDesc), ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p],
                              ctypes.c_int),
    "sdpa_cp_workspace_size": ([_P(Desc), ctypes.c_int, _P(ctypes.c_size_t)], ctypes.c_int),
    "sdpa_cp_fwd": ([_P(Desc), ctypes.c_int, _P(ctypes.c_int32)] + [_P(Tensor)] * 4
                    + [_P(RowStat), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "sdpa_cp_bwd": ([_P(Desc), ctypes.c_int, _P(ctypes.c_int32)] + [_P(Tensor)] * 4
                    + [_P(RowStat), _P(Tensor), _P(RowStat)] + [_P(Tensor)] * 3
                    + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
}

_PROFILE_SIGNATURES = {
    "sdpa_profile_enable": ([ctypes.c_int], ctypes.c_int),
    "sdpa_profile_read": ([ctypes.c_char_p, ctypes.c_size_t], ctypes.c_int),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libsdpa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m scaled_dot_product_05_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in {**_SIGNATURES, **_PROFILE_SIGNATURES}.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def exported_symbols() -> Sequence[str]:
    return tuple(_SIGNATURES)


def _check(status: int) -> None:
    if status != 0:
        raise SdpaError(status, lib().sdpa_last_error().decode())


# ---------------------------------------------------------------------------------------
# handles
# ---------------------------------------------------------------------------------------

def _dtype_name(t) -> str:
    import torch
    return {torch.float16: "f16", torch.bfloat16: "bf16", torch.float32: "f32",
            torch.float8_e4m3fn: "e4m3", torch.uint8: "e4m3"}[t.dtype]


def tensor(t) -> Tensor:
    """sdpa_tensor_t of a torch tensor whose dims are in the layout's logical order."""
    if t is None:
        return Tensor(None, (ctypes.c_int64 * 4)(0, 0, 0, 0))
    st = list(t.stride()) + [0] * (4 - t.dim())
    return Tensor(ctypes.c_void_p(t.data_ptr() if t.numel() else 0), (ctypes.c_int64 * 4)(*st[:4]))


def rowstat(t) -> RowStat:
    """sdpa_rowstat_t of an fp32 [B,H,S] (or THD [H,T]) tensor; None gives a NULL handle."""
    if t is None:
        return RowStat(None, (ctypes.c_int64 * 3)(0, 0, 0))
    st = list(t.stride()) + [0] * (3 - t.dim())
    return RowStat(ctypes.c_void_p(t.data_ptr() if t.numel() else 0), (ctypes.c_int64 * 3)(*st[:3]))


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def make_desc(layout: str, dtype: str, batch: int, seqlen_q: int, seqlen_k: int, heads_q: int,
              heads_kv: int, head_dim: int, softmax_scale: float, window=(-1, -1),
              diag_align: str | int = "top_left", cu_seqlens_q=None, cu_seqlens_k=None,
              total_q: int = 0, total_k: int = 0, cu_seqlens_q_padded=None,
              cu_seqlens_k_padded=None, block_mask=None) -> Desc:
    """Fill a sdpa_desc_t.  cu_seqlens_* are device int32 tensors (THD only); block_mask a
    BlockMask (kept alive by the caller)."""
    al = ALIGN[diag_align] if isinstance(diag_align, str) else int(diag_align)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    cq = ptr(cu_seqlens_q)
    ck = ptr(cu_seqlens_k) if cu_seqlens_k is not None else cq
    pq = ptr(cu_seqlens_q_padded)
    pk = ptr(cu_seqlens_k_padded) if cu_seqlens_k_padded is not None else pq
    bm = ctypes.cast(ctypes.pointer(block_mask.desc), ctypes.c_void_p) if block_mask is not None else None
    return Desc(LAYOUTS[layout], DTYPES[dtype], batch, seqlen_q, seqlen_k, heads_q, heads_kv,
                head_dim, cq, ck, total_q, total_k, float(softmax_scale), int(window[0]),
                int(window[1]), al, pq, pk, bm)


def make_merge_desc(layout: str, dtype: str, batch: int, seqlen: int, heads: int, head_dim: int,
                    total: int = 0, cu_seqlens=None, cu_seqlens_padded=None) -> MergeDesc:
    """cu_seqlens / cu_seqlens_padded: optional device int32 tensors (THD: merge only the rows
    of these sequences, at their padded starts)."""
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    return MergeDesc(LAYOUTS[layout], DTYPES[dtype], batch, seqlen, heads, head_dim, total,
                     ptr(cu_seqlens), ptr(cu_seqlens_padded))


# ---------------------------------------------------------------------------------------
# the C entry points, by name
# ---------------------------------------------------------------------------------------

def sdpa_version() -> int:
    return lib().sdpa_version()


def sdpa_profile_enable(on: bool) -> None:
    """Start (clearing earlier records) or stop per-launch hipEvent timing (sdpa_profile.h)."""
    _check(lib().sdpa_profile_enable(int(bool(on))))


def sdpa_profile_read() -> dict:
    """{kernel: (launches, total_ms)} over the launches recorded since the last enable."""
    buf = ctypes.create_string_buffer(4096)
    _check(lib().sdpa_profile_read(buf, len(buf)))
    out = {}
    for line in buf.value.decode().splitlines():
        name, n, ms = line.split()
        out[name] = (int(n), float(ms))
    return out


def sdpa_fwd_workspace_size(desc: Desc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().sdpa_fwd_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def sdpa_bwd_workspace_size(desc: Desc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().sdpa_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def _ws(workspace):
    if workspace is None:
        return None, 0
    return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()


def sdpa_fwd_validate(desc, q, k, v, o, lse, workspace_bytes: int = 0) -> None:
    _check(lib().sdpa_fwd_validate(ctypes.byref(desc), tensor(q), tensor(k), tensor(v), tensor(o),
                                   rowstat(lse), workspace_bytes))


def sdpa_fwd(desc, q, k, v, o, lse, workspace=None, stream=None) -> None:
    wp, wb = _ws(workspace)
    _check(lib().sdpa_fwd(ctypes.byref(desc), tensor(q), tensor(k), tensor(v), tensor(o),
                          rowstat(lse), wp, wb, _stream(stream)))


def sdpa_fwd_fp8_validate(desc, q, k, v, o, lse, workspace_bytes: int = 0) -> None:
    _check(lib().sdpa_fwd_fp8_validate(ctypes.byref(desc), tensor(q), tensor(k), tensor(v),
                                       tensor(o), rowstat(lse), workspace_bytes))


def sdpa_fwd_fp8(desc, q, k, v, descale_q, descale_k, descale_v, o, lse, workspace=None,
                 stream=None) -> None:
    """descale_*: device fp32 tensors of one element (None = 1.0)."""
    wp, wb = _ws(workspace)
    dp = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    _check(lib().sdpa_fwd_fp8(ctypes.byref(desc), tensor(q), tensor(k), tensor(v), dp(descale_q),
                              dp(descale_k), dp(descale_v), tensor(o), rowstat(lse), wp, wb,
                              _stream(stream)))


def sdpa_bwd_validate(desc, q, k, v, o, lse, dout, dlse, dq, dk, dv, workspace_bytes: int) -> None:
    _check(lib().sdpa_bwd_validate(ctypes.byref(desc), tensor(q), tensor(k), tensor(v), tensor(o),
                                   rowstat(lse), tensor(dout), rowstat(dlse), tensor(dq),
                                   tensor(dk), tensor(dv), workspace_bytes))


def sdpa_bwd(desc, q, k, v, o, lse, dout, dlse, dq, dk, dv, accumulate: bool = False,
             workspace=None, stream=None) -> None:
    wp, wb = _ws(workspace)
    _check(lib().sdpa_bwd(ctypes.byref(desc), tensor(q), tensor(k), tensor(v), tensor(o),
                          rowstat(lse), tensor(dout), rowstat(dlse), tensor(dq), tensor(dk),
                          tensor(dv), int(bool(accumulate)), wp, wb, _stream(stream)))


def sdpa_bwd_noalloc_max_workspace() -> int:
    return lib().sdpa_bwd_noalloc_max_workspace()


def sdpa_bwd_noalloc(desc, q, k, v, o, lse, dout, dlse, dq, dk, dv, accumulate: bool = False,
                     stream=None) -> None:
    """sdpa_bwd with the library's static scratch buffer as workspace (no allocation)."""
    _check(lib().sdpa_bwd_noalloc(ctypes.byref(desc), tensor(q), tensor(k), tensor(v), tensor(o),
                                  rowstat(lse), tensor(dout), rowstat(dlse), tensor(dq),
                                  tensor(dk), tensor(dv), int(bool(accumulate)), _stream(stream)))


def sdpa_merge_fwd_validate(mdesc, x_a, lse_a, x_b, lse_b, x, lse) -> None:
    _check(lib().sdpa_merge_fwd_validate(ctypes.byref(mdesc), tensor(x_a), rowstat(lse_a),
                                         tensor(x_b), rowstat(lse_b), tensor(x), rowstat(lse)))


def sdpa_merge_bwd_validate(mdesc, x_a, lse_a, x_b, lse_b, g, g_lse, dx_a, dlse_a, dx_b,
                            dlse_b) -> None:
    _check(lib().sdpa_merge_bwd_validate(ctypes.byref(mdesc), tensor(x_a), rowstat(lse_a),
                                         tensor(x_b), rowstat(lse_b), tensor(g), rowstat(g_lse),
                                         tensor(dx_a), rowstat(dlse_a), tensor(dx_b),
                                         rowstat(dlse_b)))


def sdpa_merge_fwd(mdesc, x_a, lse_a, x_b, lse_b, x, lse, stream=None) -> None:
    _check(lib().sdpa_merge_fwd(ctypes.byref(mdesc), tensor(x_a), rowstat(lse_a), tensor(x_b),
                                rowstat(lse_b), tensor(x), rowstat(lse), _stream(stream)))


def sdpa_merge_bwd(mdesc, x_a, lse_a, x_b, lse_b, g, g_lse, dx_a, dlse_a, dx_b, dlse_b,
                   stream=None) -> None:
    _check(lib().sdpa_merge_bwd(ctypes.byref(mdesc), tensor(x_a), rowstat(lse_a), tensor(x_b),
                                rowstat(lse_b), tensor(g), rowstat(g_lse), tensor(dx_a),
                                rowstat(dlse_a), tensor(dx_b), rowstat(dlse_b), _stream(stream)))


def sdpa_block_mask_build(mdesc: BlockMaskDesc, seqlen_q: int, seqlen_k: int, stream=None) -> None:
    _check(lib().sdpa_block_mask_build(ctypes.byref(mdesc), int(seqlen_q), int(seqlen_k),
                                       _stream(stream)))


class BlockMask:
    """A block-sparse mask on the device: the caller's element bits (uint64
    [batch, heads, Sq, ceil(Sk/64)], bit j of word w of row i = key 64w+j visible to query
    i; batch / heads may be 1 to share) and the block table sdpa_block_mask_build writes from
    them into arrays allocated here."""

    BLOCK = 128

    def __init__(self, bits, seqlen_q: int, seqlen_k: int, stream=None):
        import torch
        if bits.dtype not in (torch.int64, torch.uint64) or bits.dim() != 4:
            raise ValueError("bits must be a 4-D int64/uint64 tensor [batch, heads, Sq, words]")
        nb, nh = bits.shape[0], bits.shape[1]
        words = (seqlen_k + 63) // 64
        if tuple(bits.shape[2:]) != (seqlen_q, words) or not bits.is_contiguous():
            raise ValueError(f"bits must be contiguous [.., {seqlen_q}, {words}]")
        nqb, nkb = -(-seqlen_q // self.BLOCK), -(-seqlen_k // self.BLOCK)
        dev = bits.device
        self.bits = bits
        self.kv_count = torch.empty((nb, nh, nqb), dtype=torch.int32, device=dev)
        self.kv_list = torch.empty((nb, nh, nqb, nkb), dtype=torch.int32, device=dev)
        self.q_count = torch.empty((nb, nh, nkb), dtype=torch.int32, device=dev)
        self.q_list = torch.empty((nb, nh, nkb, nqb), dtype=torch.int32, device=dev)
        self.seqlen_q, self.seqlen_k = seqlen_q, seqlen_k
        ptr = lambda t: ctypes.c_void_p(t.data_ptr())
        self.desc = BlockMaskDesc(nb, nh, ptr(bits), ptr(self.kv_count), ptr(self.kv_list),
                                  ptr(self.q_count), ptr(self.q_list))
        sdpa_block_mask_build(self.desc, seqlen_q, seqlen_k, stream)


def _order(hop_order):
    if hop_order is None:
        return None
    arr = (ctypes.c_int32 * len(hop_order))(*[int(x) for x in hop_order])
    return ctypes.cast(arr, _P(ctypes.c_int32)), arr


def sdpa_cp_workspace_size(desc: Desc, cp: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().sdpa_cp_workspace_size(ctypes.byref(desc), int(cp), ctypes.byref(n)))
    return n.value


def sdpa_cp_fwd(desc, cp, hop_order, q, k, v, o, lse, workspace=None, stream=None) -> None:
    wp, wb = _ws(workspace)
    ho = _order(hop_order)
    _check(lib().sdpa_cp_fwd(ctypes.byref(desc), int(cp), ho[0] if ho else None, tensor(q),
                             tensor(k), tensor(v), tensor(o), rowstat(lse), wp, wb, _stream(stream)))


def sdpa_cp_bwd(desc, cp, hop_order, q, k, v, o, lse, dout, dlse, dq, dk, dv, workspace=None,
                stream=None) -> None:
    wp, wb = _ws(workspace)
    ho = _order(hop_order)
    _check(lib().sdpa_cp_bwd(ctypes.byref(desc), int(cp), ho[0] if ho else None, tensor(q),
                             tensor(k), tensor(v), tensor(o), rowstat(lse), tensor(dout),
                             rowstat(dlse), tensor(dq), tensor(dk), tensor(dv), wp, wb,
                             _stream(stream)))


# ---------------------------------------------------------------------------------------
# conveniences: describe a call from the tensors and allocate the outputs (torch.empty)
# ---------------------------------------------------------------------------------------

class Problem:
    """Shapes and options of one attention call, derived from q and k."""

    def __init__(self, q, k, layout: str, softmax_scale: Optional[float] = None, window=(-1, -1),
                 diag_align="top_left", cu_seqlens_q=None, cu_seqlens_k=None,
                 max_seqlen_q: Optional[int] = None, max_seqlen_k: Optional[int] = None,
                 cu_seqlens_q_padded=None, cu_seqlens_k_padded=None, block_mask=None):
        self.layout = layout
        self.dtype = _dtype_name(q)
        d = q.shape[-1]
        if softmax_scale is None:
            raise ValueError("softmax_scale is required")
        if layout == "thd":
            if cu_seqlens_q is None or max_seqlen_q is None:
                raise ValueError("THD needs cu_seqlens_q and max_seqlen_q")
            ck = cu_seqlens_q if cu_seqlens_k is None else cu_seqlens_k
            b = cu_seqlens_q.numel() - 1
            self.desc = make_desc(layout, self.dtype, b, max_seqlen_q,
                                  max_seqlen_q if max_seqlen_k is None else max_seqlen_k,
                                  q.shape[1], k.shape[1], d, softmax_scale, window, diag_align,
                                  cu_seqlens_q, ck, q.shape[0], k.shape[0], cu_seqlens_q_padded,
                                  cu_seqlens_k_padded)
            self.lse_shape = (q.shape[1], q.shape[0])
        else:
            bdim, sdim, hdim = {"bshd": (0, 1, 2), "sbhd": (1, 0, 2), "bhsd": (0, 2, 1)}[layout]
            b, sq, hq = q.shape[bdim], q.shape[sdim], q.shape[hdim]
            self.desc = make_desc(layout, self.dtype, b, sq, k.shape[sdim], hq, k.shape[hdim], d,
                                  softmax_scale, window, diag_align, block_mask=block_mask)
            self.lse_shape = (b, hq, sq)
        # device arrays must outlive the calls
        self.keep = (cu_seqlens_q, cu_seqlens_k, cu_seqlens_q_padded, cu_seqlens_k_padded,
                     block_mask)


def forward(q, k, v, layout: str, softmax_scale: float, window=(-1, -1), diag_align="top_left",
            cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None,
            out=None, lse=None, stream=None, cu_seqlens_q_padded=None, cu_seqlens_k_padded=None,
            block_mask=None):
    """Run sdpa_fwd; returns (O, LSE) with O shaped like q and LSE fp32."""
    import torch
    pr = Problem(q, k, layout, softmax_scale, window, diag_align, cu_seqlens_q, cu_seqlens_k,
                 max_seqlen_q, max_seqlen_k, cu_seqlens_q_padded, cu_seqlens_k_padded, block_mask)
    o = torch.empty_like(q, memory_format=torch.contiguous_format) if out is None else out
    l = torch.empty(pr.lse_shape, dtype=torch.float32, device=q.device) if lse is None else lse
    nws = sdpa_fwd_workspace_size(pr.desc)
    ws = torch.empty(nws, dtype=torch.uint8, device=q.device) if nws else None
    sdpa_fwd(pr.desc, q, k, v, o, l, ws, stream)
    return o, l


def forward_fp8(q, k, v, layout: str, softmax_scale: float, descale_q=None, descale_k=None,
                descale_v=None, window=(-1, -1), diag_align="top_left", cu_seqlens_q=None,
                cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None, out=None, lse=None,
                stream=None):
    """Run sdpa_fwd_fp8 on E4M3 codes (torch uint8 or float8_e4m3fn tensors); descales are
    device fp32 one-element tensors (None = 1).  Returns (O bf16 shaped like q, LSE fp32)."""
    import torch
    pr = Problem(q, k, layout, softmax_scale, window, diag_align, cu_seqlens_q, cu_seqlens_k,
                 max_seqlen_q, max_seqlen_k)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device) if out is None else out
    l = torch.empty(pr.lse_shape, dtype=torch.float32, device=q.device) if lse is None else lse
    nws = sdpa_fwd_workspace_size(pr.desc)
    ws = torch.empty(nws, dtype=torch.uint8, device=q.device) if nws else None
    sdpa_fwd_fp8(pr.desc, q, k, v, descale_q, descale_k, descale_v, o, l, ws, stream)
    return o, l


def backward(q, k, v, o, lse, dout, layout: str, softmax_scale: float, window=(-1, -1),
             diag_align="top_left", dlse=None, cu_seqlens_q=None, cu_seqlens_k=None,
             max_seqlen_q=None, max_seqlen_k=None, dq=None, dk=None, dv=None,
             accumulate: bool = False, stream=None, cu_seqlens_q_padded=None,
             cu_seqlens_k_padded=None, block_mask=None):
    """Run sdpa_bwd; returns (dQ, dK, dV)."""
    import torch
    pr = Problem(q, k, layout, softmax_scale, window, diag_align, cu_seqlens_q, cu_seqlens_k,
                 max_seqlen_q, max_seqlen_k, cu_seqlens_q_padded, cu_seqlens_k_padded, block_mask)
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    nws = sdpa_bwd_workspace_size(pr.desc)
    ws = torch.empty(nws, dtype=torch.uint8, device=q.device) if nws else None
    sdpa_bwd(pr.desc, q, k, v, o, lse, dout, dlse, dq, dk, dv, accumulate, ws, stream)
    return dq, dk, dv


def _merge_desc(x, layout: str):
    d = x.shape[-1]
    if layout == "thd":
        return make_merge_desc(layout, _dtype_name(x), 0, 0, x.shape[1], d, x.shape[0])
    bdim, sdim, hdim = {"bshd": (0, 1, 2), "sbhd": (1, 0, 2), "bhsd": (0, 2, 1)}[layout]
    return make_merge_desc(layout, _dtype_name(x), x.shape[bdim], x.shape[sdim], x.shape[hdim], d)


def merge(x_a, lse_a, x_b, lse_b, layout: str, out=None, lse=None, stream=None):
    """Run sdpa_merge_fwd; returns (x, lse)."""
    import torch
    md = _merge_desc(x_a, layout)
    x = torch.empty_like(x_a, memory_format=torch.contiguous_format) if out is None else out
    l = torch.empty_like(lse_a, memory_format=torch.contiguous_format) if lse is None else lse
    sdpa_merge_fwd(md, x_a, lse_a, x_b, lse_b, x, l, stream)
    return x, l


def merge_backward(x_a, lse_a, x_b, lse_b, g, g_lse, layout: str, stream=None):
    """Run sdpa_merge_bwd; returns (dx_a, dlse_a, dx_b, dlse_b)."""
    import torch
    md = _merge_desc(x_a, layout)
    dxa = torch.empty_like(x_a, memory_format=torch.contiguous_format)
    dxb = torch.empty_like(x_b, memory_format=torch.contiguous_format)
    dla = torch.empty_like(lse_a, memory_format=torch.contiguous_format)
    dlb = torch.empty_like(lse_b, memory_format=torch.contiguous_format)
    sdpa_merge_bwd(md, x_a, lse_a, x_b, lse_b, g, g_lse, dxa, dla, dxb, dlb, stream)
    return dxa, dla, dxb, dlb


def cp_forward(q, k, v, layout: str, softmax_scale: float, window, cp: int, hop_order=None,
               stream=None, cu_seqlens=None, max_seqlen=None, cu_seqlens_padded=None, out=None):
    """Run sdpa_cp_fwd (context-parallel ring emulated on one GPU); returns (O, LSE).  THD:
    cu_seqlens (shared by q and k), max_seqlen and optional cu_seqlens_padded."""
    import torch
    pr = Problem(q, k, layout, softmax_scale, window, "top_left", cu_seqlens, cu_seqlens,
                 max_seqlen, max_seqlen, cu_seqlens_padded, cu_seqlens_padded)
    o = torch.empty_like(q, memory_format=torch.contiguous_format) if out is None else out
    l = torch.empty(pr.lse_shape, dtype=torch.float32, device=q.device)
    ws = torch.empty(sdpa_cp_workspace_size(pr.desc, cp), dtype=torch.uint8, device=q.device)
    sdpa_cp_fwd(pr.desc, cp, hop_order, q, k, v, o, l, ws, stream)
    return o, l


def cp_backward(q, k, v, o, lse, dout, layout: str, softmax_scale: float, window, cp: int,
                hop_order=None, dlse=None, stream=None, cu_seqlens=None, max_seqlen=None,
                cu_seqlens_padded=None, dq=None, dk=None, dv=None):
    """Run sdpa_cp_bwd; returns (dQ, dK, dV)."""
    import torch
    pr = Problem(q, k, layout, softmax_scale, window, "top_left", cu_seqlens, cu_seqlens,
                 max_seqlen, max_seqlen, cu_seqlens_padded, cu_seqlens_padded)
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    ws = torch.empty(sdpa_cp_workspace_size(pr.desc, cp), dtype=torch.uint8, device=q.device)
    sdpa_cp_bwd(pr.desc, cp, hop_order, q, k, v, o, lse, dout, dlse, dq, dk, dv, ws, stream)
    return dq, dk, dv


def flops(n_visible: int, head_dim: int, backward: bool = False) -> int:
    """Algorithmic flops: 4 D per visible (query, key) pair forward, 10 D backward."""
    return (10 if backward else 4) * head_dim * n_visible


def n_visible(sq: int, sk: int, window=(-1, -1), diag_align: int = 0) -> int:
    """Number of visible (query, key) pairs of one head under a window mask (closed form)."""
    off = 0 if diag_align == 0 else sk - sq
    lo = -math.inf if window[0] == -1 else -window[0]
    hi = math.inf if window[1] == -1 else window[1]
    total = 0
    # count per query: keys j in [i + off + lo, i + off + hi] intersect [0, sk)
    for i in range(sq):
        a = 0 if lo == -math.inf else max(0, i + off + lo)
        b = sk - 1 if hi == math.inf else min(sk - 1, i + off + hi)
        if b >= a:
            total += b - a + 1
    return int(total)
