"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws numbers and arranges them in memory: it holds none of the
attention arithmetic.  Both the HIP path (through the C-ABI binding) and the fp64
oracle receive tensors built here; the oracle gets an exact fp64 promotion of the
very bytes the GPU gets.

Recipe (one stream per tensor): ``numpy.random.default_rng([seed, config, tensor])``
draws fp64 N(0,1); the values are rounded to fp32 (round-to-nearest-even) and then
to the working dtype with torch's RNE conversion.

Workloads follow the pages' problem statements:

* ``c1`` non-causal MHA, fp32, B1 S128 H4 D64, BHSD contiguous, scale 1/8.
* ``c2`` causal self-attention fwd+bwd, bf16, B4 S1024 H8 D64, BSHD contiguous, scale 1/8.
* ``c3`` MQA causal from one packed QKV tensor [2048,1,18,64] fp16 split on the head
  dim into q (16 heads), k (1), v (1): non-contiguous SBHD views with element strides
  (1152,1152,64,1), window (-1,0), scale 1.0 or 0.1  (TransformerEngine issue 1195,
  first and second repro).
* ``c4`` varlen THD causal, bf16: 8 sequences, lengths uniform on [256,4096] (integers,
  both ends inclusive), int32 cu_seqlens, 16 q heads, 4 kv heads, D128, scale 1/sqrt(128).
* ``c5`` fp32 local+global split merged by LSE: x ~ N(0,1) [1,512,256], W [256,768] and
  b [768] = 0.1 + 0.02 N(0,1), qkv = x W + b (fp64, then fp32), 4 heads of 64, BSHD views
  of the [1,512,768] projection (PyTorch issue 135161, first repro).
* ``target`` causal bf16 BSHD self-attention at long S (the throughput workload).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

LAYOUTS = ("bshd", "sbhd", "bhsd", "thd")
DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def normal(seed: int, config: int, tensor: int, shape) -> np.ndarray:
    """fp64 N(0,1) draws from the stream (seed, config, tensor)."""
    return np.random.default_rng([seed, config, tensor]).standard_normal(shape)


def cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    """RNE-cast fp64 values to a CPU torch tensor of ``dtype`` ('f16','bf16','f32')."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(DTYPES[dtype])


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy of a (possibly strided, possibly device) tensor's values."""
    return t.detach().to("cpu", torch.float64).numpy().copy()


def to_bhsd(t: torch.Tensor, layout: str) -> torch.Tensor:
    """View a 4-D tensor given in ``layout`` logical order as [B,H,S,D] (a permutation)."""
    if layout == "bshd":
        return t.permute(0, 2, 1, 3)
    if layout == "sbhd":
        return t.permute(1, 2, 0, 3)
    if layout == "bhsd":
        return t
    raise ValueError(layout)


def from_bhsd_shape(b: int, h: int, s: int, d: int, layout: str):
    """Logical shape, in ``layout`` order, of a [B,H,S,D] tensor."""
    return {"bshd": (b, s, h, d), "sbhd": (s, b, h, d), "bhsd": (b, h, s, d)}[layout]


@dataclass
class Workload:
    """One attention problem: shapes, options and the CPU input tensors."""

    name: str
    dtype: str
    layout: str
    batch: int
    seqlen_q: int
    seqlen_k: int
    heads_q: int
    heads_kv: int
    head_dim: int
    scale: float
    window: tuple = (-1, -1)
    diag_align: int = 0  # 0 = top-left, 1 = bottom-right
    q: Optional[torch.Tensor] = None
    k: Optional[torch.Tensor] = None
    v: Optional[torch.Tensor] = None
    dout: Optional[torch.Tensor] = None
    dlse: Optional[torch.Tensor] = None
    cu_seqlens_q: Optional[np.ndarray] = None
    cu_seqlens_k: Optional[np.ndarray] = None
    extra: dict = field(default_factory=dict)

    @property
    def is_thd(self) -> bool:
        return self.layout == "thd"


def lse_shape(w: Workload):
    """Shape of the fp32 LSE buffer: [B,Hq,Sq] for padded layouts, [Hq,T] for THD."""
    if w.is_thd:
        return (w.heads_q, int(w.cu_seqlens_q[-1]))
    return (w.batch, w.heads_q, w.seqlen_q)


def dense(seed: int, config: int, dtype: str, layout: str, b: int, sq: int, sk: int,
          hq: int, hk: int, d: int, scale: float, window=(-1, -1), diag_align: int = 0,
          with_grad: bool = False, with_dlse: bool = False, name: str = "dense") -> Workload:
    """Contiguous q,k,v (and dO, dLSE) in a padded layout, N(0,1) values."""
    shp_q = from_bhsd_shape(b, hq, sq, d, layout)
    shp_k = from_bhsd_shape(b, hk, sk, d, layout)
    w = Workload(name, dtype, layout, b, sq, sk, hq, hk, d, scale, tuple(window), diag_align)
    w.q = cast(normal(seed, config, 0, shp_q), dtype)
    w.k = cast(normal(seed, config, 1, shp_k), dtype)
    w.v = cast(normal(seed, config, 2, shp_k), dtype)
    if with_grad:
        w.dout = cast(normal(seed, config, 3, shp_q), dtype)
    if with_dlse:
        w.dlse = torch.from_numpy(normal(seed, config, 4, (b, hq, sq)).astype(np.float32))
    return w


def thd_lengths(seed: int, n: int = 8, lo: int = 256, hi: int = 4096) -> np.ndarray:
    """Sequence lengths uniform on the integers [lo, hi], both ends included."""
    return np.random.default_rng([seed, 4, 0]).integers(lo, hi + 1, size=n)


def cu_seqlens(lengths) -> np.ndarray:
    out = np.zeros(len(lengths) + 1, dtype=np.int32)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return out


def thd(seed: int, config: int, dtype: str, lengths, hq: int, hk: int, d: int, scale: float,
        window=(-1, 0), with_grad: bool = False, with_dlse: bool = False,
        lengths_k=None, diag_align: int = 0, name: str = "thd") -> Workload:
    """Packed varlen q [T,Hq,D], k,v [Tk,Hk,D] with int32 cu_seqlens."""
    cq = cu_seqlens(lengths)
    ck = cq if lengths_k is None else cu_seqlens(lengths_k)
    tq, tk = int(cq[-1]), int(ck[-1])
    lk = lengths if lengths_k is None else lengths_k
    w = Workload(name, dtype, "thd", len(lengths), int(max(lengths, default=0)),
                 int(max(lk, default=0)), hq, hk, d, scale, tuple(window), diag_align)
    w.q = cast(normal(seed, config, 0, (tq, hq, d)), dtype)
    w.k = cast(normal(seed, config, 1, (tk, hk, d)), dtype)
    w.v = cast(normal(seed, config, 2, (tk, hk, d)), dtype)
    if with_grad:
        w.dout = cast(normal(seed, config, 3, (tq, hq, d)), dtype)
    if with_dlse:
        w.dlse = torch.from_numpy(normal(seed, config, 4, (hq, tq)).astype(np.float32))
    w.cu_seqlens_q, w.cu_seqlens_k = cq, ck
    return w


# ---------------------------------------------------------------------------------------
# The pages' workloads
# ---------------------------------------------------------------------------------------

def c1(seed: int = 0) -> Workload:
    return dense(seed, 1, "f32", "bhsd", 1, 128, 128, 4, 4, 64, 1.0 / 8.0, name="c1")


def c2(seed: int = 0, with_grad: bool = True) -> Workload:
    return dense(seed, 2, "bf16", "bshd", 4, 1024, 1024, 8, 8, 64, 1.0 / 8.0, window=(-1, 0),
                 with_grad=with_grad, name="c2")


def packed_qkv(seed: int, config: int, dtype: str, s: int, b: int, hq: int, hk: int, d: int):
    """One [S,B,Hq+2Hk,D] buffer split on the head dim into q, k, v views (not copies)."""
    buf = cast(normal(seed, config, 0, (s, b, hq + 2 * hk, d)), dtype)
    q, k, v = buf.split([hq, hk, hk], dim=2)
    return buf, q, k, v


def c3(seed: int = 0, scale: float = 1.0, seqlen: int = 2048) -> Workload:
    buf, q, k, v = packed_qkv(seed, 3, "f16", seqlen, 1, 16, 1, 64)
    w = Workload("c3", "f16", "sbhd", 1, seqlen, seqlen, 16, 1, 64, scale, (-1, 0), 0, q, k, v)
    w.extra["packed"] = buf
    return w


def c4(seed: int = 0, with_grad: bool = True, n: int = 8) -> Workload:
    return thd(seed, 4, "bf16", thd_lengths(seed, n), 16, 4, 128, 1.0 / math.sqrt(128.0),
               window=(-1, 0), with_grad=with_grad, name="c4")


def c5_projection(seed: int = 0, n_ctx: int = 512, d_in: int = 256, d_attn: int = 256):
    """x [1,n_ctx,d_in], W [d_in,3 d_attn], b [3 d_attn]; returns fp32 qkv [1,n_ctx,3 d_attn]."""
    x = normal(seed, 5, 0, (1, n_ctx, d_in))
    wgt = 0.1 + 0.02 * normal(seed, 5, 1, (d_in, 3 * d_attn))
    bias = 0.1 + 0.02 * normal(seed, 5, 2, (3 * d_attn,))
    qkv = x @ wgt + bias  # input recipe (the pages' Linear layer), fp64 then RNE to fp32
    return x, wgt, bias, torch.from_numpy(qkv.astype(np.float32))


def c5(seed: int = 0, n_ctx: int = 512, heads: int = 4, d: int = 64) -> dict:
    """Inputs of the local+global split: BSHD q,k,v views of one [1,S,3*H*D] projection.

    local  = sliding window (128,0) over all keys;
    global = keys 0..63 only (a view), causal, top-left aligned.
    The upstream gradient is g = 1 on the merged output and g_lse = 0 (a sum loss);
    a random (g, g_lse) pair is provided as well.
    """
    x, wgt, bias, qkv = c5_projection(seed, n_ctx, 256, heads * d)
    da = heads * d
    q = qkv[:, :, 0:da].unflatten(2, (heads, d))
    k = qkv[:, :, da:2 * da].unflatten(2, (heads, d))
    v = qkv[:, :, 2 * da:3 * da].unflatten(2, (heads, d))
    g_rand = torch.from_numpy(normal(seed, 5, 3, (1, n_ctx, heads, d)).astype(np.float32))
    glse_rand = torch.from_numpy(normal(seed, 5, 4, (1, heads, n_ctx)).astype(np.float32))
    return dict(x=x, W=wgt, b=bias, qkv=qkv, q=q, k=k, v=v, scale=1.0 / math.sqrt(d),
                local_window=(128, 0), global_keys=64, n_ctx=n_ctx, heads=heads, d=d,
                g_ones=torch.ones(1, n_ctx, heads, d), glse_zero=torch.zeros(1, heads, n_ctx),
                g_rand=g_rand, glse_rand=glse_rand)


def target(seed: int = 0, b: int = 8, s: int = 4096, h: int = 8, hk: Optional[int] = None,
           d: int = 64, with_grad: bool = False, dtype: str = "bf16") -> Workload:
    """Causal bf16 BSHD self-attention, scale 1/sqrt(D): the long-sequence throughput case."""
    return dense(seed, 6, dtype, "bshd", b, s, s, h, h if hk is None else hk, d,
                 1.0 / math.sqrt(d), window=(-1, 0), with_grad=with_grad, name="target")


# ---------------------------------------------------------------------------------------
# element masks for the block-sparse path (FlexAttention mask_mod predicates of PyTorch
# issue 135161, and generic structured masks), and their bit packing
# ---------------------------------------------------------------------------------------

def flex_mask(name: str, sq: int, sk: int, band: int = 128, q_offset: int = 0,
              doc_lengths=None, seed: int = 0, density: float = 0.5) -> np.ndarray:
    """Boolean [Sq,Sk] visibility built from a named predicate over (q_idx, kv_idx).

    ``q_offset`` is added to the row index before the predicate (issue 135161's v1 form
    evaluates its global mask on query rows sliced from ``band`` on, in local indices, so
    the caller passes the local rows with q_offset = 0 there).
    Predicates:
      sliding_window_causal  (q >= kv) & (q - kv <= band)
      global_causal_v1       q > kv
      global_causal_v2       (q >= kv) & (q - kv > band)
      causal                 q >= kv
      prefix                 kv < band (every query sees the first ``band`` keys)
      document               q and kv in the same document (``doc_lengths``), causal
      random_blocks          128x128 blocks drawn empty / full / random bits
      random                 independent bits with probability ``density``
    """
    qi = np.arange(sq)[:, None] + q_offset
    kj = np.arange(sk)[None, :]
    if name == "sliding_window_causal":
        return (qi >= kj) & (qi - kj <= band)
    if name == "global_causal_v1":
        return np.broadcast_to(qi > kj, (sq, sk)).copy()
    if name == "global_causal_v2":
        return (qi >= kj) & (qi - kj > band)
    if name == "causal":
        return np.broadcast_to(qi >= kj, (sq, sk)).copy()
    if name == "prefix":
        return np.broadcast_to(kj < band, (sq, sk)).copy()
    if name == "document":
        ends = np.cumsum(np.asarray(doc_lengths))
        dq = np.searchsorted(ends, qi, side="right")
        dk = np.searchsorted(ends, kj, side="right")
        return (dq == dk) & (qi >= kj)
    rng = np.random.default_rng([seed, 9, sq, sk])
    if name == "random":
        return rng.random((sq, sk)) < density
    if name == "random_blocks":
        nqb, nkb = -(-sq // 128), -(-sk // 128)
        kind = rng.integers(0, 3, size=(nqb, nkb))  # 0 empty, 1 full, 2 random bits
        bits = rng.random((nqb * 128, nkb * 128)) < density
        full = np.kron(kind == 1, np.ones((128, 128), bool))
        part = np.kron(kind == 2, np.ones((128, 128), bool)) & bits
        return (full | part)[:sq, :sk]
    raise ValueError(f"unknown mask predicate {name!r}")


def pack_mask(mask: np.ndarray) -> np.ndarray:
    """Pack boolean [..., Sq, Sk] into uint64 [..., Sq, ceil(Sk/64)]: bit j of word w of row
    i is key 64w+j (little-endian bit order; keys past Sk are 0)."""
    mask = np.asarray(mask, dtype=bool)
    sk = mask.shape[-1]
    words = -(-sk // 64)
    pad = np.zeros(mask.shape[:-1] + (words * 64,), dtype=bool)
    pad[..., :sk] = mask
    by = np.packbits(pad, axis=-1, bitorder="little")
    return np.ascontiguousarray(by).view("<u8").reshape(mask.shape[:-1] + (words,))


# ---------------------------------------------------------------------------------------
# FP8 (E4M3) inputs: per-tensor delayed-scaling style codes
# ---------------------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_codes(x: np.ndarray):
    """Per-tensor scaled E4M3 codes of fp64 values x, with descale = amax / 448 so that the
    largest magnitude maps to the largest finite code: returns (uint8 codes as a CPU torch
    tensor, descale).  The cast is torch's round-to-nearest-even float8_e4m3fn conversion."""
    x = np.asarray(x, dtype=np.float64)
    amax = float(np.abs(x).max()) if x.size else 1.0
    descale = amax / E4M3_MAX if amax > 0 else 1.0
    scaled = torch.from_numpy(np.ascontiguousarray(x / descale, dtype=np.float32))
    return scaled.to(torch.float8_e4m3fn).view(torch.uint8), descale
