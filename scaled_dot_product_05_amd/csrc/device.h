// Device helpers shared by the gfx950 kernels: MFMA wrappers, conversions, strided row
// loads, per-sequence geometry and the window predicate.
//
// MFMA operand layouts used throughout (wave64, v_mfma_f32_32x32x16_{bf16,f16}):
//   A (32 x 16): lane l holds row l%32, contraction slots 8*(l/32) .. 8*(l/32)+7
//   B (16 x 32): lane l holds column l%32, contraction slots 8*(l/32) .. +7
//   C (32 x 32): lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4, column l%32
// and for v_mfma_f32_32x32x2_f32 one fp32 per lane, contraction slot l/32.
// A C tile therefore serves directly as the B operand of a product that contracts over
// its rows, once both operands agree on which row each contraction slot holds.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "params.h"
#include "tiles.h"

namespace sdpa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef double f64x4_t __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;

template <bool BF>
__device__ __forceinline__ f32x16_t mfma16(const uint4& a, const uint4& b, const f32x16_t& c) {
  if constexpr (BF)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma32(float a, float b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// v_mfma_f64_16x16x4_f64: fp64 inputs and accumulation.  A: lane l holds row l%16, slot
// l/16; B: column l%16, slot l/16; C: register r of lane l holds row 4*r + l/16, column l%16.
__device__ __forceinline__ f64x4_t mfma64(double a, double b, const f64x4_t& c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x4_f32.  A and B as the fp64 form; C: register r of lane l holds row
// 4*(l/16) + r, column l%16.
__device__ __forceinline__ f32x4_t mfma16x4(float a, float b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ f64x4_t zero4d() { return f64x4_t{0.0, 0.0, 0.0, 0.0}; }

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Round two fp32 values to the 16-bit type (round to nearest even) and pack lo | hi << 16.
template <bool BF>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  if constexpr (BF) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

template <bool BF>
__device__ __forceinline__ float to_f32(uint16_t x) {
  if constexpr (BF) return __uint_as_float(uint32_t(x) << 16);
  else return float(__builtin_bit_cast(_Float16, x));
}

template <bool BF>
__device__ __forceinline__ uint16_t from_f32(float x) {
  if constexpr (BF) return __builtin_bit_cast(uint16_t, __bf16(x));
  else return __builtin_bit_cast(uint16_t, _Float16(x));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// acc + a.lo * b.lo + a.hi * b.hi for packed 16-bit pairs (v_dot2c_f32_{bf16,f16})
template <bool BF>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  if constexpr (BF)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b),
                                           acc, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), acc, false);
}

// v_permlane32_swap_b32 with both operands x: the first result holds x of lanes 0-31 in
// both halves, the second x of lanes 32-63 in both halves.
__device__ __forceinline__ void halves(float x, float& lo, float& hi) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

// x of the lane 32 away (lane l ^ 32), without an LDS round trip.
__device__ __forceinline__ float xor32(float x) {
  float lo, hi;
  halves(x, lo, hi);
  return (threadIdx.x & 32) ? lo : hi;
}

// max / sum of x over lanes l and l ^ 32; both lanes get the identical result.
__device__ __forceinline__ float max_halves(float x) {
  float lo, hi;
  halves(x, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float sum_halves(float x) {
  float lo, hi;
  halves(x, lo, hi);
  return lo + hi;
}

// LDS as a byte array in its own address space (ds_* instructions with immediate offsets).
typedef __attribute__((address_space(3))) char lds_t;
typedef short s16x4_t __attribute__((ext_vector_type(4)));

// s_waitcnt vmcnt(N): wait until at most N vector memory loads of this wave are in flight
// (LDS and export counters left alone).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// Workgroup barrier that orders LDS accesses only: global loads in flight (including loads
// into LDS, which the caller waits for with vm_wait) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Buffer resource words over [base, base + bytes): loads past the end return zero per
// dword.  Word 3 is the gfx9 default format with offset-only (raw) addressing.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t make_rsrc(const void* base, int64_t bytes) {
  const int32_t n = int32_t(bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes));
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4_t{int32_t(uint32_t(a)), int32_t(uint32_t(a >> 32) & 0xffff), n, 0x00020000};
}

// 16 bytes per lane from global memory straight into LDS: lane i of the wave lands at
// dst + 16 * i (dst wave-uniform), read from the resource at byte offset voff.  Issued as
// inline assembly so that the compiler does not order later LDS reads behind it (it
// cannot tell which LDS bytes the load writes); the caller waits with vm_wait and a
// barrier before the destination is read.  The load reads its LDS address from M0, which
// the compiler writes with a scalar instruction just before; that write needs one wait
// state before an LDS DMA reads it (the compiler pads its own LDS DMA the same way, but
// does not look inside inline assembly), hence the s_nop.
__device__ __forceinline__ void dma16(i32x4_t r, lds_t* dst, uint32_t voff) {
  const uint32_t d = uint32_t(reinterpret_cast<uintptr_t>(dst));
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" : : "{m0}"(d), "v"(voff), "s"(r) : "memory");
}

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 lds_read16(const lds_t* p) {
  return __builtin_bit_cast(uint4, *(const __attribute__((address_space(3))) u32x4_t*)p);
}

// 4 bytes per lane straight into LDS: lane i lands at dst + 4 * i (dst wave-uniform);
// lanes outside the exec mask load nothing.  The same wait state after the M0 write.
__device__ __forceinline__ void dma4(i32x4_t r, lds_t* dst, uint32_t voff) {
  const uint32_t d = uint32_t(reinterpret_cast<uintptr_t>(dst));
  asm volatile("s_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds" : : "{m0}"(d), "v"(voff), "s"(r) : "memory");
}

// ds_read_b64_tr_b16: lane 16g + 4a + b receives element b of the 8-byte rows addressed by
// lanes 16g + a + 4c, c = 0..3, as its elements c.
__device__ __forceinline__ uint2 read_tr16(const lds_t* p) {
  s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p);
  return __builtin_bit_cast(uint2, v);
}

// 16 bytes from a row that is 16-byte aligned (al) or only element aligned.
template <int ES>
__device__ __forceinline__ uint4 load16(const void* p, bool al) {
  if (al) return *static_cast<const uint4*>(p);
  uint4 r;
  if constexpr (ES == 2) {
    const uint16_t* e = static_cast<const uint16_t*>(p);
    r.x = uint32_t(e[0]) | (uint32_t(e[1]) << 16);
    r.y = uint32_t(e[2]) | (uint32_t(e[3]) << 16);
    r.z = uint32_t(e[4]) | (uint32_t(e[5]) << 16);
    r.w = uint32_t(e[6]) | (uint32_t(e[7]) << 16);
  } else {
    const uint32_t* e = static_cast<const uint32_t*>(p);
    r.x = e[0]; r.y = e[1]; r.z = e[2]; r.w = e[3];
  }
  return r;
}

template <int ES>
__device__ __forceinline__ void store16(void* p, const uint4& v, bool al) {
  if (al) { *static_cast<uint4*>(p) = v; return; }
  if constexpr (ES == 2) {
    uint16_t* e = static_cast<uint16_t*>(p);
    e[0] = v.x; e[1] = v.x >> 16; e[2] = v.y; e[3] = v.y >> 16;
    e[4] = v.z; e[5] = v.z >> 16; e[6] = v.w; e[7] = v.w >> 16;
  } else {
    uint32_t* e = static_cast<uint32_t*>(p);
    e[0] = v.x; e[1] = v.y; e[2] = v.z; e[3] = v.w;
  }
}

// 8 bytes (four 16-bit elements) to a row.
__device__ __forceinline__ void store8(uint16_t* p, uint32_t lo, uint32_t hi, bool al) {
  if (al) { *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi); return; }
  p[0] = lo; p[1] = lo >> 16; p[2] = hi; p[3] = hi >> 16;
}

__device__ __forceinline__ uint32_t u4get(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// 16-bit element e (0..7) of a 16-byte vector.
__device__ __forceinline__ uint32_t elem16(const uint4& v, int e) {
  return (u4get(v, e >> 1) >> ((e & 1) * 16)) & 0xffffu;
}

// Position of key (or query) row `r` inside a transposed 16-bit LDS tile: bits 2 and 3
// swapped, so that the 8 contraction slots a lane feeds to one MFMA are contiguous.
__host__ __device__ __forceinline__ int tpos(int r) {
  return (r & ~0xC) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// One sequence of the batch: first packed row (THD) and its lengths.
// Block-sparse mask plane of (batch b, q head h): a mask of extent 1 is shared.
__device__ __forceinline__ int64_t bm_plane(const BlockMaskP& m, int b, int h) {
  return int64_t(m.nb == 1 ? 0 : b) * m.nh + (m.nh == 1 ? 0 : h);
}

// Mask bits of query row i for keys 32 dw .. 32 dw + 31 (bit k: key 32 dw + k); 0 for a row
// or keys outside the (sq, sk) plane.
__device__ __forceinline__ uint32_t bm_dword(const BlockMaskP& m, int64_t plane, int sq, int sk, int i,
                                             int dw) {
  if (i < 0 || i >= sq || dw < 0 || 32 * dw >= sk) return 0u;
  return reinterpret_cast<const uint32_t*>(m.bits + (plane * sq + i) * int64_t(m.words))[dw];
}

// 16-byte chunk swizzles of row-major LDS tiles of CPR chunks per row (chunk c of row r sits
// at slot c ^ sw(r)).
// LDS serves 256 bytes (64 banks) per cycle; a 16-byte read covers 16 lanes per cycle and
// an 8-byte read 32 lanes.  K reads take one chunk of 16 consecutive rows, so those rows
// must fall on 16 distinct 16-byte bank slots; transposed V reads take 4 consecutive rows
// x 64 bytes per 32 lanes, so those 4 rows must fall on distinct 64-byte bank quarters.
template <int CPR>
__device__ __forceinline__ int swk(int r) {
  return CPR >= 16 ? (r & 15) : CPR == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}
template <int CPR>
__device__ __forceinline__ int swv(int r) {
  return CPR >= 16 ? 4 * (r & 3) : CPR == 8 ? 2 * (r & 3) : 0;
}

struct Seq {
  int64_t qrow0, krow0;
  int32_t sq, sk, off;
};

__device__ __forceinline__ int64_t clamp64(int64_t x, int64_t lo, int64_t hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

__device__ __forceinline__ Seq seq_of(const Shape& s, int b) {
  Seq r;
  if (s.thd) {
    int64_t a0 = clamp64(s.cu_q[b], 0, s.total_q);
    int64_t a1 = clamp64(s.cu_q[b + 1], a0, s.total_q);
    int64_t c0 = clamp64(s.cu_k[b], 0, s.total_k);
    int64_t c1 = clamp64(s.cu_k[b + 1], c0, s.total_k);
    // with padding the rows start at the padded offsets; lengths still come from cu_seqlens
    r.qrow0 = s.pad_q ? clamp64(s.pad_q[b], 0, s.total_q) : a0;
    r.krow0 = s.pad_k ? clamp64(s.pad_k[b], 0, s.total_k) : c0;
    int64_t lq = a1 - a0 < s.sq ? a1 - a0 : s.sq;
    int64_t lk = c1 - c0 < s.sk ? c1 - c0 : s.sk;
    lq = lq < s.total_q - r.qrow0 ? lq : s.total_q - r.qrow0;
    lk = lk < s.total_k - r.krow0 ? lk : s.total_k - r.krow0;
    r.sq = int32_t(lq);
    r.sk = int32_t(lk);
  } else {
    r.qrow0 = 0;
    r.krow0 = 0;
    r.sq = s.sq;
    r.sk = s.sk;
  }
  r.off = s.bottom_right ? r.sk - r.sq : 0;
  return r;
}

// Keys [j0, j1) that some query in rows [i0, i1) may see (i1 > i0).
__device__ __forceinline__ void key_range(const Shape& s, const Seq& g, int i0, int i1, int& j0,
                                          int& j1) {
  int64_t lo = int64_t(i0) + g.off + s.lo_rel;
  int64_t hi = int64_t(i1 - 1) + g.off + s.hi_rel + 1;
  j0 = int(clamp64(lo, 0, g.sk));
  j1 = int(clamp64(hi, j0, g.sk));
}

// Queries [i0, i1) that may see some key in [j0, j1) (j1 > j0).
__device__ __forceinline__ void query_range(const Shape& s, const Seq& g, int j0, int j1, int& i0,
                                            int& i1) {
  int64_t lo = int64_t(j0) - g.off - s.hi_rel;
  int64_t hi = int64_t(j1 - 1) - g.off - s.lo_rel + 1;
  i0 = int(clamp64(lo, 0, g.sq));
  i1 = int(clamp64(hi, i0, g.sq));
}

__device__ __forceinline__ bool visible(const Shape& s, const Seq& g, int i, int j) {
  int rel = j - i - g.off;
  return rel >= s.lo_rel && rel <= s.hi_rel && j < g.sk && i < g.sq;
}

// Every (i, j) of rows [i0, i1) x keys [j0, j1) visible and in range.
__device__ __forceinline__ bool tile_full(const Shape& s, const Seq& g, int i0, int i1, int j0,
                                          int j1) {
  return int64_t(j0) - (i1 - 1) - g.off >= s.lo_rel && int64_t(j1 - 1) - i0 - g.off <= s.hi_rel &&
         j1 <= g.sk && i1 <= g.sq;
}

}  // namespace sdpa
