// LSE merge of two partial attention results, forward and backward.
//
// "Significant Accuracy Difference between Compiled and Eager Flex Attention" (PyTorch
// issue 135161, second repro) combines a sliding-window partial and a global partial with
// merge_attn: with m = max(lse_a, lse_b) and w = exp(lse - m),
// x = (x_a w_a + x_b w_b) / (w_a + w_b) and lse = m + log(w_a + w_b).  Per row this is
// x = alpha x_a + beta x_b with alpha = w_a / (w_a + w_b), beta = 1 - alpha, and the
// gradients are dx_a = alpha g, dx_b = beta g, dlse_a = alpha beta <g, x_a - x_b> +
// alpha g_lse and dlse_b = alpha beta <g, x_b - x_a> + beta g_lse.  A row where both
// partials saw no key (-inf, -inf) merges to (0, -inf) with zero gradients.
//
// Pure streaming work (HBM bound): a group of D/VPT lanes owns one row, each lane one
// 16-byte vector; row statistics are fp32 and all arithmetic is fp32.
#include "device.h"
#include "launch.h"
#include "profile.h"

namespace sdpa {

template <int ES, int D>
struct RowMap {
  static constexpr int VPT = 16 / ES;          // elements per lane
  static constexpr int TPR = D / VPT;          // lanes per row
  static constexpr int RPB = kThreads / TPR;   // rows per workgroup
};

struct RowPos {
  int64_t b, h, s;
};

// Row r of the launch: (batch, head, row).  THD with a sequence map enumerates the packed
// rows of the listed sequences (t = 0 .. cu[nseq] - 1) and places each at its sequence's
// row start; s = -1 marks a launch row past the last sequence.
__device__ __forceinline__ RowPos row_pos(const MergeParams& p, int64_t r) {
  RowPos q;
  if (p.thd) {
    q.b = 0;
    q.h = r / p.seqlen;
    q.s = r % p.seqlen;
    if (p.cu) {
      const int32_t t = int32_t(q.s), total = p.seqlen;
      auto at = [&](const int32_t* a, int i) { return min(max(a[i], 0), total); };
      if (t >= at(p.cu, p.nseq)) {
        q.s = -1;
        return q;
      }
      int lo = 0, hi = p.nseq;  // the sequence b with cu[b] <= t < cu[b + 1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (at(p.cu, mid) <= t) lo = mid;
        else hi = mid;
      }
      const int64_t row = int64_t(at(p.pad ? p.pad : p.cu, lo)) + (t - at(p.cu, lo));
      q.s = row < total ? row : -1;
    }
  } else {
    q.s = r % p.seqlen;
    int64_t bh = r / p.seqlen;
    q.h = bh % p.heads;
    q.b = bh / p.heads;
  }
  return q;
}

template <int ES>
__device__ __forceinline__ const char* xrow(const View& v, const RowPos& q) {
  return static_cast<const char*>(v.ptr) + (q.b * v.sb + q.h * v.sh + q.s * v.ss) * ES;
}

__device__ __forceinline__ float* srow(const StatView& v, const RowPos& q) {
  return v.ptr + q.b * v.sb + q.h * v.sh + q.s * v.ss;
}

template <int ES, bool BF>
__device__ __forceinline__ void unpack(const uint4& u, float* f) {
  if constexpr (ES == 4) {
    f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = to_f32<BF>(uint16_t(elem16(u, e)));
  }
}

template <int ES, bool BF>
__device__ __forceinline__ uint4 pack(const float* f) {
  if constexpr (ES == 4)
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  else
    return make_uint4(pack2<BF>(f[0], f[1]), pack2<BF>(f[2], f[3]), pack2<BF>(f[4], f[5]),
                      pack2<BF>(f[6], f[7]));
}

// alpha, beta and the merged lse of one row
__device__ __forceinline__ void weights(float la, float lb, float& alpha, float& beta, float& lse) {
  float m = fmaxf(la, lb);
  if (m == kNegInf) {
    alpha = beta = 0.f;
    lse = kNegInf;
    return;
  }
  float wa = expf(la - m), wb = expf(lb - m);
  float den = wa + wb;
  alpha = wa / den;
  beta = wb / den;
  lse = m + logf(den);
}

template <int ES, bool BF, int D>
__device__ __forceinline__ void merge_fwd_row(const MergeParams& p, int64_t r) {
  using M = RowMap<ES, D>;
  const int tid = threadIdx.x;
  if (r >= p.rows) return;
  const int c = (tid % M::TPR) * M::VPT;
  const RowPos q = row_pos(p, r);
  if (q.s < 0) return;
  float alpha, beta, lse;
  weights(*srow(p.la, q), *srow(p.lb, q), alpha, beta, lse);
  float a[M::VPT], b[M::VPT], x[M::VPT];
  unpack<ES, BF>(load16<ES>(xrow<ES>(p.xa, q) + c * ES, p.aligned), a);
  unpack<ES, BF>(load16<ES>(xrow<ES>(p.xb, q) + c * ES, p.aligned), b);
#pragma unroll
  for (int e = 0; e < M::VPT; ++e) x[e] = alpha * a[e] + beta * b[e];
  store16<ES>(const_cast<char*>(xrow<ES>(p.x, q)) + c * ES, pack<ES, BF>(x), p.aligned);
  if (p.l.ptr && c == 0) *srow(p.l, q) = lse;
}

template <int ES, bool BF, int D>
__device__ __forceinline__ void merge_bwd_row(const MergeParams& p, int64_t r) {
  using M = RowMap<ES, D>;
  const int tid = threadIdx.x;
  const int c = (tid % M::TPR) * M::VPT;
  const RowPos q = row_pos(p, r < p.rows ? r : 0);
  const bool live = r < p.rows && q.s >= 0;  // every lane takes part in the row reduction below
  float alpha = 0.f, beta = 0.f, lse, dot = 0.f;
  float a[M::VPT], b[M::VPT], gg[M::VPT], da[M::VPT], dbv[M::VPT];
  if (live) {
    weights(*srow(p.la, q), *srow(p.lb, q), alpha, beta, lse);
    unpack<ES, BF>(load16<ES>(xrow<ES>(p.xa, q) + c * ES, p.aligned), a);
    unpack<ES, BF>(load16<ES>(xrow<ES>(p.xb, q) + c * ES, p.aligned), b);
    unpack<ES, BF>(load16<ES>(xrow<ES>(p.g, q) + c * ES, p.aligned), gg);
#pragma unroll
    for (int e = 0; e < M::VPT; ++e) {
      dot += gg[e] * (a[e] - b[e]);
      da[e] = alpha * gg[e];
      dbv[e] = beta * gg[e];
    }
  }
#pragma unroll
  for (int off = M::TPR / 2; off > 0; off >>= 1) dot += __shfl_xor(dot, off);
  if (!live) return;
  store16<ES>(const_cast<char*>(xrow<ES>(p.dxa, q)) + c * ES, pack<ES, BF>(da), p.aligned);
  store16<ES>(const_cast<char*>(xrow<ES>(p.dxb, q)) + c * ES, pack<ES, BF>(dbv), p.aligned);
  if (c == 0) {
    float gl = p.glse.ptr ? *srow(p.glse, q) : 0.f;
    float ab = alpha * beta * dot;
    *srow(p.dla, q) = ab + alpha * gl;
    *srow(p.dlb, q) = -ab + beta * gl;
  }
}

// RPB rows per workgroup; a grid capped at kMaxRowBlocks loops over the rest, with the same
// row group across the workgroup in every pass (the backward's row reduction needs all its
// lanes)
template <int ES, bool BF, int D>
__global__ __launch_bounds__(kThreads) void merge_fwd_kernel(MergeParams p) {
  using M = RowMap<ES, D>;
  const int64_t r0 = int64_t(blockIdx.x) * M::RPB, step = int64_t(gridDim.x) * M::RPB;
  merge_fwd_row<ES, BF, D>(p, r0 + threadIdx.x / M::TPR);
  if (gridDim.x == kMaxRowBlocks)
    for (int64_t r = r0 + step; r < p.rows; r += step) merge_fwd_row<ES, BF, D>(p, r + threadIdx.x / M::TPR);
}

template <int ES, bool BF, int D>
__global__ __launch_bounds__(kThreads) void merge_bwd_kernel(MergeParams p) {
  using M = RowMap<ES, D>;
  const int64_t r0 = int64_t(blockIdx.x) * M::RPB, step = int64_t(gridDim.x) * M::RPB;
  merge_bwd_row<ES, BF, D>(p, r0 + threadIdx.x / M::TPR);
  if (gridDim.x == kMaxRowBlocks)
    for (int64_t r = r0 + step; r < p.rows; r += step) merge_bwd_row<ES, BF, D>(p, r + threadIdx.x / M::TPR);
}

template <template <int, bool, int> class K, int ES, bool BF>
static hipError_t merge_go(const MergeParams& p, hipStream_t st, bool fwd) {
  auto pick = [&](auto kernel, int rpb) {
    int64_t blocks = (p.rows + rpb - 1) / rpb;
    if (blocks > kMaxRowBlocks) blocks = kMaxRowBlocks;
    if (blocks <= 0) return hipSuccess;
    prof_begin(st, fwd ? "merge_fwd" : "merge_bwd");
    hipLaunchKernelGGL(kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, st, p);
    prof_end(st);
    return hipGetLastError();
  };
  if (p.d == 32) return pick(K<ES, BF, 32>::fn(), RowMap<ES, 32>::RPB);
  if (p.d == 64) return pick(K<ES, BF, 64>::fn(), RowMap<ES, 64>::RPB);
  return pick(K<ES, BF, 128>::fn(), RowMap<ES, 128>::RPB);
}

template <int ES, bool BF, int D>
struct FwdK {
  static auto fn() { return merge_fwd_kernel<ES, BF, D>; }
};
template <int ES, bool BF, int D>
struct BwdK {
  static auto fn() { return merge_bwd_kernel<ES, BF, D>; }
};

hipError_t launch_merge_fwd(const MergeParams& p, DType dt, hipStream_t st) {
  if (dt == DType::F32) return merge_go<FwdK, 4, false>(p, st, true);
  if (dt == DType::BF16) return merge_go<FwdK, 2, true>(p, st, true);
  return merge_go<FwdK, 2, false>(p, st, true);
}

hipError_t launch_merge_bwd(const MergeParams& p, DType dt, hipStream_t st) {
  if (dt == DType::F32) return merge_go<BwdK, 4, false>(p, st, false);
  if (dt == DType::BF16) return merge_go<BwdK, 2, true>(p, st, false);
  return merge_go<BwdK, 2, false>(p, st, false);
}

}  // namespace sdpa
