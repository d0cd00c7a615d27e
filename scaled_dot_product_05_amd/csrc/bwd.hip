// Fused attention backward for gfx950, recomputing P from the saved LSE.
//
// Gradient of a loss through O and through the returned LSE (PyTorch issue 135161,
// "Significant Accuracy Difference between Compiled and Eager Flex Attention": the merged
// LSE is differentiated, so the backward receives dLSE):
//   Delta_i = dO_i . O_i - dLSE_i,   P_ij = exp(s_ij - LSE_i),   dP = dO V^T,
//   dS_ij = P_ij (dP_ij - Delta_i),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
// Launches on one stream.  No gradient is ever accumulated with atomics: every element of
// dQ, dK and dV has one writer.  The only atomic operation is an arrival counter of the
// GQA dK/dV split (two workgroups per small-grid dK/dV block, see bwd_fused16p_kernel):
// the half that arrives second adds the other's fp32 partial sums, in a fixed order.
//   pre   Delta and LSE log2(e) for every query row (streaming, HBM bound);
//   dq    one workgroup per 64 (16-bit) or 128 (fp32) query rows of a q head, streaming
//         the key tiles;
//   dkdv  one workgroup per 64 (16-bit) or 128 (fp32) keys of a kv head, streaming the
//         query tiles of every q head of its group, so dK and dV of a GQA group are summed
//         in registers.
// With 16-byte aligned rows and head_dim 64 or 128, dq and dkdv are the pipelined kernels
// near the end of this file (streamed tiles loaded straight into LDS, transposed operands
// read with ds_read_b64_tr_b16) and run as one launch; on large grids (no block mask, no
// split) they run as two launches of four-wave workgroups instead, dq first (128 query
// rows per workgroup, forming Delta and LSE log2(e) in place of the pre-pass), then dkdv
// (128 keys per workgroup, the four waves sharing each Q/dO tile); under THD the longest
// dkdv items may run as two half blocks whose fp32 partial sums a combine launch adds (no
// atomics: each half writes its own slot).  Otherwise the register-staged
// kernels below keep the row-contracted operands (K in dq; Q and dO in dkdv) transposed in
// LDS, written once per tile from the registers that fill the row-major copy, and split the
// streamed tile between wave pairs so small problems still launch enough waves.  fp32 mode
// uses true fp32 MFMA and reads the transposed operand element-wise from the row-major tile.
#include "device.h"
#include "launch.h"
#include "profile.h"

namespace sdpa {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int64_t delta_index(const Shape& s, int b, int h, const Seq& g, int i) {
  return s.thd ? int64_t(h) * s.total_q + g.qrow0 + i : (int64_t(b) * s.hq + h) * s.sq + i;
}

// ----------------------------------------------------------------------------------------
// pre-pass: Delta_i = dO_i . O_i - dLSE_i, and LSE_i log2(e) as a contiguous array
// ----------------------------------------------------------------------------------------
template <int ES, bool BF, int D>
__device__ __forceinline__ void bwd_pre_rows(const BwdParams& p, int64_t rows, int64_t r) {
  constexpr int VPT = 16 / ES, TPR = D / VPT;
  const Shape& s = p.s;
  const int tid = threadIdx.x;
  const bool live = r < rows;
  int64_t b = 0, h, t;
  if (s.thd) {
    h = live ? r / s.total_q : 0;
    t = live ? r % s.total_q : 0;
  } else {
    t = live ? r % s.sq : 0;
    int64_t bh = live ? r / s.sq : 0;
    h = bh % s.hq;
    b = bh / s.hq;
  }
  const int c = (tid % TPR) * VPT;
  float dot = 0.f;
  if (live) {
    const char* orow = static_cast<const char*>(p.o.ptr) + (b * p.o.sb + h * p.o.sh + t * p.o.ss + c) * ES;
    const char* grow = static_cast<const char*>(p.dout.ptr) +
                       (b * p.dout.sb + h * p.dout.sh + t * p.dout.ss + c) * ES;
    uint4 ov = load16<ES>(orow, p.aligned & kAlO);
    uint4 gv = load16<ES>(grow, p.aligned & kAlDO);
    if constexpr (ES == 4) {
      dot = __uint_as_float(ov.x) * __uint_as_float(gv.x) + __uint_as_float(ov.y) * __uint_as_float(gv.y) +
            __uint_as_float(ov.z) * __uint_as_float(gv.z) + __uint_as_float(ov.w) * __uint_as_float(gv.w);
    } else {
      // one fma chain per 8-element chunk (the four-wave dQ kernel repeats these roundings)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        dot = __builtin_fmaf(to_f32<BF>(uint16_t(elem16(ov, e))), to_f32<BF>(uint16_t(elem16(gv, e))), dot);
    }
  }
  // butterfly over the row's TPR chunks
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) dot += __shfl_xor(dot, off);
  if (live && c == 0) {
    float dl = p.dlse.ptr ? p.dlse.ptr[b * p.dlse.sb + h * p.dlse.sh + t * p.dlse.ss] : 0.f;
    p.delta[r] = dot - dl;
    const float l = p.lse.ptr[b * p.lse.sb + h * p.lse.sh + t * p.lse.ss];
    p.lse2[r] = l == kNegInf ? __builtin_inff() : l * kLog2e;
  }
}

// RPB rows per workgroup per pass; the grid is capped and loops over the rest, with the same
// row group across the workgroup in every pass (the row reduction needs all its lanes)
template <int ES, bool BF, int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(BwdParams p) {
  constexpr int TPR = D / (16 / ES), RPB = kThreads / TPR;
  const Shape& s = p.s;
  const int64_t rows = s.thd ? int64_t(s.hq) * s.total_q : int64_t(s.batch) * s.hq * s.sq;
  if (p.nsplit > 1) {
    // counters of the split dK/dV blocks of the launch that follows on this stream
    for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < p.split_blocks;
         i += int64_t(gridDim.x) * kThreads)
      p.split_cnt[i] = 0;
  }
  for (int64_t r0 = int64_t(blockIdx.x) * RPB; r0 < rows; r0 += int64_t(gridDim.x) * RPB)
    bwd_pre_rows<ES, BF, D>(p, rows, r0 + threadIdx.x / TPR);
}

// ----------------------------------------------------------------------------------------
// work decode shared by dq (query tiles, heaviest last tile first) and dkdv (key tiles)
// ----------------------------------------------------------------------------------------
struct BwdPos {
  int b, h, tile;
  int item = 0;   // THD: index in the work list
};

// GROUPED (head_dim 128 kernels): THD grids with a multiple of 8 heads give each XCD a
// contiguous range of heads; causal/window grids with more than kBwdHeadGroup kv heads'
// pairs per XCD take them in groups of kBwdHeadGroup (q heads: times the GQA group), tiles
// longest first within a group (measured: B8 S4096 D128 2596 -> 2520 us, B16 S2048 D128
// 1571 -> 1474 us; at head_dim 64 it lost 1-5%).
template <bool GROUPED = false>
__device__ __forceinline__ bool bwd_decode(const Shape& s, const WorkItem* work,
                                           const int32_t* count, int heads, int len, int tile_rows,
                                           bool reverse, BwdPos& w, int bid = -1) {
  if (bid < 0) bid = blockIdx.x;
  if (s.thd) {
    int item, h;
    if (GROUPED && heads % kXcds == 0) {
      // XCD x (block b on XCD b % 8) runs the contiguous heads [x per, (x + 1) per), so a kv
      // group's q heads share an XCD (head_dim 128 kernels; C4's THD GQA backward
      // 1045 -> 988 us)
      const int per = heads / kXcds, j = bid / kXcds;
      item = j / per;
      h = (bid % kXcds) * per + j % per;
    } else {
      item = bid / heads;
      h = bid % heads;
    }
    w.h = h;
    w.item = item;
    if (item >= *count) return false;
    WorkItem it = work[item];
    w.b = it.seq;
    w.tile = it.tile;
    return true;
  }
  int bh = s.batch * heads;
  int nt = (len + tile_rows - 1) / tile_rows;
  int t = 0, r = 0;
  const bool uniform = s.uniform != 0;
  bool grouped = false;
  if constexpr (GROUPED) {
    const int hg = kBwdHeadGroup * (heads == s.hk ? 1 : s.group);
    grouped = bh % kXcds == 0 && !uniform &&
              (bh / kXcds) % hg == 0 && bh / kXcds > hg;
    if (grouped) {
      const int per = bh / kXcds, x = bid % kXcds, k = bid / kXcds;
      const int gi = k / (hg * nt), kk = k - gi * hg * nt;
      r = x * per + gi * hg + kk % hg;
      t = kk / hg;
    }
  }
  if (grouped) {
    // r and t set above
  } else if (bh % kXcds == 0 && (uniform || s.group > 1)) {
    // Block b runs on XCD b % 8 (dQ blocks follow a multiple of 8 dK/dV blocks in the fused
    // launch).  XCD x owns the pairs [x per, (x + 1) per): for dK/dV the (batch, kv head)
    // pairs and for dQ the (batch, q head) pairs of the same kv heads, so a kv group's K/V
    // and its q heads' Q/dO meet in one XCD's L2.  Tiles of equal cost: pair after pair
    // (fewer heads resident); causal or window masks: tiles longest first across the XCD's
    // pairs, and only under GQA (with one q head per kv head the order below measured the
    // same or slightly faster: C2 39.3 vs 39.7 us).
    const int per = bh / kXcds, x = bid % kXcds, k = bid / kXcds;
    const int dv = uniform ? nt : per, q = k / dv, m = k - q * dv;  // one division
    r = x * per + (uniform ? q : m);
    t = uniform ? m : q;
  } else {
    t = bid / bh;
    r = bid % bh;
  }
  w.b = r / heads;
  w.h = r % heads;
  w.tile = reverse ? nt - 1 - t : t;
  return true;
}

// Load a [64 rows x D] 16-bit tile into registers so that this thread holds RPT
// consecutive rows of one 8-element column chunk (the layout both LDS copies need).
template <int D>
struct Tile16 {
  static constexpr int ROWS = 64;
  static constexpr int RPT = ROWS * D / 8 / kThreads;  // rows per thread
  static constexpr int RP = D + 8;                     // row-major pitch (elements)
  static constexpr int TP = ROWS + 8;                  // transposed pitch (elements)
  static_assert(RPT >= 1 && RPT <= 4, "tile split");
  uint4 r[RPT];
  // Rows past nrows read the last row instead (in bounds, branch-free); callers give them
  // P = 0.  nrows >= 1.
  __device__ __forceinline__ void load(const uint16_t* base, int64_t ss, int row0, int nrows, bool al) {
    const int dc = threadIdx.x % (D / 8), rg = threadIdx.x / (D / 8);
#pragma unroll
    for (int x = 0; x < RPT; ++x) {
      const int row = min(row0 + rg * RPT + x, nrows - 1);
      r[x] = load16<2>(base + int64_t(row) * ss + dc * 8, al);
    }
  }
  __device__ __forceinline__ void store_rows(uint16_t* lds) const {
    const int dc = threadIdx.x % (D / 8), rg = threadIdx.x / (D / 8);
#pragma unroll
    for (int x = 0; x < RPT; ++x)
      *reinterpret_cast<uint4*>(&lds[(rg * RPT + x) * RP + dc * 8]) = r[x];
  }
  __device__ __forceinline__ void store_transposed(uint16_t* lds) const {
    const int dc = threadIdx.x % (D / 8), rg = threadIdx.x / (D / 8);
    const int pos = tpos(rg * RPT);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t* dst = &lds[(dc * 8 + e) * TP + pos];
      if constexpr (RPT == 4) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(elem16(r[0], e) | (elem16(r[1], e) << 16),
                                                    elem16(r[2], e) | (elem16(r[3], e) << 16));
      } else if constexpr (RPT == 2) {
        *reinterpret_cast<uint32_t*>(dst) = elem16(r[0], e) | (elem16(r[1], e) << 16);
      } else {
        *dst = uint16_t(elem16(r[0], e));
      }
    }
  }
};

// Write 4 consecutive d values (scaled) of one row, adding to the old ones if asked.
template <bool BF>
__device__ __forceinline__ void out4_16(uint16_t* p, const float* v, float scale, bool al, bool acc) {
  float x[4] = {v[0] * scale, v[1] * scale, v[2] * scale, v[3] * scale};
  if (acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] += to_f32<BF>(p[i]);
  }
  store8(p, pack2<BF>(x[0], x[1]), pack2<BF>(x[2], x[3]), al);
}

__device__ __forceinline__ void out4_32(float* p, const float* v, float scale, bool al, bool acc) {
  float x[4] = {v[0] * scale, v[1] * scale, v[2] * scale, v[3] * scale};
  if (acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] += p[i];
  }
  store16<4>(p, make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                           __float_as_uint(x[3])), al);
}

// ----------------------------------------------------------------------------------------
// dQ, 16-bit.  A workgroup owns 64 query rows of one q head and streams 64-key tiles.
// Wave w takes query block w&1 (32 rows) and key half w>>1 of every tile; the two key
// halves' partial dQ are summed once through LDS at the end (fixed order, no atomics).
// ----------------------------------------------------------------------------------------
template <bool BF, int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq16_kernel(BwdParams p) {
  constexpr int BM = kBwdQ16, BN = kBwdQInner;
  using T = Tile16<D>;
  static_assert(BN == T::ROWS && BM == 64, "tile split");
  constexpr int NC = D / 16, NDB = D / 32;
  constexpr int OFF_KT = BN * T::RP, OFF_V = OFF_KT + D * T::TP, SMEM = OFF_V + BN * T::RP;
  static_assert(2 * NDB * 16 * 64 * 4 <= SMEM * 2, "reduction buffer");
  __shared__ __align__(16) uint16_t smem[SMEM];
  uint16_t* sk_ = smem;
  uint16_t* skt_ = smem + OFF_KT;
  uint16_t* sv_ = smem + OFF_V;

  const Shape& s = p.s;
  BwdPos w;
  if (!bwd_decode(s, p.work_q, p.count_q, s.hq, s.sq, BM, true, w)) return;
  const Seq g = seq_of(s, w.b);
  const int q0 = w.tile * BM;
  if (q0 >= g.sq) return;
  const int qend = min(q0 + BM, g.sq);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hf = lane >> 5;
  const int qblk = wave & 1, khalf = wave >> 1;
  const int hk = w.h / s.group;
  const uint16_t* qb = static_cast<const uint16_t*>(p.q.ptr) + w.b * p.q.sb + w.h * p.q.sh + g.qrow0 * p.q.ss;
  const uint16_t* gb = static_cast<const uint16_t*>(p.dout.ptr) + w.b * p.dout.sb + w.h * p.dout.sh +
                       g.qrow0 * p.dout.ss;
  const uint16_t* kb = static_cast<const uint16_t*>(p.k.ptr) + w.b * p.k.sb + hk * p.k.sh + g.krow0 * p.k.ss;
  const uint16_t* vb = static_cast<const uint16_t*>(p.v.ptr) + w.b * p.v.sb + hk * p.v.sh + g.krow0 * p.v.ss;
  uint16_t* dqb = static_cast<uint16_t*>(p.dq.ptr) + w.b * p.dq.sb + w.h * p.dq.sh + g.qrow0 * p.dq.ss;

  int j0, j1;
  key_range(s, g, q0, qend, j0, j1);
  const int kt0 = j0 / BN, kt1 = j1 > j0 ? (j1 + BN - 1) / BN : kt0;
  const int qw0 = q0 + qblk * 32, qw1 = min(qw0 + 32, g.sq);
  const int qi = qw0 + l32;
  const bool qvalid = qi < g.sq;
  int wj0 = 0, wj1 = 0;
  if (qw0 < qw1) key_range(s, g, qw0, qw1, wj0, wj1);

  uint4 qf[NC], gf[NC];
  {
    const int qr = min(qi, g.sq - 1);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qf[c] = load16<2>(qb + qr * p.q.ss + 16 * c + 8 * hf, p.aligned & kAlQ);
      gf[c] = load16<2>(gb + qr * p.dout.ss + 16 * c + 8 * hf, p.aligned & kAlDO);
    }
  }
  float lse2 = __builtin_inff(), dl = 0.f;
  if (qvalid) {
    float l = p.lse.ptr[w.b * p.lse.sb + w.h * p.lse.sh + (g.qrow0 + qi) * p.lse.ss];
    lse2 = l == kNegInf ? __builtin_inff() : l * kLog2e;
    dl = p.delta[delta_index(s, w.b, w.h, g, qi)];
  }
  f32x16_t acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = zero16();

  T kt, vt;
  if (kt0 < kt1) {
    kt.load(kb, p.k.ss, kt0 * BN, g.sk, p.aligned & kAlK);
    vt.load(vb, p.v.ss, kt0 * BN, g.sk, p.aligned & kAlV);
  }
  for (int t = kt0; t < kt1; ++t) {
    const int kbase = t * BN;
    __syncthreads();  // previous tile fully consumed
    kt.store_rows(sk_);
    kt.store_transposed(skt_);
    vt.store_rows(sv_);
    __syncthreads();
    if (t + 1 < kt1) {  // next tile's global loads overlap this tile's compute
      kt.load(kb, p.k.ss, kbase + BN, g.sk, p.aligned & kAlK);
      vt.load(vb, p.v.ss, kbase + BN, g.sk, p.aligned & kAlV);
    }
    const int kw = kbase + 32 * khalf;  // this wave's 32 keys
    if (kw < wj1 && kw + 32 > wj0) {
      const bool full = tile_full(s, g, qw0, qw1, kw, kw + 32);
      f32x16_t st = zero16(), dp = zero16();
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        uint4 a = *reinterpret_cast<const uint4*>(&sk_[(32 * khalf + l32) * T::RP + 16 * c + 8 * hf]);
        uint4 bv = *reinterpret_cast<const uint4*>(&sv_[(32 * khalf + l32) * T::RP + 16 * c + 8 * hf]);
        st = mfma16<BF>(a, qf[c], st);
        dp = mfma16<BF>(bv, gf[c], dp);
      }
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pr = fast_exp2(st[r] * s.scale_log2 - lse2);
        if (!full && !visible(s, g, qi, kw + 8 * (r >> 2) + 4 * hf + (r & 3))) pr = 0.f;
        ds[r] = pr * (dp[r] - dl);
      }
      uint4 dsf[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        dsf[h2] = make_uint4(pack2<BF>(ds[8 * h2], ds[8 * h2 + 1]), pack2<BF>(ds[8 * h2 + 2], ds[8 * h2 + 3]),
                             pack2<BF>(ds[8 * h2 + 4], ds[8 * h2 + 5]), pack2<BF>(ds[8 * h2 + 6], ds[8 * h2 + 7]));
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          uint4 a = *reinterpret_cast<const uint4*>(&skt_[(db * 32 + l32) * T::TP + 32 * khalf + 16 * c + 8 * hf]);
          acc[db] = mfma16<BF>(a, dsf[c], acc[db]);
        }
    }
  }
  // sum the two key halves: khalf 1 parks its partial in LDS, khalf 0 adds and writes
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
  if (khalf == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[((qblk * NDB + db) * 16 + r) * 64 + lane] = acc[db][r];
  }
  __syncthreads();
  if (khalf == 0 && qvalid) {
    uint16_t* row = dqb + qi * p.dq.ss;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = acc[db][4 * gq + e] + red[((qblk * NDB + db) * 16 + 4 * gq + e) * 64 + lane];
        out4_16<BF>(row + db * 32 + 8 * gq + 4 * hf, v, s.scale, p.aligned & kAlDQ, p.accumulate);
      }
  }
}

// ----------------------------------------------------------------------------------------
// dK, dV, 16-bit.  A workgroup owns 64 keys of one kv head and streams 64-row query tiles
// of every q head of the group.  Wave w takes key block w&1 (32 keys) and query half w>>1
// of every tile; the two query halves' partial dK, dV are summed once through LDS.
// ----------------------------------------------------------------------------------------
template <bool BF, int D>
__global__ __launch_bounds__(kThreads, D == 128 ? 1 : 2) void bwd_dkdv16_kernel(BwdParams p) {
  constexpr int BK = kBwdK16, BQ = kBwdKInner;
  using T = Tile16<D>;
  static_assert(BQ == T::ROWS && BK == 64, "tile split");
  constexpr int NC = D / 16, NDB = D / 32;
  constexpr int OFF_QT = BQ * T::RP, OFF_G = OFF_QT + D * T::TP, OFF_GT = OFF_G + BQ * T::RP;
  constexpr int SMEM = OFF_GT + D * T::TP;
  static_assert(2 * 2 * NDB * 16 * 64 * 4 <= SMEM * 2, "reduction buffer");
  __shared__ __align__(16) uint16_t smem[SMEM];
  __shared__ __align__(16) float slse_[BQ];
  __shared__ __align__(16) float sdl_[BQ];
  uint16_t* sq_ = smem;
  uint16_t* sqt_ = smem + OFF_QT;
  uint16_t* sg_ = smem + OFF_G;
  uint16_t* sgt_ = smem + OFF_GT;

  const Shape& s = p.s;
  BwdPos w;
  if (!bwd_decode(s, p.work_k, p.count_k, s.hk, s.sk, BK, false, w)) return;
  const Seq g = seq_of(s, w.b);
  const int k0 = w.tile * BK;
  if (k0 >= g.sk) return;
  const int kend = min(k0 + BK, g.sk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hf = lane >> 5;
  const int kblk = wave & 1, qhalf = wave >> 1;
  const int hk = w.h;
  const uint16_t* kb = static_cast<const uint16_t*>(p.k.ptr) + w.b * p.k.sb + hk * p.k.sh + g.krow0 * p.k.ss;
  const uint16_t* vb = static_cast<const uint16_t*>(p.v.ptr) + w.b * p.v.sb + hk * p.v.sh + g.krow0 * p.v.ss;
  uint16_t* dkb = static_cast<uint16_t*>(p.dk.ptr) + w.b * p.dk.sb + hk * p.dk.sh + g.krow0 * p.dk.ss;
  uint16_t* dvb = static_cast<uint16_t*>(p.dv.ptr) + w.b * p.dv.sb + hk * p.dv.sh + g.krow0 * p.dv.ss;

  int i0, i1;
  query_range(s, g, k0, kend, i0, i1);
  const int qt0 = i0 / BQ, qt1 = i1 > i0 ? (i1 + BQ - 1) / BQ : qt0;
  const int kw0 = k0 + kblk * 32, kw1 = min(kw0 + 32, g.sk);
  const int kj = kw0 + l32;
  const bool kvalid = kj < g.sk;
  int wi0 = 0, wi1 = 0;
  if (kw0 < kw1) query_range(s, g, kw0, kw1, wi0, wi1);

  uint4 kf[NC], vf[NC];
  {
    const int kr = min(kj, g.sk - 1);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      kf[c] = load16<2>(kb + kr * p.k.ss + 16 * c + 8 * hf, p.aligned & kAlK);
      vf[c] = load16<2>(vb + kr * p.v.ss + 16 * c + 8 * hf, p.aligned & kAlV);
    }
  }
  f32x16_t adk[NDB], adv[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    adk[i] = zero16();
    adv[i] = zero16();
  }

  // items = (q head of the group, q tile); the next item's global loads overlap compute
  T qt, gt;
  const int nq = qt1 - qt0, nitems = s.group * nq;
  float lv = __builtin_inff(), dv = 0.f;
  auto load_item = [&](int it) {
    const int h = hk * s.group + it / nq, qbase = (qt0 + it % nq) * BQ;
    qt.load(static_cast<const uint16_t*>(p.q.ptr) + w.b * p.q.sb + h * p.q.sh + g.qrow0 * p.q.ss,
            p.q.ss, qbase, g.sq, p.aligned & kAlQ);
    gt.load(static_cast<const uint16_t*>(p.dout.ptr) + w.b * p.dout.sb + h * p.dout.sh + g.qrow0 * p.dout.ss,
            p.dout.ss, qbase, g.sq, p.aligned & kAlDO);
    if (tid < BQ) {
      const int i = qbase + tid, ic = min(i, g.sq - 1);
      const float l = p.lse.ptr[w.b * p.lse.sb + h * p.lse.sh + (g.qrow0 + ic) * p.lse.ss];
      const float d = p.delta[delta_index(s, w.b, h, g, ic)];
      lv = (i < g.sq && l != kNegInf) ? l * kLog2e : __builtin_inff();
      dv = i < g.sq ? d : 0.f;
    }
  };
  if (nitems > 0) load_item(0);
  for (int it = 0; it < nitems; ++it) {
    const int qbase = (qt0 + it % nq) * BQ;
    __syncthreads();
    qt.store_rows(sq_);
    qt.store_transposed(sqt_);
    gt.store_rows(sg_);
    gt.store_transposed(sgt_);
    if (tid < BQ) {
      slse_[tid] = lv;
      sdl_[tid] = dv;
    }
    __syncthreads();
    if (it + 1 < nitems) load_item(it + 1);
    const int qr0 = qbase + 32 * qhalf;  // this wave's 32 query rows
    if (qr0 < wi1 && qr0 + 32 > wi0) {
      const bool full = tile_full(s, g, qr0, min(qr0 + 32, g.sq), kw0, kw1);
      f32x16_t st = zero16(), dp = zero16();
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        uint4 a = *reinterpret_cast<const uint4*>(&sq_[(32 * qhalf + l32) * T::RP + 16 * c + 8 * hf]);
        uint4 b2 = *reinterpret_cast<const uint4*>(&sg_[(32 * qhalf + l32) * T::RP + 16 * c + 8 * hf]);
        st = mfma16<BF>(a, kf[c], st);
        dp = mfma16<BF>(b2, vf[c], dp);
      }
      float pr[16], ds[16];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int ql = 32 * qhalf + 8 * g4 + 4 * hf;
        float4 l4 = *reinterpret_cast<const float4*>(&slse_[ql]);
        float4 d4 = *reinterpret_cast<const float4*>(&sdl_[ql]);
        float la[4] = {l4.x, l4.y, l4.z, l4.w}, da[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g4 + e;
          float x = fast_exp2(st[r] * s.scale_log2 - la[e]);
          if (!full && !visible(s, g, qbase + ql + e, kj)) x = 0.f;
          pr[r] = x;
          ds[r] = x * (dp[r] - da[e]);
        }
      }
      uint4 pf[2], dsf[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        pf[h2] = make_uint4(pack2<BF>(pr[8 * h2], pr[8 * h2 + 1]), pack2<BF>(pr[8 * h2 + 2], pr[8 * h2 + 3]),
                            pack2<BF>(pr[8 * h2 + 4], pr[8 * h2 + 5]), pack2<BF>(pr[8 * h2 + 6], pr[8 * h2 + 7]));
        dsf[h2] = make_uint4(pack2<BF>(ds[8 * h2], ds[8 * h2 + 1]), pack2<BF>(ds[8 * h2 + 2], ds[8 * h2 + 3]),
                             pack2<BF>(ds[8 * h2 + 4], ds[8 * h2 + 5]), pack2<BF>(ds[8 * h2 + 6], ds[8 * h2 + 7]));
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int off = (db * 32 + l32) * T::TP + 32 * qhalf + 16 * c + 8 * hf;
          uint4 a = *reinterpret_cast<const uint4*>(&sgt_[off]);
          uint4 b2 = *reinterpret_cast<const uint4*>(&sqt_[off]);
          adv[db] = mfma16<BF>(a, pf[c], adv[db]);
          adk[db] = mfma16<BF>(b2, dsf[c], adk[db]);
        }
    }
  }
  // sum the two query halves: qhalf 1 parks its partials in LDS, qhalf 0 adds and writes
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
  if (qhalf == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        red[(((kblk * 2 + 0) * NDB + db) * 16 + r) * 64 + lane] = adk[db][r];
        red[(((kblk * 2 + 1) * NDB + db) * 16 + r) * 64 + lane] = adv[db][r];
      }
  }
  __syncthreads();
  if (qhalf == 0 && kvalid) {
    uint16_t* krow = dkb + kj * p.dk.ss;
    uint16_t* vrow = dvb + kj * p.dv.ss;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = db * 32 + 8 * gq + 4 * hf;
        float a[4], b2[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * gq + e;
          a[e] = adk[db][r] + red[(((kblk * 2 + 0) * NDB + db) * 16 + r) * 64 + lane];
          b2[e] = adv[db][r] + red[(((kblk * 2 + 1) * NDB + db) * 16 + r) * 64 + lane];
        }
        out4_16<BF>(krow + d, a, s.scale, p.aligned & kAlDK, p.accumulate);
        out4_16<BF>(vrow + d, b2, 1.f, p.aligned & kAlDV, p.accumulate);
      }
  }
}

// ----------------------------------------------------------------------------------------
// fp32: true fp32 MFMA 32x32x2, inner tiles of 32 rows, row-major LDS only
// ----------------------------------------------------------------------------------------
template <int D>
struct Tile32 {
  static constexpr int ROWS = 32;
  static constexpr int RP = D + 4;
  static constexpr int LDC = ROWS * D / 4 / kThreads;
  static_assert(LDC >= 1, "tile split");
  uint4 r[LDC];
  __device__ __forceinline__ void load(const float* base, int64_t ss, int row0, int nrows, bool al) {
#pragma unroll
    for (int u = 0; u < LDC; ++u) {
      const int ci = threadIdx.x + u * kThreads;
      const int row = min(row0 + ci / (D / 4), nrows - 1), col = (ci % (D / 4)) * 4;
      r[u] = load16<4>(base + int64_t(row) * ss + col, al);
    }
  }
  __device__ __forceinline__ void store(float* lds) const {
#pragma unroll
    for (int u = 0; u < LDC; ++u) {
      int ci = threadIdx.x + u * kThreads;
      *reinterpret_cast<uint4*>(&lds[(ci / (D / 4)) * RP + (ci % (D / 4)) * 4]) = r[u];
    }
  }
};

template <int D, bool BSM>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq32_kernel(BwdParams p) {
  constexpr int BM = kBwdQ32, BN = 32, H2 = D / 2, NDB = D / 32;
  using T = Tile32<D>;
  __shared__ __align__(16) float sk_[BN * T::RP];
  __shared__ __align__(16) float sv_[BN * T::RP];

  const Shape& s = p.s;
  BwdPos w;
  if (!bwd_decode(s, p.work_q, p.count_q, s.hq, s.sq, BM, true, w)) return;
  const Seq g = seq_of(s, w.b);
  const int q0 = w.tile * BM;
  if (q0 >= g.sq) return;
  const int qend = min(q0 + BM, g.sq);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hf = lane >> 5;
  const int hk = w.h / s.group;
  const float* qb = static_cast<const float*>(p.q.ptr) + w.b * p.q.sb + w.h * p.q.sh + g.qrow0 * p.q.ss;
  const float* gb = static_cast<const float*>(p.dout.ptr) + w.b * p.dout.sb + w.h * p.dout.sh + g.qrow0 * p.dout.ss;
  const float* kb = static_cast<const float*>(p.k.ptr) + w.b * p.k.sb + hk * p.k.sh + g.krow0 * p.k.ss;
  const float* vb = static_cast<const float*>(p.v.ptr) + w.b * p.v.sb + hk * p.v.sh + g.krow0 * p.v.ss;
  float* dqb = static_cast<float*>(p.dq.ptr) + w.b * p.dq.sb + w.h * p.dq.sh + g.qrow0 * p.dq.ss;

  int j0, j1;
  key_range(s, g, q0, qend, j0, j1);
  const int kt0 = j0 / BN, kt1 = j1 > j0 ? (j1 + BN - 1) / BN : kt0;
  const int qw0 = q0 + wave * 32, qw1 = min(qw0 + 32, g.sq);
  const int qi = qw0 + l32;
  const bool qvalid = qi < g.sq;
  int wj0 = 0, wj1 = 0;
  if (qw0 < qw1) key_range(s, g, qw0, qw1, wj0, wj1);

  float qf[H2], gf[H2];
#pragma unroll
  for (int u = 0; u < H2 / 4; ++u) {
    uint4 a = qvalid ? load16<4>(qb + qi * p.q.ss + hf * H2 + 4 * u, p.aligned & kAlQ) : make_uint4(0, 0, 0, 0);
    uint4 b = qvalid ? load16<4>(gb + qi * p.dout.ss + hf * H2 + 4 * u, p.aligned & kAlDO) : make_uint4(0, 0, 0, 0);
    qf[4 * u] = __uint_as_float(a.x); qf[4 * u + 1] = __uint_as_float(a.y);
    qf[4 * u + 2] = __uint_as_float(a.z); qf[4 * u + 3] = __uint_as_float(a.w);
    gf[4 * u] = __uint_as_float(b.x); gf[4 * u + 1] = __uint_as_float(b.y);
    gf[4 * u + 2] = __uint_as_float(b.z); gf[4 * u + 3] = __uint_as_float(b.w);
  }
  float lse2 = __builtin_inff(), dl = 0.f;
  if (qvalid) {
    float l = p.lse.ptr[w.b * p.lse.sb + w.h * p.lse.sh + (g.qrow0 + qi) * p.lse.ss];
    lse2 = l == kNegInf ? __builtin_inff() : l * kLog2e;
    dl = p.delta[delta_index(s, w.b, w.h, g, qi)];
  }
  f32x16_t acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = zero16();

  // block-sparse mask: the 128-key blocks of this 128-row block row replace [kt0, kt1)
  constexpr int TPB = kMaskBlock / BN;
  int64_t plane = 0, lrow = 0;
  int nt = kt1 - kt0;
  if constexpr (BSM) {
    static_assert(BM == kMaskBlock, "block rows");
    plane = bm_plane(s.bm, w.b, w.h);
    lrow = plane * s.bm.nqb + q0 / kMaskBlock;
    nt = min(max(s.bm.kv_count[lrow], 0), s.bm.nkb) * TPB;
  }
  T ktile, vtile;
  for (int it = 0; it < nt; ++it) {
    int t = kt0 + it;
    bool part = false;
    if constexpr (BSM) {
      const int e = s.bm.kv_list[lrow * s.bm.nkb + it / TPB];
      t = min(max(e >> 1, 0), s.bm.nkb - 1) * TPB + it % TPB;
      part = (e & 1) != 0;
    }
    const int kbase = t * BN;
    ktile.load(kb, p.k.ss, kbase, g.sk, p.aligned & kAlK);
    vtile.load(vb, p.v.ss, kbase, g.sk, p.aligned & kAlV);
    __syncthreads();
    ktile.store(sk_);
    vtile.store(sv_);
    __syncthreads();
    if (kbase < wj1 && kbase + BN > wj0) {
      const bool full = tile_full(s, g, qw0, qw1, kbase, kbase + BN) && !part;
      // element bits of this row's 32 keys (a 32-key tile is dword t of the row)
      const uint32_t mb = part ? bm_dword(s.bm, plane, s.sq, s.sk, qi, t) : ~0u;
      f32x16_t st = zero16(), dp = zero16();
#pragma unroll
      for (int u = 0; u < H2 / 4; ++u) {
        float4 kv = *reinterpret_cast<const float4*>(&sk_[l32 * T::RP + hf * H2 + 4 * u]);
        float4 vv = *reinterpret_cast<const float4*>(&sv_[l32 * T::RP + hf * H2 + 4 * u]);
        st = mfma32(kv.x, qf[4 * u], st); st = mfma32(kv.y, qf[4 * u + 1], st);
        st = mfma32(kv.z, qf[4 * u + 2], st); st = mfma32(kv.w, qf[4 * u + 3], st);
        dp = mfma32(vv.x, gf[4 * u], dp); dp = mfma32(vv.y, gf[4 * u + 1], dp);
        dp = mfma32(vv.z, gf[4 * u + 2], dp); dp = mfma32(vv.w, gf[4 * u + 3], dp);
      }
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pr = fast_exp2(st[r] * s.scale_log2 - lse2);
        if (!full && !(visible(s, g, qi, kbase + 8 * (r >> 2) + 4 * hf + (r & 3)) &&
                       ((mb >> (8 * (r >> 2) + 4 * hf + (r & 3))) & 1u)))
          pr = 0.f;
        ds[r] = pr * (dp[r] - dl);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          int key = 8 * (i >> 2) + 4 * hf + (i & 3);
          acc[db] = mfma32(sk_[key * T::RP + db * 32 + l32], ds[i], acc[db]);
        }
    }
  }
  if (qvalid) {
    float* row = dqb + qi * p.dq.ss;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float v[4] = {acc[db][4 * gq], acc[db][4 * gq + 1], acc[db][4 * gq + 2], acc[db][4 * gq + 3]};
        out4_32(row + db * 32 + 8 * gq + 4 * hf, v, s.scale, p.aligned & kAlDQ, p.accumulate);
      }
  }
}

template <int D, bool BSM>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv32_kernel(BwdParams p) {
  constexpr int BK = kBwdK32, BQ = 32, H2 = D / 2, NDB = D / 32;
  using T = Tile32<D>;
  __shared__ __align__(16) float sq_[BQ * T::RP];
  __shared__ __align__(16) float sg_[BQ * T::RP];
  __shared__ __align__(16) float slse_[BQ];
  __shared__ __align__(16) float sdl_[BQ];

  const Shape& s = p.s;
  BwdPos w;
  if (!bwd_decode(s, p.work_k, p.count_k, s.hk, s.sk, BK, false, w)) return;
  const Seq g = seq_of(s, w.b);
  const int k0 = w.tile * BK;
  if (k0 >= g.sk) return;
  const int kend = min(k0 + BK, g.sk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hf = lane >> 5;
  const int hk = w.h;
  const float* kb = static_cast<const float*>(p.k.ptr) + w.b * p.k.sb + hk * p.k.sh + g.krow0 * p.k.ss;
  const float* vb = static_cast<const float*>(p.v.ptr) + w.b * p.v.sb + hk * p.v.sh + g.krow0 * p.v.ss;
  float* dkb = static_cast<float*>(p.dk.ptr) + w.b * p.dk.sb + hk * p.dk.sh + g.krow0 * p.dk.ss;
  float* dvb = static_cast<float*>(p.dv.ptr) + w.b * p.dv.sb + hk * p.dv.sh + g.krow0 * p.dv.ss;

  int i0, i1;
  query_range(s, g, k0, kend, i0, i1);
  const int qt0 = i0 / BQ, qt1 = i1 > i0 ? (i1 + BQ - 1) / BQ : qt0;
  const int kw0 = k0 + wave * 32, kw1 = min(kw0 + 32, g.sk);
  const int kj = kw0 + l32;
  const bool kvalid = kj < g.sk;
  int wi0 = 0, wi1 = 0;
  if (kw0 < kw1) query_range(s, g, kw0, kw1, wi0, wi1);

  float kf[H2], vf[H2];
#pragma unroll
  for (int u = 0; u < H2 / 4; ++u) {
    uint4 a = kvalid ? load16<4>(kb + kj * p.k.ss + hf * H2 + 4 * u, p.aligned & kAlK) : make_uint4(0, 0, 0, 0);
    uint4 b = kvalid ? load16<4>(vb + kj * p.v.ss + hf * H2 + 4 * u, p.aligned & kAlV) : make_uint4(0, 0, 0, 0);
    kf[4 * u] = __uint_as_float(a.x); kf[4 * u + 1] = __uint_as_float(a.y);
    kf[4 * u + 2] = __uint_as_float(a.z); kf[4 * u + 3] = __uint_as_float(a.w);
    vf[4 * u] = __uint_as_float(b.x); vf[4 * u + 1] = __uint_as_float(b.y);
    vf[4 * u + 2] = __uint_as_float(b.z); vf[4 * u + 3] = __uint_as_float(b.w);
  }
  f32x16_t adk[NDB], adv[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    adk[i] = zero16();
    adv[i] = zero16();
  }

  T qtile, gtile;
  for (int gi = 0; gi < s.group; ++gi) {
    const int h = hk * s.group + gi;
    const float* qb = static_cast<const float*>(p.q.ptr) + w.b * p.q.sb + h * p.q.sh + g.qrow0 * p.q.ss;
    const float* gb = static_cast<const float*>(p.dout.ptr) + w.b * p.dout.sb + h * p.dout.sh + g.qrow0 * p.dout.ss;
    // block-sparse mask: the 128-row blocks of this 128-key block column replace [qt0, qt1)
    constexpr int TPQ = kMaskBlock / BQ;
    int64_t plane = 0, lcol = 0;
    int nt = qt1 - qt0;
    if constexpr (BSM) {
      static_assert(BK == kMaskBlock, "block columns");
      plane = bm_plane(s.bm, w.b, h);
      lcol = plane * s.bm.nkb + k0 / kMaskBlock;
      nt = min(max(s.bm.q_count[lcol], 0), s.bm.nqb) * TPQ;
    }
    for (int it = 0; it < nt; ++it) {
      int t = qt0 + it;
      bool part = false;
      if constexpr (BSM) {
        const int e = s.bm.q_list[lcol * s.bm.nqb + it / TPQ];
        t = min(max(e >> 1, 0), s.bm.nqb - 1) * TPQ + it % TPQ;
        part = (e & 1) != 0;
      }
      const int qbase = t * BQ;
      qtile.load(qb, p.q.ss, qbase, g.sq, p.aligned & kAlQ);
      gtile.load(gb, p.dout.ss, qbase, g.sq, p.aligned & kAlDO);
      float lv = __builtin_inff(), dv = 0.f;
      if (tid < BQ) {
        int i = qbase + tid;
        if (i < g.sq) {
          float l = p.lse.ptr[w.b * p.lse.sb + h * p.lse.sh + (g.qrow0 + i) * p.lse.ss];
          lv = l == kNegInf ? __builtin_inff() : l * kLog2e;
          dv = p.delta[delta_index(s, w.b, h, g, i)];
        }
      }
      __syncthreads();
      qtile.store(sq_);
      gtile.store(sg_);
      if (tid < BQ) {
        slse_[tid] = lv;
        sdl_[tid] = dv;
      }
      __syncthreads();
      if (qbase < wi1 && qbase + BQ > wi0) {
        const bool full = tile_full(s, g, qbase, min(qbase + BQ, g.sq), kw0, kw1) && !part;
        f32x16_t st = zero16(), dp = zero16();
#pragma unroll
        for (int u = 0; u < H2 / 4; ++u) {
          float4 qv = *reinterpret_cast<const float4*>(&sq_[l32 * T::RP + hf * H2 + 4 * u]);
          float4 gv = *reinterpret_cast<const float4*>(&sg_[l32 * T::RP + hf * H2 + 4 * u]);
          st = mfma32(qv.x, kf[4 * u], st); st = mfma32(qv.y, kf[4 * u + 1], st);
          st = mfma32(qv.z, kf[4 * u + 2], st); st = mfma32(qv.w, kf[4 * u + 3], st);
          dp = mfma32(gv.x, vf[4 * u], dp); dp = mfma32(gv.y, vf[4 * u + 1], dp);
          dp = mfma32(gv.z, vf[4 * u + 2], dp); dp = mfma32(gv.w, vf[4 * u + 3], dp);
        }
        float pr[16], ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = 8 * (r >> 2) + 4 * hf + (r & 3);
          float x = fast_exp2(st[r] * s.scale_log2 - slse_[ql]);
          // element bit of (query row, this lane's key): bit l32 of dword kw0 / 32 of the row
          if (!full && !(visible(s, g, qbase + ql, kj) &&
                         (!part || ((bm_dword(s.bm, plane, s.sq, s.sk, qbase + ql, kw0 / 32) >> l32) & 1u))))
            x = 0.f;
          pr[r] = x;
          ds[r] = x * (dp[r] - sdl_[ql]);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int ql = 8 * (i >> 2) + 4 * hf + (i & 3);
            adv[db] = mfma32(sg_[ql * T::RP + db * 32 + l32], pr[i], adv[db]);
            adk[db] = mfma32(sq_[ql * T::RP + db * 32 + l32], ds[i], adk[db]);
          }
      }
    }
  }
  if (kvalid) {
    float* krow = dkb + kj * p.dk.ss;
    float* vrow = dvb + kj * p.dv.ss;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = db * 32 + 8 * gq + 4 * hf;
        float a[4] = {adk[db][4 * gq], adk[db][4 * gq + 1], adk[db][4 * gq + 2], adk[db][4 * gq + 3]};
        float b2[4] = {adv[db][4 * gq], adv[db][4 * gq + 1], adv[db][4 * gq + 2], adv[db][4 * gq + 3]};
        out4_32(krow + d, a, s.scale, p.aligned & kAlDK, p.accumulate);
        out4_32(vrow + d, b2, 1.f, p.aligned & kAlDV, p.accumulate);
      }
  }
}

// ----------------------------------------------------------------------------------------
// Pipelined 16-bit backward kernels (16-byte aligned rows, head_dim 64 / 128).
//
// Streamed tiles go from HBM straight into LDS (buffer loads with an LDS destination, as
// in the forward) and stay row-major; their 16-byte chunks are XOR-swizzled by row with
// swb(), which keeps both access patterns free of bank conflicts: 16-byte row reads of 16
// consecutive rows (A operands) and transposed 8-byte reads of 4 rows x 64 bytes
// (ds_read_b64_tr_b16, operands contracted over the tile's rows).
// ----------------------------------------------------------------------------------------
template <int CPR>
__device__ __forceinline__ int swb(int r) {
  if constexpr (CPR >= 16)
    return ((r >> 2) & 1) | (((r >> 3) & 1) << 1) | ((r & 1) << 2) | (((r >> 1) & 1) << 3);
  else if constexpr (CPR == 8)
    return (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1);
  else
    return (r >> 2) & 3;
}

// Lane part of the byte offset of a transposed read inside a [rows x CPR chunks] tile:
// lane 16g + 4c + a supplies row 8h + 4(g/2) + c (plus 16 cc, an immediate), 8-byte half
// a&1 of chunk 4db + 2(g&1) + a/2.  The swizzle depends on h, so each h has its own offset.
template <int CPR>
__device__ __forceinline__ int tr_offset(int lane, int db, int h) {
  const int g = lane >> 4, c = (lane >> 2) & 3, a = lane & 3;
  const int row = 8 * h + 4 * (g >> 1) + c;
  return (row * CPR + ((4 * db + 2 * (g & 1) + (a >> 1)) ^ swb<CPR>(row))) * 16 + (a & 1) * 8;
}

// dQ.  A workgroup of W waves owns 32 W query rows of one q head (lane = query, as the
// forward) and streams 32-key tiles:
//   S^T  = K Q^T     (A: K rows from LDS, B: Q^T in registers)
//   dP^T = V dO^T    (A: V rows from LDS, B: dO^T in registers)
//   dS^T = P^T (dP^T - Delta),  P^T = exp2(S^T scale log2e - LSE log2e)
//   dQ^T += K^T dS^T (A: K^T by transposed reads, B: dS^T straight from registers)
// K and V rings of 4 slots: step t reads K(t) (transposed, for dQ) and K(t+1), V(t+1) (the
// next tile's products), and issues the loads of K(t+3), V(t+3) into the slots step t-1
// read.
template <int D, int W>
struct DqP {
  static constexpr int BN = 32, TB = BN * D * 2, NSK = 4, NSV = 4;
  static constexpr int LDS = (NSK + NSV) * TB;
};

// DELTA: the block also forms Delta_i = dO_i . O_i - dLSE_i and LSE_i log2(e) of its rows and
// stores them for the dK/dV launch that follows (in place of the pre-pass)
template <bool BF, int D, int W, bool BSM, bool DELTA = false>
__device__ __forceinline__ void dq16p_body(const BwdParams& p, lds_t* const lds, int bid) {
  constexpr int BM = 32 * W, BN = DqP<D, W>::BN, NT = 64 * W;
  constexpr int CPR = D / 8, TB = DqP<D, W>::TB, NDMA = BN * CPR / NT;
  constexpr int NC = D / 16, NDB = D / 32, NPC = BN / 16;
  constexpr int NSK = DqP<D, W>::NSK;  // K slots; the V slots follow them
  static_assert(NDMA >= 1 && NPC == 2, "tile split");

  const Shape& s = p.s;
  BwdPos w;
  if (!bwd_decode<(D >= 128)>(s, p.work_q, p.count_q, s.hq, s.sq, BM, true, w, bid)) return;
  const Seq g = seq_of(s, w.b);
  const int q0 = w.tile * BM;
  if (q0 >= g.sq) return;
  const int qend = min(q0 + BM, g.sq);
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hk = w.h / s.group;
  const uint16_t* qb = static_cast<const uint16_t*>(p.q.ptr) + w.b * p.q.sb + w.h * p.q.sh + g.qrow0 * p.q.ss;
  const uint16_t* gb = static_cast<const uint16_t*>(p.dout.ptr) + w.b * p.dout.sb + w.h * p.dout.sh +
                       g.qrow0 * p.dout.ss;
  const uint16_t* kb = static_cast<const uint16_t*>(p.k.ptr) + w.b * p.k.sb + hk * p.k.sh + g.krow0 * p.k.ss;
  const uint16_t* vb = static_cast<const uint16_t*>(p.v.ptr) + w.b * p.v.sb + hk * p.v.sh + g.krow0 * p.v.ss;
  uint16_t* dqb = static_cast<uint16_t*>(p.dq.ptr) + w.b * p.dq.sb + w.h * p.dq.sh + g.qrow0 * p.dq.ss;

  int j0, j1;
  key_range(s, g, q0, qend, j0, j1);
  const int kt0 = j0 / BN, kt1 = j1 > j0 ? (j1 + BN - 1) / BN : kt0;
  const int qw0 = q0 + wave * 32, qw1 = min(qw0 + 32, g.sq);
  const int qi = qw0 + l32;
  int wf0 = 0, wf1 = 0;  // key tiles every row of this wave sees in full
  if (qw0 < qw1) {
    const int64_t lo_full = int64_t(qw1 - 1) + g.off + s.lo_rel;
    const int64_t hi_full = min(int64_t(qw0) + g.off + s.hi_rel, int64_t(g.sk) - 1);
    const int64_t a = lo_full <= 0 ? 0 : (lo_full + BN - 1) / BN;
    const int64_t b = hi_full < 0 ? 0 : (hi_full + 1) / BN;
    wf0 = int(clamp64(a, 0, int64_t(1) << 30));
    wf1 = int(clamp64(b, wf0, int64_t(1) << 30));
  }

  // Block-sparse mask: the 128-key block list of this 128-row block row, staged in LDS,
  // replaces the tile range [kt0, kt1); past the last step a tile beyond every key.
  constexpr int TPB = kMaskBlock / BN;
  __shared__ int32_t bm_list[BSM ? kMaskMaxList : 1];
  // element bits of partial tiles, loaded with their K tile into the same ring slot: row
  // 32 w + l of the workgroup, dword t (the tile's 32 keys), one dword per lane of 32
  __shared__ __align__(16) uint32_t bm_bits[BSM ? 4 * BM : 1];
  int nbm = 0;
  int64_t plane = 0;
  if constexpr (BSM) {
    plane = bm_plane(s.bm, w.b, w.h);
    const int64_t row = plane * s.bm.nqb + q0 / kMaskBlock;
    nbm = min(max(s.bm.kv_count[row], 0), s.bm.nkb);
    for (int i = tid; i < nbm; i += NT) bm_list[i] = s.bm.kv_list[row * s.bm.nkb + i];
    __syncthreads();
  }
  auto tile_at = [&](int i) -> int {
    if constexpr (BSM) {
      if (i >= nbm * TPB) return s.bm.nkb * TPB;
      const int e = __builtin_amdgcn_readfirstlane(bm_list[i / TPB]);
      return min(max(e >> 1, 0), s.bm.nkb - 1) * TPB + i % TPB;
    } else {
      return kt0 + i;
    }
  };
  auto partial_at = [&](int i) -> bool {
    if constexpr (BSM) return (__builtin_amdgcn_readfirstlane(bm_list[i / TPB]) & 1) != 0;
    return false;
  };

  // Scores enter exp2 as fma(s, c, -LSE log2e) with c = |scale| log2e; a negative scale
  // is applied by negating q (exact).  dQ takes the signed scale at the end.
  const float c = fmaxf(fabsf(s.scale_log2), 1e-30f);
  const uint32_t qsign = s.scale_log2 < 0.f ? 0x80008000u : 0u;
  uint4 qf[NC], gf[NC];
  float lse2 = __builtin_inff(), dl = 0.f;
  {
    const int qr = min(qi, g.sq - 1);
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      const uint4 t = *reinterpret_cast<const uint4*>(qb + qr * p.q.ss + 16 * cc + 8 * hf);
      qf[cc] = make_uint4(t.x ^ qsign, t.y ^ qsign, t.z ^ qsign, t.w ^ qsign);
      gf[cc] = *reinterpret_cast<const uint4*>(gb + qr * p.dout.ss + 16 * cc + 8 * hf);
    }
    if constexpr (DELTA) {
      // The same value as the pre-pass, bit for bit: one fma chain per 8-element chunk, then
      // its butterfly over the row's 16 chunks.  This lane holds chunks c = 2 cc + hf, so the
      // partners c^8, c^4, c^2 are chunks cc^4, cc^2, cc^1 of this lane and c^1 is the same
      // chunk of lane l^32.
      static_assert(NC == 8 || NC == 4, "the butterfly below is the pre-pass's at head_dim 128 and 64");
      const uint16_t* ob = static_cast<const uint16_t*>(p.o.ptr) + w.b * p.o.sb + w.h * p.o.sh + g.qrow0 * p.o.ss;
      float pc[NC];
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const uint4 ov = *reinterpret_cast<const uint4*>(ob + qr * p.o.ss + 16 * cc + 8 * hf);
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          d = __builtin_fmaf(to_f32<BF>(uint16_t(elem16(ov, e))), to_f32<BF>(uint16_t(elem16(gf[cc], e))), d);
        pc[cc] = d;
      }
      float dot;
      if constexpr (NC == 8)
        dot = ((pc[0] + pc[4]) + (pc[2] + pc[6])) + ((pc[1] + pc[5]) + (pc[3] + pc[7]));
      else  // head_dim 64: 8 chunks a row, partners c^4, c^2 in this lane (cc^2, cc^1)
        dot = (pc[0] + pc[2]) + (pc[1] + pc[3]);
      dot += __shfl_xor(dot, 32);
      if (qi < g.sq) {
        const float l = p.lse.ptr[w.b * p.lse.sb + w.h * p.lse.sh + (g.qrow0 + qi) * p.lse.ss];
        lse2 = l == kNegInf ? __builtin_inff() : l * kLog2e;
        const float dlse = p.dlse.ptr ? p.dlse.ptr[w.b * p.dlse.sb + w.h * p.dlse.sh + (g.qrow0 + qi) * p.dlse.ss] : 0.f;
        dl = dot - dlse;
        if (hf == 0) {
          const int64_t r = delta_index(s, w.b, w.h, g, qi);
          p.delta[r] = dl;
          p.lse2[r] = lse2;
        }
      }
    } else if (qi < g.sq) {
      const float l = p.lse.ptr[w.b * p.lse.sb + w.h * p.lse.sh + (g.qrow0 + qi) * p.lse.ss];
      lse2 = l == kNegInf ? __builtin_inff() : l * kLog2e;
      dl = p.delta[delta_index(s, w.b, w.h, g, qi)];
    }
  }

  // ---- HBM -> LDS: one resource per tensor, a tile is a 32-bit offset ----
  const int64_t kss = p.k.ss, vss = p.v.ss;
  const i32x4_t rk = make_rsrc(kb, (int64_t(g.sk) - 1) * kss * 2 + D * 2);
  const i32x4_t rv = make_rsrc(vb, (int64_t(g.sk) - 1) * vss * 2 + D * 2);
  const uint32_t kstep = uint32_t(BN * kss * 2), vstep = uint32_t(BN * vss * 2);
  uint32_t koff_g[NDMA], voff_g[NDMA];
#pragma unroll
  for (int u = 0; u < NDMA; ++u) {
    const int P = (u * W + wave) * 64 + lane;
    const int row = P / CPR, pos = P % CPR;
    koff_g[u] = uint32_t(row * kss * 2 + ((pos ^ swb<CPR>(row)) * 16));
    voff_g[u] = uint32_t(row * vss * 2 + ((pos ^ swb<CPR>(row)) * 16));
  }
  constexpr int NB = BSM ? 1 : 0;  // extra loads per K tile
  i32x4_t rbits = {0, 0, 0, 0};
  uint32_t boff = 0;
  if constexpr (BSM) {
    rbits = make_rsrc(s.bm.bits + (plane * s.sq + q0) * int64_t(s.bm.words),
                      int64_t(s.sq - q0) * s.bm.words * 8);
    boff = uint32_t((wave * 32 + l32) * s.bm.words * 8);
  }
  auto issue_k = [&](int t, int slot, bool part) {
    const uint32_t o = uint32_t(t) * kstep;
#pragma unroll
    for (int u = 0; u < NDMA; ++u) dma16(rk, lds + slot * TB + (u * W + wave) * 1024, koff_g[u] + o);
    if constexpr (BSM) {
      // not partial: a load from past the buffer end (fills zeros, reads nothing)
      if (lane < 32)
        dma4(rbits, (lds_t*)(bm_bits + slot * BM + wave * 32), part ? boff + uint32_t(t) * 4u : 0x80000000u);
    }
  };
  auto issue_v = [&](int t, int slot) {
    const uint32_t o = uint32_t(t) * vstep;
#pragma unroll
    for (int u = 0; u < NDMA; ++u) dma16(rv, lds + (NSK + slot) * TB + (u * W + wave) * 1024, voff_g[u] + o);
  };

  // LDS operand offsets (lane part)
  int ra[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) ra[cc] = (l32 * CPR + ((2 * cc + hf) ^ swb<CPR>(l32))) * 16;
  int ta[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    ta[db][0] = tr_offset<CPR>(lane, db, 0);
    ta[db][1] = tr_offset<CPR>(lane, db, 1);
  }

  f32x16_t acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = zero16();

  // S^T and dP^T of one tile: independent chains, interleaved
  // At head_dim 128 with two waves (one wave per SIMD, registers to spare) every A operand
  // of the tile is read before the first product, so the LDS latency is paid once per tile
  // rather than before every pair of products; with four waves the other wave of the SIMD
  // hides it.
  constexpr bool kPrefetch = D >= 128 && W == 2;
  auto products = [&](int ks, int vs, f32x16_t& st, f32x16_t& dp) {
    st = zero16();
    dp = zero16();
    if constexpr (kPrefetch) {
      uint4 a[NC], b2[NC];
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        a[cc] = lds_read16(lds + ks * TB + ra[cc]);
        b2[cc] = lds_read16(lds + (NSK + vs) * TB + ra[cc]);
      }
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        st = mfma16<BF>(a[cc], qf[cc], st);
        dp = mfma16<BF>(b2[cc], gf[cc], dp);
      }
    } else {
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const uint4 a = lds_read16(lds + ks * TB + ra[cc]);
        const uint4 b2 = lds_read16(lds + (NSK + vs) * TB + ra[cc]);
        st = mfma16<BF>(a, qf[cc], st);
        dp = mfma16<BF>(b2, gf[cc], dp);
      }
    }
  };
  // key j visible to query i iff lo_rel <= j - i - off <= min(hi_rel, sk - 1 - i - off)
  // x = s c - LSE log2e and y = dP - Delta of the current tile: the first uses of its S and
  // dP, taken before the next tile's products overwrite those registers
  auto consume = [&](const f32x16_t& st, const f32x16_t& dp, float(&x)[16], float(&y)[16]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      x[r] = __builtin_fmaf(st[r], c, -lse2);
      y[r] = dp[r] - dl;
    }
  };
  auto grad = [&](int t, bool part, int slot, const float(&x)[16], const float(&y)[16], uint4(&dsf)[NPC]) {
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) ds[r] = fast_exp2(x[r]) * y[r];
    if (part || t < wf0 || t >= wf1) {
      asm volatile("" ::: "memory");
      const int base_rel = t * BN - qi - g.off + 4 * hf;
      const int hi_eff = qi < g.sq ? min(s.hi_rel, g.sk - 1 - qi - g.off) : s.lo_rel - 1;
      // element bits of this row's 32 keys (a 32-key tile is dword t of the row)
      uint32_t mb = ~0u;
      if constexpr (BSM) {
        if (part) mb = bm_bits[slot * BM + wave * 32 + l32];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rel = base_rel + 8 * (r >> 2) + (r & 3);
        const bool bit = (mb >> (8 * (r >> 2) + 4 * hf + (r & 3))) & 1u;
        ds[r] = (rel >= s.lo_rel && rel <= hi_eff && bit) ? ds[r] : 0.f;
      }
    }
#pragma unroll
    for (int h2 = 0; h2 < NPC; ++h2)
      dsf[h2] = make_uint4(pack2<BF>(ds[8 * h2], ds[8 * h2 + 1]), pack2<BF>(ds[8 * h2 + 2], ds[8 * h2 + 3]),
                           pack2<BF>(ds[8 * h2 + 4], ds[8 * h2 + 5]), pack2<BF>(ds[8 * h2 + 6], ds[8 * h2 + 7]));
  };
  auto dq_update = [&](int ks, const uint4(&dsf)[NPC]) {
    if constexpr (kPrefetch) {
      uint2 lo[NPC][NDB], hi[NPC][NDB];
#pragma unroll
      for (int cc = 0; cc < NPC; ++cc)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const lds_t* base = lds + ks * TB + 16 * cc * CPR * 16;
          lo[cc][db] = read_tr16(base + ta[db][0]);
          hi[cc][db] = read_tr16(base + ta[db][1]);
        }
#pragma unroll
      for (int cc = 0; cc < NPC; ++cc)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          acc[db] = mfma16<BF>(make_uint4(lo[cc][db].x, lo[cc][db].y, hi[cc][db].x, hi[cc][db].y), dsf[cc], acc[db]);
    } else {
#pragma unroll
      for (int cc = 0; cc < NPC; ++cc)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const lds_t* base = lds + ks * TB + 16 * cc * CPR * 16;
          const uint2 lo = read_tr16(base + ta[db][0]), hi = read_tr16(base + ta[db][1]);
          acc[db] = mfma16<BF>(make_uint4(lo.x, lo.y, hi.x, hi.y), dsf[cc], acc[db]);
        }
    }
  };

  const int n = BSM ? nbm * TPB : kt1 - kt0;
  if (n > 0) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      issue_k(tile_at(j), j, j < n && partial_at(j));
      issue_v(tile_at(j), j);
    }
    vm_wait<2 * NDMA + NB>();
    lds_barrier();
  }
  // Step i: tile t = kt0 + i in K and V slot t % 4.  The products of tile t+1 are issued
  // before tile t's dS, so the matrix cores run while the VALU works; before its barrier a
  // step waits for every load but its own, so tile t+2 has landed.
  // head_dim <= 64 (two waves per SIMD): one pair of score registers; each step first takes
  // the current tile's S and dP into their first uses, then issues the next tile's
  // products into the same registers (their MFMAs run while the VALU exponentiates), so no
  // register copies carry them over.  head_dim 128 (one wave per SIMD) gains more from the
  // compiler interleaving the next products with the whole softmax, at the price of the
  // copies (measured: D64 B8 S4096 backward 568 -> 548 us, D128 B4 S4096 1180 -> 1273 us).
  // This wave's own tiles [ia, ib): those with a key visible to one of its rows.  The block
  // walks the keys of all its rows, so below the causal diagonal a wave's last tiles, and
  // past the sequence end all of a wave's tiles, are masked for it; it skips their products,
  // exponentials and dQ update and only issues loads and meets the barriers.
  int ia = 0, ib = n;
  if constexpr (!BSM) {
    int wj0 = 0, wj1 = 0;
    if (qw0 < qw1) key_range(s, g, qw0, qw1, wj0, wj1);
    if (wj1 > wj0) {
      ia = min(max(wj0 / BN - kt0, 0), n);
      ib = min(max((wj1 + BN - 1) / BN - kt0, ia), n);
    } else {
      ia = ib = 0;
    }
    ia = __builtin_amdgcn_readfirstlane(ia);
    ib = __builtin_amdgcn_readfirstlane(ib);
  }
  auto skip = [&](int i) {
    const int ph = i & 3;
    issue_k(tile_at(i + 3), (ph + 3) & 3, i + 3 < n && partial_at(i + 3));
    issue_v(tile_at(i + 3), (ph + 3) & 3);
    vm_wait<2 * NDMA + NB>();
    lds_barrier();
  };
  f32x16_t sa, da, sb, db_;
  for (int i = 0; i < ia; ++i) skip(i);
  if (ia < ib) products(ia & 3, ia & 3, sa, da);
  // one step: tile i's S and dP are in (cs, cd); the next tile's products go to (ns, nd)
  auto step = [&](int i, f32x16_t& cs, f32x16_t& cd, f32x16_t& ns, f32x16_t& nd) {
    const int ph = i & 3;
    issue_k(tile_at(i + 3), (ph + 3) & 3, i + 3 < n && partial_at(i + 3));
    issue_v(tile_at(i + 3), (ph + 3) & 3);
    float x[16], y[16];
    if constexpr (D <= 64) {
      consume(cs, cd, x, y);
      __builtin_amdgcn_sched_barrier(0);
      products((ph + 1) & 3, (ph + 1) & 3, ns, nd);  // past the last tile: unused
    } else {
      products((ph + 1) & 3, (ph + 1) & 3, ns, nd);
      consume(cs, cd, x, y);
    }
    uint4 dsf[NPC];
    grad(tile_at(i), partial_at(i), ph, x, y, dsf);
    dq_update(ph, dsf);
    vm_wait<2 * NDMA + NB>();
    lds_barrier();
  };
  for (int i = ia; i < ib; ++i) {
    if constexpr (D <= 64) {
      step(i, sa, da, sa, da);
    } else {
      step(i, sa, da, sb, db_);
      sa = sb;
      da = db_;
    }
  }
  for (int i = ib; i < n; ++i) skip(i);
  vm_wait<0>();  // no load may land in LDS after the workgroup ends

  if (qi < g.sq) {
    uint16_t* row = dqb + qi * p.dq.ss;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float v[4] = {acc[db][4 * gq], acc[db][4 * gq + 1], acc[db][4 * gq + 2], acc[db][4 * gq + 3]};
        out4_16<BF>(row + db * 32 + 8 * gq + 4 * hf, v, s.scale, true, p.accumulate);
      }
  }
}

// dK, dV.  A workgroup of W waves (2, or 4 in the separate head_dim-128 launch) owns 32 W
// keys of one kv head, 32 per wave (lane = key), and streams
// 32-row query tiles of every q head of its group:
//   S  = Q K^T   (A: Q rows from LDS, B: K^T in registers)
//   dP = dO V^T  (A: dO rows from LDS, B: V^T in registers)
//   P = exp2(S scale log2e - LSE log2e),  dS = P (dP - Delta)
//   dV^T += dO^T P   (A: dO^T by transposed reads, B: P straight from registers)
//   dK^T += Q^T dS   (A: Q^T by transposed reads, B: dS from registers)
// Query tiles, with their rows' LSE log2e and Delta from the pre-pass, go to a ring of 4
// LDS slots, loaded 3 tiles ahead.
template <int D, int W>
struct DkdvP {
  static constexpr int BQ = 32, TB = BQ * D * 2, NS = 4;
  static constexpr int SB = 2 * TB + 256;  // slot: Q tile, dO tile, 32 LSE log2e, 32 Delta
  static constexpr int LDS = NS * SB;
};

// HALVES (separate THD launch): split items of the list come as two half blocks (see below)
template <bool BF, int D, int W, bool BSM, bool SPLIT = false, bool HALVES = false>
__device__ __forceinline__ void dkdv16p_body(const BwdParams& p, lds_t* const lds, int bid, int split = 0) {
  constexpr int BK = 32 * W, BQ = DkdvP<D, W>::BQ, NT = 64 * W;
  constexpr int CPR = D / 8, TB = DkdvP<D, W>::TB, NDMA = BQ * CPR / NT;
  constexpr int NC = D / 16, NDB = D / 32, NPC = BQ / 16;
  constexpr int NS = DkdvP<D, W>::NS, SB = DkdvP<D, W>::SB;
  constexpr int NL = 2 * NDMA + 1 + (BSM ? 1 : 0);  // loads per wave per tile
  static_assert((W == 2 || (W == 4 && !BSM && !SPLIT)) && NDMA >= 1 && NPC == 2, "tile split");

  const Shape& s = p.s;
  BwdPos w;
  static_assert(!HALVES || (W == 4 && !BSM && !SPLIT), "halves: the separate launch only");
  if (!bwd_decode<(D >= 128)>(s, p.work_k, p.count_k, s.hk, s.sk, BK, false, w, bid)) return;
  // a split THD item comes twice in the list, with (half + 1) << 24 in its tile field; its
  // halves' partial-sum slot is the pair's index
  int half = -1, slot = 0;
  if constexpr (HALVES) {
    half = (w.tile >> 24) - 1;
    w.tile &= 0xffffff;
    slot = w.item >> 1;
  }
  const Seq g = seq_of(s, w.b);
  const int k0 = w.tile * BK;
  if (k0 >= g.sk) return;
  const int kend = min(k0 + BK, g.sk);
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hk = w.h;
  const uint16_t* kb = static_cast<const uint16_t*>(p.k.ptr) + w.b * p.k.sb + hk * p.k.sh + g.krow0 * p.k.ss;
  const uint16_t* vb = static_cast<const uint16_t*>(p.v.ptr) + w.b * p.v.sb + hk * p.v.sh + g.krow0 * p.v.ss;
  uint16_t* dkb = static_cast<uint16_t*>(p.dk.ptr) + w.b * p.dk.sb + hk * p.dk.sh + g.krow0 * p.dk.ss;
  uint16_t* dvb = static_cast<uint16_t*>(p.dv.ptr) + w.b * p.dv.sb + hk * p.dv.sh + g.krow0 * p.dv.ss;

  int i0, i1;
  query_range(s, g, k0, kend, i0, i1);
  const int qt0 = i0 / BQ, qt1 = i1 > i0 ? (i1 + BQ - 1) / BQ : qt0;
  const int nq = qt1 - qt0;
  // Block-sparse mask: this key block's column lists of 128-row blocks, staged in LDS.  A
  // mask shared by all q heads has one list (item it: head it / nper, list position
  // (it % nper) / TPQ); per-head masks are staged head after head with the head's index in
  // bits 16.. of each entry (entries are below 2 * nqb <= 1024, and the host bounds
  // group * nqb by the LDS list length).
  constexpr int TPQ = kMaskBlock / BQ;
  __shared__ int32_t bm_list[BSM ? kMaskMaxList : 1];
  // element bits of partial items, loaded with the item into the same ring slot: rows
  // qbase .. qbase + 31, dword kw0 / 32 (the wave's 32 keys), one dword per lane of 32
  __shared__ __align__(16) uint32_t bm_bits[BSM ? NS * 64 : 1];
  int n = s.group * nq, nper = 0;
  if constexpr (BSM) {
    const int kblk = k0 / kMaskBlock;
    if (s.bm.nh == 1) {
      const int64_t col = bm_plane(s.bm, w.b, 0) * s.bm.nkb + kblk;
      const int cnt = min(min(max(s.bm.q_count[col], 0), s.bm.nqb), kMaskMaxList);
      for (int i = tid; i < cnt; i += NT) bm_list[i] = s.bm.q_list[col * s.bm.nqb + i];
      nper = cnt * TPQ;
      n = s.group * nper;
    } else {
      int tot = 0;
      for (int gi = 0; gi < s.group; ++gi) {
        const int64_t col = bm_plane(s.bm, w.b, hk * s.group + gi) * s.bm.nkb + kblk;
        const int cnt = min(min(max(s.bm.q_count[col], 0), s.bm.nqb), kMaskMaxList - tot);
        for (int i = tid; i < cnt; i += NT) bm_list[tot + i] = (gi << 16) | (s.bm.q_list[col * s.bm.nqb + i] & 0xffff);
        tot += cnt;
      }
      n = tot * TPQ;
    }
    __syncthreads();
  }
  const int n_all = n;  // items of the whole block (before a split)
  // a split block (or half of a split THD item) takes the first or the second half of the
  // items
  int ib = 0;
  if constexpr (SPLIT) half = split;
  if (SPLIT || (HALVES && half >= 0)) {
    const int n1 = (n + 1) / 2;
    if (half == 0) {
      n = n1;
    } else {
      ib = n1;
      n -= n1;
    }
  }
  // item it -> q head (within the group), q tile, and whether its block needs the bits
  auto item = [&](int it, int& gi, int& qt, bool& part) {
    if constexpr (SPLIT || HALVES) it += ib;
    if constexpr (BSM) {
      // the same order as without a mask: last listed tile first; one shared list: every q
      // head at one tile before the next, per-head lists: head after head (last head first)
      int e, r;
      if (s.bm.nh == 1) {
        gi = it % s.group;
        r = nper - 1 - it / s.group;
        e = __builtin_amdgcn_readfirstlane(bm_list[r / TPQ]);
      } else {
        r = n_all - 1 - it;
        const int v = __builtin_amdgcn_readfirstlane(bm_list[r / TPQ]);
        gi = v >> 16;
        e = v & 0xffff;
      }
      qt = min(max(e >> 1, 0), s.bm.nqb - 1) * TPQ + r % TPQ;
      part = (e & 1) != 0;
    } else {
      // last query tile first, every q head of the group at one tile before the next: the
      // dK/dV blocks of a (sequence, kv head) that run at one time read the same Q and dO
      // rows at about the same time, so the repeats hit in L2 (C4's backward: 2.77 -> 1.76
      // GB read from beyond L2 per launch; ascending tiles head after head let the blocks
      // drift apart by one tile per block)
      gi = it % s.group;
      qt = qt1 - 1 - it / s.group;
      part = false;
    }
  };
  const int kw0 = k0 + wave * 32, kw1 = min(kw0 + 32, g.sk);
  const int kj = kw0 + l32;
  // query tiles [wq0, wq1) in which every (query, key) pair of this wave is visible and
  // every query row exists
  int wq0 = 0, wq1 = 0;
  if (kw0 < kw1) {
    const int64_t lo = int64_t(kw1 - 1) - g.off - s.hi_rel;                      // qbase >= lo
    const int64_t hi = min(int64_t(kw0) - g.off - s.lo_rel - (BQ - 1), int64_t(g.sq) - BQ);  // qbase <= hi
    const int64_t a = lo <= 0 ? 0 : (lo + BQ - 1) / BQ;
    const int64_t b = hi < 0 ? 0 : hi / BQ + 1;
    wq0 = int(clamp64(a, 0, int64_t(1) << 30));
    wq1 = int(clamp64(b, wq0, int64_t(1) << 30));
  }

  // K^T and V^T operands in registers; a negative scale is applied by negating k (exact)
  const float c = fmaxf(fabsf(s.scale_log2), 1e-30f);
  const uint32_t ksign = s.scale_log2 < 0.f ? 0x80008000u : 0u;
  uint4 kf[NC], vf[NC];
  {
    const int kr = min(kj, g.sk - 1);
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      const uint4 t = *reinterpret_cast<const uint4*>(kb + kr * p.k.ss + 16 * cc + 8 * hf);
      kf[cc] = make_uint4(t.x ^ ksign, t.y ^ ksign, t.z ^ ksign, t.w ^ ksign);
      vf[cc] = *reinterpret_cast<const uint4*>(vb + kr * p.v.ss + 16 * cc + 8 * hf);
    }
  }

  // ---- HBM -> LDS ----
  const int64_t qss = p.q.ss, gss = p.dout.ss;
  uint32_t qoff[NDMA], goff[NDMA];
#pragma unroll
  for (int u = 0; u < NDMA; ++u) {
    const int P = (u * W + wave) * 64 + lane;
    const int row = P / CPR, pos = P % CPR;
    qoff[u] = uint32_t(row * qss * 2 + ((pos ^ swb<CPR>(row)) * 16));
    goff[u] = uint32_t(row * gss * 2 + ((pos ^ swb<CPR>(row)) * 16));
  }
  // wave 0 loads the tile rows' LSE log2e, wave 1 their Delta (lanes 0..31); the host keeps
  // the whole array below 2^31 bytes for this kernel
  const i32x4_t rstat = make_rsrc(wave == 0 ? p.lse2 : p.delta, p.ws_rows * 4);
  auto issue_at = [&](int gi, int qt, bool part, int slot) {
    const int h = hk * s.group + gi, qbase = qt * BQ;
    const uint16_t* qh = static_cast<const uint16_t*>(p.q.ptr) + w.b * p.q.sb + h * p.q.sh + g.qrow0 * qss;
    const uint16_t* gh = static_cast<const uint16_t*>(p.dout.ptr) + w.b * p.dout.sb + h * p.dout.sh +
                         g.qrow0 * gss;
    const i32x4_t rq = make_rsrc(qh, (int64_t(g.sq) - 1) * qss * 2 + D * 2);
    const i32x4_t rg = make_rsrc(gh, (int64_t(g.sq) - 1) * gss * 2 + D * 2);
    const uint32_t oq = uint32_t(qbase) * uint32_t(qss * 2), og = uint32_t(qbase) * uint32_t(gss * 2);
    lds_t* dst = lds + slot * SB;
#pragma unroll
    for (int u = 0; u < NDMA; ++u) dma16(rq, dst + (u * W + wave) * 1024, qoff[u] + oq);
#pragma unroll
    for (int u = 0; u < NDMA; ++u) dma16(rg, dst + TB + (u * W + wave) * 1024, goff[u] + og);
    if (wave < 2 && lane < 32)
      dma4(rstat, dst + 2 * TB + wave * 128, uint32_t(delta_index(s, w.b, h, g, qbase + lane)) * 4u);
    if constexpr (BSM) {
      // not partial: a load from past the buffer end (fills zeros, reads nothing)
      const i32x4_t rb = make_rsrc(s.bm.bits + bm_plane(s.bm, w.b, h) * s.sq * int64_t(s.bm.words),
                                   int64_t(s.sq) * s.bm.words * 8);
      const uint32_t o = part ? uint32_t((qbase + l32) * s.bm.words * 8 + (kw0 / 32) * 4) : 0x80000000u;
      if (lane < 32) dma4(rb, (lds_t*)(bm_bits + slot * 64 + wave * 32), o);
    }
  };
  auto issue = [&](int it, int slot) {
    it = min(it, n - 1);  // past the last item: reload it (never read), keeps wait counts fixed
    int gi, qt;
    bool part;
    item(it, gi, qt, part);
    issue_at(gi, qt, part, slot);
  };

  int ra[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) ra[cc] = (l32 * CPR + ((2 * cc + hf) ^ swb<CPR>(l32))) * 16;
  int ta[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    ta[db][0] = tr_offset<CPR>(lane, db, 0);
    ta[db][1] = tr_offset<CPR>(lane, db, 1);
  }

  f32x16_t adk[NDB], adv[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    adk[i] = zero16();
    adv[i] = zero16();
  }

  // S and dP of the tile in slot sl
  // (head_dim 128: every A operand read before the first product, as in dQ)
  auto products = [&](int sl, f32x16_t& st, f32x16_t& dp) {
    const lds_t* base = lds + sl * SB;
    st = zero16();
    dp = zero16();
    if constexpr (D >= 128) {
      uint4 a[NC], b2[NC];
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        a[cc] = lds_read16(base + ra[cc]);
        b2[cc] = lds_read16(base + TB + ra[cc]);
      }
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        st = mfma16<BF>(a[cc], kf[cc], st);
        dp = mfma16<BF>(b2[cc], vf[cc], dp);
      }
    } else {
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const uint4 a = lds_read16(base + ra[cc]);
        const uint4 b2 = lds_read16(base + TB + ra[cc]);
        st = mfma16<BF>(a, kf[cc], st);
        dp = mfma16<BF>(b2, vf[cc], dp);
      }
    }
  };
  // x = s c - LSE log2e and y = dP - Delta of item in slot sl: the first uses of its S and
  // dP, taken before the next item's products overwrite those registers.
  // lane = key; register r holds query 8(r/4) + 4hf + r%4 of the tile
  auto consume = [&](int sl, const f32x16_t& st, const f32x16_t& dp, float(&x)[16], float(&y)[16]) {
    const lds_t* base = lds + sl * SB;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 l4 = lds_read16(base + 2 * TB + (8 * j + 4 * hf) * 4);
      const uint4 d4 = lds_read16(base + 2 * TB + 128 + (8 * j + 4 * hf) * 4);
      const float la[4] = {__uint_as_float(l4.x), __uint_as_float(l4.y), __uint_as_float(l4.z), __uint_as_float(l4.w)};
      const float da[4] = {__uint_as_float(d4.x), __uint_as_float(d4.y), __uint_as_float(d4.z), __uint_as_float(d4.w)};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[4 * j + e] = __builtin_fmaf(st[4 * j + e], c, -la[e]);
        y[4 * j + e] = dp[4 * j + e] - da[e];
      }
    }
  };
  // P, dS and the dV, dK updates of the item of tile qt (slot sl), given consume's x and y
  auto update_at = [&](int sl, int qt, bool part, const float(&x)[16], const float(&y)[16]) {
    const lds_t* base = lds + sl * SB;
    const int qbase = qt * BQ;
    float pr[16], ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pr[r] = fast_exp2(x[r]);
      ds[r] = pr[r] * y[r];
    }
    if (part || qt < wq0 || qt >= wq1) {
      asm volatile("" ::: "memory");
      const int rel0 = kj - qbase - g.off - 4 * hf;
      // element bits of (query row, this lane's key): bit l32 of row 8 j + 4 hf + e's dword
      uint32_t rb[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) rb[r] = ~0u;
      if constexpr (BSM) {
        if (part) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint4 b4 = *reinterpret_cast<const uint4*>(bm_bits + sl * 64 + wave * 32 + 8 * j + 4 * hf);
            rb[4 * j] = b4.x;
            rb[4 * j + 1] = b4.y;
            rb[4 * j + 2] = b4.z;
            rb[4 * j + 3] = b4.w;
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qrow = 8 * (r >> 2) + (r & 3);
        const bool bit = (rb[r] >> l32) & 1u;
        const bool vis = rel0 - qrow >= s.lo_rel && rel0 - qrow <= s.hi_rel && qbase + 4 * hf + qrow < g.sq && bit;
        pr[r] = vis ? pr[r] : 0.f;
        ds[r] = vis ? ds[r] : 0.f;
      }
    }
    uint4 pf[NPC], dsf[NPC];
#pragma unroll
    for (int h2 = 0; h2 < NPC; ++h2) {
      pf[h2] = make_uint4(pack2<BF>(pr[8 * h2], pr[8 * h2 + 1]), pack2<BF>(pr[8 * h2 + 2], pr[8 * h2 + 3]),
                          pack2<BF>(pr[8 * h2 + 4], pr[8 * h2 + 5]), pack2<BF>(pr[8 * h2 + 6], pr[8 * h2 + 7]));
      dsf[h2] = make_uint4(pack2<BF>(ds[8 * h2], ds[8 * h2 + 1]), pack2<BF>(ds[8 * h2 + 2], ds[8 * h2 + 3]),
                           pack2<BF>(ds[8 * h2 + 4], ds[8 * h2 + 5]), pack2<BF>(ds[8 * h2 + 6], ds[8 * h2 + 7]));
    }
    if constexpr (D >= 128) {
      uint2 g2[NPC][NDB][2], q2[NPC][NDB][2];
#pragma unroll
      for (int cc = 0; cc < NPC; ++cc)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const lds_t* rb = base + 16 * cc * CPR * 16;
          g2[cc][db][0] = read_tr16(rb + TB + ta[db][0]);
          g2[cc][db][1] = read_tr16(rb + TB + ta[db][1]);
          q2[cc][db][0] = read_tr16(rb + ta[db][0]);
          q2[cc][db][1] = read_tr16(rb + ta[db][1]);
        }
#pragma unroll
      for (int cc = 0; cc < NPC; ++cc)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          adv[db] = mfma16<BF>(make_uint4(g2[cc][db][0].x, g2[cc][db][0].y, g2[cc][db][1].x, g2[cc][db][1].y),
                               pf[cc], adv[db]);
          adk[db] = mfma16<BF>(make_uint4(q2[cc][db][0].x, q2[cc][db][0].y, q2[cc][db][1].x, q2[cc][db][1].y),
                               dsf[cc], adk[db]);
        }
    } else {
#pragma unroll
      for (int cc = 0; cc < NPC; ++cc)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const lds_t* rb = base + 16 * cc * CPR * 16;
          const uint2 glo = read_tr16(rb + TB + ta[db][0]), ghi = read_tr16(rb + TB + ta[db][1]);
          adv[db] = mfma16<BF>(make_uint4(glo.x, glo.y, ghi.x, ghi.y), pf[cc], adv[db]);
          const uint2 qlo = read_tr16(rb + ta[db][0]), qhi = read_tr16(rb + ta[db][1]);
          adk[db] = mfma16<BF>(make_uint4(qlo.x, qlo.y, qhi.x, qhi.y), dsf[cc], adk[db]);
        }
    }
  };

  auto update = [&](int sl, int it, const float(&x)[16], const float(&y)[16]) {
    int gi, qt;
    bool part;
    item(it, gi, qt, part);
    update_at(sl, qt, part, x, y);
  };
  // Without a block mask a cursor (q head gi, q tile qt) steps to the next item with an
  // increment, not a division by the group size
  auto advance = [&](int& gi, int& qt) {
    if (++gi == s.group) {
      gi = 0;
      --qt;
    }
  };

  // Step it reads item it (slot it % 4) and item it+1 (the next S and dP, issued before
  // this item's softmax so the matrix cores run while the VALU works), loads item it+3 and
  // before its barrier waits for every load but its own, so item it+2 has landed.  At
  // head_dim <= 64 one pair of score registers: the current item's S and dP are taken into
  // their first uses before the next item's products are issued into the same registers
  // (no copies); head_dim 128 keeps two pairs and lets the compiler interleave (as in dQ).
  // every load of this wave but the last tile's (waves 2 and 3 of a four-wave block load no
  // LSE log2e or Delta)
  auto wait_tiles = [&]() {
    if constexpr (W == 2) {
      vm_wait<NL>();
    } else {
      if (wave < 2)
        vm_wait<NL>();
      else
        vm_wait<NL - 1>();
    }
  };
  f32x16_t sa, da, sb, db_;
  if (n > 0) {
    issue(0, 0);
    issue(1, 1);
    issue(2, 2);
    wait_tiles();
    lds_barrier();
    products(0, sa, da);
  }
  // cursors of item it and of item min(it + 3, n - 1), the one the step loads
  int gi_c = 0, qt_c = 0, gi_a = 0, qt_a = 0;
  bool pt_a = false;
  if (!BSM && n > 0) {
    item(0, gi_c, qt_c, pt_a);
    item(min(3, n - 1), gi_a, qt_a, pt_a);
  }
  // one step: item it's S and dP are in (cs, cd); the next item's products go to (ns, nd)
  auto step = [&](int it, f32x16_t& cs, f32x16_t& cd, f32x16_t& ns, f32x16_t& nd) {
    const int ph = it & (NS - 1);
    if constexpr (BSM) {
      issue(it + 3, (ph + 3) & (NS - 1));
    } else {
      issue_at(gi_a, qt_a, false, (ph + 3) & (NS - 1));
      if (it + 3 < n - 1) advance(gi_a, qt_a);
    }
    float x[16], y[16];
    if constexpr (D <= 64) {
      consume(ph, cs, cd, x, y);
      __builtin_amdgcn_sched_barrier(0);
      products((ph + 1) & (NS - 1), ns, nd);  // past the last item: a reloaded tile, unused
    } else {
      products((ph + 1) & (NS - 1), ns, nd);
      consume(ph, cs, cd, x, y);
    }
    if constexpr (BSM) {
      update(ph, it, x, y);
    } else {
      update_at(ph, qt_c, false, x, y);
      advance(gi_c, qt_c);
    }
    wait_tiles();
    lds_barrier();
  };
  for (int it = 0; it < n; ++it) {
    if constexpr (D <= 64) {
      step(it, sa, da, sa, da);
    } else {
      step(it, sa, da, sb, db_);
      sa = sb;
      da = db_;
    }
  }
  vm_wait<0>();  // no load may land in LDS after the workgroup ends

  if constexpr (SPLIT) {
    // Each half stores its fp32 sums (in register order, one 256-byte row per register),
    // makes them visible at device scope and counts itself in; the half that arrives second
    // adds the other half's sums (a + b: the same value whichever half it is) and writes.
    constexpr int PR = 2 * NDB * 16 * 64;  // floats per wave and half
    float* mine = p.split_part + (int64_t(bid) * 2 * W + split * W + wave) * PR;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        mine[(db * 16 + r) * 64 + lane] = adk[db][r];
        mine[((NDB + db) * 16 + r) * 64 + lane] = adv[db][r];
      }
    __threadfence();
    __shared__ int32_t arrived;
    __syncthreads();
    if (tid == 0) arrived = __hip_atomic_fetch_add(p.split_cnt + bid, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (arrived != 1) return;
    __threadfence();
    const float* other = p.split_part + (int64_t(bid) * 2 * W + (split ^ 1) * W + wave) * PR;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        adk[db][r] += other[(db * 16 + r) * 64 + lane];
        adv[db][r] += other[((NDB + db) * 16 + r) * 64 + lane];
      }
  }
  if (HALVES && half >= 0) {
    // half of a split THD item: fp32 partial sums in register order, one 256-byte row per
    // register, for the combine launch
    constexpr int PR = 2 * NDB * 16 * 64;  // floats per wave
    float* mine = p.ksplit_part + ((int64_t(slot) * s.hk + hk) * 2 + half) * (PR * W) + wave * PR;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        mine[(db * 16 + r) * 64 + lane] = adk[db][r];
        mine[((NDB + db) * 16 + r) * 64 + lane] = adv[db][r];
      }
    return;
  }
  if (kj < g.sk) {
    uint16_t* krow = dkb + kj * p.dk.ss;
    uint16_t* vrow = dvb + kj * p.dv.ss;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = db * 32 + 8 * gq + 4 * hf;
        const float a[4] = {adk[db][4 * gq], adk[db][4 * gq + 1], adk[db][4 * gq + 2], adk[db][4 * gq + 3]};
        const float b2[4] = {adv[db][4 * gq], adv[db][4 * gq + 1], adv[db][4 * gq + 2], adv[db][4 * gq + 3]};
        out4_16<BF>(krow + d, a, s.scale, true, p.accumulate);
        out4_16<BF>(vrow + d, b2, 1.f, true, p.accumulate);
      }
  }
}

// Second launch bound: waves per SIMD that registers and LDS allow.  D128 dQ with four waves
// (128 query rows sharing one K/V ring): 240 registers and two 64 KB workgroups per CU, so
// two waves per SIMD; with two waves (64 rows) the LDS allows one.
template <bool BF, int D, int W, bool DELTA = false>
__global__ __launch_bounds__(64 * W, (D == 128 && W == 2) ? 1 : 2) void bwd_dq16p_kernel(BwdParams p) {
  __shared__ __align__(16) char smem_[DqP<D, W>::LDS];
  dq16p_body<BF, D, W, false, DELTA>(p, (lds_t*)smem_, blockIdx.x);
}

template <bool BF, int D, int W, bool HALVES = false>
__global__ __launch_bounds__(64 * W, D == 128 ? 1 : 2) void bwd_dkdv16p_kernel(BwdParams p) {
  __shared__ __align__(16) char smem_[DkdvP<D, W>::LDS];
  dkdv16p_body<BF, D, W, false, false, HALVES>(p, (lds_t*)smem_, blockIdx.x);
}

// The split THD items of the separate dK/dV launch: block (slot, kv head) adds the two halves'
// partial sums in a fixed order (first + second) and writes dK (scaled) and dV as the dK/dV
// body's own epilogue does, the same lane for the same (key, d).
template <bool BF, int D>
__global__ __launch_bounds__(256) void bwd_dkdv_combine_kernel(BwdParams p) {
  constexpr int W = 4, NDB = D / 32, PR = 2 * NDB * 16 * 64;
  const Shape& s = p.s;
  const int slot = blockIdx.x / s.hk, hk = blockIdx.x % s.hk;
  if (slot >= *p.ksplit_count) return;
  const WorkItem it = p.work_k[2 * slot];  // half 0 of the pair (tile | 1 << 24)
  const Seq g = seq_of(s, it.seq);
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5, wave = tid >> 6;
  const int kj = (it.tile & 0xffffff) * (32 * W) + wave * 32 + l32;
  if (kj >= g.sk) return;
  const float* a = p.ksplit_part + (int64_t(slot) * s.hk + hk) * 2 * (PR * W) + wave * PR;
  const float* c = a + PR * W;
  uint16_t* krow = static_cast<uint16_t*>(p.dk.ptr) + it.seq * p.dk.sb + hk * p.dk.sh + (g.krow0 + kj) * p.dk.ss;
  uint16_t* vrow = static_cast<uint16_t*>(p.dv.ptr) + it.seq * p.dv.sb + hk * p.dv.sh + (g.krow0 + kj) * p.dv.ss;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d = db * 32 + 8 * gq + 4 * hf;
      float vk[4], vv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * gq + e;
        vk[e] = a[(db * 16 + r) * 64 + lane] + c[(db * 16 + r) * 64 + lane];
        vv[e] = a[((NDB + db) * 16 + r) * 64 + lane] + c[((NDB + db) * 16 + r) * 64 + lane];
      }
      out4_16<BF>(krow + d, vk, s.scale, true, p.accumulate);
      out4_16<BF>(vrow + d, vv, 1.f, true, p.accumulate);
    }
}

// dK/dV and dQ in one launch: blocks [0, nk) take key tiles, the rest query tiles.  The two
// halves are independent, so on small problems they fill the chip together instead of one
// after the other.
template <bool BF, int D, int W, bool BSM, bool SPLIT>
__global__ __launch_bounds__(64 * W, D == 128 ? 1 : 2) void bwd_fused16p_kernel(BwdParams p, int nk) {
  constexpr int L = DqP<D, W>::LDS > DkdvP<D, W>::LDS ? DqP<D, W>::LDS : DkdvP<D, W>::LDS;
  __shared__ __align__(16) char smem_[L];
  const int bid = blockIdx.x;
  if constexpr (SPLIT) {
    // GQA: block 2 i + h is half h of dK/dV block i
    static_assert(!BSM, "no split under a block mask");
    if (bid < 2 * nk)
      dkdv16p_body<BF, D, W, BSM, true>(p, (lds_t*)smem_, bid >> 1, bid & 1);
    else
      dq16p_body<BF, D, W, BSM>(p, (lds_t*)smem_, bid - 2 * nk);
    return;
  }
  if (bid < nk)
    dkdv16p_body<BF, D, W, BSM>(p, (lds_t*)smem_, bid);
  else
    dq16p_body<BF, D, W, BSM>(p, (lds_t*)smem_, bid - nk);
}

// ----------------------------------------------------------------------------------------
// Short sequences, 16-bit inputs, head_dim <= 64: at most 32 queries and 32 keys per
// sequence.  The tiled kernels then run on mostly empty 64-row tiles and the call is bound
// by HBM bytes in flight.  Here each wave is a work unit of its own: the keys of one
// (sequence, kv head), and in turn every q head of its group.  Delta_i = dO_i . O_i - dLSE_i
// is formed in the wave (no pre-pass).  Every global access is row-contiguous (lane chunk
// 64 u + lane of a 32-row tile is row (64 u + lane) / CPR, 16-byte column
// (64 u + lane) % CPR); rows pass through private LDS tiles into the MFMA layouts:
//   S = Q K^T and dP = dO V^T with the key as the MFMA column (lane = key, registers =
//     queries 8 (r / 4) + 4 half + r % 4);
//   dV^T += dO^T P and dK^T += Q^T dS, with dO^T and Q^T from transposed LDS reads whose
//     query order matches the registers of P and dS;
//   dQ^T = K^T dS^T, with dS staged in LDS as [key][query] and read back transposed.
// dK, dV accumulate in registers over the group; dQ leaves after each head.  LDS accesses of
// one wave take effect in issue order, so there is no barrier.
// ----------------------------------------------------------------------------------------
template <bool BF, int D>
__global__ __launch_bounds__(kThreads, 2) void bwd16w_kernel(BwdParams p) {
  constexpr int BN = 32;
  constexpr int CPR = D / 8;         // 16-byte chunks per row
  constexpr int NC = D / 16;         // contraction chunks over d
  constexpr int NDB = D / 32;        // 32-column blocks of d
  constexpr int NU = BN * CPR / 64;  // 16-byte chunks per lane per 32-row tile
  constexpr int TB = BN * D * 2;     // bytes of a 32-row tile
  constexpr int WB = 4 * TB + 2 * BN * 4;
  static_assert(NU >= 1 && D <= 64, "tile split");
  __shared__ __align__(16) char smem_[kWaves * WB];

  const Shape& s = p.s;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  lds_t* const tq = (lds_t*)smem_ + wave * WB;  // Q tile, then the dQ tile
  lds_t* const tk = tq + TB;                    // K tile, then the dK tile
  lds_t* const tdo = tk + TB;                   // dO tile, then the dV tile
  lds_t* const tvs = tdo + TB;                  // V tile, then dS [key][query]
  lds_t* const tst = tvs + TB;                  // LSE log2(e) [32], Delta [32]

  const int64_t item = int64_t(blockIdx.x) * kWaves + wave;
  if (item >= int64_t(s.batch) * s.hk) return;
  const int b = int(item / s.hk), hk = int(item % s.hk);
  const Seq g = seq_of(s, b);

  auto at_v = [](int r, int c) { return (r * CPR + (c ^ swv<CPR>(r))) * 16; };
  auto at_k = [](int r, int c) { return (r * CPR + (c ^ swk<CPR>(r))) * 16; };
  typedef __attribute__((address_space(3))) u32x4_t lds_u4;
  typedef __attribute__((address_space(3))) float lds_f;
  auto load_rows = [&](const uint16_t* base, int64_t ss, int nrows, uint4(&r)[NU]) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int P = 64 * u + lane, row = P / CPR;
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (row < nrows) x = *reinterpret_cast<const uint4*>(base + row * ss + (P % CPR) * 8);
      r[u] = x;
    }
  };
  auto put = [&](lds_t* dst, const uint4(&r)[NU]) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int P = 64 * u + lane;
      *(lds_u4*)(dst + at_v(P / CPR, P % CPR)) = __builtin_bit_cast(u32x4_t, r[u]);
    }
  };
  // transposed-read addresses: tiles [32 rows][D] (V layout) and dS [32 keys][32 queries]
  int va[NDB], vs;
  {
    const int gg = lane >> 4, cr = (lane >> 2) & 3, a = lane & 3;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      va[db] = ((4 * (gg >> 1) + cr) * CPR + ((4 * db + 2 * (gg & 1) + (a >> 1)) ^ swv<CPR>(cr))) * 16 +
               (a & 1) * 8;
    vs = ((4 * (gg >> 1) + cr) * 4 + 2 * (gg & 1) + (a >> 1)) * 16 + (a & 1) * 8;
  }
  auto tr = [&](const lds_t* base, int pitch_chunks, int cc) {
    const lds_t* q = base + 16 * cc * pitch_chunks * 16;
    const uint2 lo = read_tr16(q), hi = read_tr16(q + 8 * pitch_chunks * 16);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  };
  // a [32 rows][D] C-layout result (lane = row l32, d = 32 db + 8 gq + 4 hf + 0..3) to rows
  // of dst, through an LDS tile; scaled, and added to the old values if asked
  auto store_tile = [&](lds_t* stage, const f32x16_t(&acc)[NDB], float scale, uint16_t* dst, int64_t ss, int nrows) {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t v = {pack2<BF>(acc[db][4 * gq] * scale, acc[db][4 * gq + 1] * scale),
                           pack2<BF>(acc[db][4 * gq + 2] * scale, acc[db][4 * gq + 3] * scale)};
        *(__attribute__((address_space(3))) u32x2_t*)(stage + at_k(l32, 4 * db + gq) + 8 * hf) = v;
      }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int P = 64 * u + lane, row = P / CPR;
      uint4 x = lds_read16(stage + at_k(row, P % CPR));
      if (row < nrows) {
        uint4* o = reinterpret_cast<uint4*>(dst + row * ss + (P % CPR) * 8);
        if (p.accumulate) {
          const uint4 old = *o;
          float a[8], c[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            a[e] = to_f32<BF>(uint16_t(elem16(x, e)));
            c[e] = to_f32<BF>(uint16_t(elem16(old, e)));
          }
          x = make_uint4(pack2<BF>(a[0] + c[0], a[1] + c[1]), pack2<BF>(a[2] + c[2], a[3] + c[3]),
                         pack2<BF>(a[4] + c[4], a[5] + c[5]), pack2<BF>(a[6] + c[6], a[7] + c[7]));
        }
        *o = x;
      }
    }
  };

  const uint16_t* kb = static_cast<const uint16_t*>(p.k.ptr) + b * p.k.sb + hk * p.k.sh + g.krow0 * p.k.ss;
  const uint16_t* vb = static_cast<const uint16_t*>(p.v.ptr) + b * p.v.sb + hk * p.v.sh + g.krow0 * p.v.ss;
  uint4 ra[NU], rb[NU], rc[NU];
  load_rows(kb, p.k.ss, g.sk, ra);
  load_rows(vb, p.v.ss, g.sk, rb);
  put(tk, ra);
  put(tvs, rb);
  asm volatile("" ::: "memory");
  uint4 kf[NC], vf[NC];  // lane = key l32, d chunk 16 cc + 8 hf
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    kf[cc] = lds_read16(tk + at_v(l32, 2 * cc + hf));
    vf[cc] = lds_read16(tvs + at_v(l32, 2 * cc + hf));
  }
  f32x16_t dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dk[db] = dv[db] = zero16();
  const int j = l32;  // this lane's key

  for (int h = hk * s.group; h < (hk + 1) * s.group; ++h) {
    const uint16_t* qb = static_cast<const uint16_t*>(p.q.ptr) + b * p.q.sb + h * p.q.sh + g.qrow0 * p.q.ss;
    const uint16_t* gb = static_cast<const uint16_t*>(p.dout.ptr) + b * p.dout.sb + h * p.dout.sh + g.qrow0 * p.dout.ss;
    const uint16_t* ob = static_cast<const uint16_t*>(p.o.ptr) + b * p.o.sb + h * p.o.sh + g.qrow0 * p.o.ss;
    load_rows(qb, p.q.ss, g.sq, ra);
    load_rows(gb, p.dout.ss, g.sq, rb);
    load_rows(ob, p.o.ss, g.sq, rc);
    // Delta of each row: 8-element partial dots, summed over the CPR lanes of the row
    float dl = 0.f, l2 = __builtin_inff();
    if (hf == 0 && l32 < g.sq) {
      const int64_t so = b * p.lse.sb + h * p.lse.sh + (g.qrow0 + l32) * p.lse.ss;
      const float l = p.lse.ptr[so];
      l2 = l == kNegInf ? __builtin_inff() : l * kLog2e;
      if (p.dlse.ptr) dl = p.dlse.ptr[b * p.dlse.sb + h * p.dlse.sh + (g.qrow0 + l32) * p.dlse.ss];
    }
    asm volatile("" ::: "memory");
    if (hf == 0) ((lds_f*)tst)[l32] = l2;
    // the dS reads of the previous head were issued before these writes (in-order LDS)
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        dot += to_f32<BF>(uint16_t(elem16(rb[u], e))) * to_f32<BF>(uint16_t(elem16(rc[u], e)));
#pragma unroll
      for (int off = CPR / 2; off > 0; off >>= 1) dot += __shfl_xor(dot, off);
      const int P = 64 * u + lane;
      if (P % CPR == 0) ((lds_f*)tst)[BN + P / CPR] = dot;
    }
    put(tq, ra);
    put(tdo, rb);
    asm volatile("" ::: "memory");
    if (hf == 0) ((lds_f*)tst)[BN + l32] -= dl;
    asm volatile("" ::: "memory");

    f32x16_t st = zero16(), dp = zero16();
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      st = mfma16<BF>(lds_read16(tq + at_v(l32, 2 * cc + hf)), kf[cc], st);
      dp = mfma16<BF>(lds_read16(tdo + at_v(l32, 2 * cc + hf)), vf[cc], dp);
    }
    float pr[16], ds[16];
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int i0 = 8 * gi + 4 * hf;
      const f32x4_t L = *(const __attribute__((address_space(3))) f32x4_t*)(tst + 4 * i0);
      const f32x4_t Dl = *(const __attribute__((address_space(3))) f32x4_t*)(tst + 4 * (BN + i0));
      const float lv[4] = {L[0], L[1], L[2], L[3]}, dv4[4] = {Dl[0], Dl[1], Dl[2], Dl[3]};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * gi + e, i = i0 + e, rel = j - i - g.off;
        const bool vis = i < g.sq && j < g.sk && rel >= s.lo_rel && rel <= s.hi_rel;
        pr[r] = vis ? fast_exp2(__builtin_fmaf(st[r], s.scale_log2, -lv[e])) : 0.f;
        ds[r] = pr[r] * (dp[r] - dv4[e]);
      }
    }
    uint4 pf[2], sf[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      pf[cc] = make_uint4(pack2<BF>(pr[8 * cc], pr[8 * cc + 1]), pack2<BF>(pr[8 * cc + 2], pr[8 * cc + 3]),
                          pack2<BF>(pr[8 * cc + 4], pr[8 * cc + 5]), pack2<BF>(pr[8 * cc + 6], pr[8 * cc + 7]));
      sf[cc] = make_uint4(pack2<BF>(ds[8 * cc], ds[8 * cc + 1]), pack2<BF>(ds[8 * cc + 2], ds[8 * cc + 3]),
                          pack2<BF>(ds[8 * cc + 4], ds[8 * cc + 5]), pack2<BF>(ds[8 * cc + 6], ds[8 * cc + 7]));
    }
    // dS as [key][query]: registers 4 gi .. 4 gi + 3 are queries 8 gi + 4 hf + 0..3
    asm volatile("" ::: "memory");
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
      const uint4 w = sf[gi >> 1];
      const u32x2_t v = (gi & 1) ? u32x2_t{w.z, w.w} : u32x2_t{w.x, w.y};
      *(__attribute__((address_space(3))) u32x2_t*)(tvs + j * 64 + (8 * gi + 4 * hf) * 2) = v;
    }
    asm volatile("" ::: "memory");
    f32x16_t dq[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dq[db] = zero16();
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const uint4 sT = tr(tvs + vs, 4, cc);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        dv[db] = mfma16<BF>(tr(tdo + va[db], CPR, cc), pf[cc], dv[db]);
        dk[db] = mfma16<BF>(tr(tq + va[db], CPR, cc), sf[cc], dk[db]);
        dq[db] = mfma16<BF>(tr(tk + va[db], CPR, cc), sT, dq[db]);
      }
    }
    uint16_t* dqb = static_cast<uint16_t*>(p.dq.ptr) + b * p.dq.sb + h * p.dq.sh + g.qrow0 * p.dq.ss;
    store_tile(tq, dq, s.scale, dqb, p.dq.ss, g.sq);
  }
  uint16_t* dkb = static_cast<uint16_t*>(p.dk.ptr) + b * p.dk.sb + hk * p.dk.sh + g.krow0 * p.dk.ss;
  uint16_t* dvb = static_cast<uint16_t*>(p.dv.ptr) + b * p.dv.sb + hk * p.dv.sh + g.krow0 * p.dv.ss;
  store_tile(tdo, dv, 1.f, dvb, p.dv.ss, g.sk);
  store_tile(tk, dk, s.scale, dkb, p.dk.ss, g.sk);
}

// ----------------------------------------------------------------------------------------
// launches
// ----------------------------------------------------------------------------------------
#ifndef SDPA_BWD_KERNELS_ONLY
// The separate-launch dQ kernels at head_dim 128 are compiled in bwd_dq128.hip, with a
// scheduling strategy of their own; this unit only declares them.
extern template __global__ void bwd_dq16p_kernel<true, 128, 4, true>(BwdParams);
extern template __global__ void bwd_dq16p_kernel<false, 128, 4, true>(BwdParams);

template <class K>
static hipError_t go(K kernel, const char* name, int64_t blocks, hipStream_t st, const BwdParams& p,
                     int threads = kThreads) {
  if (blocks <= 0) return hipSuccess;
  if (!grid_fits(blocks, threads)) return hipErrorInvalidConfiguration;
  prof_begin(st, name);
  hipLaunchKernelGGL(kernel, dim3(unsigned(blocks)), dim3(threads), 0, st, p);
  prof_end(st);
  return hipGetLastError();
}

// The pipelined kernels read the streamed rows with 16-byte buffer loads at 32-bit offsets
// and need rows of at least D elements (rows past the sequence end then lie wholly outside
// the buffer range).
template <int D>
static bool pipelined_ok(const BwdParams& p, int64_t rows, int64_t ss_a, int64_t ss_b, int32_t need) {
  const int64_t ss = ss_a > ss_b ? ss_a : ss_b;
  return D >= 64 && (p.aligned & need) == need && ss_a >= D && ss_b >= D &&
         (rows + 4 * 64) * ss * 2 < (int64_t(1) << 31);
}

// The pipelined dK/dV kernels: the streamed Q/dO rows as above, and LSE log2(e) and Delta read
// through one buffer resource over the whole workspace array (one fp32 per q head and row), so
// that array must stay below 2^31 bytes; larger problems take the kernels with 64-bit
// addressing
template <int D>
static bool kv_pipelined(const BwdParams& p) {
  const int64_t rows = int64_t(p.s.hq) * (p.s.thd ? p.s.total_q : int64_t(p.s.batch) * p.s.sq);
  return pipelined_ok<D>(p, p.s.sq, p.q.ss, p.dout.ss, kAlQ | kAlK | kAlV | kAlDO | kAlDK | kAlDV) &&
         rows * 4 < (int64_t(1) << 31);
}

// head_dim 64 or 128, 16-bit, both pipelined kernels usable, no block mask, no dK/dV split
// and a large grid: dQ and dK/dV run as two launches of four-wave workgroups (at D128 the dQ
// half then runs two waves per SIMD instead of the dK/dV body's one; both halves share each
// streamed tile between four waves, and dQ forms Delta in place of the pre-pass).  Measured:
// B8 S4096 H16/4 backward 2180 -> 2010 us, H16/16 2175 -> 2040 us; varlen THD GQA (C4) 802
// -> 811 us of kernels but a 0.5% shorter step (the fused launch filled the tail of the
// longest dK/dV chain with dQ blocks).  Splitting the long dK/dV blocks into halves in the
// separate launch took 495 -> 871 us (each half's release of its partial sums).
template <int D>
static bool dq_wide_d(const BwdParams& p) {
  return kv_pipelined<D>(p) && pipelined_ok<D>(p, p.s.sk, p.k.ss, p.v.ss, kAlQ | kAlK | kAlV | kAlDO | kAlDQ) &&
         (p.aligned & kAlO) && p.o.ss >= D;
}
// The two launches pay off once the fused launch would have more than kBwdWideMinPerCU
// dK/dV plus dQ blocks per CU of the current device; on smaller grids the fused launch
// fills the tail of each half with the other (measured, causal bf16: D64 B1 S4096 H8
// fused 107 vs 163 us, B4 S2048 85 vs 101 us, B4 S4096 280 vs 275 us, B8 S4096 530 vs
// 500 us; D128 H16 B4 S1024 106 vs 113 us, B2 S2048 163 vs 164 us, B2 S4096 546 vs 515 us).
static bool dq_wide(const BwdParams& p, DType dt) {
  const Shape& s = p.s;
  if (dt == DType::F32 || s.bm.bits || p.nsplit == 2) return false;
  if (!(s.d == 128 ? dq_wide_d<128>(p) : (s.d == 64 && dq_wide_d<64>(p)))) return false;
  const int64_t tq = kBwdQ16, tk = kBwdK16;
  const int64_t nq = s.thd ? ((s.total_q + tq - 1) / tq + s.batch) * s.hq : ((s.sq + tq - 1) / tq) * s.batch * s.hq;
  const int64_t nk = s.thd ? ((s.total_k + tk - 1) / tk + s.batch) * s.hk : ((s.sk + tk - 1) / tk) * s.batch * s.hk;
  return nq + nk > int64_t(kBwdWideMinPerCU) * device_cus();
}

int bwd_q_tile_rows(const BwdParams& p, DType dt) {
  if (dt == DType::F32) return kBwdQ32;
  return dq_wide(p, dt) ? kBwdQ16Wide : kBwdQ16;
}

int bwd_k_tile_rows(const BwdParams& p, DType dt) {
  if (dt == DType::F32) return kBwdK32;
  return dq_wide(p, dt) ? kBwdK16Wide : kBwdK16;
}

// Split THD dK/dV items (their partial-sum slots): only on the separate dK/dV launch, and only
// when an item could exceed 1.5 times the mean cost per workgroup slot (the scheduler's own
// rule, decided there on the actual lengths).  The cost of a key tile is the number of
// 64-row query tiles it sees, at most ceil(max q length / 64); under a causal mask a
// sequence of L tokens costs about L^2 / (2 x 64 x 128) over its key tiles, and the sum of
// squares of the lengths is at least total^2 / batch, which bounds the mean from below.
int bwd_k_split_cap(const BwdParams& p, DType dt) {
  const Shape& s = p.s;
  if (!(s.thd && p.ksplit_cap > 0 && p.ksplit_count && p.ksplit_part && dq_wide(p, dt))) return 0;
  const double slots = double(device_cus()) * (s.d == 128 ? 1 : 2);
  if (slots <= 0 || s.batch <= 0) return 0;
  const double mean_lo = double(s.total_k) * double(s.total_k) / s.batch /
                         (2.0 * kBwdKInner * kBwdK16Wide) * s.hk / slots;
  const double max_item = double((int64_t(s.sq) + kBwdKInner - 1) / kBwdKInner);
  return max_item * 10 > mean_lo * 15 ? p.ksplit_cap : 0;
}

template <int ES, bool BF>
static hipError_t pre(const BwdParams& p, hipStream_t st) {
  const Shape& s = p.s;
  int64_t rows = s.thd ? int64_t(s.hq) * s.total_q : int64_t(s.batch) * s.hq * s.sq;
  auto launch = [&](auto kernel, int d) {
    int rpb = kThreads / (d / (16 / ES));
    int64_t blocks = (rows + rpb - 1) / rpb;
    if (blocks > kMaxRowBlocks) blocks = kMaxRowBlocks;
    return go(kernel, "bwd_pre", p.nsplit > 1 && blocks < 1 ? 1 : blocks, st, p);  // it zeroes the split counters
  };
  if (s.d == 32) return launch(bwd_pre_kernel<ES, BF, 32>, 32);
  if (s.d == 64) return launch(bwd_pre_kernel<ES, BF, 64>, 64);
  return launch(bwd_pre_kernel<ES, BF, 128>, 128);
}

template <bool BF, int D>
static hipError_t main16(const BwdParams& p, hipStream_t st, int64_t bq, int64_t bk) {
  if constexpr (D >= 64) {
    static_assert(kBwdQ16 == 64 && kBwdK16 == 64, "tile rows of the pipelined kernels");
    const bool kv = kv_pipelined<D>(p);
    const bool q = pipelined_ok<D>(p, p.s.sk, p.k.ss, p.v.ss, kAlQ | kAlK | kAlV | kAlDO | kAlDQ);
    if constexpr (D == 128 || D == 64) {
      if (dq_wide(p, BF ? DType::BF16 : DType::F16)) {
        // dQ first: its blocks form Delta and LSE log2(e) of their rows for dK/dV (no pre-pass)
        hipError_t e = go(bwd_dq16p_kernel<BF, D, 4, true>, "bwd_dq", bq, st, p, 256);
        if (e != hipSuccess) return e;
        if (p.ksplit_cap <= 0) return go(bwd_dkdv16p_kernel<BF, D, 4>, "bwd_dkdv", bk, st, p, 256);
        // THD that may have items far above the mean: the longest items run as two half
        // blocks each (listed first, ksplit_cap items at most), then a combine
        const int64_t xk = int64_t(p.ksplit_cap) * p.s.hk;
        e = go(bwd_dkdv16p_kernel<BF, D, 4, true>, "bwd_dkdv", bk + xk, st, p, 256);
        if (e != hipSuccess) return e;
        return go(bwd_dkdv_combine_kernel<BF, D>, "bwd_dkdv_combine", xk, st, p, 256);
      }
    }
    if (kv && q) {
      if (bk + bq <= 0) return hipSuccess;
      const bool split = !p.s.bm.bits && p.nsplit == 2 && bk == p.split_blocks;
      const int64_t grid = bk * (split ? 2 : 1) + bq;
      if (!grid_fits(grid, 128)) return hipErrorInvalidConfiguration;
      prof_begin(st, "bwd_main");
      if (p.s.bm.bits)
        hipLaunchKernelGGL((bwd_fused16p_kernel<BF, D, 2, true, false>), dim3(unsigned(grid)), dim3(128), 0, st, p, int(bk));
      else if (split)
        hipLaunchKernelGGL((bwd_fused16p_kernel<BF, D, 2, false, true>), dim3(unsigned(grid)), dim3(128), 0, st, p, int(bk));
      else
        hipLaunchKernelGGL((bwd_fused16p_kernel<BF, D, 2, false, false>), dim3(unsigned(grid)), dim3(128), 0, st, p, int(bk));
      prof_end(st);
      return hipGetLastError();
    }
    if (p.s.bm.bits) return hipErrorInvalidValue;  // rejected by validation
    hipError_t e = kv ? go(bwd_dkdv16p_kernel<BF, D, 2>, "bwd_dkdv", bk, st, p, 128)
                      : go(bwd_dkdv16_kernel<BF, D>, "bwd_dkdv", bk, st, p);
    if (e != hipSuccess) return e;
    return q ? go(bwd_dq16p_kernel<BF, D, 2>, "bwd_dq", bq, st, p, 128)
             : go(bwd_dq16_kernel<BF, D>, "bwd_dq", bq, st, p);
  } else {
    if (p.s.bm.bits) return hipErrorInvalidValue;  // rejected by validation
    hipError_t e = go(bwd_dkdv16_kernel<BF, D>, "bwd_dkdv", bk, st, p);
    if (e != hipSuccess) return e;
    return go(bwd_dq16_kernel<BF, D>, "bwd_dq", bq, st, p);
  }
}

template <int D>
static hipError_t main32(const BwdParams& p, hipStream_t st, int64_t bq, int64_t bk) {
  if (p.s.bm.bits) {
    hipError_t e = go(bwd_dkdv32_kernel<D, true>, "bwd_dkdv", bk, st, p);
    if (e != hipSuccess) return e;
    return go(bwd_dq32_kernel<D, true>, "bwd_dq", bq, st, p);
  }
  hipError_t e = go(bwd_dkdv32_kernel<D, false>, "bwd_dkdv", bk, st, p);
  if (e != hipSuccess) return e;
  return go(bwd_dq32_kernel<D, false>, "bwd_dq", bq, st, p);
}

bool bwd_block_mask_ok(const BwdParams& p, DType dt) {
  if (dt == DType::F32) return true;
  if (p.s.d < 64) return false;
  constexpr int32_t need_q = kAlQ | kAlK | kAlV | kAlDO | kAlDQ;
  const bool kv = p.s.d == 64 ? kv_pipelined<64>(p) : kv_pipelined<128>(p);
  const bool q = p.s.d == 64 ? pipelined_ok<64>(p, p.s.sk, p.k.ss, p.v.ss, need_q)
                             : pipelined_ok<128>(p, p.s.sk, p.k.ss, p.v.ss, need_q);
  // per-head masks stage every head's column list of a key block in LDS
  return kv && q && (p.s.bm.nh == 1 || int64_t(p.s.group) * p.s.bm.nqb <= kMaskMaxList);
}

// Sequences of at most kBwdShortRows queries and keys, head_dim <= 64: one work unit per wave
// (bwd16w_kernel, no pre-pass); its row-contiguous 16-byte accesses need every row start of
// q, k, v, o, dO, dq, dk, dv 16-byte aligned.
static bool bwd_short(const BwdParams& p, DType dt) {
  constexpr int need = kAlQ | kAlK | kAlV | kAlO | kAlDO | kAlDQ | kAlDK | kAlDV;
  return dt != DType::F32 && p.s.d <= 64 && p.s.sq <= kBwdShortRows &&
         p.s.sk <= kBwdShortRows && !p.s.bm.bits && (p.aligned & need) == need;
}

template <bool BF>
static hipError_t go_bwd_short(const BwdParams& p, hipStream_t st) {
  const int64_t blocks = (int64_t(p.s.batch) * p.s.hk + kWaves - 1) / kWaves;
  if (blocks <= 0) return hipSuccess;
  if (!grid_fits(blocks, kThreads)) return hipErrorInvalidConfiguration;
  prof_begin(st, "bwd_short");
  if (p.s.d == 32)
    hipLaunchKernelGGL((bwd16w_kernel<BF, 32>), dim3(unsigned(blocks)), dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL((bwd16w_kernel<BF, 64>), dim3(unsigned(blocks)), dim3(kThreads), 0, st, p);
  prof_end(st);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams& p, DType dt, hipStream_t st) {
  const Shape& s = p.s;
  if (bwd_short(p, dt)) return dt == DType::BF16 ? go_bwd_short<true>(p, st) : go_bwd_short<false>(p, st);
  if (!dq_wide(p, dt)) {
    hipError_t e = dt == DType::F32 ? pre<4, false>(p, st)
                                     : (dt == DType::BF16 ? pre<2, true>(p, st) : pre<2, false>(p, st));
    if (e != hipSuccess) return e;
  }
  const int tq = bwd_q_tile_rows(p, dt), tk = bwd_k_tile_rows(p, dt);
  int64_t bq = s.thd ? ((s.total_q + tq - 1) / tq + s.batch) * s.hq : int64_t((s.sq + tq - 1) / tq) * s.batch * s.hq;
  int64_t bk = s.thd ? ((s.total_k + tk - 1) / tk + s.batch) * s.hk : int64_t((s.sk + tk - 1) / tk) * s.batch * s.hk;
  switch (dt) {
    case DType::BF16:
      if (s.d == 32) return main16<true, 32>(p, st, bq, bk);
      if (s.d == 64) return main16<true, 64>(p, st, bq, bk);
      return main16<true, 128>(p, st, bq, bk);
    case DType::F16:
      if (s.d == 32) return main16<false, 32>(p, st, bq, bk);
      if (s.d == 64) return main16<false, 64>(p, st, bq, bk);
      return main16<false, 128>(p, st, bq, bk);
    default:
      if (s.d == 32) return main32<32>(p, st, bq, bk);
      if (s.d == 64) return main32<64>(p, st, bq, bk);
      return main32<128>(p, st, bq, bk);
  }
}

#endif  // SDPA_BWD_KERNELS_ONLY

}  // namespace sdpa
