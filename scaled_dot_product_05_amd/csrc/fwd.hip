// Fused attention forward for gfx950: O = softmax(scale Q K^T + mask) V and LSE.
//
// The method (online softmax over key tiles, LSE = m + log l) reaches the plain
// definition exactly up to rounding; the pages define the result, not the tiling:
// "Significant Accuracy Difference between Compiled and Eager Flex Attention" (PyTorch
// issue 135161, return_lse and merge_attn) and "[PyTorch] fused CUDNN attention kernel not
// properly handling strides" (TransformerEngine issue 1195, strided packed q/k/v, causal
// window (-1,0), softmax_scale, MQA/GQA).
//
// One workgroup (4 waves) owns 128 query rows of one (sequence, q head); each wave owns 32
// of them.  The wave computes S^T = K Q^T for a 32-key block with the query as the MFMA
// column, so each lane holds one query and 16 of its keys: the row max and row sum are
// in-lane reductions plus one exchange with the lane 32 away.  P^T then feeds O^T += V^T P^T
// straight from registers.  K tiles sit in LDS row-major; V tiles are transposed on the way
// into LDS so a lane's 8 contraction keys are one 16-byte read.  K/V tiles are double
// buffered: the global loads of tile t+1 are in flight while tile t is computed.
// Key tiles outside the window are never visited; only tiles that straddle the window edge
// or the sequence end evaluate the mask.  Work is issued longest-first (for causal masks the
// last query tiles see the most keys).
#include "device.h"
#include "launch.h"
#include "profile.h"

#include <type_traits>

namespace sdpa {

struct WorkPos {
  int b, h, tile;
};

// Decode blockIdx.x into (sequence, q head, q tile).  Returns false for idle blocks.
// Workgroups are dispatched to the 8 XCDs round-robin (block b on XCD b % 8).  Padded
// layouts with batch * heads a multiple of 8: each XCD owns a contiguous range of
// (batch, head) pairs and takes its tiles longest first (reversed q tile index), in groups
// of kFwdHeadGroup pairs when it owns more, or pair after pair when every tile costs the
// same.  Otherwise the q tile index is outermost (longest first), (batch, head) fastest.
// THD: the scheduler's cost-sorted items, with contiguous q-head ranges per XCD when the
// head count is a multiple of 8.
__device__ __forceinline__ bool decode_work(const FwdParams& p, int rows_per_tile, WorkPos& w) {
  const Shape& s = p.s;
  if (s.thd) {
    int item, h;
    if (s.hq % kXcds == 0) {
      // XCD x (block b on XCD b % 8) runs the contiguous q heads [x per, (x + 1) per), so
      // the q heads of one kv group share an XCD's L2
      const int per = s.hq / kXcds, j = blockIdx.x / kXcds;
      item = j / per;
      h = (blockIdx.x % kXcds) * per + j % per;
    } else {
      item = blockIdx.x / s.hq;
      h = blockIdx.x % s.hq;
    }
    w.h = h;
    if (item >= *p.work_count) return false;
    WorkItem it = p.work[item];
    w.b = it.seq;
    w.tile = it.tile;
    return true;
  }
  int bh = s.batch * s.hq;
  int nt = (s.sq + rows_per_tile - 1) / rows_per_tile;
  int t, r;
  // every q tile sees all sk keys (no window bound cuts any tile's range, no block mask)
  const bool uniform = s.uniform != 0;
  if (bh % kXcds == 0) {
    // XCD x (block b runs on XCD b % 8) owns the (batch, head) pairs [x per, (x + 1) per),
    // so the q heads of one kv group share an XCD and its L2.  Tiles of equal cost: the XCD
    // walks its pairs one after the other, so the workgroups resident at one time cover a
    // few heads.  Otherwise (causal or window masks) its tiles go longest first across its
    // pairs, which balances the CUs better.
    const int per = bh / kXcds, x = blockIdx.x % kXcds, k = blockIdx.x / kXcds;
    if (!uniform && per % kFwdHeadGroup == 0 && per > kFwdHeadGroup) {
      // many pairs per XCD: groups of kFwdHeadGroup pairs one after the other, longest
      // tile first within a group (fewer heads' K/V resident than longest first over all
      // the XCD's pairs, with most of its balance; causal B8 S4096 D128 672 -> 638 us,
      // B16 S2048 D128 438 -> 404 us, D64 B8 S4096 201 -> 199 us)
      constexpr int G = kFwdHeadGroup;
      const int gi = k / (G * nt), kk = k - gi * G * nt;
      r = x * per + gi * G + kk % G;
      t = kk / G;
    } else {
      const int dv = uniform ? nt : per, q = k / dv, m = k - q * dv;  // one division
      r = x * per + (uniform ? q : m);
      t = uniform ? m : q;
    }
  } else {
    t = blockIdx.x / bh;
    r = blockIdx.x % bh;
  }
  w.b = r / s.hq;
  w.h = r % s.hq;
  w.tile = nt - 1 - t;
  return true;
}

// ----------------------------------------------------------------------------------------
// bf16 / fp16 inputs: MFMA 32x32x16, fp32 accumulation
//
// Each wave owns 32 query rows.  Key tiles are double-buffered in LDS: the global loads of
// tile t+1 are in flight while tile t is computed, one barrier per tile.  Only tiles on the
// window edges or past the end of the sequence evaluate the mask.  AL = every row start is
// 16-byte aligned.
// ----------------------------------------------------------------------------------------
template <bool BF, int D, int BN, int MINB, bool AL>
__global__ __launch_bounds__(kThreads, MINB) void fwd16_kernel(FwdParams p) {
  constexpr int BM = 32 * kWaves;
  constexpr int KP = D + 8;   // K row pitch in elements (+16 B: conflict-free 16 B reads)
  constexpr int VP = BN + 8;  // V^T row pitch
  constexpr int NG = BN / 8;  // 16-byte key groups per V^T row
  constexpr int NC = D / 16;  // contraction chunks of Q K^T
  constexpr int NKB = BN / 32;
  constexpr int NDB = D / 32;
  constexpr int NPC = BN / 16;  // contraction chunks of P V
  constexpr int LDC = BN * D / 8 / kThreads;  // 16-byte chunks per thread per tile
  static_assert(LDC >= 1 && LDC <= 4, "tile split");
  // Lazy rescaling: the reference max only moves when a tile's max exceeds it by more than
  // kTau (log2 units), so P <= 2^kTau and the O accumulator is rarely rescaled.
  constexpr float kTau = 8.f;
  __shared__ __align__(16) uint16_t sk_[2][BN * KP];
  __shared__ __align__(16) uint16_t sv_[2][D * VP];

  const Shape& s = p.s;
  WorkPos w;
  if (!decode_work(p, BM, w)) return;
  const Seq g = seq_of(s, w.b);
  const int q0 = w.tile * BM;
  if (q0 >= g.sq) return;
  const int qend = min(q0 + BM, g.sq);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hf = lane >> 5;
  const int hk = w.h / s.group;

  const uint16_t* qb = static_cast<const uint16_t*>(p.q.ptr) + w.b * p.q.sb + w.h * p.q.sh +
                       g.qrow0 * p.q.ss;
  const uint16_t* kb = static_cast<const uint16_t*>(p.k.ptr) + w.b * p.k.sb + hk * p.k.sh +
                       g.krow0 * p.k.ss;
  const uint16_t* vb = static_cast<const uint16_t*>(p.v.ptr) + w.b * p.v.sb + hk * p.v.sh +
                       g.krow0 * p.v.ss;
  uint16_t* ob = static_cast<uint16_t*>(p.o.ptr) + w.b * p.o.sb + w.h * p.o.sh + g.qrow0 * p.o.ss;

  // key tiles the workgroup visits [kt0, kt1), and those every one of its rows sees in full
  int j0, j1;
  key_range(s, g, q0, qend, j0, j1);
  const int kt0 = j0 / BN;
  const int kt1 = j1 > j0 ? (j1 + BN - 1) / BN : kt0;
  int kf0, kf1;
  {
    const int64_t lo_full = int64_t(qend - 1) + g.off + s.lo_rel;  // first key every row sees
    const int64_t hi_full = min(int64_t(q0) + g.off + s.hi_rel, int64_t(g.sk) - 1);
    const int64_t a = lo_full <= 0 ? 0 : (lo_full + BN - 1) / BN;
    const int64_t b = hi_full < 0 ? 0 : (hi_full + 1) / BN;
    kf0 = int(clamp64(a, kt0, kt1));
    kf1 = int(clamp64(b, kf0, kt1));
  }

  const int qw0 = q0 + wave * 32;
  const int qw1 = min(qw0 + 32, g.sq);
  const int qi = qw0 + l32;
  int wj0 = 0, wj1 = 0;
  if (qw0 < qw1) key_range(s, g, qw0, qw1, wj0, wj1);

  // scores enter exp2 as fma(s, c, -m) with c = |scale| * log2(e) > 0; a negative scale
  // is applied by negating q (exact).
  const float c = fmaxf(fabsf(s.scale_log2), 1e-30f);
  const uint32_t qsign = s.scale_log2 < 0.f ? 0x80008000u : 0u;
  uint4 qf[NC];
  {
    const int qr = min(qi, g.sq - 1);
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      uint4 t = load16<2>(qb + qr * p.q.ss + 16 * cc + 8 * hf, AL);
      qf[cc] = make_uint4(t.x ^ qsign, t.y ^ qsign, t.z ^ qsign, t.w ^ qsign);
    }
  }

  f32x16_t acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = zero16();
  float m_run = kNegInf, l_run = 0.f;

  // ---- global -> LDS staging ----
  uint4 kst[LDC], vst[LDC];
  const int vdc = tid % (D / 8), vkg = tid / (D / 8);
  const int jlast = g.sk - 1;
  auto loadK = [&](int t) {
#pragma unroll
    for (int u = 0; u < LDC; ++u) {
      const int ci = tid + u * kThreads;
      kst[u] = load16<2>(kb + int64_t(min(t * BN + ci / (D / 8), jlast)) * p.k.ss + (ci % (D / 8)) * 8, AL);
    }
  };
  auto loadV = [&](int t) {
#pragma unroll
    for (int u = 0; u < LDC; ++u)
      vst[u] = load16<2>(vb + int64_t(min(t * BN + vkg * LDC + u, jlast)) * p.v.ss + vdc * 8, AL);
  };
  auto storeK = [&](int buf) {
#pragma unroll
    for (int u = 0; u < LDC; ++u) {
      const int ci = tid + u * kThreads;
      *reinterpret_cast<uint4*>(&sk_[buf][(ci / (D / 8)) * KP + (ci % (D / 8)) * 8]) = kst[u];
    }
  };
  // V^T rows d = vdc*8 + e hold keys in transposed order (tpos) with the 16-byte key groups
  // XOR-swizzled by d/8, so the 8 lanes writing rows 8 apart hit different banks.
  const int vpos = tpos(vkg * LDC);
  const int vcol = (((vpos >> 3) ^ (vdc & (NG - 1))) << 3) | (vpos & 7);
  auto storeV = [&](int buf) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t* dst = &sv_[buf][(vdc * 8 + e) * VP + vcol];
      if constexpr (LDC == 4) {
        uint32_t lo = elem16(vst[0], e) | (elem16(vst[1], e) << 16);
        uint32_t hi = elem16(vst[2], e) | (elem16(vst[3], e) << 16);
        *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
      } else if constexpr (LDC == 2) {
        *reinterpret_cast<uint32_t*>(dst) = elem16(vst[0], e) | (elem16(vst[1], e) << 16);
      } else {
        *dst = uint16_t(elem16(vst[0], e));
      }
    }
  };
  int voff[NDB][NPC];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int cc = 0; cc < NPC; ++cc) {
      const int d = db * 32 + l32;
      voff[db][cc] = d * VP + (((2 * cc + hf) ^ ((d >> 3) & (NG - 1))) << 3);
    }
  const int koff = l32 * KP + 8 * hf;

  // ---- building blocks ----
  auto scores = [&](int buf, f32x16_t (&st)[NKB]) {
#pragma unroll
    for (int k2 = 0; k2 < NKB; ++k2) {
      st[k2] = zero16();
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        uint4 a = *reinterpret_cast<const uint4*>(&sk_[buf][koff + k2 * 32 * KP + 16 * cc]);
        st[k2] = mfma16<BF>(a, qf[cc], st[k2]);
      }
    }
  };
  auto pv = [&](int buf, const uint4 (&pf)[NPC]) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int cc = 0; cc < NPC; ++cc) {
        uint4 a = *reinterpret_cast<const uint4*>(&sv_[buf][voff[db][cc]]);
        acc[db] = mfma16<BF>(a, pf[cc], acc[db]);
      }
  };
  // Row max of a score tile against the reference; returns true when some lane's reference
  // has to move (then the caller settles pending P V work before rescale()).
  auto tile_max = [&](const f32x16_t (&st)[NKB], float& m_tile) {
    float mx = kNegInf;
#pragma unroll
    for (int k2 = 0; k2 < NKB; ++k2)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[k2][r]);
    mx = fmaxf(mx, xor32(mx));
    m_tile = mx == kNegInf ? kNegInf : mx * c;
    return __builtin_amdgcn_ballot_w64(m_tile > m_run + kTau) != 0;
  };
  auto rescale = [&](float m_tile) {
    const bool raise = m_tile > m_run + kTau;
    const float alpha = raise ? fast_exp2(m_run - m_tile) : 1.f;
    m_run = raise ? m_tile : m_run;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
  };
  auto probs = [&](const f32x16_t (&st)[NKB], uint4 (&pf)[NPC]) {
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int cc = 0; cc < NPC; ++cc) {
      const int k2 = cc >> 1, rb = (cc & 1) * 8;
      float e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = fast_exp2(__builtin_fmaf(st[k2][rb + j], c, -m_use));
      ps0 += (e[0] + e[1]) + (e[2] + e[3]);
      ps1 += (e[4] + e[5]) + (e[6] + e[7]);
      pf[cc] = make_uint4(pack2<BF>(e[0], e[1]), pack2<BF>(e[2], e[3]), pack2<BF>(e[4], e[5]),
                          pack2<BF>(e[6], e[7]));
    }
    l_run += ps0 + ps1;
  };

  // ---- key tiles kt0 .. kt1-1, double-buffered: tile t+1 is loaded while t is computed ----
  if (kt0 < kt1) {
    loadK(kt0);
    loadV(kt0);
    storeK(0);
    storeV(0);
  }
  __syncthreads();
  for (int t = kt0; t < kt1; ++t) {
    const int buf = (t - kt0) & 1;
    const bool more = t + 1 < kt1;
    if (more) {
      loadK(t + 1);
      loadV(t + 1);
    }
    const int kbase = t * BN;
    if (kbase < wj1 && kbase + BN > wj0) {  // this wave sees part of the tile
      f32x16_t st[NKB];
      scores(buf, st);
      if (!(t >= kf0 && t < kf1) && !tile_full(s, g, qw0, qw1, kbase, kbase + BN)) {
        // key j visible to query i iff lo_rel <= j - i - off <= min(hi_rel, sk - 1 - i - off)
        const int base_rel = kbase - qi - g.off + 4 * hf;
        const int hi_eff = qi < g.sq ? min(s.hi_rel, g.sk - 1 - qi - g.off) : s.lo_rel - 1;
#pragma unroll
        for (int k2 = 0; k2 < NKB; ++k2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rel = base_rel + k2 * 32 + 8 * (r >> 2) + (r & 3);
            st[k2][r] = (rel >= s.lo_rel && rel <= hi_eff) ? st[k2][r] : kNegInf;
          }
      }
      float m_tile;
      if (tile_max(st, m_tile)) rescale(m_tile);
      uint4 pf[NPC];
      probs(st, pf);
      pv(buf, pf);
    }
    if (more) {
      storeK(buf ^ 1);
      storeV(buf ^ 1);
    }
    __syncthreads();
  }

  const float lt = l_run + xor32(l_run);
  if (qi < g.sq) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* orow = ob + qi * p.o.ss;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        int d = db * 32 + 8 * gq + 4 * hf;
        uint32_t lo = pack2<BF>(acc[db][4 * gq] * inv, acc[db][4 * gq + 1] * inv);
        uint32_t hi = pack2<BF>(acc[db][4 * gq + 2] * inv, acc[db][4 * gq + 3] * inv);
        store8(orow + d, lo, hi, AL);
      }
    }
    if (hf == 0 && p.lse.ptr) {
      float* lp = p.lse.ptr + w.b * p.lse.sb + w.h * p.lse.sh + (g.qrow0 + qi) * p.lse.ss;
      *lp = lt > 0.f ? (m_run + __log2f(lt)) * kLn2 : kNegInf;
    }
  }
}

// ----------------------------------------------------------------------------------------
// bf16 / fp16 inputs, software-pipelined: the main path for 16-byte aligned rows.
//
// K and V tiles go from HBM straight into LDS (buffer loads with the LDS destination), so
// no registers stage them and rows past the end of the sequence arrive as zeros.  Both
// tiles stay row-major in LDS with their 16-byte chunks XOR-swizzled by row:
//   K: chunk c of row r sits at slot c ^ swk(r), so the 32 rows one A-operand read touches
//      spread over all banks;
//   V: chunk c of row r sits at slot c ^ swv(r); V^T operands come from transposed LDS
//      reads (ds_read_b64_tr_b16), two per 8-key contraction slot group.
// The loop runs one tile ahead on the matrix cores: while the VALU turns tile t's scores
// into probabilities, the QK^T products of tile t+1 are already issued, and the P V
// products of tile t follow.  Loads for K(t+2) and V(t+1) are issued at the top of step t
// and waited for at its end, one barrier per tile.
// ----------------------------------------------------------------------------------------

// QB = query blocks of 32 per wave: with QB = 2 every K or V operand read from LDS feeds two
// products, halving LDS reads per flop, and each K/V tile serves 256 query rows.
// A block-sparse mask asks for one more workgroup per CU at head_dim <= 64 (its lists and
// bits fit the LDS of three).
template <bool BF, int D, int MINB, int QB, int BN, bool BSM>
__global__ __launch_bounds__(kThreads, (D == 64 && MINB < 3) ? 3 : MINB) void fwd16p_kernel(FwdParams p) {
  constexpr int BM = 32 * QB * kWaves;
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int TB = BN * D * 2;          // bytes per K or V tile
  constexpr int NDMA = BN * CPR / kThreads;  // DMA instructions per thread per tile
  constexpr int NC = D / 16;              // contraction chunks of Q K^T
  constexpr int NKB = BN / 32;
  constexpr int NDB = D / 32;
  constexpr int NPC = BN / 16;            // contraction chunks of P V
  static_assert(NDMA >= 1 && BN % 32 == 0, "tile split");
  constexpr float kTau = 8.f;
  constexpr int NS = D >= 128 ? kFwdStagesD128 : kFwdStages;  // K and V slots each
  // direct-to-LDS loads are kept below 128 KiB of LDS (with the block-mask lists and bits):
  // a backward layout that reached past it lost data it had staged at the bottom of LDS
  static_assert(2 * NS * TB + 8192 <= 131072, "LDS load destinations below 128 KiB");
  __shared__ __align__(16) char smem_[2 * NS * TB];  // K slots, then V slots
  lds_t* const lds = (lds_t*)smem_;

  const Shape& s = p.s;
  WorkPos w;
  if (!decode_work(p, BM, w)) return;
  const Seq g = seq_of(s, w.b);
  const int q0 = w.tile * BM;
  if (q0 >= g.sq) return;
  const int qend = min(q0 + BM, g.sq);
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hk = w.h / s.group;

  const uint16_t* qb = static_cast<const uint16_t*>(p.q.ptr) + w.b * p.q.sb + w.h * p.q.sh +
                       g.qrow0 * p.q.ss;
  const uint16_t* kb = static_cast<const uint16_t*>(p.k.ptr) + w.b * p.k.sb + hk * p.k.sh +
                       g.krow0 * p.k.ss;
  const uint16_t* vb = static_cast<const uint16_t*>(p.v.ptr) + w.b * p.v.sb + hk * p.v.sh +
                       g.krow0 * p.v.ss;
  uint16_t* ob = static_cast<uint16_t*>(p.o.ptr) + w.b * p.o.sb + w.h * p.o.sh + g.qrow0 * p.o.ss;

  int j0, j1;
  key_range(s, g, q0, qend, j0, j1);
  const int kt0 = j0 / BN;
  const int kt1 = j1 > j0 ? (j1 + BN - 1) / BN : kt0;
  // Block-sparse mask: the workgroup's query rows are one 128-row block row; its list of
  // 128-key blocks (each TPB tiles) is staged in LDS and replaces the range [kt0, kt1).
  constexpr int TPB = kMaskBlock / BN;
  __shared__ int32_t bm_list[BSM ? kMaskMaxList : 1];
  __shared__ __align__(16) uint32_t bm_bits[BSM ? NS * kThreads : 1];
  int nbm = 0;
  int64_t plane = 0;
  if constexpr (BSM) {
    static_assert(BM == kMaskBlock && kMaskBlock % BN == 0, "block rows");
    plane = bm_plane(s.bm, w.b, w.h);
    const int64_t row = plane * s.bm.nqb + q0 / kMaskBlock;
    nbm = min(max(s.bm.kv_count[row], 0), s.bm.nkb);
    for (int i = tid; i < nbm; i += kThreads) bm_list[i] = s.bm.kv_list[row * s.bm.nkb + i];
    __syncthreads();
  }
  // tile of step i and whether its block needs the element bits; past the last step a tile
  // beyond every key (its loads fill with zeros)
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
  const int qw0 = q0 + wave * 32 * QB;
  const int qw1 = min(qw0 + 32 * QB, g.sq);
  // key tiles [wf0, wf1) that every row of this wave sees in full (no mask needed); a wave
  // without rows masks everything (its lanes are never stored)
  int wf0 = 0, wf1 = 0;
  if (qw0 < qw1) {
    const int64_t lo_full = int64_t(qw1 - 1) + g.off + s.lo_rel;
    const int64_t hi_full = min(int64_t(qw0) + g.off + s.hi_rel, int64_t(g.sk) - 1);
    const int64_t a = lo_full <= 0 ? 0 : (lo_full + BN - 1) / BN;
    const int64_t b = hi_full < 0 ? 0 : (hi_full + 1) / BN;
    wf0 = int(clamp64(a, 0, int64_t(1) << 30));
    wf1 = int(clamp64(b, wf0, int64_t(1) << 30));
  }

  // This wave's step bound: after the last key tile one of its rows sees (the block's later
  // tiles are masked for it below the causal diagonal, and all of them for a wave past the
  // sequence end) it only issues its loads and meets the barriers.
  int wb = 1 << 30;
  if constexpr (!BSM) {
    int wj0 = 0, wj1 = 0;
    if (qw0 < qw1) key_range(s, g, qw0, qw1, wj0, wj1);
    wb = __builtin_amdgcn_readfirstlane(wj1 > wj0 ? (wj1 + BN - 1) / BN - kt0 : 0);
  }

  const float c = fmaxf(fabsf(s.scale_log2), 1e-30f);
  const uint32_t qsign = s.scale_log2 < 0.f ? 0x80008000u : 0u;
  uint4 qf[QB][NC];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const int qr = min(qw0 + 32 * j + l32, g.sq - 1);
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      uint4 t = *reinterpret_cast<const uint4*>(qb + qr * p.q.ss + 16 * cc + 8 * hf);
      qf[j][cc] = make_uint4(t.x ^ qsign, t.y ^ qsign, t.z ^ qsign, t.w ^ qsign);
    }
  }

  // ---- HBM -> LDS ----
  const int64_t kss = p.k.ss, vss = p.v.ss;
  uint32_t koff_g[NDMA], voff_g[NDMA];
#pragma unroll
  for (int u = 0; u < NDMA; ++u) {
    const int P = (u * kWaves + wave) * 64 + lane;
    const int row = P / CPR, pos = P % CPR;
    koff_g[u] = uint32_t(row * kss * 2 + ((pos ^ swk<CPR>(row)) * 16));
    voff_g[u] = uint32_t(row * vss * 2 + ((pos ^ swv<CPR>(row)) * 16));
  }
  // One resource per tensor over the sequence's rows; a tile is a 32-bit offset (the host
  // guarantees that every tile issued, up to NS past the last, stays below 2^31 bytes).
  const i32x4_t rk = make_rsrc(kb, (int64_t(g.sk) - 1) * kss * 2 + D * 2);
  const i32x4_t rv = make_rsrc(vb, (int64_t(g.sk) - 1) * vss * 2 + D * 2);
  const uint32_t kstep = uint32_t(BN * kss * 2), vstep = uint32_t(BN * vss * 2);
  auto issue_k = [&](int t, int buf) {
    const uint32_t o = uint32_t(t) * kstep;
#pragma unroll
    for (int u = 0; u < NDMA; ++u) dma16(rk, lds + buf * TB + (u * kWaves + wave) * 1024, koff_g[u] + o);
  };
  auto issue_v = [&](int t, int buf) {
    const uint32_t o = uint32_t(t) * vstep;
#pragma unroll
    for (int u = 0; u < NDMA; ++u) dma16(rv, lds + (NS + buf) * TB + (u * kWaves + wave) * 1024, voff_g[u] + o);
  };

  // ---- LDS operand addresses (lane part; tile, block and buffer parts are immediates) ----
  int ka[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) ka[cc] = (l32 * CPR + ((2 * cc + hf) ^ swk<CPR>(l32))) * 16;
  int va[NDB];
  {
    const int gg = lane >> 4, cr = (lane >> 2) & 3, a = lane & 3;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      va[db] = ((4 * (gg >> 1) + cr) * CPR + ((4 * db + 2 * (gg & 1) + (a >> 1)) ^ swv<CPR>(cr))) * 16 +
               (a & 1) * 8;
  }

  f32x16_t acc[QB][NDB];
  float m_run[QB], l_run[QB];
  bool live[QB];  // the lane's row lies inside the sequence
#pragma unroll
  for (int j = 0; j < QB; ++j) {
#pragma unroll
    for (int i = 0; i < NDB; ++i) acc[j][i] = zero16();
    m_run[j] = kNegInf;
    l_run[j] = 0.f;
    live[j] = qw0 + 32 * j + l32 < g.sq;
  }

  // The key blocks and query blocks are independent accumulation chains; alternating them
  // keeps the previous product of a chain in flight while the next one issues.
  auto scores = [&](auto B, f32x16_t(&st)[QB][NKB]) {
    constexpr int b = decltype(B)::value;
#pragma unroll
    for (int j = 0; j < QB; ++j)
#pragma unroll
      for (int k2 = 0; k2 < NKB; ++k2) st[j][k2] = zero16();
    if constexpr (D >= 128) {
      // head_dim 128: the tile's 16 A operands are read four products ahead of their use
      // (the compiler otherwise read each just before its product and waited for it; four
      // more registers per slot fit the two-wave budget: 564 -> 554 us at B8 S4096 H16, a
      // full prefetch at one wave per SIMD took 741 us)
      constexpr int NA = NC * NKB, PF = 4;
      uint4 a[NA];
#pragma unroll
      for (int u = 0; u < PF && u < NA; ++u)
        a[u] = lds_read16(lds + b * TB + (u % NKB) * 32 * CPR * 16 + ka[u / NKB]);
#pragma unroll
      for (int u = 0; u < NA; ++u) {
        if (u + PF < NA)
          a[u + PF] = lds_read16(lds + b * TB + ((u + PF) % NKB) * 32 * CPR * 16 + ka[(u + PF) / NKB]);
#pragma unroll
        for (int j = 0; j < QB; ++j)
          st[j][u % NKB] = mfma16<BF>(a[u], qf[j][u / NKB], st[j][u % NKB]);
      }
    } else {
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
#pragma unroll
      for (int k2 = 0; k2 < NKB; ++k2) {
        const uint4 a = lds_read16(lds + b * TB + k2 * 32 * CPR * 16 + ka[cc]);
#pragma unroll
        for (int j = 0; j < QB; ++j) st[j][k2] = mfma16<BF>(a, qf[j][cc], st[j][k2]);
      }
    }
  };
  auto pv = [&](auto B, const uint4(&pf)[QB][NPC]) {
    constexpr int b = decltype(B)::value;
#pragma unroll
    for (int cc = 0; cc < NPC; ++cc)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const lds_t* base = lds + (NS + b) * TB + 16 * cc * CPR * 16 + va[db];
        const uint2 lo = read_tr16(base), hi = read_tr16(base + 8 * CPR * 16);
        const uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
        for (int j = 0; j < QB; ++j) acc[j][db] = mfma16<BF>(a, pf[j][cc], acc[j][db]);
      }
  };
  // key j visible to query i iff lo_rel <= j - i - off <= min(hi_rel, sk - 1 - i - off)
  // (and, in a partial block of a block-sparse mask, the element bit of (query, key), as a
  // pass of its own so that neither pass holds the other's values)
  auto mask = [&](int t, bool part, int bslot, f32x16_t(&st)[QB][NKB]) {
    const int kbase = t * BN;
    if constexpr (BSM) {
      if (part) {
        asm volatile("" ::: "memory");
        static_assert(QB == 1 && NKB == 2, "one 64-key word per row");
        const int qi = qw0 + l32;
        const uint2 wb = *reinterpret_cast<const uint2*>(bm_bits + bslot * kThreads + 2 * (qi - q0));
        const uint32_t mb[2] = {wb.x >> (4 * hf), wb.y >> (4 * hf)};
#pragma unroll
        for (int k2 = 0; k2 < NKB; ++k2)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            st[0][k2][r] = (mb[k2] >> (8 * (r >> 2) + (r & 3))) & 1u ? st[0][k2][r] : kNegInf;
      }
    }
    if (t < wf0 || t >= wf1) {
      // keeps the compiler from evaluating the mask on every tile as selects
      asm volatile("" ::: "memory");
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        const int qi = qw0 + 32 * j + l32;
        const int base_rel = kbase - qi - g.off + 4 * hf;
        const int hi_eff = qi < g.sq ? min(s.hi_rel, g.sk - 1 - qi - g.off) : s.lo_rel - 1;
#pragma unroll
        for (int k2 = 0; k2 < NKB; ++k2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rel = base_rel + k2 * 32 + 8 * (r >> 2) + (r & 3);
            st[j][k2][r] = (rel >= s.lo_rel && rel <= hi_eff) ? st[j][k2][r] : kNegInf;
          }
      }
    }
  };
  // Lazy rescaling: the reference max m_run only moves when a tile's max exceeds it by more
  // than kTau (log2 units), so the O accumulator is rarely rescaled.  A tile is first
  // exponentiated against the current m_run with no max taken; the per-lane partial sums,
  // which are needed anyway, then show whether that was safe: every P is at most its lane's
  // sum, so a sum <= kSumMax bounds every P by 2^13 (fp16 P stays finite).  Only a lane
  // whose sum is larger (or not finite), or a live row with no reference yet, sends the
  // wave through the max and rescale below and a second exponentiation.  The second case
  // cannot be read off the sum: when every visible score of the row lies ~126 (log2 units)
  // or more below 0, exp2 against the stand-in reference 0 underflows to a zero sum, and
  // the row would keep no reference and lose its keys.  A row's first tile with a visible
  // key therefore always takes the max; rows past the sequence end never do.
  constexpr float kSumMax = 8192.f;
  auto softmax_ref = [&](const f32x16_t(&st)[QB][NKB]) {
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      float mx = kNegInf;
#pragma unroll
      for (int k2 = 0; k2 < NKB; ++k2)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[j][k2][r]);
      mx = max_halves(mx);
      const float m_tile = mx == kNegInf ? kNegInf : mx * c;
      const bool raise = m_tile > m_run[j] + kTau;
      const float alpha = raise ? fast_exp2(m_run[j] - m_tile) : 1.f;
      m_run[j] = raise ? m_tile : m_run[j];
      l_run[j] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][db][r] *= alpha;
    }
  };
  // P of the tile against m_run (0 while a row has no reference) and this lane's partial
  // row sums
  auto probs = [&](const f32x16_t(&st)[QB][NKB], uint4(&pf)[QB][NPC], float(&ps)[QB]) {
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      const float m_use = m_run[j] == kNegInf ? 0.f : m_run[j];
      float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
      for (int cc = 0; cc < NPC; ++cc) {
        const int k2 = cc >> 1, rb = (cc & 1) * 8;
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = fast_exp2(__builtin_fmaf(st[j][k2][rb + i], c, -m_use));
        ps0 += (e[0] + e[1]) + (e[2] + e[3]);
        ps1 += (e[4] + e[5]) + (e[6] + e[7]);
        pf[j][cc] = make_uint4(pack2<BF>(e[0], e[1]), pack2<BF>(e[2], e[3]), pack2<BF>(e[4], e[5]),
                               pack2<BF>(e[6], e[7]));
      }
      ps[j] = ps0 + ps1;
    }
  };
  auto softmax = [&](const f32x16_t(&st)[QB][NKB], uint4(&pf)[QB][NPC]) {
    float ps[QB];
    probs(st, pf, ps);
    bool bad = false;
#pragma unroll
    for (int j = 0; j < QB; ++j) bad = bad || (m_run[j] == kNegInf ? live[j] : !(ps[j] <= kSumMax));
    if (__builtin_amdgcn_ballot_w64(bad) != 0) {
      softmax_ref(st);
      probs(st, pf, ps);
    }
#pragma unroll
    for (int j = 0; j < QB; ++j) l_run[j] += ps[j];
  };

  // Slots: K(t) lives in K slot t % NS, V(t) in V slot t % NS.  Step t reads K(t+1) (the
  // next tile's scores) and V(t), issues the loads of K(t+NS) and V(t+NS-1), and before its
  // barrier waits only for the loads issued one step earlier (NS = 3) or for all (NS = 2).
  // Loads are issued whether or not the tile exists: past the sequence end the buffer
  // range is empty and the slot fills with zeros, which keeps the wait counts fixed.
  const int n = BSM ? nbm * TPB : kt1 - kt0;
  // Element bits of a partial tile come into LDS with its V tile and in the V tile's ring
  // slot (both are read at the tile's own step): one dword per thread (row T / 2, dword
  // T % 2 of the tile's 64-key word).  A tile that is not partial loads from past the
  // buffer end, which fills zeros and reads nothing.
  constexpr int NB = BSM ? 1 : 0;  // extra loads per V tile
  i32x4_t rbits = {0, 0, 0, 0};
  uint32_t boff = 0;
  if constexpr (BSM) {
    rbits = make_rsrc(s.bm.bits + (plane * s.sq + q0) * int64_t(s.bm.words),
                      int64_t(s.sq - q0) * s.bm.words * 8);
    boff = uint32_t((tid >> 1) * s.bm.words * 8 + (tid & 1) * 4);
  }
  auto issue_bits = [&](int i, int slot) {
    if constexpr (BSM) {
      const bool part = i < n && partial_at(i);
      const uint32_t o = part ? boff + uint32_t(tile_at(i)) * 8u : 0x80000000u;
      dma4(rbits, (lds_t*)(bm_bits + slot * kThreads + wave * 64), o);
    }
  };
  f32x16_t sa[QB][NKB], sb[QB][NKB];
  if (n > 0) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      issue_k(tile_at(j), j);
      if (j + 1 < NS) {
        issue_v(tile_at(j), j);
        issue_bits(j, j);
      }
    }
    vm_wait<(NS - 2) * (2 * NDMA + NB)>();
    lds_barrier();
    scores(std::integral_constant<int, 0>(), sa);
    // step 0 reloads K slot 0: every wave must be done reading it first
    lds_barrier();
  }
  // step i (phase I = i % U): the scores of tile kt0+i are in `cur`.  The QK^T products of
  // the next tile are issued even past the last tile (their result is then unused), so a
  // step has no branch between the two cases.
  auto step = [&](auto I, int i, f32x16_t(&cur)[QB][NKB], f32x16_t(&nxt)[QB][NKB]) {
    constexpr int ph = decltype(I)::value % NS;
    issue_k(tile_at(i + NS), ph);
    issue_v(tile_at(i + NS - 1), (ph + NS - 1) % NS);
    issue_bits(i + NS - 1, (ph + NS - 1) % NS);
    if (i < wb) {
      mask(tile_at(i), partial_at(i), ph, cur);
      uint4 pf[QB][NPC];
      scores(std::integral_constant<int, (ph + 1) % NS>(), nxt);
      softmax(cur, pf);
      pv(std::integral_constant<int, ph>(), pf);
    }
    vm_wait<(NS - 2) * (2 * NDMA + NB)>();
    lds_barrier();
  };
  constexpr int U = NS == 2 ? 2 : 6;  // a multiple of NS and of the two score buffers
  for (int i = 0; i < n; i += U) {
    step(std::integral_constant<int, 0>(), i, sa, sb);
    if (i + 1 >= n) break;
    step(std::integral_constant<int, 1>(), i + 1, sb, sa);
    if constexpr (U > 2) {
      if (i + 2 >= n) break;
      step(std::integral_constant<int, 2>(), i + 2, sa, sb);
      if (i + 3 >= n) break;
      step(std::integral_constant<int, 3>(), i + 3, sb, sa);
      if (i + 4 >= n) break;
      step(std::integral_constant<int, 4>(), i + 4, sa, sb);
      if (i + 5 >= n) break;
      step(std::integral_constant<int, 5>(), i + 5, sb, sa);
    }
  }
  vm_wait<0>();  // no load may land in LDS after the workgroup ends

#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const float lt = sum_halves(l_run[j]);
    const int qi = qw0 + 32 * j + l32;
    if (qi < g.sq) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      uint16_t* orow = ob + qi * p.o.ss;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          int d = db * 32 + 8 * gq + 4 * hf;
          uint32_t lo = pack2<BF>(acc[j][db][4 * gq] * inv, acc[j][db][4 * gq + 1] * inv);
          uint32_t hi = pack2<BF>(acc[j][db][4 * gq + 2] * inv, acc[j][db][4 * gq + 3] * inv);
          *reinterpret_cast<uint2*>(orow + d) = make_uint2(lo, hi);
        }
      }
      if (hf == 0 && p.lse.ptr) {
        float* lp = p.lse.ptr + w.b * p.lse.sb + w.h * p.lse.sh + (g.qrow0 + qi) * p.lse.ss;
        *lp = lt > 0.f ? (m_run[j] + __log2f(lt)) * kLn2 : kNegInf;
      }
    }
  }
}

// ----------------------------------------------------------------------------------------
// Short query sequences, 16-bit inputs.  With only a few dozen queries per (sequence, head)
// a 128-row workgroup leaves most of its waves without rows, and the call is bound by the
// HBM bytes in flight rather than by the matrix cores.  Here each wave is a work unit of its
// own: 32 query rows of one (sequence, q head), over 32-key tiles, with a private LDS area
// of two 32-row tiles (Q, then K tiles; V tiles, then the O tile).  Every global access is
// row-contiguous: lane chunk P = 64 u + lane of a tile is row P / CPR, 16-byte column
// P % CPR.  Rows then go from LDS into the MFMA operand layouts (K rows as the A operand of
// S^T = K Q^T, Q rows as its B operand, V through the transposed reads of O^T += V^T P^T),
// and the O tile returns through LDS to leave as whole rows.  There is no workgroup barrier:
// the four waves of a block run unrelated items, and the LDS accesses of one wave take
// effect in issue order.  The next tile's K rows load into registers while the current tile
// is computed, its V rows once the current P V products are issued.  The softmax takes the exact running max of every tile (VALU time is
// not what bounds this kernel), so P <= 1.
// ----------------------------------------------------------------------------------------
template <bool BF, int D>
__global__ __launch_bounds__(kThreads, D >= 128 ? 2 : kFwdShortMinB) void fwd16w_kernel(FwdParams p) {
  constexpr int BN = 32;
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int NC = D / 16;          // contraction chunks of Q K^T
  constexpr int NDB = D / 32;         // 32-column blocks of O
  constexpr int NU = BN * CPR / 64;   // 16-byte chunks per lane per 32-row tile
  constexpr int TB = BN * D * 2;      // bytes of one 32-row tile
  static_assert(NU >= 1 && BN * CPR % 64 == 0, "tile split");
  __shared__ __align__(16) char smem_[kWaves * 2 * TB];

  const Shape& s = p.s;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  lds_t* const ra = (lds_t*)smem_ + wave * 2 * TB;  // Q, then K tiles
  lds_t* const rb = ra + TB;                        // V tiles, then the O tile

  // item = (q tile, sequence, q head), (sequence, head) fastest
  const int64_t bh = int64_t(s.batch) * s.hq;
  const int64_t item = int64_t(blockIdx.x) * kWaves + wave;
  const int64_t nt = (s.sq + BN - 1) / BN;
  if (item >= bh * nt) return;
  const int b = int((item % bh) / s.hq), h = int(item % s.hq);
  const int q0 = int(item / bh) * BN;
  const Seq g = seq_of(s, b);
  if (q0 >= g.sq) return;
  const int qend = min(q0 + BN, g.sq);
  const int hk = h / s.group;

  const uint16_t* qb = static_cast<const uint16_t*>(p.q.ptr) + b * p.q.sb + h * p.q.sh + g.qrow0 * p.q.ss;
  const uint16_t* kb = static_cast<const uint16_t*>(p.k.ptr) + b * p.k.sb + hk * p.k.sh + g.krow0 * p.k.ss;
  const uint16_t* vb = static_cast<const uint16_t*>(p.v.ptr) + b * p.v.sb + hk * p.v.sh + g.krow0 * p.v.ss;
  uint16_t* ob = static_cast<uint16_t*>(p.o.ptr) + b * p.o.sb + h * p.o.sh + g.qrow0 * p.o.ss;

  int j0, j1;
  key_range(s, g, q0, qend, j0, j1);
  const int kt0 = j0 / BN;
  const int kt1 = j1 > j0 ? (j1 + BN - 1) / BN : kt0;
  // key tiles [wf0, wf1) that every row of the wave sees in full (no mask needed)
  int wf0, wf1;
  {
    const int64_t lo_full = int64_t(qend - 1) + g.off + s.lo_rel;
    const int64_t hi_full = min(int64_t(q0) + g.off + s.hi_rel, int64_t(g.sk) - 1);
    const int64_t a = lo_full <= 0 ? 0 : (lo_full + BN - 1) / BN;
    const int64_t e = hi_full < 0 ? 0 : (hi_full + 1) / BN;
    wf0 = int(clamp64(a, 0, int64_t(1) << 30));
    wf1 = int(clamp64(e, wf0, int64_t(1) << 30));
  }

  // LDS byte offset of 16-byte column c of tile row r: K-like tiles (read 16 rows per
  // cycle, one column) and V tiles (transposed reads of 4 rows)
  auto at_k = [](int r, int c) { return (r * CPR + (c ^ swk<CPR>(r))) * 16; };
  auto at_v = [](int r, int c) { return (r * CPR + (c ^ swv<CPR>(r))) * 16; };
  typedef __attribute__((address_space(3))) u32x4_t lds_u4;
  uint4 kr[NU], vr[NU];
  auto load_rows = [&](const uint16_t* base, int64_t ss, int row0, int nrows, uint4(&r)[NU]) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int P = 64 * u + lane, row = row0 + P / CPR;
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (row < nrows) x = *reinterpret_cast<const uint4*>(base + row * ss + (P % CPR) * 8);
      r[u] = x;
    }
  };
  auto put = [&](lds_t* dst, bool vt, const uint4(&r)[NU]) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int P = 64 * u + lane;
      const int o = vt ? at_v(P / CPR, P % CPR) : at_k(P / CPR, P % CPR);
      *(lds_u4*)(dst + o) = __builtin_bit_cast(u32x4_t, r[u]);
    }
  };
  int ka[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) ka[cc] = at_k(l32, 2 * cc + hf);
  int va[NDB];
  {
    const int gg = lane >> 4, cr = (lane >> 2) & 3, a = lane & 3;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      va[db] = ((4 * (gg >> 1) + cr) * CPR + ((4 * db + 2 * (gg & 1) + (a >> 1)) ^ swv<CPR>(cr))) * 16 +
               (a & 1) * 8;
  }

  const float c = fmaxf(fabsf(s.scale_log2), 1e-30f);
  const uint32_t qsign = s.scale_log2 < 0.f ? 0x80008000u : 0u;
  uint4 qf[NC];
  load_rows(qb, p.q.ss, q0, g.sq, kr);
  if (kt0 < kt1) {
    load_rows(vb, p.v.ss, kt0 * BN, g.sk, vr);
  }
  put(ra, false, kr);
  asm volatile("" ::: "memory");
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    const uint4 t = lds_read16(ra + ka[cc]);
    qf[cc] = make_uint4(t.x ^ qsign, t.y ^ qsign, t.z ^ qsign, t.w ^ qsign);
  }
  if (kt0 < kt1) load_rows(kb, p.k.ss, kt0 * BN, g.sk, kr);

  f32x16_t acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = zero16();
  float m_run = kNegInf, l_run = 0.f;
  const int qi = q0 + l32;
  const int hi_eff = qi < g.sq ? min(s.hi_rel, g.sk - 1 - qi - g.off) : s.lo_rel - 1;

  for (int t = kt0; t < kt1; ++t) {
    if (t > kt0) {
      load_rows(kb, p.k.ss, t * BN, g.sk, kr);
      load_rows(vb, p.v.ss, t * BN, g.sk, vr);
    }
    // the previous tile's LDS reads were issued before these writes (in-order LDS)
    asm volatile("" ::: "memory");
    put(ra, false, kr);
    put(rb, true, vr);
    asm volatile("" ::: "memory");
    f32x16_t st = zero16();
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) st = mfma16<BF>(lds_read16(ra + ka[cc]), qf[cc], st);

    if (t < wf0 || t >= wf1) {
      const int base_rel = t * BN - qi - g.off + 4 * hf;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rel = base_rel + 8 * (r >> 2) + (r & 3);
        st[r] = (rel >= s.lo_rel && rel <= hi_eff) ? st[r] : kNegInf;
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[r]);
    mx = max_halves(mx);
    const float m_new = fmaxf(m_run, mx == kNegInf ? kNegInf : mx * c);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    uint4 pf[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) e[i] = fast_exp2(__builtin_fmaf(st[8 * cc + i], c, -m_use));
      l_run += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
      pf[cc] = make_uint4(pack2<BF>(e[0], e[1]), pack2<BF>(e[2], e[3]), pack2<BF>(e[4], e[5]),
                          pack2<BF>(e[6], e[7]));
    }
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const lds_t* base = rb + 16 * cc * CPR * 16 + va[db];
        const uint2 lo = read_tr16(base), hi = read_tr16(base + 8 * CPR * 16);
        acc[db] = mfma16<BF>(make_uint4(lo.x, lo.y, hi.x, hi.y), pf[cc], acc[db]);
      }
  }

  // O tile: lane (row l32, d = 32 db + 8 gq + 4 hf .. +3) into LDS, then whole rows out
  const float lt = sum_halves(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  asm volatile("" ::: "memory");
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const uint32_t lo = pack2<BF>(acc[db][4 * gq] * inv, acc[db][4 * gq + 1] * inv);
      const uint32_t hi = pack2<BF>(acc[db][4 * gq + 2] * inv, acc[db][4 * gq + 3] * inv);
      typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
      *(__attribute__((address_space(3))) u32x2_t*)(rb + at_k(l32, 4 * db + gq) + 8 * hf) = u32x2_t{lo, hi};
    }
  asm volatile("" ::: "memory");
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int P = 64 * u + lane, row = q0 + P / CPR;
    const uint4 x = lds_read16(rb + at_k(P / CPR, P % CPR));
    if (row < g.sq) *reinterpret_cast<uint4*>(ob + row * p.o.ss + (P % CPR) * 8) = x;
  }
  if (hf == 0 && qi < g.sq && p.lse.ptr) {
    float* lp = p.lse.ptr + b * p.lse.sb + h * p.lse.sh + (g.qrow0 + qi) * p.lse.ss;
    *lp = lt > 0.f ? (m_run + __log2f(lt)) * kLn2 : kNegInf;
  }
}

// ----------------------------------------------------------------------------------------
// fp32 inputs.  Nothing is rounded below fp32 (PyTorch issue 135161 traces its large
// gradient errors to a tensor-core shortcut inside an "fp32" kernel), and the scores are
// formed in fp64: fp32 inputs widen exactly, v_mfma_f64_16x16x4 accumulates q.k in fp64,
// and the row max is subtracted in fp64 before the fp32 exp2.  With the pages' fp32
// local/global workload (q, k, v from a Linear layer filled with 0.1) scores reach ~2e2,
// where fp32 score rounding alone moves O by ~1e-5.  P V uses fp32 MFMA 16x16x4.
//
// 16x16 tiles: v_mfma_{f64_16x16x4_f64, f32_16x16x4_f32} put lane l on column l%16 and
// contraction slot l/16.  Their C layouts differ: register r of lane l is row 4*r + l/16
// for the fp64 form and row 4*(l/16) + r for the fp32 form.  Each wave owns 32 queries
// (two 16-column blocks); a K/V tile is 32 keys (two 16-row blocks).
// ----------------------------------------------------------------------------------------
template <int D, bool BSM>
__global__ __launch_bounds__(kThreads, D == 128 ? 1 : 2) void fwd32_kernel(FwdParams p) {
  constexpr int BM = kFwdBM, BN = kFwdBN32;
  constexpr int KP = D + 4;  // row pitch in floats
  constexpr int Q4 = D / 4;  // d values per contraction slot group
  constexpr int NDB = D / 16;
  constexpr int LDC = BN * D / 4 / kThreads;
  static_assert(BN == 32 && LDC >= 1, "tile split");
  __shared__ __align__(16) float sk_[2][BN * KP];
  __shared__ __align__(16) float sv_[2][BN * KP];

  const Shape& s = p.s;
  WorkPos w;
  if (!decode_work(p, BM, w)) return;
  const Seq g = seq_of(s, w.b);
  const int q0 = w.tile * BM;
  if (q0 >= g.sq) return;
  const int qend = min(q0 + BM, g.sq);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, sg = lane >> 4;
  const int hk = w.h / s.group;

  const float* qb = static_cast<const float*>(p.q.ptr) + w.b * p.q.sb + w.h * p.q.sh + g.qrow0 * p.q.ss;
  const float* kb = static_cast<const float*>(p.k.ptr) + w.b * p.k.sb + hk * p.k.sh + g.krow0 * p.k.ss;
  const float* vb = static_cast<const float*>(p.v.ptr) + w.b * p.v.sb + hk * p.v.sh + g.krow0 * p.v.ss;
  float* ob = static_cast<float*>(p.o.ptr) + w.b * p.o.sb + w.h * p.o.sh + g.qrow0 * p.o.ss;
  const bool alq = p.aligned & kAlQ, alk = p.aligned & kAlK, alv = p.aligned & kAlV,
             alo = p.aligned & kAlO;

  int j0, j1;
  key_range(s, g, q0, qend, j0, j1);
  const int kt0 = j0 / BN;
  const int kt1 = j1 > j0 ? (j1 + BN - 1) / BN : kt0;
  const int qw0 = q0 + wave * 32;
  const int qw1 = min(qw0 + 32, g.sq);
  int wj0 = 0, wj1 = 0;
  if (qw0 < qw1) key_range(s, g, qw0, qw1, wj0, wj1);
  // block-sparse mask: the list of 128-key blocks of this 128-row block row, in LDS
  constexpr int TPB = kMaskBlock / BN;
  __shared__ int32_t bm_list[BSM ? kMaskMaxList : 1];
  int nbm = 0;
  int64_t plane = 0;
  if constexpr (BSM) {
    static_assert(BM == kMaskBlock, "block rows");
    plane = bm_plane(s.bm, w.b, w.h);
    const int64_t row = plane * s.bm.nqb + q0 / kMaskBlock;
    nbm = min(max(s.bm.kv_count[row], 0), s.bm.nkb);
    for (int i = tid; i < nbm; i += kThreads) bm_list[i] = s.bm.kv_list[row * s.bm.nkb + i];
    __syncthreads();
  }
  const int nt = BSM ? nbm * TPB : kt1 - kt0;
  auto tile_at = [&](int i) -> int {
    if constexpr (BSM) {
      const int e = __builtin_amdgcn_readfirstlane(bm_list[i / TPB]);
      return min(max(e >> 1, 0), s.bm.nkb - 1) * TPB + i % TPB;
    } else {
      return kt0 + i;
    }
  };
  const double scale = double(s.scale);
  const double log2e = 1.4426950408889634;

  float qf[2][Q4];
#pragma unroll
  for (int qb2 = 0; qb2 < 2; ++qb2) {
    const int qi = qw0 + 16 * qb2 + l16;
#pragma unroll
    for (int u = 0; u < Q4 / 4; ++u) {
      uint4 t = qi < g.sq ? load16<4>(qb + qi * p.q.ss + sg * Q4 + 4 * u, alq) : make_uint4(0, 0, 0, 0);
      qf[qb2][4 * u] = __uint_as_float(t.x);
      qf[qb2][4 * u + 1] = __uint_as_float(t.y);
      qf[qb2][4 * u + 2] = __uint_as_float(t.z);
      qf[qb2][4 * u + 3] = __uint_as_float(t.w);
    }
  }
  f32x4_t acc[NDB][2];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i][0] = acc[i][1] = zero4();
  double m_run[2] = {-__builtin_inf(), -__builtin_inf()};
  float l_run[2] = {0.f, 0.f};

  uint4 kst[LDC], vst[LDC];
  auto gload = [&](int kt) {
    const int base = kt * BN;
#pragma unroll
    for (int u = 0; u < LDC; ++u) {
      int ci = tid + u * kThreads;
      int row = ci / (D / 4), col = (ci % (D / 4)) * 4;
      int j = base + row;
      bool in = j < g.sk;
      kst[u] = in ? load16<4>(kb + j * p.k.ss + col, alk) : make_uint4(0, 0, 0, 0);
      vst[u] = in ? load16<4>(vb + j * p.v.ss + col, alv) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < LDC; ++u) {
      int ci = tid + u * kThreads;
      int row = ci / (D / 4), col = (ci % (D / 4)) * 4;
      *reinterpret_cast<uint4*>(&sk_[buf][row * KP + col]) = kst[u];
      *reinterpret_cast<uint4*>(&sv_[buf][row * KP + col]) = vst[u];
    }
  };

  if (nt > 0) {
    gload(tile_at(0));
    sstore(0);
  }
  __syncthreads();

  for (int it = 0; it < nt; ++it) {
    const int kt = tile_at(it);
    const int buf = it & 1;
    const bool more = it + 1 < nt;
    if (more) gload(tile_at(it + 1));
    const int kbase = kt * BN;
    bool part = false;
    if constexpr (BSM) part = (__builtin_amdgcn_readfirstlane(bm_list[it / TPB]) & 1) != 0;
    if (kbase < wj1 && kbase + BN > wj0) {
      // S^T blocks (key block kb, query block qb) in fp64
      f64x4_t st[2][2];
#pragma unroll
      for (int a = 0; a < 2; ++a) st[a][0] = st[a][1] = zero4d();
#pragma unroll
      for (int u = 0; u < Q4 / 4; ++u) {
        float4 kv[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
          kv[k2] = *reinterpret_cast<const float4*>(&sk_[buf][(16 * k2 + l16) * KP + sg * Q4 + 4 * u]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const double kd = double(e == 0 ? kv[k2].x : e == 1 ? kv[k2].y : e == 2 ? kv[k2].z : kv[k2].w);
#pragma unroll
            for (int qb2 = 0; qb2 < 2; ++qb2) st[k2][qb2] = mfma64(kd, double(qf[qb2][4 * u + e]), st[k2][qb2]);
          }
        }
      }
      const bool full = tile_full(s, g, qw0, qw1, kbase, kbase + BN) && !part;
#pragma unroll
      for (int qb2 = 0; qb2 < 2; ++qb2) {
        const int qi = qw0 + 16 * qb2 + l16;
        // element bits of this row's 32 keys (tile kt is dword kt of the row)
        const uint32_t mb = part ? bm_dword(s.bm, plane, s.sq, s.sk, qi, kt) : ~0u;
        double mx = -__builtin_inf();
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            double t = st[k2][qb2][r] * scale;
            if (!full && !(visible(s, g, qi, kbase + 16 * k2 + 4 * r + sg) &&
                           ((mb >> (16 * k2 + 4 * r + sg)) & 1u)))
              t = -__builtin_inf();
            st[k2][qb2][r] = t;
            mx = fmax(mx, t);
          }
        mx = fmax(mx, __shfl_xor(mx, 16));
        mx = fmax(mx, __shfl_xor(mx, 32));
        const double m_new = fmax(m_run[qb2], mx);
        const double m_use = m_new == -__builtin_inf() ? 0.0 : m_new;
        const float alpha = fast_exp2(float((m_run[qb2] - m_use) * log2e));
        float ps = 0.f;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float e = fast_exp2(float((st[k2][qb2][r] - m_use) * log2e));
            st[k2][qb2][r] = e;  // P^T kept in the fp64 slots, exact in fp32
            ps += e;
          }
        l_run[qb2] = l_run[qb2] * alpha + ps;
        m_run[qb2] = m_new;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[db][qb2][r] *= alpha;
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[db][qb2] = mfma16x4(sv_[buf][(16 * k2 + 4 * r + sg) * KP + 16 * db + l16],
                                      float(st[k2][qb2][r]), acc[db][qb2]);
        }
      }
    }
    if (more) sstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int qb2 = 0; qb2 < 2; ++qb2) {
    float lt = l_run[qb2];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const int qi = qw0 + 16 * qb2 + l16;
    if (qi < g.sq) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      float* orow = ob + qi * p.o.ss;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        uint4 v = make_uint4(__float_as_uint(acc[db][qb2][0] * inv), __float_as_uint(acc[db][qb2][1] * inv),
                             __float_as_uint(acc[db][qb2][2] * inv), __float_as_uint(acc[db][qb2][3] * inv));
        store16<4>(orow + 16 * db + 4 * sg, v, alo);
      }
      if (sg == 0 && p.lse.ptr) {
        float* lp = p.lse.ptr + w.b * p.lse.sb + w.h * p.lse.sh + (g.qrow0 + qi) * p.lse.ss;
        *lp = lt > 0.f ? float(m_run[qb2] + double(__logf(lt))) : kNegInf;
      }
    }
  }
}

// Grid for a tile of `rows` query rows: THD uses the scheduler's work list (rows past the
// packed total plus one partial tile per sequence), padded layouts one block per tile.
static int64_t fwd_grid(const FwdParams& p, int rows) {
  const Shape& s = p.s;
  const int64_t tiles = s.thd ? (s.total_q + rows - 1) / rows + s.batch
                              : int64_t((s.sq + rows - 1) / rows) * s.batch;
  return tiles * s.hq;
}

template <class K>
static hipError_t go(K kernel, int blocks, hipStream_t st, const FwdParams& p) {
  if (!grid_fits(blocks, kThreads)) return hipErrorInvalidConfiguration;
  prof_begin(st, "attn_fwd");
  hipLaunchKernelGGL(kernel, dim3(blocks), dim3(kThreads), 0, st, p);
  prof_end(st);
  return hipGetLastError();
}

// The pipelined kernel addresses K/V rows with 32-bit buffer offsets (a tile spans kFwdBNP
// rows) and relies on rows of at least D elements, so that every row past the sequence end
// lies wholly outside the buffer range.
static bool fwd_pipelined(const FwdParams& p) {
  constexpr int need = kAlQ | kAlK | kAlV | kAlO;
  const int64_t kv_ss = p.k.ss > p.v.ss ? p.k.ss : p.v.ss;
  return (p.aligned & need) == need && p.k.ss >= p.s.d && p.v.ss >= p.s.d &&
         (int64_t(p.s.sk) + 4 * kFwdBNP) * kv_ss * 2 < (int64_t(1) << 31);
}

bool fwd_block_mask_ok(const FwdParams& p, DType dt) { return dt == DType::F32 || fwd_pipelined(p); }

// Sequences of at most kFwdShortRows queries: one work unit per wave (fwd16w_kernel), which
// reads rows with 16-byte vector loads, so every row start must be 16-byte aligned.
static bool fwd_short(const FwdParams& p) {
  constexpr int need = kAlQ | kAlK | kAlV | kAlO;
  return p.s.sq <= kFwdShortRows && !p.s.bm.bits && (p.aligned & need) == need;
}

template <bool BF, int D>
static hipError_t go_short(const FwdParams& p, hipStream_t st) {
  const int64_t items = int64_t(p.s.batch) * p.s.hq * ((p.s.sq + 31) / 32);
  const int64_t blocks = (items + kWaves - 1) / kWaves;
  if (blocks <= 0) return hipSuccess;
  if (!grid_fits(blocks, kThreads)) return hipErrorInvalidConfiguration;
  prof_begin(st, "attn_fwd_short");
  hipLaunchKernelGGL((fwd16w_kernel<BF, D>), dim3(unsigned(blocks)), dim3(kThreads), 0, st, p);
  prof_end(st);
  return hipGetLastError();
}

template <bool BF, int D, int BN, int MINB>
static hipError_t go16(const FwdParams& p, hipStream_t st) {
  if (fwd_short(p)) return go_short<BF, D>(p, st);
  constexpr int BM = 32 * kWaves;
  static_assert(BM == kFwdBM16, "host and kernel tile rows differ");
  const int64_t blocks = fwd_grid(p, BM);
  if (blocks <= 0) return hipSuccess;
  if (!grid_fits(blocks, kThreads)) return hipErrorInvalidConfiguration;
  const bool al = (p.aligned & (kAlQ | kAlK | kAlV | kAlO)) == (kAlQ | kAlK | kAlV | kAlO);
  if (fwd_pipelined(p)) {
    if (p.s.bm.bits) return go(fwd16p_kernel<BF, D, MINB, 1, kFwdBNP, true>, int(blocks), st, p);
    return go(fwd16p_kernel<BF, D, MINB, 1, kFwdBNP, false>, int(blocks), st, p);
  }
  if (p.s.bm.bits) return hipErrorInvalidValue;  // rejected by validation
  return al ? go(fwd16_kernel<BF, D, BN, MINB, true>, int(blocks), st, p)
            : go(fwd16_kernel<BF, D, BN, MINB, false>, int(blocks), st, p);
}

template <bool BF>
static hipError_t fwd16_dispatch(const FwdParams& p, hipStream_t st) {
  switch (p.s.d) {
    case 32: return go16<BF, 32, 64, 2>(p, st);
    case 64: return go16<BF, 64, kFwdBN16_D64, kFwdMinB_D64>(p, st);
    default: return go16<BF, 128, kFwdBN16_D128, kFwdMinB_D128>(p, st);
  }
}

// ----------------------------------------------------------------------------------------
// FP8 (E4M3) inputs, bf16 output.  "[PyTorch] fused CUDNN attention kernel not properly
// handling strides" (TransformerEngine issue 1195) hands its fused attention an FP8 recipe
// (DelayedScaling): tensors as 8-bit codes with one fp32 scale each, value = code *
// descale.  Both products run on v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 operands, unit
// block scales, 64-deep contraction).  That instruction pairs byte idx of an A lane with
// byte idx of the B lane in the same half of the wave, so each operand only has to agree on
// which key or d each (half, byte) holds:
//   Q K^T: A = K rows, B = Q rows, byte idx of half h = d 64 e + 32 h + idx;
//   P V:   B = P^T straight from the score registers (byte 16 k2 + r = register r of key
//          block k2, i.e. key 32 k2 + 8 (r / 4) + 4 h + r % 4), A = V^T gathered in that key
//          order by ds_read_b64_tr_b8 (lane 16g + 8a + b receives byte b of the rows the
//          lanes 16g + a + 2c address, c = 0..7): four reads of 8 bytes per 32 columns.
// The softmax takes the exact running max every tile, so P is in [0, 1]; it is scaled by
// 2^8 (added to the exponent) so that P * 256 uses E4M3's normal range down to 2^-14, and
// the row sum carries the same factor (O unaffected, LSE takes -8).
// ----------------------------------------------------------------------------------------
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16_t mfma_e4m3(const i32x8_t& a, const i32x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x2_t read_tr8(const lds_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2_t*)p);
}

// V rows of an FP8 tile: 16-byte chunk c of row r sits at slot c ^ swv8(r).  With it the
// eight rows × two chunks one transposed read touches per 32 lanes fall on 64 distinct
// banks (checked on the CPU for D 64 and 128).
template <int CPR>
__device__ __forceinline__ int swv8(int r) {
  return CPR == 4 ? ((r & 1) | (((r >> 3) & 1) << 1))
                  : ((r & 1) | (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2));
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd8_kernel(FwdParams p) {
  constexpr int BM = 32 * kWaves, BN = 64;
  constexpr int CPR = D / 16;                 // 16-byte chunks per row
  constexpr int TB = BN * D;                  // bytes per K or V tile
  constexpr int NDMA = BN * CPR / kThreads;   // 16-byte loads per thread per tile
  constexpr int NE = D / 64;                  // 64-deep contraction blocks of Q K^T
  constexpr int NDB = D / 32;                 // 32-column blocks of O
  constexpr int NS = 3;                       // K and V slots each
  static_assert(NDMA >= 1 && (D == 64 || D == 128), "tile split");
  __shared__ __align__(16) char smem_[2 * NS * TB];
  lds_t* const lds = (lds_t*)smem_;

  const Shape& s = p.s;
  WorkPos w;
  if (!decode_work(p, BM, w)) return;
  const Seq g = seq_of(s, w.b);
  const int q0 = w.tile * BM;
  if (q0 >= g.sq) return;
  const int qend = min(q0 + BM, g.sq);
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hk = w.h / s.group;
  const uint8_t* qb = static_cast<const uint8_t*>(p.q.ptr) + w.b * p.q.sb + w.h * p.q.sh + g.qrow0 * p.q.ss;
  const uint8_t* kb = static_cast<const uint8_t*>(p.k.ptr) + w.b * p.k.sb + hk * p.k.sh + g.krow0 * p.k.ss;
  const uint8_t* vb = static_cast<const uint8_t*>(p.v.ptr) + w.b * p.v.sb + hk * p.v.sh + g.krow0 * p.v.ss;
  uint16_t* ob = static_cast<uint16_t*>(p.o.ptr) + w.b * p.o.sb + w.h * p.o.sh + g.qrow0 * p.o.ss;

  int j0, j1;
  key_range(s, g, q0, qend, j0, j1);
  const int kt0 = j0 / BN;
  const int kt1 = j1 > j0 ? (j1 + BN - 1) / BN : kt0;
  const int qw0 = q0 + wave * 32;
  const int qw1 = min(qw0 + 32, g.sq);
  int wf0 = 0, wf1 = 0;  // key tiles every row of this wave sees in full
  if (qw0 < qw1) {
    const int64_t lo_full = int64_t(qw1 - 1) + g.off + s.lo_rel;
    const int64_t hi_full = min(int64_t(qw0) + g.off + s.hi_rel, int64_t(g.sk) - 1);
    const int64_t a = lo_full <= 0 ? 0 : (lo_full + BN - 1) / BN;
    const int64_t b = hi_full < 0 ? 0 : (hi_full + 1) / BN;
    wf0 = int(clamp64(a, 0, int64_t(1) << 30));
    wf1 = int(clamp64(b, wf0, int64_t(1) << 30));
  }

  // descales and the score multiplier in log2 units; a negative product flips q's signs
  const float dsq = p.descale_q ? *p.descale_q : 1.f;
  const float dsk = p.descale_k ? *p.descale_k : 1.f;
  const float dsv = p.descale_v ? *p.descale_v : 1.f;
  const float craw = s.scale_log2 * dsq * dsk;
  const float c = fmaxf(fabsf(craw), 1e-30f);
  const uint32_t qsign = craw < 0.f ? 0x80808080u : 0u;

  // Q fragments: lane (query l32, half hf) holds d = 64 e + 32 hf + 0..31 of its row
  i32x8_t qf[NE];
  {
    const int qr = min(qw0 + l32, g.sq - 1);
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const uint4* src = reinterpret_cast<const uint4*>(qb + int64_t(qr) * p.q.ss + 64 * e + 32 * hf);
      const uint4 x0 = src[0], x1 = src[1];
      qf[e] = i32x8_t{int(x0.x ^ qsign), int(x0.y ^ qsign), int(x0.z ^ qsign), int(x0.w ^ qsign),
                      int(x1.x ^ qsign), int(x1.y ^ qsign), int(x1.z ^ qsign), int(x1.w ^ qsign)};
    }
  }

  // ---- HBM -> LDS (rows past the sequence end read as zeros) ----
  const int64_t kss = p.k.ss, vss = p.v.ss;
  uint32_t koff_g[NDMA], voff_g[NDMA];
#pragma unroll
  for (int u = 0; u < NDMA; ++u) {
    const int P = (u * kWaves + wave) * 64 + lane;
    const int row = P / CPR, pos = P % CPR;
    koff_g[u] = uint32_t(row * kss + ((pos ^ swk<CPR>(row)) * 16));
    voff_g[u] = uint32_t(row * vss + ((pos ^ swv8<CPR>(row)) * 16));
  }
  const i32x4_t rk = make_rsrc(kb, (int64_t(g.sk) - 1) * kss + D);
  const i32x4_t rv = make_rsrc(vb, (int64_t(g.sk) - 1) * vss + D);
  const uint32_t kstep = uint32_t(BN * kss), vstep = uint32_t(BN * vss);
  auto issue_k = [&](int t, int slot) {
    const uint32_t o = uint32_t(t) * kstep;
#pragma unroll
    for (int u = 0; u < NDMA; ++u) dma16(rk, lds + slot * TB + (u * kWaves + wave) * 1024, koff_g[u] + o);
  };
  auto issue_v = [&](int t, int slot) {
    const uint32_t o = uint32_t(t) * vstep;
#pragma unroll
    for (int u = 0; u < NDMA; ++u) dma16(rv, lds + (NS + slot) * TB + (u * kWaves + wave) * 1024, voff_g[u] + o);
  };

  // ---- LDS operand offsets (lane part) ----
  int ka[NE][2];
#pragma unroll
  for (int e = 0; e < NE; ++e)
#pragma unroll
    for (int part = 0; part < 2; ++part)
      ka[e][part] = l32 * D + (((4 * e + 2 * hf + part) ^ swk<CPR>(l32)) * 16);
  int va[NDB][4];
  {
    const int g4 = lane >> 4, a = lane & 1, cc = (lane & 15) >> 1;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = 16 * j + 8 * (cc >> 2) + 4 * (g4 >> 1) + (cc & 3);
        const int unit = 2 * db + (g4 & 1);
        va[db][j] = key * D + ((unit ^ swv8<CPR>(key)) * 16) + 8 * a;
      }
  }

  f32x16_t acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = zero16();
  float m_run = kNegInf, l_run = 0.f;

  // S^T of the K tile in slot sl: two 32-key blocks, NE MFMAs each
  auto scores = [&](int sl, f32x16_t(&st)[2]) {
    const lds_t* base = lds + sl * TB;
    st[0] = zero16();
    st[1] = zero16();
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const uint4 a0 = lds_read16(base + k2 * 32 * D + ka[e][0]);
        const uint4 a1 = lds_read16(base + k2 * 32 * D + ka[e][1]);
        const i32x8_t a = {int(a0.x), int(a0.y), int(a0.z), int(a0.w), int(a1.x), int(a1.y), int(a1.z), int(a1.w)};
        st[k2] = mfma_e4m3(a, qf[e], st[k2]);
      }
  };
  auto pv = [&](int sl, const i32x8_t& pf) {
    const lds_t* base = lds + (NS + sl) * TB;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const i32x2_t r0 = read_tr8(base + va[db][0]), r1 = read_tr8(base + va[db][1]);
      const i32x2_t r2 = read_tr8(base + va[db][2]), r3 = read_tr8(base + va[db][3]);
      const i32x8_t a = {r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y};
      acc[db] = mfma_e4m3(a, pf, acc[db]);
    }
  };
  // key j visible to query i iff lo_rel <= j - i - off <= min(hi_rel, sk - 1 - i - off)
  auto mask = [&](int t, f32x16_t(&st)[2]) {
    if (t < wf0 || t >= wf1) {
      asm volatile("" ::: "memory");
      const int qi = qw0 + l32;
      const int base_rel = t * BN - qi - g.off + 4 * hf;
      const int hi_eff = qi < g.sq ? min(s.hi_rel, g.sk - 1 - qi - g.off) : s.lo_rel - 1;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rel = base_rel + k2 * 32 + 8 * (r >> 2) + (r & 3);
          st[k2][r] = (rel >= s.lo_rel && rel <= hi_eff) ? st[k2][r] : kNegInf;
        }
    }
  };
  // exact running max, P * 256 packed to E4M3 as the B operand of P V
  auto softmax = [&](const f32x16_t(&st)[2], i32x8_t& pf) {
    float mx = kNegInf;
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[k2][r]);
    mx = max_halves(mx);
    const float m_tile = mx == kNegInf ? kNegInf : mx * c;
    const float m_new = fmaxf(m_run, m_tile);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
      const float alpha = m_new > m_run ? fast_exp2(m_run - m_new) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      m_run = m_new;
    }
    const float off = 8.f - (m_run == kNegInf ? 0.f : m_run);
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int wd = 0; wd < 8; ++wd) {
      const int k2 = wd >> 2, rb = 4 * (wd & 3);
      const float e0 = fast_exp2(__builtin_fmaf(st[k2][rb], c, off));
      const float e1 = fast_exp2(__builtin_fmaf(st[k2][rb + 1], c, off));
      const float e2 = fast_exp2(__builtin_fmaf(st[k2][rb + 2], c, off));
      const float e3 = fast_exp2(__builtin_fmaf(st[k2][rb + 3], c, off));
      ps0 += e0 + e1;
      ps1 += e2 + e3;
      pf[wd] = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false), true);
    }
    l_run += ps0 + ps1;
  };

  // Slots: K(t) and V(t) in slot t % 3.  Step t reads K(t+1) and V(t), issues the loads of
  // K(t+3) and V(t+2) and waits, before its barrier, for all loads but its own.
  const int n = kt1 - kt0;
  f32x16_t sa[2], sb[2];
  if (n > 0) {
    issue_k(kt0, 0);
    issue_v(kt0, 0);
    issue_k(kt0 + 1, 1);
    issue_v(kt0 + 1, 1);
    issue_k(kt0 + 2, 2);
    vm_wait<2 * NDMA>();
    lds_barrier();
    scores(0, sa);
    lds_barrier();  // step 0 reloads K slot 0
  }
  int ph = 0;
  for (int i = 0; i < n; ++i) {
    const int t = kt0 + i;
    const int p1 = ph == NS - 1 ? 0 : ph + 1, p2 = p1 == NS - 1 ? 0 : p1 + 1;
    issue_k(t + NS, ph);
    issue_v(t + NS - 1, p2);
    mask(t, sa);
    scores(p1, sb);  // past the last tile: zeros, unused
    i32x8_t pf;
    softmax(sa, pf);
    pv(ph, pf);
    vm_wait<2 * NDMA>();
    lds_barrier();
    sa[0] = sb[0];
    sa[1] = sb[1];
    ph = p1;
  }
  vm_wait<0>();  // no load may land in LDS after the workgroup ends

  const float lt = sum_halves(l_run);
  const int qi = qw0 + l32;
  if (qi < g.sq) {
    const float inv = lt > 0.f ? dsv / lt : 0.f;
    uint16_t* orow = ob + int64_t(qi) * p.o.ss;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = db * 32 + 8 * gq + 4 * hf;
        const uint32_t lo = pack2<true>(acc[db][4 * gq] * inv, acc[db][4 * gq + 1] * inv);
        const uint32_t hi = pack2<true>(acc[db][4 * gq + 2] * inv, acc[db][4 * gq + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d) = make_uint2(lo, hi);
      }
    if (hf == 0 && p.lse.ptr) {
      float* lp = p.lse.ptr + w.b * p.lse.sb + w.h * p.lse.sh + (g.qrow0 + qi) * p.lse.ss;
      *lp = lt > 0.f ? (m_run + __log2f(lt) - 8.f) * kLn2 : kNegInf;
    }
  }
}

// The FP8 kernel needs 16-byte aligned rows of q, k, v and o, k/v row strides of at least
// D bytes and 32-bit tile offsets (as the pipelined 16-bit kernel).
bool fwd8_ok(const FwdParams& p) {
  constexpr int need = kAlQ | kAlK | kAlV | kAlO;
  const int64_t kv_ss = p.k.ss > p.v.ss ? p.k.ss : p.v.ss;
  return (p.s.d == 64 || p.s.d == 128) && (p.aligned & need) == need && p.k.ss >= p.s.d &&
         p.v.ss >= p.s.d && (int64_t(p.s.sk) + 4 * 64) * kv_ss < (int64_t(1) << 31);
}

hipError_t launch_fwd8(const FwdParams& p, hipStream_t st) {
  const int64_t blocks = fwd_grid(p, 32 * kWaves);
  if (blocks <= 0) return hipSuccess;
  if (!grid_fits(blocks, kThreads)) return hipErrorInvalidConfiguration;
  prof_begin(st, "attn_fwd_fp8");
  if (p.s.d == 64)
    hipLaunchKernelGGL(fwd8_kernel<64>, dim3(unsigned(blocks)), dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL(fwd8_kernel<128>, dim3(unsigned(blocks)), dim3(kThreads), 0, st, p);
  prof_end(st);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams& p, DType dt, hipStream_t st) {
  const Shape& s = p.s;
  if (dt == DType::BF16) return fwd16_dispatch<true>(p, st);
  if (dt == DType::F16) return fwd16_dispatch<false>(p, st);
  const int64_t blocks = fwd_grid(p, kFwdBM);
  if (blocks <= 0) return hipSuccess;
  if (!grid_fits(blocks, kThreads)) return hipErrorInvalidConfiguration;
  if (s.bm.bits) {
    if (s.d == 32) return go(fwd32_kernel<32, true>, int(blocks), st, p);
    if (s.d == 64) return go(fwd32_kernel<64, true>, int(blocks), st, p);
    return go(fwd32_kernel<128, true>, int(blocks), st, p);
  }
  if (s.d == 32) return go(fwd32_kernel<32, false>, int(blocks), st, p);
  if (s.d == 64) return go(fwd32_kernel<64, false>, int(blocks), st, p);
  return go(fwd32_kernel<128, false>, int(blocks), st, p);
}

}  // namespace sdpa
