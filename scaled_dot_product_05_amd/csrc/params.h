// Kernel-side parameter blocks, shared by the host launch code and the HIP kernels.
// Every tensor reaches a kernel as a base pointer plus element strides for
// (batch, head, row); the d stride is 1 (checked at the C-ABI boundary).
#pragma once
#include <stdint.h>

namespace sdpa {

enum class DType : int32_t { F16 = 0, BF16 = 1, F32 = 2 };

// Strided [batch, head, row, d] view.  For packed varlen (THD) tensors sb is 0 and a
// row index is the packed row t = cu_seqlens[b] + i.
struct View {
  void* ptr;
  int64_t sb, sh, ss;
};

// fp32 row statistic [batch, head, row] (THD: [head, packed row], sb = 0).
struct StatView {
  float* ptr;
  int64_t sb, sh, ss;
};

// Window bounds relative to the aligned diagonal: key j is visible to query i iff
// lo_rel <= j - (i + off) <= hi_rel, off = 0 (top-left) or sk - sq (bottom-right).
// Unbounded sides are clamped to +-kUnbounded so int32 arithmetic never overflows.
constexpr int32_t kUnbounded = 1 << 30;
constexpr int32_t kMaxSeqlen = (1 << 28) - 1;

struct Shape {
  int32_t batch, sq, sk, hq, hk, group, d;
  int32_t thd;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* pad_q;  // THD with padding: first packed row of each sequence (else null)
  const int32_t* pad_k;
  int64_t total_q, total_k;
  int32_t lo_rel, hi_rel;
  int32_t bottom_right;
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
};

// THD work item: sequence index and tile index within that sequence.
struct WorkItem {
  int32_t seq, tile;
};

// Bits of FwdParams::aligned / BwdParams::aligned: every row start of that tensor is
// 16-byte aligned (vector loads and stores allowed).
enum AlignBit : int32_t {
  kAlQ = 1, kAlK = 2, kAlV = 4, kAlO = 8, kAlDO = 16, kAlDQ = 32, kAlDK = 64, kAlDV = 128
};

struct FwdParams {
  Shape s;
  View q, k, v, o;
  StatView lse;  // ptr may be null
  const WorkItem* work;  // THD: longest-first list of (seq, q tile)
  const int32_t* work_count;
  int32_t aligned;
};

struct BwdParams {
  Shape s;
  View q, k, v, o, dout, dq, dk, dv;
  StatView lse, dlse;  // dlse.ptr may be null
  float* delta;        // workspace: Delta_i = dO_i . O_i - dLSE_i, laid out [b][h][row] / [h][t]
  float* lse2;         // workspace: LSE_i log2(e) (+inf for rows without a visible key), same layout
  int64_t ws_rows;     // rows of delta and lse2
  const WorkItem* work_q;  // THD: (seq, q tile) list for dQ
  const int32_t* count_q;
  const WorkItem* work_k;  // THD: (seq, k tile) list for dK/dV
  const int32_t* count_k;
  int32_t aligned;
  int32_t accumulate;
};

struct MergeParams {
  int64_t rows;          // batch * heads * seqlen, or heads * total
  int32_t batch, seqlen, heads, d, thd;
  View xa, xb, x, g, dxa, dxb;
  StatView la, lb, l, glse, dla, dlb;
  int32_t aligned;       // all x-like row starts 16-byte aligned
};

// THD scheduler: builds a work list sorted by decreasing cost from device cu_seqlens.
struct SchedParams {
  const int32_t* cu_own;    // sequences whose tiles become work items
  const int32_t* cu_other;  // the other side (keys for q tiles, queries for k tiles)
  int64_t total_own, total_other;
  int32_t batch, max_own, max_other;
  int32_t tile_own, tile_other;
  int32_t lo_rel, hi_rel, bottom_right;
  int32_t own_is_query;  // 1: items are q tiles, cost = k tiles seen; 0: k tiles, cost = q tiles
  int32_t max_items;
  WorkItem* items;
  int32_t* count;
};

}  // namespace sdpa
