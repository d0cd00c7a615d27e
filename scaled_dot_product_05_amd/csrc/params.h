// Kernel-side parameter blocks, shared by the host launch code and the HIP kernels.
// Every tensor reaches a kernel as a base pointer plus element strides for
// (batch, head, row); the d stride is 1 (checked at the C-ABI boundary).
#pragma once
#include <stdint.h>

namespace sdpa {

enum class DType : int32_t { F16 = 0, BF16 = 1, F32 = 2, E4M3 = 3 };

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

// Block-sparse mask: element bits plus the block table built from them (128 x 128 blocks).
// bits == nullptr: no block mask.
constexpr int kMaskBlock = 128;
constexpr int kMaskMaxList = 512;  // longest block list a workgroup stages in LDS
struct BlockMaskP {
  const uint64_t* bits;     // [nb][nh][sq][words]: bit j of word w of row i = key 64w+j
  const int32_t* kv_count;  // [nb][nh][nqb]
  const int32_t* kv_list;   // [nb][nh][nqb][nkb]: 2*kb + partial, increasing kb
  const int32_t* q_count;   // [nb][nh][nkb]
  const int32_t* q_list;    // [nb][nh][nkb][nqb]: 2*qb + partial, increasing qb
  int32_t nb, nh;           // 1 = shared over batch / q heads
  int32_t nqb, nkb, words;
};

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
  int32_t uniform;   // padded layout, no block mask, and every query row may see all sk keys
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
  BlockMaskP bm;
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
  const float* descale_q;  // FP8 inputs: value = code * descale (null: 1)
  const float* descale_k;
  const float* descale_v;
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
  // dK/dV blocks split in two over their (q head, q tile) items (GQA): fp32 partial sums of
  // each half and a per-block counter (zeroed by the pre-pass); nsplit = 1: no split
  int32_t nsplit;
  int32_t split_blocks;  // dK/dV blocks (counters)
  int32_t* split_cnt;
  float* split_part;
  // THD, separate dK/dV launch: the first *ksplit_count items of work_k (the longest) run as
  // two half blocks each, whose fp32 partial sums a combine launch adds; ksplit_cap = 0: none
  int32_t ksplit_cap;          // most items split (the partial-sum slots)
  const int32_t* ksplit_count;
  float* ksplit_part;          // [slot][kv head][half][{dK, dV} 128 keys x D, register order]
};

struct MergeParams {
  int64_t rows;          // batch * heads * seqlen, or heads * total
  int32_t batch, seqlen, heads, d, thd;
  const int32_t* cu;     // THD with a sequence map: cu_seqlens [nseq + 1] (else null)
  const int32_t* pad;    // ... and sequence row starts (null: cu)
  int32_t nseq;
  View xa, xb, x, g, dxa, dxb;
  StatView la, lb, l, glse, dla, dlb;
  int32_t aligned;       // all x-like row starts 16-byte aligned
};

// Block-table builder (sdpa_block_mask_build).
struct BmBuildParams {
  const uint64_t* bits;
  int32_t* kv_count;
  int32_t* kv_list;
  int32_t* q_count;
  int32_t* q_list;
  int64_t planes;
  int32_t sq, sk, nqb, nkb, words;
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
  // split count (split_cap > 0): the number of items, at most split_cap, whose cost exceeds
  // the mean cost per work slot, total cost x split_heads / split_slots
  int32_t split_cap, split_heads, split_slots;
  int32_t* nsplit;
};

}  // namespace sdpa
