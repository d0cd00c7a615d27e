// Tile sizes shared by the host (grid sizing, THD work-list bounds) and the kernels.
#pragma once

namespace sdpa {

constexpr int kWaves = 4;              // waves per workgroup
constexpr int kThreads = 64 * kWaves;  // threads per workgroup

// forward: one workgroup owns the query rows of its waves (32 per wave) of one (batch, q head)
constexpr int kFwdBM = 128;  // fp32
#ifndef SDPA_FWD_BN_D64
#define SDPA_FWD_BN_D64 64
#endif
#ifndef SDPA_FWD_MINB_D64
#define SDPA_FWD_MINB_D64 2
#endif
#ifndef SDPA_FWD_BN_D128
#define SDPA_FWD_BN_D128 64
#endif
#ifndef SDPA_FWD_MINB_D128
#define SDPA_FWD_MINB_D128 2
#endif
constexpr int kFwdBM16 = 32 * kWaves;
constexpr int kFwdBN16 = 64;         // keys per K/V tile, 16-bit inputs, head_dim 32
constexpr int kFwdBN16_D64 = SDPA_FWD_BN_D64;    // keys per tile and minimum workgroups
constexpr int kFwdMinB_D64 = SDPA_FWD_MINB_D64;  // per CU, head_dim 64
constexpr int kFwdBN16_D128 = SDPA_FWD_BN_D128;
constexpr int kFwdMinB_D128 = SDPA_FWD_MINB_D128;
constexpr int kFwdBN32 = 32;  // keys per K/V tile, fp32 inputs
#ifndef SDPA_FWD_BNP
#define SDPA_FWD_BNP 64
#endif
constexpr int kFwdBNP = SDPA_FWD_BNP;  // keys per K/V tile, pipelined 16-bit kernel
#ifndef SDPA_FWD_NS
#define SDPA_FWD_NS 3
#endif
#ifndef SDPA_FWD_NS_D128
#define SDPA_FWD_NS_D128 2
#endif
constexpr int kFwdStages = SDPA_FWD_NS;            // K/V LDS slots, head_dim <= 64
#ifndef SDPA_FWD_XCD_ORDER
#define SDPA_FWD_XCD_ORDER 1
#endif
constexpr int kXcds = 8;  // workgroups go to the XCDs round-robin by block index
// padded-layout forward grids: each XCD walks its own (batch, head) pairs one after the
// other (0: q tile outermost, (batch, head) fastest)
constexpr bool kFwdXcdOrder = SDPA_FWD_XCD_ORDER;
#ifndef SDPA_FWD_HEAD_GROUP
#define SDPA_FWD_HEAD_GROUP 4
#endif
// causal/window forward grids with more than this many pairs per XCD: the XCD takes its
// pairs in groups of this many, tiles longest first within a group (0: one group)
constexpr int kFwdHeadGroup = SDPA_FWD_HEAD_GROUP;
constexpr int kFwdStagesD128 = SDPA_FWD_NS_D128;  // K/V LDS slots, head_dim 128
#ifndef SDPA_FWD_WIDE_D64
#define SDPA_FWD_WIDE_D64 0
#endif
#ifndef SDPA_FWD_WIDE_MIN
#define SDPA_FWD_WIDE_MIN 1024
#endif
constexpr bool kFwdWideD64 = SDPA_FWD_WIDE_D64;      // 64 query rows per wave, head_dim 64
constexpr int kFwdWideMinBlocks = SDPA_FWD_WIDE_MIN;  // ... when the grid has this many blocks
#ifndef SDPA_FWD_SHORT_ROWS
#define SDPA_FWD_SHORT_ROWS 32
#endif
// queries per sequence up to which every wave of the 16-bit forward is a work unit of its own
// (32 query rows of one (sequence, q head)); 0 turns that kernel off
constexpr int kFwdShortRows = SDPA_FWD_SHORT_ROWS;
#ifndef SDPA_FWD_SHORT_MINB
#define SDPA_FWD_SHORT_MINB 3
#endif
constexpr int kFwdShortMinB = SDPA_FWD_SHORT_MINB;  // its workgroups per CU, head_dim <= 64

// backward dQ: one workgroup owns kBwdQ16 (16-bit) or kBwdQ32 (fp32) query rows; keys stream
// in kBwdQInner tiles (16-bit) or 32-key tiles (fp32)
constexpr int kBwdQ16 = 64;
constexpr int kBwdQ32 = 128;
constexpr int kBwdQInner = 64;
// backward dK/dV: one workgroup owns kBwdK16 / kBwdK32 keys of one (batch, kv head); query
// rows of every head of the group stream in kBwdKInner tiles (16-bit) or 32-row tiles (fp32)
constexpr int kBwdK16 = 64;
constexpr int kBwdK32 = 128;
constexpr int kBwdKInner = 64;

// backward: queries and keys per sequence up to which every wave is a work unit of its own
// (head_dim <= 64); 0 turns that kernel off
#ifndef SDPA_BWD_SHORT_ROWS
#define SDPA_BWD_SHORT_ROWS 32
#endif
constexpr int kBwdShortRows = SDPA_BWD_SHORT_ROWS;

// backward: GQA dK/dV blocks of the fused 16-bit kernel run as two halves (0: off)
#ifndef SDPA_BWD_SPLIT
#define SDPA_BWD_SPLIT 1
#endif
constexpr int kBwdSplit = SDPA_BWD_SPLIT;
constexpr int kBwdSplitPerCU = 8;  // ... when the grid has at most this many blocks per CU
#ifndef SDPA_BWD_XCD_ORDER
#define SDPA_BWD_XCD_ORDER 1
#endif
// padded-layout backward grids: each XCD owns a contiguous range of (batch, head) pairs
// (0: tile outermost, (batch, head) fastest)
constexpr bool kBwdXcdOrder = SDPA_BWD_XCD_ORDER;
#ifndef SDPA_BWD_HEAD_GROUP
#define SDPA_BWD_HEAD_GROUP 4
#endif
// head_dim 128 backward, causal/window grids: kv heads per group of the XCD order (0: none)
constexpr int kBwdHeadGroup = SDPA_BWD_HEAD_GROUP;

// THD scheduler buckets (costs above the last bucket share it)
constexpr int kSchedBuckets = 4096;

}  // namespace sdpa
