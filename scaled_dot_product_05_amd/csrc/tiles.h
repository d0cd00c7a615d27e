// Tile sizes shared by the host (grid sizing, THD work-list bounds) and the kernels.
#pragma once

namespace sdpa {

constexpr int kWaves = 4;              // waves per workgroup
constexpr int kThreads = 64 * kWaves;  // threads per workgroup

// forward: one workgroup owns the query rows of its waves (32 per wave) of one (batch, q head)
constexpr int kFwdBM = 128;  // fp32
constexpr int kFwdBM16 = 32 * kWaves;
constexpr int kFwdBN16 = 64;       // keys per K/V tile, 16-bit inputs, head_dim 32
constexpr int kFwdBN16_D64 = 64;   // keys per tile and minimum workgroups per CU of the
constexpr int kFwdMinB_D64 = 2;    // register-staged 16-bit kernel, head_dim 64
constexpr int kFwdBN16_D128 = 64;  // ... and head_dim 128
constexpr int kFwdMinB_D128 = 2;
constexpr int kFwdBN32 = 32;       // keys per K/V tile, fp32 inputs
constexpr int kFwdBNP = 64;        // keys per K/V tile, pipelined 16-bit kernel
constexpr int kFwdStages = 3;      // K/V LDS slots, head_dim <= 64
constexpr int kFwdStagesD128 = 2;  // K/V LDS slots, head_dim 128
constexpr int kXcds = 8;  // workgroups go to the XCDs round-robin by block index
// causal/window forward grids with more than this many pairs per XCD: the XCD takes its
// pairs in groups of this many, tiles longest first within a group
constexpr int kFwdHeadGroup = 4;
// queries per sequence up to which every wave of the 16-bit forward is a work unit of its own
// (32 query rows of one (sequence, q head))
constexpr int kFwdShortRows = 32;
constexpr int kFwdShortMinB = 3;  // its workgroups per CU, head_dim <= 64

// backward dQ: one workgroup owns kBwdQ16 (16-bit) or kBwdQ32 (fp32) query rows; keys stream
// in kBwdQInner tiles (16-bit) or 32-key tiles (fp32)
constexpr int kBwdQ16 = 64;
constexpr int kBwdQ32 = 128;
// dQ rows per tile of the separate four-wave dQ launch
constexpr int kBwdQ16Wide = 128;
constexpr int kBwdQInner = 64;
// backward dK/dV: one workgroup owns kBwdK16 / kBwdK32 keys of one (batch, kv head); query
// rows of every head of the group stream in kBwdKInner tiles (16-bit) or 32-row tiles (fp32)
constexpr int kBwdK16 = 64;
constexpr int kBwdK32 = 128;
// keys per workgroup of the separate four-wave dK/dV launch
constexpr int kBwdK16Wide = 128;
// fused-launch blocks (dK/dV plus dQ, 64-row tiles) per CU above which the backward runs as
// the two four-wave launches
constexpr int kBwdWideMinPerCU = 12;
constexpr int kBwdKInner = 64;

// backward: queries and keys per sequence up to which every wave is a work unit of its own
// (head_dim <= 64)
constexpr int kBwdShortRows = 32;

// backward: GQA dK/dV blocks of the fused 16-bit kernel run as two halves when the grid has
// at most this many blocks per CU
constexpr int kBwdSplitPerCU = 8;
// head_dim 128 backward, causal/window grids: kv heads per group of the XCD order
constexpr int kBwdHeadGroup = 4;

// THD scheduler buckets (costs above the last bucket share it)
constexpr int kSchedBuckets = 4096;

}  // namespace sdpa
