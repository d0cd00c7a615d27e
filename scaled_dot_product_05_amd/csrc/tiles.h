// Tile sizes shared by the host (grid sizing, THD work-list bounds) and the kernels.
#pragma once

namespace sdpa {

constexpr int kWaves = 4;              // waves per workgroup
constexpr int kThreads = 64 * kWaves;  // threads per workgroup

// forward: one workgroup owns kFwdBM query rows (32 per wave) of one (batch, q head)
constexpr int kFwdBM = 128;
constexpr int kFwdBN16 = 64;  // keys per K/V tile, 16-bit inputs
constexpr int kFwdBN32 = 32;  // keys per K/V tile, fp32 inputs

// backward dQ: one workgroup owns kBwdQ query rows (32 per wave); keys stream in kBwdQInner tiles
constexpr int kBwdQ = 128;
constexpr int kBwdQInner = 64;
// backward dK/dV: one workgroup owns kBwdK keys (32 per wave) of one (batch, kv head);
// query rows of every head of the group stream in kBwdKInner tiles
constexpr int kBwdK = 128;
constexpr int kBwdKInner = 64;

// THD scheduler buckets (costs above the last bucket share it)
constexpr int kSchedBuckets = 4096;

}  // namespace sdpa
