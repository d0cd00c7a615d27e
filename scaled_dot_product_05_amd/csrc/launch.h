// Host-side launch functions defined next to their kernels.
#pragma once
#include <hip/hip_runtime_api.h>

#include "params.h"

namespace sdpa {

// A dispatch carries its grid size in work-items as a 32-bit value, so blocks x threads must
// stay below 2^32 (a larger grid would be cut short, not refused).
constexpr int64_t kMaxGridItems = 0xffffffffLL;
inline bool grid_fits(int64_t blocks, int threads) {
  return blocks >= 0 && threads > 0 && blocks <= kMaxGridItems / threads;
}
// Grids of the kernels that take a few rows per workgroup and loop over the rest.
constexpr int64_t kMaxRowBlocks = int64_t(1) << 20;

hipError_t launch_schedule(const SchedParams& p, hipStream_t stream);
// two lists in one launch (one workgroup each)
hipError_t launch_schedule2(const SchedParams& a, const SchedParams& b, hipStream_t stream);
// Context parallelism over THD: per chunk c of 2 cp, the per-sequence row starts and the
// prefix of chunk lengths (out: int32 [2 cp][2][batch + 1]: starts, then prefix).
hipError_t launch_cp_chunks(const int32_t* cu, const int32_t* padded, int32_t batch, int64_t total,
                            int32_t cp, int32_t* out, hipStream_t stream);
hipError_t launch_fwd(const FwdParams& p, DType dtype, hipStream_t stream);
// FP8 (E4M3) q, k, v with per-tensor descales, bf16 O
hipError_t launch_fwd8(const FwdParams& p, hipStream_t stream);
bool fwd8_ok(const FwdParams& p);
hipError_t launch_bwd(const BwdParams& p, DType dtype, hipStream_t stream);
// Query rows per dQ tile (and THD dQ work item) of the kernels launch_bwd picks for p
// (strides, alignment, head_dim, block mask and split set).
int bwd_q_tile_rows(const BwdParams& p, DType dtype);
// Keys per dK/dV tile (and THD dK/dV work item), likewise.
int bwd_k_tile_rows(const BwdParams& p, DType dtype);
// THD items of the separate dK/dV launch that may run as two halves (0: none), given the
// partial-sum slots the workspace holds in p.ksplit_cap.
int bwd_k_split_cap(const BwdParams& p, DType dtype);
// Compute units of the current device (0 if unknown), cached per device.
int device_cus();
hipError_t launch_merge_fwd(const MergeParams& p, DType dtype, hipStream_t stream);
hipError_t launch_merge_bwd(const MergeParams& p, DType dtype, hipStream_t stream);
hipError_t launch_block_mask_build(const BmBuildParams& p, hipStream_t stream);
// Whether the kernels chosen for these parameters take a block-sparse mask.
bool fwd_block_mask_ok(const FwdParams& p, DType dtype);
bool bwd_block_mask_ok(const BwdParams& p, DType dtype);

}  // namespace sdpa
