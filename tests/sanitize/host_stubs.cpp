// Host-only stand-ins for the kernel launchers and kernel-choice predicates, so that the C-ABI
// entry points (api.cpp, cp.cpp) link into a host library built with AddressSanitizer and
// UndefinedBehaviorSanitizer for the validation tests.  Validation never launches anything:
// every launcher reports an error, and the predicates of the block-mask and FP8 paths say
// "unsupported" (those paths are not what the sanitizer run checks).
#include <hip/hip_runtime_api.h>

#include "../../scaled_dot_product_05_amd/csrc/launch.h"

namespace sdpa {

hipError_t launch_schedule(const SchedParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_schedule2(const SchedParams&, const SchedParams&, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_cp_chunks(const int32_t*, const int32_t*, int32_t, int64_t, int32_t, int32_t*,
                            hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_fwd(const FwdParams&, DType, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fwd8(const FwdParams&, hipStream_t) { return hipErrorNotSupported; }
bool fwd8_ok(const FwdParams&) { return false; }
hipError_t launch_bwd(const BwdParams&, DType, hipStream_t) { return hipErrorNotSupported; }
int bwd_q_tile_rows(const BwdParams&, DType) { return 64; }
int bwd_k_tile_rows(const BwdParams&, DType) { return 64; }
int bwd_k_split_cap(const BwdParams&, DType) { return 0; }
hipError_t launch_merge_fwd(const MergeParams&, DType, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_merge_bwd(const MergeParams&, DType, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_block_mask_build(const BmBuildParams&, hipStream_t) { return hipErrorNotSupported; }
bool fwd_block_mask_ok(const FwdParams&, DType) { return false; }
bool bwd_block_mask_ok(const BwdParams&, DType) { return false; }

}  // namespace sdpa
