// Host-side launch functions defined next to their kernels.
#pragma once
#include <hip/hip_runtime_api.h>

#include "params.h"

namespace sdpa {

hipError_t launch_schedule(const SchedParams& p, hipStream_t stream);
hipError_t launch_fwd(const FwdParams& p, DType dtype, hipStream_t stream);
hipError_t launch_bwd(const BwdParams& p, DType dtype, hipStream_t stream);
hipError_t launch_merge_fwd(const MergeParams& p, DType dtype, hipStream_t stream);
hipError_t launch_merge_bwd(const MergeParams& p, DType dtype, hipStream_t stream);

}  // namespace sdpa
