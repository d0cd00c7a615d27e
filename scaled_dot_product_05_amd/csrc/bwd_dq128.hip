// The separate-launch dQ kernels at head_dim 128 (bf16 and fp16), in a translation unit of their
// own so that they can be built with the machine scheduler's max-ilp strategy: it takes these
// kernels 2-3% down (varlen THD GQA 308 -> 303 us, B8 S4096 H16/4 765 -> 749 us), while the
// default strategy suits every other kernel of bwd.hip (max-ilp costs the head_dim 128 dK/dV
// launch 5% and the forward 1%).
#define SDPA_BWD_KERNELS_ONLY
#include "bwd.hip"

namespace sdpa {
template __global__ void bwd_dq16p_kernel<true, 128, 4, true>(BwdParams);
template __global__ void bwd_dq16p_kernel<false, 128, 4, true>(BwdParams);
}  // namespace sdpa
