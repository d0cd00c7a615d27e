// sdpa_bwd_noalloc: the backward for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  It is sdpa_bwd
// with its workspace (Delta, LSE log2(e), the THD work lists and the GQA split's partial
// sums and arrival counters) taken from one static device array instead of the caller.
//
// The array, `scratch`, holds kScratchBytes on every GPU the library runs on, until the
// process ends.  In host code its name is only a stand-in for the symbol: the device address
// comes from hipGetSymbolAddress, once per device (with that device current), and only that
// address is passed on.  Nothing in it has to start at zero: the THD scheduler writes its
// lists and the Delta pre-pass writes Delta, LSE log2(e) and zeroes the split counters on
// every call, before the kernels that read them.  Every call on one GPU uses the same array,
// so calls that overlap on one GPU (different streams, or host threads) race; calls on one
// stream are ordered.
#include <stdio.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/sdpa.h"

namespace sdpa {
int set_error(int code, const char* msg);
int bwd_workspace_min(const sdpa_desc_t* desc, size_t* bytes);
}

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's copy of `scratch` (looked up on first use).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return sdpa::set_error(SDPA_ERR_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return sdpa::set_error(SDPA_ERR_UNSUPPORTED, "sdpa_bwd_noalloc: device index beyond 63");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return sdpa::set_error(SDPA_ERR_HIP, e != hipSuccess ? hipGetErrorString(e)
                                                           : "scratch has no device address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SDPA_OK;
}

}  // namespace

extern "C" {

size_t sdpa_bwd_noalloc_max_workspace(void) { return kScratchBytes; }

int sdpa_bwd_noalloc(const sdpa_desc_t* desc, const sdpa_tensor_t* q, const sdpa_tensor_t* k,
                     const sdpa_tensor_t* v, const sdpa_tensor_t* o, const sdpa_rowstat_t* lse,
                     const sdpa_tensor_t* dout, const sdpa_rowstat_t* dlse,
                     const sdpa_tensor_t* dq, const sdpa_tensor_t* dk, const sdpa_tensor_t* dv,
                     int accumulate, void* stream) {
  // the smallest workspace the backward runs with (room for split THD dK/dV items is used
  // only when the buffer holds it too)
  size_t need = 0;
  int rc = sdpa::bwd_workspace_min(desc, &need);
  if (rc) return rc;
  if (need > kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof(msg),
             "sdpa_bwd_noalloc: this problem needs %zu bytes of workspace, more than the %zu of "
             "the static scratch buffer; call sdpa_bwd with a workspace",
             need, kScratchBytes);
    return sdpa::set_error(SDPA_ERR_WORKSPACE, msg);
  }
  void* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  return sdpa_bwd(desc, q, k, v, o, lse, dout, dlse, dq, dk, dv, accumulate, ws, kScratchBytes,
                  stream);
}

}  // extern "C"
