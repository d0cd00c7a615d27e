// Launch-timing hooks used by the kernel launchers (no-ops unless enabled through
// sdpa_profile_enable).
#pragma once
#include <hip/hip_runtime_api.h>

namespace sdpa {

void prof_begin(hipStream_t stream, const char* kernel);
void prof_end(hipStream_t stream);

}  // namespace sdpa
