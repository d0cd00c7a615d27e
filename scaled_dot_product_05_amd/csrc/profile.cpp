// Per-kernel launch timing: hipEvent pairs around each launch while enabled.
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "../../include/sdpa.h"
#include "../../include/sdpa_profile.h"
#include "profile.h"

namespace sdpa {
namespace {

struct Rec {
  const char* name;
  hipEvent_t start, stop;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

void prof_begin(hipStream_t st, const char* name) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  Rec r{name, take_event(), take_event()};
  if (!r.start || !r.stop) return;
  (void)hipEventRecord(r.start, st);
  g_recs.push_back(r);
}

void prof_end(hipStream_t st) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_recs.empty()) (void)hipEventRecord(g_recs.back().stop, st);
}

}  // namespace sdpa

extern "C" {

int sdpa_profile_enable(int on) {
  using namespace sdpa;
  std::lock_guard<std::mutex> lk(g_mu);
  if (on) {
    for (const Rec& r : g_recs) {
      g_pool.push_back(r.start);
      g_pool.push_back(r.stop);
    }
    g_recs.clear();
  }
  g_on.store(on != 0);
  return SDPA_OK;
}

int sdpa_profile_read(char* buf, size_t len) {
  using namespace sdpa;
  std::lock_guard<std::mutex> lk(g_mu);
  std::map<std::string, std::pair<long, double>> agg;
  for (const Rec& r : g_recs) {
    if (hipEventSynchronize(r.stop) != hipSuccess) return SDPA_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return SDPA_ERR_HIP;
    auto& a = agg[r.name];
    a.first += 1;
    a.second += ms;
  }
  std::string out;
  char line[160];
  for (const auto& kv : agg) {
    snprintf(line, sizeof(line), "%s %ld %.6f\n", kv.first.c_str(), kv.second.first, kv.second.second);
    out += line;
  }
  if (buf && len) {
    size_t n = out.size() < len - 1 ? out.size() : len - 1;
    memcpy(buf, out.data(), n);
    buf[n] = 0;
  }
  return SDPA_OK;
}

}  // extern "C"
