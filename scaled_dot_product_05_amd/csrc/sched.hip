// Varlen (THD) scheduler: turns device cu_seqlens into a work list of (sequence, tile)
// items, most expensive first, so that the long causal tiles of the long sequences start
// before the short ones fill the machine.  Packed THD sequences with int32 cu_seqlens come
// from "Add support for cuDNN FusedAttention + THD + CP" (TransformerEngine issue 885).
//
// One workgroup: histogram of item costs (cost = number of tiles on the other side that
// the window lets the item see), an exclusive scan of the histogram from the most to the
// least expensive bucket, then a scatter through LDS atomic counters.  The order inside a
// bucket does not matter: every item writes its own output rows.
#include "device.h"
#include "launch.h"
#include "profile.h"

namespace sdpa {

constexpr int kSchedThreads = 1024;

struct SeqLens {
  int own, other, off;  // lengths and the diagonal offset of this sequence
};

__device__ __forceinline__ SeqLens sched_lens(const SchedParams& p, int b) {
  int64_t a0 = clamp64(p.cu_own[b], 0, p.total_own);
  int64_t a1 = clamp64(p.cu_own[b + 1], a0, p.total_own);
  int64_t c0 = clamp64(p.cu_other[b], 0, p.total_other);
  int64_t c1 = clamp64(p.cu_other[b + 1], c0, p.total_other);
  SeqLens r;
  r.own = int(min<int64_t>(a1 - a0, p.max_own));
  r.other = int(min<int64_t>(c1 - c0, p.max_other));
  int sq = p.own_is_query ? r.own : r.other;
  int sk = p.own_is_query ? r.other : r.own;
  r.off = p.bottom_right ? sk - sq : 0;
  return r;
}

__device__ __forceinline__ int item_cost(const SchedParams& p, const SeqLens& L, int t) {
  int r0 = t * p.tile_own;
  int r1 = min(r0 + p.tile_own, L.own);
  int64_t lo, hi;
  if (p.own_is_query) {  // keys seen by query rows [r0, r1)
    lo = int64_t(r0) + L.off + p.lo_rel;
    hi = int64_t(r1 - 1) + L.off + p.hi_rel + 1;
  } else {  // queries that see key rows [r0, r1)
    lo = int64_t(r0) - L.off - p.hi_rel;
    hi = int64_t(r1 - 1) - L.off - p.lo_rel + 1;
  }
  lo = clamp64(lo, 0, L.other);
  hi = clamp64(hi, lo, L.other);
  if (hi <= lo) return 0;
  int64_t c = (hi + p.tile_other - 1) / p.tile_other - lo / p.tile_other;
  return int(min<int64_t>(c, kSchedBuckets - 1));
}

// Workgroup b builds list b (the backward's query-tile and key-tile lists in one launch).
struct SchedPair {
  SchedParams p[2];
};

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(SchedPair pp) {
  const SchedParams& p = pp.p[blockIdx.x];
  __shared__ int hist[kSchedBuckets];
  __shared__ int part[2 * (kSchedThreads / 64) + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int nwaves = kSchedThreads / 64;
  constexpr int PER = kSchedBuckets / kSchedThreads;
  __shared__ unsigned long long total_cost;
  __shared__ int max_cost, split_at;
  for (int i = tid; i < kSchedBuckets; i += kSchedThreads) hist[i] = 0;
  if (tid == 0) {
    total_cost = 0;
    max_cost = 0;
    split_at = 0;
  }
  __syncthreads();
  unsigned long long my_sum = 0;
  int my_max = 0;
  for (int b = wave; b < p.batch; b += nwaves) {
    SeqLens L = sched_lens(p, b);
    int nt = (L.own + p.tile_own - 1) / p.tile_own;
    for (int t = lane; t < nt; t += 64) {
      const int c = item_cost(p, L, t);
      atomicAdd(&hist[c], 1);
      if (p.split_cap > 0) {
        my_sum += unsigned(c);
        my_max = max(my_max, c);
      }
    }
  }
  if (p.split_cap > 0) {  // total and largest cost: wave sums, one LDS atomic per wave
    for (int o = 32; o > 0; o >>= 1) {
      my_sum += __shfl_xor(my_sum, o);
      my_max = max(my_max, __shfl_xor(my_max, o));
    }
    if (lane == 0) {
      atomicAdd(&total_cost, my_sum);
      atomicMax(&max_cost, my_max);
    }
  }
  __syncthreads();
  // Split items: those of cost above the mean per work slot, thr, when the largest cost
  // exceeds 1.5 thr (below that the tail of the unsplit list costs less than the halves'
  // partial sums and their combine); they are the list's first split_at entries.
  int64_t thr = kSchedBuckets;
  if (p.split_cap > 0 && p.split_slots > 0) {
    thr = int64_t(total_cost) * p.split_heads / p.split_slots;
    if (int64_t(max_cost) * 10 <= thr * 15) thr = kSchedBuckets;
  }
  // exclusive scan in decreasing cost order: thread i owns reversed buckets PER*i .. PER*i+PER-1;
  // an inclusive scan inside each wave, then one over the wave totals in wave 0
  int local = 0;
  for (int k = 0; k < PER; ++k) local += hist[kSchedBuckets - 1 - (PER * tid + k)];
  int incl = local;
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) part[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int t = lane < nwaves ? part[lane] : 0;
    int x = t;
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d);
      if (lane >= d) x += y;
    }
    if (lane < nwaves) part[nwaves + lane] = x - t;  // items before wave `lane`
    if (lane == nwaves - 1) part[2 * nwaves] = x;
  }
  __syncthreads();
  int run = part[nwaves + wave] + incl - local;  // exclusive prefix of this thread's first bucket
  const int total = part[2 * nwaves];
  for (int k = 0; k < PER; ++k) {
    int c = kSchedBuckets - 1 - (PER * tid + k);
    int n = hist[c];
    hist[c] = run;  // becomes the next free slot of bucket c
    if (c == thr) split_at = run;  // items of cost above thr come before bucket thr
    run += n;
  }
  __syncthreads();
  // the first ns items appear twice, as halves 0 and 1 (tile | (half + 1) << 24), then the rest
  const int ns = p.split_cap > 0 ? min(split_at, p.split_cap) : 0;
  if (tid == 0 && p.nsplit) *p.nsplit = ns;
  for (int b = wave; b < p.batch; b += nwaves) {
    SeqLens L = sched_lens(p, b);
    int nt = (L.own + p.tile_own - 1) / p.tile_own;
    for (int t = lane; t < nt; t += 64) {
      const int pos = atomicAdd(&hist[item_cost(p, L, t)], 1);
      WorkItem it;
      it.seq = b;
      if (pos < ns) {
        it.tile = t | (1 << 24);
        p.items[2 * pos] = it;
        it.tile = t | (2 << 24);
        p.items[2 * pos + 1] = it;
      } else if (pos + ns < p.max_items) {
        it.tile = t;
        p.items[pos + ns] = it;
      }
    }
  }
  if (tid == 0) *p.count = min(total + ns, p.max_items);
}

hipError_t launch_schedule(const SchedParams& p, hipStream_t st) {
  prof_begin(st, "thd_schedule");
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, st, SchedPair{{p, p}});
  prof_end(st);
  return hipGetLastError();
}

hipError_t launch_schedule2(const SchedParams& a, const SchedParams& b, hipStream_t st) {
  prof_begin(st, "thd_schedule");
  hipLaunchKernelGGL(schedule_kernel, dim3(2), dim3(kSchedThreads), 0, st, SchedPair{{a, b}});
  prof_end(st);
  return hipGetLastError();
}

// Context parallelism over THD ("Add support for cuDNN FusedAttention + THD + CP",
// TransformerEngine issue 885: every sequence of a packed batch is cut into 2 cp chunks).
// Chunk c of a sequence of length L is rows [floor(c L / 2cp), floor((c+1) L / 2cp)) of it,
// so a query chunk and the key chunk of the same index cover the same rows.  Thread c
// writes, for every sequence, the packed row where its chunk c starts (from the padded
// starts if given) and the prefix sum of the chunk lengths: a padded-THD view of chunk c of
// every sequence at once.  Entries are clamped to [0, total].
__global__ __launch_bounds__(128) void cp_chunks_kernel(const int32_t* cu, const int32_t* padded,
                                                       int32_t batch, int64_t total, int32_t cp,
                                                       int32_t* out) {
  const int c = threadIdx.x, n = 2 * cp;
  if (c >= n) return;
  int32_t* start = out + int64_t(c) * 2 * (batch + 1);
  int32_t* pre = start + (batch + 1);
  auto at = [&](const int32_t* a, int i) { return int64_t(min(max(int64_t(a[i]), int64_t(0)), total)); };
  int64_t acc = 0;
  pre[0] = 0;
  for (int b = 0; b < batch; ++b) {
    const int64_t len = max(at(cu, b + 1) - at(cu, b), int64_t(0));
    const int64_t lo = int64_t(c) * len / n, hi = int64_t(c + 1) * len / n;
    start[b] = int32_t(min(at(padded ? padded : cu, b) + lo, total));
    acc += hi - lo;
    pre[b + 1] = int32_t(min(acc, total));
  }
  start[batch] = int32_t(total);
}

hipError_t launch_cp_chunks(const int32_t* cu, const int32_t* padded, int32_t batch, int64_t total,
                            int32_t cp, int32_t* out, hipStream_t st) {
  prof_begin(st, "cp_chunks");
  hipLaunchKernelGGL(cp_chunks_kernel, dim3(1), dim3(128), 0, st, cu, padded, batch, total, cp, out);
  prof_end(st);
  return hipGetLastError();
}

}  // namespace sdpa
