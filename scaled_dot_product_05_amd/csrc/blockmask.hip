// Block table of a block-sparse mask (FlexAttention's BlockMask model).
//
// "Significant Accuracy Difference between Compiled and Eager Flex Attention" (PyTorch
// issue 135161, second repro) builds its sliding-window and global masks with
// create_block_mask from predicates over (q_idx, kv_idx).  Here the predicate arrives
// evaluated, as one bit per (query, key), and this file classifies every 128 x 128 block
// of the (Sq, Sk) plane over the pairs inside the plane: no bit set (skipped), every bit
// set (full: no element test), or mixed (partial).  It then writes each block row's list
// (kv_count, kv_list: 2 kb + partial in increasing kb) and each block column's list
// (q_count, q_list: 2 qb + partial in increasing qb).
//
// Two launches.  The row kernel reads every mask word once (a workgroup per block row,
// 64 block columns per pass, four row groups per column), compacts the row list with a
// ballot scan and parks each block's kind in q_list[kb][qb].  The column kernel then
// compacts every column of q_list in place (an entry only moves to a lower index, and a
// pass reads its whole chunk before it writes).
#include "device.h"
#include "launch.h"
#include "profile.h"

namespace sdpa {

// bits of word w that belong to keys < sk
__device__ __forceinline__ uint64_t valid_bits(int sk, int w) {
  const int lo = 64 * w;
  if (lo + 64 <= sk) return ~0ull;
  if (sk <= lo) return 0ull;
  return (1ull << (sk - lo)) - 1ull;
}

__global__ __launch_bounds__(256) void bm_rows_kernel(BmBuildParams p) {
  const int qb = int(blockIdx.x % unsigned(p.nqb));
  const int64_t plane = int64_t(blockIdx.x / unsigned(p.nqb));
  const int tid = threadIdx.x, c = tid & 63, grp = tid >> 6;
  const int r0 = qb * kMaskBlock, r1 = min(r0 + kMaskBlock, p.sq);
  const uint64_t* rows = p.bits + plane * p.sq * int64_t(p.words);
  int32_t* kvl = p.kv_list + (plane * p.nqb + qb) * int64_t(p.nkb);
  __shared__ uint32_t s_any[4][64], s_all[4][64];
  int base = 0;  // entries written so far (wave 0)
  for (int kb0 = 0; kb0 < p.nkb; kb0 += 64) {
    const int kb = kb0 + c;
    bool any = false, all = true;
    if (kb < p.nkb) {
      const int w0 = 2 * kb, w1 = 2 * kb + 1;
      const uint64_t v0 = valid_bits(p.sk, w0), v1 = w1 < p.words ? valid_bits(p.sk, w1) : 0ull;
      for (int r = r0 + grp; r < r1; r += 4) {
        const uint64_t* wr = rows + int64_t(r) * p.words;
        const uint64_t a = wr[w0] & v0;
        const uint64_t b = w1 < p.words ? (wr[w1] & v1) : 0ull;
        any = any || (a | b) != 0ull;
        all = all && a == v0 && b == v1;
      }
    }
    s_any[grp][c] = any;
    s_all[grp][c] = all;
    __syncthreads();
    if (grp == 0) {
      const bool A = s_any[0][c] | s_any[1][c] | s_any[2][c] | s_any[3][c];
      const bool L = s_all[0][c] & s_all[1][c] & s_all[2][c] & s_all[3][c];
      const int kind = kb < p.nkb ? (!A ? 0 : L ? 1 : 2) : 0;
      const uint64_t bal = __builtin_amdgcn_ballot_w64(kind != 0);
      const int pos = base + __popcll(bal & ((1ull << c) - 1ull));
      if (kind != 0) kvl[pos] = 2 * kb + (kind == 2 ? 1 : 0);
      if (kb < p.nkb) p.q_list[(plane * p.nkb + kb) * int64_t(p.nqb) + qb] = kind;
      base += __popcll(bal);
    }
    __syncthreads();
  }
  if (tid == 0) p.kv_count[plane * p.nqb + qb] = base;
}

__global__ __launch_bounds__(256) void bm_cols_kernel(BmBuildParams p) {
  const int kb = int(blockIdx.x % unsigned(p.nkb));
  const int64_t plane = int64_t(blockIdx.x / unsigned(p.nkb));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t* col = p.q_list + (plane * p.nkb + kb) * int64_t(p.nqb);
  __shared__ int s_cnt[4];
  int base = 0;
  for (int qb0 = 0; qb0 < p.nqb; qb0 += 256) {
    const int qb = qb0 + tid;
    const int kind = qb < p.nqb ? col[qb] : 0;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(kind != 0);
    if (lane == 0) s_cnt[wave] = __popcll(bal);
    __syncthreads();  // every read of this chunk precedes every write
    int off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      off += w < wave ? s_cnt[w] : 0;
      tot += s_cnt[w];
    }
    if (kind != 0) col[base + off + __popcll(bal & ((1ull << lane) - 1ull))] = 2 * qb + (kind == 2 ? 1 : 0);
    base += tot;
    __syncthreads();  // s_cnt reuse
  }
  if (tid == 0) p.q_count[plane * p.nkb + kb] = base;
}

hipError_t launch_block_mask_build(const BmBuildParams& p, hipStream_t st) {
  if (!grid_fits(int64_t(p.planes) * p.nqb, 256) || !grid_fits(int64_t(p.planes) * p.nkb, 256))
    return hipErrorInvalidConfiguration;
  prof_begin(st, "mask_rows");
  hipLaunchKernelGGL(bm_rows_kernel, dim3(unsigned(p.planes * p.nqb)), dim3(256), 0, st, p);
  prof_end(st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_begin(st, "mask_cols");
  hipLaunchKernelGGL(bm_cols_kernel, dim3(unsigned(p.planes * p.nkb)), dim3(256), 0, st, p);
  prof_end(st);
  return hipGetLastError();
}

}  // namespace sdpa
