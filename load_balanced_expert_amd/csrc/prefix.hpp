// Device-side prefix sums shared by the route and dispatch kernels: the last
// workgroup of a grid turns per-chunk expert counts into the quantities that
// capacity slots need ([Switch review] "Expert Capacity와 토큰 드롭"):
//   kept_j            = min(c_j, capacity)
//   expert_offsets    = exclusive scan of kept_j over experts (+ total)
//   super_prefix[s,j] = Σ_{c < s*sup} chunk_counts[c, j]   (chunks grouped by sup)
// A chunk's base for expert j is then super_prefix[c/sup, j] plus at most
// sup-1 chunk counts, so no grid-wide serial scan is needed.
#pragma once
#include "common.hpp"

namespace moe {

struct PrefixArgs {
  const int32_t* chunk_counts;  // [nch, n]
  int nch, sup, n;
  int32_t capacity;
  int32_t* expert_offsets;      // [n + 1]
  int32_t* super_prefix;        // [ceil(nch / sup), n]
};

inline int super_chunk(int nch) {  // chunks per super chunk: at most 16 super chunks
  return nch <= 16 ? 1 : (nch + 15) / 16;
}

// Exclusive scan of v[0..n) held in LDS (n <= 4096) by one workgroup of
// `threads` threads into out[0..n] (global); fixed order, deterministic.
__device__ __forceinline__ void block_exclusive_scan(const int* v, int n, int32_t* out, int* part, int threads) {
  const int per = ceil_div(n, threads);
  const int j0 = threadIdx.x * per;
  int s = 0;
  for (int j = j0; j < min(j0 + per, n); ++j) s += v[j];
  // wave-level inclusive scan of the per-thread sums, then across waves
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) part[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < threads / 64; ++w) {
      const int t = part[w];
      part[w] = run;
      run += t;
    }
    out[n] = run;
  }
  __syncthreads();
  int run = part[wave] + incl - s;
  for (int j = j0; j < min(j0 + per, n); ++j) {
    out[j] = run;
    run += v[j];
  }
  __syncthreads();
}

// Runs in the last workgroup.  cnt: per-expert totals in LDS (overwritten with
// kept counts); part: LDS scratch of threads/64 ints.
__device__ __forceinline__ void dispatch_prefix(const PrefixArgs& p, int* cnt, int* part, int threads) {
  for (int j = threadIdx.x; j < p.n; j += threads) cnt[j] = min(cnt[j], p.capacity);
  __syncthreads();
  block_exclusive_scan(cnt, p.n, p.expert_offsets, part, threads);
  const int nsup = ceil_div(p.nch, p.sup);
  for (int q = threadIdx.x; q < nsup * p.n; q += threads) {
    const int s = q / p.n, j = q - s * p.n;
    int sum = 0;
    const int c1 = min(p.nch, (s + 1) * p.sup);
    for (int c = s * p.sup; c < c1; ++c)
      sum += __hip_atomic_load(p.chunk_counts + int64_t(c) * p.n + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    p.super_prefix[int64_t(s) * p.n + j] = sum;
  }
  __syncthreads();
  for (int j = threadIdx.x; j < p.n; j += threads) {
    int run = 0;
    for (int s = 0; s < nsup; ++s) {
      int32_t* q = p.super_prefix + int64_t(s) * p.n + j;
      const int v = *q;
      *q = run;
      run += v;
    }
  }
}

}  // namespace moe
