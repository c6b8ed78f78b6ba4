// Capacity slots in token order, drop mask, permutation maps and the
// permute-dispatch copy.
//
// [Switch review] "Expert Capacity와 토큰 드롭": capacity = (tokens / experts) x
// capacity factor; overflow tokens skip the expert (residual only).
// [Switch impl] "forward pass에서는 토큰 순서를 두 번 변경한다": tokens of the
// same expert are gathered together; each keeps its gate and capacity slot.
//
// The slot of pair p = (t, r) is its rank among earlier pairs (token-major)
// with the same expert.  Atomic return order is not deterministic, so ranks
// come from counting instead:
//   1. histogram kernel: per-chunk (1024 pairs) expert counts in LDS; the
//      last block turns them into per-chunk exclusive bases (scan over chunks
//      for each expert), clamps totals at the capacity and scans those into
//      the expert offsets;
//   2. rank kernel: inside a chunk, each wave ranks its 64-pair groups with a
//      match-any built from ballots over the expert-id bits; per-wave counts
//      in LDS give the offset of each wave inside the chunk;
//   3. copy kernel: every kept row is copied with 16-byte loads and stores.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kDispThreads = 256;
constexpr int kPairsPerWave = kDispChunk / (kDispThreads / 64);  // 256

size_t dispatch_ws_bytes(int64_t pairs, int n) {
  const int64_t nch = ceil_div64(pairs, kDispChunk);
  return size_t(nch) * n * sizeof(int32_t);
}

__global__ __launch_bounds__(kDispThreads) void k_disp_hist(DispatchArgs a) {
  extern __shared__ int lds[];
  int* hist = lds;                  // [n]
  const int n = a.n;
  const int64_t c = blockIdx.x;
  const int nch = gridDim.x;
  for (int j = threadIdx.x; j < n; j += kDispThreads) hist[j] = 0;
  __syncthreads();
  const int64_t p0 = c * kDispChunk;
  for (int u = 0; u < kDispChunk / kDispThreads; ++u) {
    const int64_t p = p0 + u * kDispThreads + threadIdx.x;
    if (p < a.pairs) {
      const int e = a.idx[p];
      if (unsigned(e) < unsigned(n)) atomicAdd(&hist[e], 1);   // ids outside [0, n) are dropped
    }
  }
  __syncthreads();
  int32_t* cc = a.chunk_counts + c * n;
  for (int j = threadIdx.x; j < n; j += kDispThreads) cc[j] = hist[j];

  // last block: exclusive scan over chunks per expert, capacity clamp, offsets
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = atomicAdd(a.done, 1u) == unsigned(nch) - 1;
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  int* kept = lds;  // reuse: [n]
  for (int j = threadIdx.x; j < n; j += kDispThreads) {
    int run = 0;
    for (int cc2 = 0; cc2 < nch; ++cc2) {
      int32_t* q = a.chunk_counts + int64_t(cc2) * n + j;
      const int v = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *q = run;
      run += v;
    }
    kept[j] = min(run, a.capacity);
  }
  __syncthreads();
  // exclusive scan of kept[0..n) into expert_offsets (n <= 4096: 16 per thread)
  __shared__ int part[kDispThreads];
  const int per = ceil_div(n, kDispThreads);
  const int j0 = threadIdx.x * per;
  int s = 0;
  for (int j = j0; j < min(j0 + per, n); ++j) s += kept[j];
  part[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int t = 0; t < kDispThreads; ++t) {
      const int v = part[t];
      part[t] = run;
      run += v;
    }
    a.expert_offsets[n] = run;
  }
  __syncthreads();
  int run = part[threadIdx.x];
  for (int j = j0; j < min(j0 + per, n); ++j) {
    a.expert_offsets[j] = run;
    run += kept[j];
  }
  if (threadIdx.x == 0) atomicExch(a.done, 0u);
}

__global__ __launch_bounds__(kDispThreads) void k_disp_rank(DispatchArgs a) {
  extern __shared__ uint16_t whist[];   // [4][n] per-wave counts, then per-wave bases
  const int n = a.n;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int j = threadIdx.x; j < 4 * n; j += kDispThreads) whist[j] = 0;
  __syncthreads();
  const int64_t pw = int64_t(blockIdx.x) * kDispChunk + int64_t(wave) * kPairsPerWave;
  uint16_t* wh = whist + wave * n;
  uint64_t peers[kPairsPerWave / 64];
  int ex[kPairsPerWave / 64];
#pragma unroll
  for (int it = 0; it < kPairsPerWave / 64; ++it) {
    const int64_t p = pw + it * 64 + lane;
    const bool inside = p < a.pairs;
    const int e0 = inside ? a.idx[p] : 0;
    const bool valid = inside && unsigned(e0) < unsigned(n);
    const int e = valid ? e0 : 0;
    const uint64_t active = __ballot(valid);
    const uint64_t pr = match_any(uint32_t(e), a.nbits, active);
    ex[it] = e;
    peers[it] = pr;
    if (valid && (pr & lanemask_lt()) == 0) wh[e] = uint16_t(wh[e] + __popcll(pr));
  }
  __syncthreads();
  for (int j = threadIdx.x; j < n; j += kDispThreads) {
    int run = 0;
    for (int w = 0; w < 4; ++w) {
      const int v = whist[w * n + j];
      whist[w * n + j] = uint16_t(run);
      run += v;
    }
  }
  __syncthreads();
  const int32_t* base = a.chunk_counts + int64_t(blockIdx.x) * n;
#pragma unroll
  for (int it = 0; it < kPairsPerWave / 64; ++it) {
    const int64_t p = pw + it * 64 + lane;
    const uint64_t pr = peers[it];
    const bool inside = p < a.pairs;
    const bool valid = inside && (pr >> lane) & 1;
    const int e = ex[it];
    int slot = 0;
    if (valid) slot = base[e] + wh[e] + __popcll(pr & lanemask_lt());
    // every lane has read wh[e] above before the group leader advances it
    __builtin_amdgcn_wave_barrier();
    if (valid && (pr & lanemask_lt()) == 0) wh[e] = uint16_t(wh[e] + __popcll(pr));
    if (inside && !valid) {
      a.token_to_row[p] = -1;
      if (a.drop_mask) a.drop_mask[p] = 1;
    }
    if (valid) {
      const bool kept = slot < a.capacity;
      const int row = kept ? a.expert_offsets[e] + slot : -1;
      a.token_to_row[p] = row;
      if (a.drop_mask) a.drop_mask[p] = kept ? 0 : 1;
      if (kept && a.row_to_token) a.row_to_token[row] = int32_t(p / a.k);
    }
  }
}

template <typename V>
__global__ __launch_bounds__(256) void k_disp_copy(const char* __restrict__ x, char* __restrict__ out,
                                                   const int32_t* __restrict__ row_to_token,
                                                   const int32_t* __restrict__ offsets_end, int64_t vpr,
                                                   int64_t items) {
  const int64_t total_rows = *offsets_end;
  const int64_t limit = min<int64_t>(items, total_rows * vpr);
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < limit; i += int64_t(gridDim.x) * 256) {
    const int64_t row = i / vpr, v = i - row * vpr;
    const int64_t t = row_to_token[row];
    reinterpret_cast<V*>(out)[row * vpr + v] = reinterpret_cast<const V*>(x)[t * vpr + v];
  }
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
  const int nch = int(ceil_div64(a.pairs, kDispChunk));
  hipLaunchKernelGGL(k_disp_hist, dim3(nch), dim3(kDispThreads), a.n * sizeof(int), s, a);
  hipLaunchKernelGGL(k_disp_rank, dim3(nch), dim3(kDispThreads), 4 * a.n * sizeof(uint16_t), s, a);
  if (a.dispatched) {
    int64_t vpr;
    const int64_t items_per_row_16 = a.row_bytes / 16;
    const bool v16 = a.row_bytes % 16 == 0;
    const bool v4 = a.row_bytes % 4 == 0;
    vpr = v16 ? items_per_row_16 : (v4 ? a.row_bytes / 4 : a.row_bytes / 2);
    const int64_t items = a.max_rows * vpr;
    const int64_t blocks = std::min<int64_t>(ceil_div64(items, 256), 16384);
    if (blocks > 0) {
      if (v16)
        hipLaunchKernelGGL(k_disp_copy<u32x4>, dim3(unsigned(blocks)), dim3(256), 0, s,
                           static_cast<const char*>(a.x), static_cast<char*>(a.dispatched), a.row_to_token,
                           a.expert_offsets + a.n, vpr, items);
      else if (v4)
        hipLaunchKernelGGL(k_disp_copy<uint32_t>, dim3(unsigned(blocks)), dim3(256), 0, s,
                           static_cast<const char*>(a.x), static_cast<char*>(a.dispatched), a.row_to_token,
                           a.expert_offsets + a.n, vpr, items);
      else
        hipLaunchKernelGGL(k_disp_copy<uint16_t>, dim3(unsigned(blocks)), dim3(256), 0, s,
                           static_cast<const char*>(a.x), static_cast<char*>(a.dispatched), a.row_to_token,
                           a.expert_offsets + a.n, vpr, items);
    }
  }
  return hipGetLastError();
}

}  // namespace moe
