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
// come from counting instead.  Tokens are cut into chunks of `chunk_tokens`
// (the route workgroup size, so the route kernel can produce the counts):
//   1. per-chunk dense expert counts and totals (from the route kernel, or
//      from the histogram kernel here); the last workgroup turns them into
//      expert offsets and super-chunk prefix sums (prefix.hpp);
//   2. one workgroup per chunk: wave 0 ranks the chunk's pairs in order with
//      a match-any built from ballots over the expert-id bits and per-expert
//      LDS counters; every pair adds its chunk base (a super-chunk prefix plus
//      at most sup-1 chunk counts) and, if kept, its expert offset.  The other
//      waves read the chunk's source rows meanwhile and write the kept ones
//      with 16-byte accesses once the rows are known.
#include "common.hpp"
#include "kernels.hpp"
#include "prefix.hpp"

namespace moe {

constexpr int kDispThreads = 1024;
constexpr int kDispPrefixBuf = 4096;   // LDS ints for the last block's super-chunk pass

size_t dispatch_ws_bytes(int64_t m, int k, int n, int chunk_tokens) {
  const int64_t nch = ceil_div64(m, chunk_tokens);
  (void)k;
  // packed chunk rows (count, route score sum), super-chunk prefixes
  return size_t(nch) * n * sizeof(uint64_t) + 256 + size_t(kMaxSuperChunks) * n * sizeof(int32_t) + 256;
}

__global__ __launch_bounds__(kDispThreads) void k_disp_hist(DispatchArgs a) {
  extern __shared__ int lds[];
  int* hist = lds;                  // [n], then the finishing scratch
  const int n = a.n;
  const int64_t c = blockIdx.x;
  for (int j = threadIdx.x; j < n; j += kDispThreads) hist[j] = 0;
  __syncthreads();
  const int64_t p0 = c * a.chunk_tokens * a.k;
  const int64_t p1 = min<int64_t>(a.pairs, p0 + int64_t(a.chunk_tokens) * a.k);
  for (int64_t p = p0 + threadIdx.x; p < p1; p += kDispThreads) {
    const int e = a.idx[p];
    if (unsigned(e) < unsigned(n)) atomicAdd(&hist[e], 1);   // ids outside [0, n) are dropped
  }
  __syncthreads();
  for (int j = threadIdx.x; j < n; j += kDispThreads) store_agent(a.chunks + c * n + j, pack_chunk(hist[j], 0.f));
  __shared__ int s_flag;
  if (!last_workgroup(a.done, gridDim.x, &s_flag)) return;
  FinalizeArgs f{};
  f.chunks = a.chunks;
  f.nch = a.nch;
  f.sup = a.sup;
  f.n = n;
  f.m = a.pairs;
  f.capacity = a.capacity;
  f.expert_offsets = a.expert_offsets;
  f.super_prefix = a.super_prefix;
  f.expert_rows = a.expert_rows;
  f.padded = a.padded;
  finalize_chunks(f, lds, n + kDispPrefixBuf, kDispThreads);
}

// Wave 0 loads the chunk's expert ids and ranks them, waves 1-2 load the
// prefix data, and waves 3-15 read the chunk's source rows (only their
// destinations depend on the slots), all at once: up to kDispPrefetch
// 16-byte items per thread of those waves, the rest after the slots.
constexpr int kDispPrefetch = 4;
constexpr int kDispCopyWave0 = 3;
constexpr int kDispCopyThreads = kDispThreads - 64 * kDispCopyWave0;

// Self prefix (n <= 256): the route kernel left per-chunk count rows
// [nch][n] int32 and, per super chunk of `sup` chunks, the expert counts and
// fixed-point score sums (integer atomics, so order-free).  Expert e's total
// is the sum of its super-chunk counts; this chunk's slot base adds the
// super-chunk counts before this chunk's super chunk and the count rows of
// the earlier chunks inside it.  Those sources are spread over the whole
// workgroup, every thread loading its share first thing (before the row
// reads, so the prefix loads are not queued behind them): thread t takes
// expert t % n and every (1024 / n)-th source.  The partial sums meet in LDS
// through integer atomics (order-free); then the offsets follow, and
// workgroup 0 publishes counts, f, P, aux, the kept counts and the offsets.
constexpr int kPrefixBatch = 8;   // sources per thread loaded up front
struct PrefixPart {
  int e, sl, slices, nsrc, nsup, sc;
  int v[kPrefixBatch];
  unsigned long long pq[kPrefixBatch];
};
__device__ __forceinline__ int prefix_source(const DispatchArgs& a, const PrefixPart& P, int c, int i) {
  const int32_t* crow = reinterpret_cast<const int32_t*>(a.chunks);
  return i < P.nsup ? a.sup_counts[i * a.n + P.e] : crow[int64_t(P.sc * a.sup + (i - P.nsup)) * a.n + P.e];
}
__device__ __forceinline__ void prefix_issue(const DispatchArgs& a, int c, PrefixPart& P) {
  const int n = a.n, t = threadIdx.x;
  P.nsup = ceil_div(a.nch, a.sup);
  P.sc = c / a.sup;
  P.nsrc = P.nsup + (c - P.sc * a.sup);
  P.slices = kDispThreads / n;
  P.e = t % n;
  P.sl = t / n;
  const bool stats = c == 0;
#pragma unroll
  for (int u = 0; u < kPrefixBatch; ++u) {
    const int i = P.sl + u * P.slices;
    const bool in = P.sl < P.slices && i < P.nsrc;
    P.v[u] = in ? prefix_source(a, P, c, i) : 0;
    P.pq[u] = stats && P.sl < P.slices && i < P.nsup ? a.sup_psum[i * n + P.e] : 0ull;
  }
}
__device__ __forceinline__ void derive_prefix(const DispatchArgs& a, int c, PrefixPart& P, int* lbase, int* loff,
                                              int* ltot_raw, unsigned long long* lps) {
  const int n = a.n, t = threadIdx.x;
  const bool stats = c == 0;
  int* ltot = loff + n + 1;   // kept counts
  // partial sums of this thread's sources (the batch loaded up front, then any rest)
  int tot = 0, base = 0;
  unsigned long long ps = 0;
  if (P.sl < P.slices) {
#pragma unroll
    for (int u = 0; u < kPrefixBatch; ++u) {
      const int i = P.sl + u * P.slices;
      tot += i < P.nsup ? P.v[u] : 0;
      base += i < P.sc || i >= P.nsup ? P.v[u] : 0;
      ps += P.pq[u];
    }
    for (int i = P.sl + kPrefixBatch * P.slices; i < P.nsrc; i += P.slices) {
      const int v = prefix_source(a, P, c, i);
      tot += i < P.nsup ? v : 0;
      base += i < P.sc || i >= P.nsup ? v : 0;
    }
  }
  __syncthreads();   // the LDS sums were zeroed before the row reads
  if (P.sl < P.slices) {
    if (tot) atomicAdd(ltot_raw + P.e, tot);
    if (base) atomicAdd(lbase + P.e, base);
    if (stats && ps) atomicAdd(lps + P.e, ps);
  }
  __syncthreads();
  double auxp = 0.0;
  for (int e = t; e < n; e += kDispThreads) {
    const int tt = ltot_raw[e];
    ltot[e] = min(tt, a.capacity);
    if (stats) {
      if (a.expert_rows) a.expert_rows[e] = ltot[e];
      const double psum = double(lps[e]) / double(kPsumScale);   // integer sum: order-free
      const int64_t m = a.pairs / a.k;
      if (a.counts) a.counts[e] = tt;
      if (a.prob_sum) a.prob_sum[e] = float(psum);
      if (a.f) a.f[e] = float(tt) / float(m);
      if (a.P) a.P[e] = float(psum / double(m));
      auxp += (double(tt) / double(m)) * (psum / double(m));
      // [Qwen global] global batch; [MoE tour 6] eq. (2): the sign of F_j - 1/n taken
      // exactly as the sign of c_j n - m k, one fp32 step of the bias
      if (a.gcounts) a.gcounts[e] += tt;
      if (a.lf_bias) {
        const int64_t diff = int64_t(tt) * n - m * a.k;
        const float sgn = diff > 0 ? 1.f : (diff < 0 ? -1.f : 0.f);
        a.lf_bias[e] = a.lf_bias[e] - a.gamma * sgn;
      }
    }
  }
  if (stats && a.gtokens && t == 0) a.gtokens[0] += a.pairs / a.k;
  if (stats && a.aux) {   // fixed-order fp64 sum over the experts
    __shared__ double red[kDispThreads / 64];
    const double v = wave_sum_f64(auxp);
    if ((t & 63) == 0) red[t >> 6] = v;
    __syncthreads();
    if (t == 0) {
      double s = 0.0;
      for (int w = 0; w < kDispThreads / 64; ++w) s += red[w];
      a.aux[0] = float(double(a.alpha) * double(n) * s);
    }
  }
  if (a.padded) {   // capacity regions: expert j starts at row j * capacity (no scan, no barrier)
    if (stats)
      for (int j = t; j <= n; j += kDispThreads) a.expert_offsets[j] = j * a.capacity;
    return;
  }
  __syncthreads();
  if (t < 64) {   // exclusive scan of the kept counts: lane l owns a contiguous run
    const int per = (n + 63) / 64, j0 = t * per, j1 = min(j0 + per, n);
    int sum = 0;
    for (int j = j0; j < j1; ++j) sum += ltot[j];
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (t >= off) incl += o;
    }
    int run = incl - sum;
    for (int j = j0; j < j1; ++j) {
      loff[j] = run;
      run += ltot[j];
    }
    if (t == 63) loff[n] = incl;
  }
  __syncthreads();
  if (stats)
    for (int j = t; j <= n; j += kDispThreads) a.expert_offsets[j] = loff[j];
}

template <typename V, bool SELF>
__global__ __launch_bounds__(kDispThreads) void k_disp_rank_copy(DispatchArgs a) {
  extern __shared__ __attribute__((aligned(16))) int lds[];
  const int n = a.n;
  const int cp = a.chunk_tokens * a.k;          // pairs per chunk
  int* cnt = lds;                                // [n] running counts inside the chunk
  int* lrow = cnt + n;                           // [cp] expert id, then dispatched row (-1: dropped)
  int* lslot = lrow + cp;                        // [cp] slot inside the chunk
  int* lbase = lslot + cp;                       // SELF: [n] slot base of this chunk
  int* loff = lbase + n;                         // SELF: [n + 1] expert offsets, then [n] kept counts
  int* ltot_raw = loff + 2 * n + 1;              // SELF: [n] expert totals
  const int c = blockIdx.x;
  PrefixPart pp;
  __shared__ unsigned long long lps[kSelfPrefixMaxN];   // SELF, workgroup 0: score sums
  if constexpr (SELF) {
    prefix_issue(a, c, pp);
    for (int j = threadIdx.x; j < n; j += kDispThreads) {
      lbase[j] = 0;
      ltot_raw[j] = 0;
      lps[j] = 0ull;
    }
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t p0 = int64_t(c) * cp;
  const int np = int(min<int64_t>(cp, a.pairs - p0));
  // copy items i = q * vpr + v (pair q, vector v) are walked with (q, v) stepped
  // incrementally: no integer division per item (np * vpr < 2^31 by the API limits)
  const int vpr = int(a.row_bytes / int64_t(sizeof(V)));
  const int qend = a.dispatched ? np : 0;
  const V* __restrict__ x = static_cast<const V*>(a.x);
  V* __restrict__ out = static_cast<V*>(a.dispatched);
  auto src_row = [&](int q) -> int64_t {   // token of pair p0 + q
    return a.k == 1 ? p0 + q : int64_t(uint32_t(p0 + q) / uint32_t(a.k));
  };
  const int ct = threadIdx.x - 64 * kDispCopyWave0;   // copy thread index (waves 3-15)
  const int q0 = ct / vpr, v0 = ct - q0 * vpr;
  const int dq = kDispCopyThreads / vpr, dv = kDispCopyThreads - dq * vpr;
  V pv[kDispPrefetch];
  if (wave >= kDispCopyWave0) {
    int q = q0, v = v0;
#pragma unroll
    for (int u = 0; u < kDispPrefetch; ++u) {
      if (q < qend) pv[u] = x[src_row(q) * vpr + v];
      q += dq;
      v += dv;
      if (v >= vpr) {
        v -= vpr;
        ++q;
      }
    }
  }
  if (wave == 0) {   // rank the chunk's pairs in token-major order
    for (int j = lane; j < n; j += 64) cnt[j] = 0;
    __builtin_amdgcn_wave_barrier();
    for (int g = 0; g < np; g += 64) {
      const bool inside = g + lane < np;
      const int e0 = inside ? a.idx[p0 + g + lane] : 0;
      const bool valid = inside && unsigned(e0) < unsigned(n);
      const int e = valid ? e0 : 0;
      const uint64_t active = __ballot(valid);
      const uint64_t pr = match_any(uint32_t(e), a.nbits, active);
      const int before = valid ? cnt[e] : 0;
      // every lane has read cnt[e] before the group's first lane advances it
      __builtin_amdgcn_wave_barrier();
      if (valid && (pr & lanemask_lt()) == 0) cnt[e] = before + __popcll(pr);
      if (inside) {
        lrow[g + lane] = valid ? e : -1;
        lslot[g + lane] = before + __popcll(pr & lanemask_lt());
      }
    }
  }
  if constexpr (SELF) derive_prefix(a, c, pp, lbase, loff, ltot_raw, lps);   // has barriers
  else __syncthreads();
  // slots -> rows and maps, one thread per pair
  const int s = c / a.sup;
  const int32_t* cw = reinterpret_cast<const int32_t*>(a.chunks);   // counts: low words of the chunk rows
  for (int q = threadIdx.x; q < np; q += kDispThreads) {
    const int e = lrow[q];
    int row = -1;
    if (e >= 0) {
      int base, off;
      if constexpr (SELF) {
        base = lbase[e];
        off = a.padded ? e * a.capacity : loff[e];
      } else {
        // chunk base of expert e: its super-chunk prefix plus the earlier chunks of the super chunk
        base = a.super_prefix[int64_t(s) * n + e];
        off = a.expert_offsets[e];
        for (int cc = s * a.sup; cc < c; cc += 16) {
          int v[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) v[u] = cw[2 * (int64_t(min(cc + u, c - 1)) * n + e)];
#pragma unroll
          for (int u = 0; u < 16; ++u)
            if (cc + u < c) base += v[u];
        }
      }
      const int slot = base + lslot[q];
      if (slot < a.capacity) row = off + slot;
    }
    const int64_t p = p0 + q;
    a.token_to_row[p] = row;
    if (a.drop_mask) a.drop_mask[p] = row < 0 ? 1 : 0;
    if (row >= 0 && a.row_to_token) a.row_to_token[row] = int32_t(src_row(q));
    lrow[q] = row;
  }
  if (!a.dispatched) return;
  __syncthreads();
  // rows are stored non-temporally: nothing in this kernel reads them again
  if (wave >= kDispCopyWave0) {
    int q = q0, v = v0;
#pragma unroll
    for (int u = 0; u < kDispPrefetch; ++u) {
      if (q < qend) {
        const int row = lrow[q];
        if (row >= 0) __builtin_nontemporal_store(pv[u], &out[int64_t(row) * vpr + v]);
      }
      q += dq;
      v += dv;
      if (v >= vpr) {
        v -= vpr;
        ++q;
      }
    }
  }
  // items past the prefetched ones (long rows or many pairs): every thread, stride kDispThreads
  const int first = kDispPrefetch * kDispCopyThreads + threadIdx.x;
  int q = first / vpr, v = first - (first / vpr) * vpr;
  const int sq = kDispThreads / vpr, sv = kDispThreads - sq * vpr;
  while (q < qend) {
    V val[4];
    int64_t dst[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      dst[u] = -1;
      if (q < qend) {
        const int row = lrow[q];
        if (row >= 0) {
          val[u] = x[src_row(q) * vpr + v];
          dst[u] = int64_t(row) * vpr + v;
        }
      }
      q += sq;
      v += sv;
      if (v >= vpr) {
        v -= vpr;
        ++q;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (dst[u] >= 0) __builtin_nontemporal_store(val[u], &out[dst[u]]);
  }
}

template <bool SELF>
static void launch_rank_copy(const DispatchArgs& a, size_t lds, hipStream_t s) {
  const uintptr_t al = reinterpret_cast<uintptr_t>(a.x) | reinterpret_cast<uintptr_t>(a.dispatched);
  if (a.row_bytes % 16 == 0 && al % 16 == 0)
    hipLaunchKernelGGL((k_disp_rank_copy<u32x4, SELF>), dim3(a.nch), dim3(kDispThreads), lds, s, a);
  else if (a.row_bytes % 4 == 0 && al % 4 == 0)
    hipLaunchKernelGGL((k_disp_rank_copy<uint32_t, SELF>), dim3(a.nch), dim3(kDispThreads), lds, s, a);
  else
    hipLaunchKernelGGL((k_disp_rank_copy<uint16_t, SELF>), dim3(a.nch), dim3(kDispThreads), lds, s, a);
}

bool dispatch_self_prefix_ok(int nch, int n) {
  return n <= kSelfPrefixMaxN && super_chunk(nch) <= 64;   // at most 63 in-super count rows per expert
}

hipError_t launch_dispatch(const DispatchArgs& a, bool prefix_ready, hipStream_t s) {
  if (a.self_prefix) {
    // cnt [n], lrow [cp], lslot [cp], lbase [n], loff [n + 1] + kept [n], totals [n]
    const size_t lds = (5 * size_t(a.n) + 1 + 2 * size_t(a.chunk_tokens) * a.k) * sizeof(int);
    launch_rank_copy<true>(a, lds, s);
    return hipGetLastError();
  }
  if (!prefix_ready)
    hipLaunchKernelGGL(k_disp_hist, dim3(a.nch), dim3(kDispThreads), (a.n + kDispPrefixBuf) * sizeof(int), s, a);
  const size_t lds = (size_t(a.n) + 2 * size_t(a.chunk_tokens) * a.k) * sizeof(int);
  launch_rank_copy<false>(a, lds, s);
  return hipGetLastError();
}

}  // namespace moe
