// Grid-wide finish of per-chunk partials, shared by the route and dispatch
// kernels.  Every workgroup (one chunk of tokens) writes its dense per-expert
// counts (and score sums) with agent-scope stores, waits for them to be
// acknowledged and takes a ticket; the workgroup that takes the last ticket
// sums the partials in a fixed order and publishes
//   counts_j, Σ score_j                         (route: f_i, P_i inputs)
//   f, P, aux                                   ([Switch review] "로드 밸런싱 손실")
//   kept_j = min(c_j, capacity), expert_offsets ([Switch review] "Expert
//                                                Capacity와 토큰 드롭")
//   super_prefix[s, j] = Σ_{c < s*sup} counts[c, j]
// so that a chunk's slot base for expert j is super_prefix[c/sup, j] plus at
// most sup-1 chunk counts.  Data crosses workgroups only through agent-scope
// (L2-bypassing) stores and loads, so no cache-wide fence is needed; every
// sum has a fixed order, so results are bit-reproducible.
#pragma once
#include "common.hpp"

namespace moe {

__host__ __device__ inline int super_chunk(int nch) {  // chunks per super chunk: at most kMaxSuperChunks super chunks
  return nch <= kMaxSuperChunks ? 1 : (nch + kMaxSuperChunks - 1) / kMaxSuperChunks;
}

template <typename T>
__device__ __forceinline__ void store_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T load_agent(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// All of this workgroup's agent-scope stores are acknowledged; then one ticket.
// Returns true in the workgroup that took the last ticket (which also resets it).
__device__ __forceinline__ bool last_workgroup(uint32_t* ticket, unsigned nblocks, int* s_flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) *s_flag = atomicAdd(ticket, 1u) == nblocks - 1;
  __syncthreads();
  const bool last = *s_flag;
  if (last && threadIdx.x == 0) atomicExch(ticket, 0u);
  return last;
}

// A chunk row entry: count in the low 32 bits, fp32 score sum in the high 32.
__device__ __forceinline__ uint64_t pack_chunk(int count, float psum) {
  return uint64_t(uint32_t(count)) | (uint64_t(__float_as_uint(psum)) << 32);
}
__device__ __forceinline__ int chunk_count(uint64_t v) { return int(uint32_t(v)); }
__device__ __forceinline__ float chunk_psum(uint64_t v) { return __uint_as_float(uint32_t(v >> 32)); }

struct FinalizeArgs {
  const uint64_t* chunks;       // [nch, n]  agent-scope stores of every chunk (pack_chunk)
  int nch, sup, n;
  int64_t m;                    // tokens (for f and P)
  int32_t* counts;              // [n] out or nullptr
  float* prob_sum;              // [n] out or nullptr
  float* f;                     // [n] out or nullptr
  float* P;                     // [n] out or nullptr
  float* aux;                   // [1] out or nullptr
  float alpha;
  int32_t capacity;             // < 0: no capacity prefix sums
  int32_t* expert_offsets;      // [n + 1]
  int32_t* super_prefix;        // [ceil(nch / sup), n]
  int32_t* expert_rows;         // [n] kept rows per expert, or nullptr
  bool padded;                  // capacity-padded layout: expert j starts at row j * capacity
  // the Loss-Free step of the same micro-batch, fused into the finish (all optional)
  int k;                        // picks per token
  int64_t* gcounts;             // [n] global-batch counts += counts
  int64_t* gtokens;             // [1] global-batch tokens += m
  float* lf_bias;               // [n] b_j -= gamma * sign(counts_j * n - m * k), in place
  float gamma;
};

// Global-batch accumulation and the Loss-Free bias step for expert j with count c, as the
// statistics kernel does them ([MoE tour 6] "방법 회고" eq. (2): b_j moves against the sign of
// F_j - 1/n, i.e. of c·n - m·k; [Qwen global] "글로벌-배치 로드 밸런스 구현": counts summed over
// the micro-batches).  The finishing workgroup runs after every workgroup of the launch has read
// the bias, so the in-place update races with none of them.
__device__ __forceinline__ void lossfree_step(const FinalizeArgs& a, int j, int c) {
  if (a.gcounts) a.gcounts[j] += c;
  if (a.lf_bias) {
    const int64_t diff = int64_t(c) * a.n - a.m * a.k;
    const float sgn = diff > 0 ? 1.f : (diff < 0 ? -1.f : 0.f);
    a.lf_bias[j] = a.lf_bias[j] - a.gamma * sgn;
  }
}

// Exclusive scan of v[0..n) held in LDS by one workgroup into out[0..n];
// fixed order, deterministic.  part: LDS of threads/64 ints.
__device__ __forceinline__ void block_exclusive_scan(const int* v, int n, int32_t* out, int* part, int threads) {
  const int per = ceil_div(n, threads);
  const int j0 = threadIdx.x * per;
  int s = 0;
  for (int j = j0; j < min(j0 + per, n); ++j) s += v[j];
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

// Runs in the last workgroup.  lds: >= n + 2 * nsup * 64 ints.
__device__ __forceinline__ void finalize_chunks(const FinalizeArgs& a, int* lds, int lds_ints, int threads) {
  __shared__ int part[16];
  __shared__ double red[16];
  const int n = a.n;
  const int nsup = ceil_div(a.nch, a.sup);
  int* tot = lds;                                   // [n] totals, then kept counts
  int* sc = tot + n;                                // [nsup][cb] super-chunk counts
  float* sp = reinterpret_cast<float*>(sc) + 0;     // reused below: [nsup][cb] score sums
  const int cb = max(1, min(n, (lds_ints - n) / (2 * nsup)));
  sp = reinterpret_cast<float*>(sc + nsup * cb);
  const double dm = double(a.m);
  double auxp = 0.0;
  for (int j0 = 0; j0 < n; j0 += cb) {
    const int w = min(cb, n - j0);
    // two (super chunk, expert) pairs per thread per pass, 32 independent loads
    // in flight (these bypass the L2), then fixed-order sums
    for (int q0 = threadIdx.x; q0 < nsup * w; q0 += 2 * threads) {
      const int q1 = min(q0 + threads, nsup * w - 1);
      const bool two = q0 + threads < nsup * w;
      const int s0 = q0 / w, j0q = q0 - s0 * w, s1 = q1 / w, j1q = q1 - s1 * w;
      const int b0 = s0 * a.sup, e0 = min(a.nch, b0 + a.sup), b1 = s1 * a.sup, e1 = min(a.nch, b1 + a.sup);
      int cs0 = 0, cs1 = 0;
      float ps0 = 0.f, ps1 = 0.f;
      for (int o = 0; o < a.sup; o += 16) {
        uint64_t v0[16], v1[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          v0[u] = load_agent(a.chunks + int64_t(min(b0 + o + u, e0 - 1)) * n + j0 + j0q);
          v1[u] = load_agent(a.chunks + int64_t(min(b1 + o + u, e1 - 1)) * n + j0 + j1q);
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          if (b0 + o + u < e0) {
            cs0 += chunk_count(v0[u]);
            ps0 += chunk_psum(v0[u]);
          }
          if (b1 + o + u < e1) {
            cs1 += chunk_count(v1[u]);
            ps1 += chunk_psum(v1[u]);
          }
        }
      }
      sc[s0 * w + j0q] = cs0;
      sp[s0 * w + j0q] = ps0;
      if (two) {
        sc[s1 * w + j1q] = cs1;
        sp[s1 * w + j1q] = ps1;
      }
    }
    __syncthreads();
    for (int jj = threadIdx.x; jj < w; jj += threads) {
      const int j = j0 + jj;
      int run = 0;
      float ps = 0.f;
      for (int s = 0; s < nsup; ++s) {
        if (a.capacity >= 0) a.super_prefix[int64_t(s) * n + j] = run;
        run += sc[s * w + jj];
        ps += sp[s * w + jj];
      }
      tot[j] = run;
      if (a.counts) a.counts[j] = run;
      lossfree_step(a, j, run);
      if (a.prob_sum) a.prob_sum[j] = ps;
      if (a.f) a.f[j] = float(run) / float(a.m);
      if (a.P) a.P[j] = ps / float(a.m);
      auxp += (double(run) / dm) * (double(ps) / dm);
    }
    __syncthreads();
  }
  if (a.gtokens && threadIdx.x == 0) a.gtokens[0] += a.m;
  if (a.aux) {
    double v = wave_sum_f64(auxp);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
      double t = 0.0;
      for (int q = 0; q < threads / 64; ++q) t += red[q];
      a.aux[0] = float(double(a.alpha) * double(n) * t);
    }
  }
  if (a.capacity >= 0) {
    for (int j = threadIdx.x; j < n; j += threads) {
      tot[j] = min(tot[j], a.capacity);
      if (a.expert_rows) a.expert_rows[j] = tot[j];
    }
    __syncthreads();
    if (a.padded) {
      for (int j = threadIdx.x; j <= n; j += threads) a.expert_offsets[j] = j * a.capacity;
    } else {
      block_exclusive_scan(tot, n, a.expert_offsets, part, threads);
    }
  }
}

// Runs in the last workgroup when every workgroup added its counts and fixed-point (2^-32) score
// sums into the per-super-chunk rows [nsup][n] with integer atomics (order-free, so deterministic):
// reads the rows (one round of L2-bypassing loads), publishes what finalize_chunks publishes and
// leaves the rows zero for the next call.  lds: >= n ints.
__device__ __forceinline__ void finalize_super(const FinalizeArgs& a, int32_t* sup_counts,
                                               unsigned long long* sup_psum, bool want_psum, int* lds,
                                               int threads) {
  __shared__ int part[16];
  __shared__ double red[16];
  const int n = a.n;
  const int nsup = ceil_div(a.nch, a.sup);
  int* tot = lds;
  const double dm = double(a.m);
  double auxp = 0.0;
  for (int j = threadIdx.x; j < n; j += threads) {
    int c[kMaxSuperChunks];
    unsigned long long p[kMaxSuperChunks];
#pragma unroll
    for (int s = 0; s < kMaxSuperChunks; ++s) {
      c[s] = s < nsup ? load_agent(sup_counts + s * n + j) : 0;
      p[s] = s < nsup && want_psum ? load_agent(sup_psum + s * n + j) : 0ull;
    }
    int run = 0;
    unsigned long long ps = 0;
#pragma unroll
    for (int s = 0; s < kMaxSuperChunks; ++s) {
      if (s < nsup) {
        if (a.capacity >= 0) a.super_prefix[int64_t(s) * n + j] = run;
        run += c[s];
        ps += p[s];
        store_agent(sup_counts + s * n + j, 0);
        if (want_psum) store_agent(sup_psum + s * n + j, 0ull);
      }
    }
    const float psf = float(double(ps) / double(kPsumScale));
    tot[j] = run;
    if (a.counts) a.counts[j] = run;
    lossfree_step(a, j, run);
    if (a.prob_sum) a.prob_sum[j] = psf;
    if (a.f) a.f[j] = float(run) / float(a.m);
    if (a.P) a.P[j] = psf / float(a.m);
    auxp += (double(run) / dm) * (double(psf) / dm);
  }
  if (a.gtokens && threadIdx.x == 0) a.gtokens[0] += a.m;
  if (a.aux) {
    double v = wave_sum_f64(auxp);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
      double t = 0.0;
      for (int q = 0; q < threads / 64; ++q) t += red[q];
      a.aux[0] = float(double(a.alpha) * double(n) * t);
    }
  }
  __syncthreads();
  if (a.capacity >= 0) {
    for (int j = threadIdx.x; j < n; j += threads) {
      tot[j] = min(tot[j], a.capacity);
      if (a.expert_rows) a.expert_rows[j] = tot[j];
    }
    __syncthreads();
    if (a.padded) {
      for (int j = threadIdx.x; j <= n; j += threads) a.expert_offsets[j] = j * a.capacity;
    } else {
      block_exclusive_scan(tot, n, a.expert_offsets, part, threads);
    }
  }
}

}  // namespace moe
