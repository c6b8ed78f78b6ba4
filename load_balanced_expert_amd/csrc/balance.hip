// Balanced optimal assignment ([MoE tour 6]):
//   "선형계획" eq. (3)/(4): maximise Σ x_ij s_ij with Σ_j x_ij = k and
//   Σ_i x_ij = q = mk/n;
//   "교대 반복" (Quantile Balancing): α_i ← (k+1)-th largest of s_i − β,
//   β_j ← (q+1)-th largest of s_·j − α, x_i = top-k of s_i − β;
//   "함정에 주의": the online form routes with the old β, then updates it.
//
// Kernels
//  * row kernel: one wave per token row.  For n <= 256 the lanes keep their
//    experts sorted in registers and each of the k+1 rounds pops the wave's
//    best head (DPP max); wider rows take k+1 rounds of a wave-wide arg-best
//    over fl32(s_i − β).  The rounds give the top-k (idx) and the (k+1)-th
//    value (α).
//  * column kernel: one 1024-thread workgroup per expert on a transposed copy
//    of s (each column contiguous): the (q+1)-th largest of fl32(s_·j − α) by
//    an exact radix select over order-preserving uint32 keys (12 + 12 + 8
//    bits), the last two digits over the keys of the chosen bin held in LDS.
//  * exact completion: one persistent workgroup runs successive shortest
//    paths on the expert graph in fp64 (the move cost a -> j is the cheapest
//    s_ia − s_ij over tokens holding a but not j; Dijkstra runs on one wave)
//    until every expert has q tokens.  The LDS-resident form (n <= 128, the
//    assignment within LDS) is below; k_qb_complete keeps its token lists in
//    global memory for larger assignments (n <= 64).
#include "common.hpp"
#include "dpp.hpp"
#include "kernels.hpp"
#include "prefix.hpp"

namespace moe {

constexpr int kQbRowsPerBlock = 16;
constexpr int kCompleteMaxN = 64;

static size_t al256(size_t b) { return (b + 255) / 256 * 256; }

size_t balance_ws_bytes(int64_t m, int n, int k, bool exact) {
  size_t b = al256(size_t(m) * n * sizeof(float));   // s transposed
  b += al256(size_t(m) * sizeof(float));              // alpha
  b += al256(size_t(ceil_div64(m, kQbRowsPerBlock)) * n * sizeof(uint64_t));  // per-workgroup chunk rows
  if (exact) {
    b += 2 * al256(size_t(m) * k * sizeof(int32_t));   // assignment, list positions
    b += al256(size_t(n) * m * sizeof(int32_t));       // per-expert token lists
    b += al256(size_t(n) * sizeof(double));            // final potentials
    b += 2 * al256(size_t(128) * 128 * sizeof(double)) + al256(size_t(128) * 128 * sizeof(int));   // M, W (n > 64)
  }
  return b;
}

// ------------------------------------------------------------------ transpose
__global__ __launch_bounds__(256) void k_qb_transpose(const float* __restrict__ s, float* __restrict__ sT, int64_t m,
                                                      int n) {
  __shared__ float tile[64][65];
  const int64_t ib = int64_t(blockIdx.x) * 64;
  const int jb = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const int64_t i = ib + r;
    const int j = jb + tx;
    tile[r][tx] = (i < m && j < n) ? s[i * n + j] : 0.f;
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int j = jb + r;
    const int64_t i = ib + tx;
    if (j < n && i < m) sT[int64_t(j) * m + i] = tile[tx][r];
  }
}

// numpy's linear interpolation of two neighbouring order statistics, in fp32
// with no contraction (the demo's quantile of fp32 differences is computed so)
__device__ __forceinline__ float lerp_np(float a, float b, float t) {
#pragma clang fp contract(off)
  const float d = b - a;
  return t >= 0.5f ? b - d * (1.0f - t) : a + d * t;
}

// ------------------------------------------------------------------ rows: top-k and α
template <bool IDX, bool ALPHA>
__global__ __launch_bounds__(256) void k_qb_rows(BalanceArgs a, const float* __restrict__ beta,
                                                 float* __restrict__ alpha, uint64_t* __restrict__ chunks) {
  extern __shared__ int hist[];   // [n], then the finishing scratch
  const int n = a.n, k = a.k;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (IDX) {
    for (int j = threadIdx.x; j < n; j += 256) hist[j] = 0;
    __syncthreads();
  }
  for (int rr = wave; rr < kQbRowsPerBlock; rr += 4) {
    const int64_t i = int64_t(blockIdx.x) * kQbRowsPerBlock + rr;
    if (i >= a.m) break;
    const float* row = a.s + i * n;
    const float* bi = a.nblocks > 1 ? beta + (i / a.beta_rows) * n : beta;   // the row's β block
    float last_key = INFINITY, hi_key = INFINITY, lo_key = INFINITY;
    int last_j = -1, my_j = 0;
    // α: the (k+1)-th largest (exact form), or the order statistics of descending
    // ranks rank_row and rank_row - 1 (quantile form)
    const int arank = a.quantile ? a.rank_row : k;
    const int rounds = ALPHA ? max(k, arank + 1) : k;
    for (int r = 0; r < rounds; ++r) {
      float bk = -INFINITY;
      int bj = 0x7FFFFFFF;
      for (int j = lane; j < n; j += 64) {
        const float v = row[j] - bi[j];
        if (better(last_key, last_j, v, j) && better(v, j, bk, bj)) {
          bk = v;
          bj = j;
        }
      }
      wave_argbest(bk, bj);
      last_key = bk;
      last_j = bj;
      if (r == arank - 1) hi_key = bk;
      if (r == arank) lo_key = bk;
      if (IDX && r < k) {
        if (lane == r) my_j = bj;
        if (lane == 0) atomicAdd(&hist[bj], 1);
      }
    }
    if (ALPHA && lane == 0) {
      float al = lo_key;
      if (a.quantile) al = lerp_np(lo_key, arank >= 1 ? hi_key : lo_key, a.g_row);
      if (a.bip) al = fmaxf(al, 0.f);
      alpha[i] = al;
    }
    if (IDX && lane < k) a.idx[i * k + lane] = my_j;
  }
  if (!IDX) return;
  __syncthreads();
  for (int j = threadIdx.x; j < n; j += 256) store_agent(chunks + int64_t(blockIdx.x) * n + j, pack_chunk(hist[j], 0.f));
  __shared__ int s_flag;
  if (!last_workgroup(a.done, gridDim.x, &s_flag)) return;
  FinalizeArgs f{};
  f.chunks = chunks;
  f.nch = int(gridDim.x);
  f.sup = super_chunk(f.nch);
  f.n = n;
  f.m = a.m;
  f.counts = a.counts;
  f.capacity = -1;
  finalize_chunks(f, hist, n + 4096, 256);
  __shared__ int s_bal;
  if (threadIdx.x == 0) s_bal = 1;
  __syncthreads();
  for (int j = threadIdx.x; j < n; j += 256)
    if (int64_t(hist[j]) != a.q) atomicAnd(&s_bal, 0);
  __syncthreads();
  if (threadIdx.x == 0 && a.info) a.info[2] = s_bal;
}

// ------------------------------------------------------------------ rows, n <= 256
// Lane l holds experts l + 64u (u < NPL) in registers, sorted by (value
// descending, index ascending); each round the wave's best head (a DPP max, and
// among equal heads the lowest expert) is popped by the lane that holds it, so a
// round costs a few DPP steps instead of a pass over the row.
// compare-exchange into (value desc, index asc) order; by value alone when the
// indices are not wanted
template <bool USEJ, int NPL>
__device__ __forceinline__ void ce_desc(float (&v)[NPL], int (&j)[NPL], int p, int q) {
  if (!USEJ) {
    const float hi = fmaxf(v[p], v[q]), lo = fminf(v[p], v[q]);
    v[p] = hi;
    v[q] = lo;
    return;
  }
  if (better(v[q], j[q], v[p], j[p])) {
    const float tv = v[p];
    v[p] = v[q];
    v[q] = tv;
    const int tj = j[p];
    j[p] = j[q];
    j[q] = tj;
  }
}

constexpr int kRowsRegThreads = 1024;
template <bool IDX, bool ALPHA, int NPL>
__global__ __launch_bounds__(kRowsRegThreads) void k_qb_rows_reg(BalanceArgs a, const float* __restrict__ beta,
                                                     float* __restrict__ alpha, uint64_t* __restrict__ chunks) {
  extern __shared__ __attribute__((aligned(16))) int hist[];   // [n], then the finishing scratch
  const int n = a.n, k = a.k;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (IDX) {
    for (int j = threadIdx.x; j < n; j += kRowsRegThreads) hist[j] = 0;
    __syncthreads();
  }
  const int arank = a.quantile ? a.rank_row : k;
  const int rounds = ALPHA ? max(k, arank + 1) : k;
  float bl[NPL];
#pragma unroll
  for (int u = 0; u < NPL; ++u) bl[u] = lane + 64 * u < n ? beta[lane + 64 * u] : 0.f;
  constexpr int kWaves = kRowsRegThreads / 64;
  const int64_t stride = int64_t(gridDim.x) * kWaves;
  int64_t i = int64_t(blockIdx.x) * kWaves + wave;
  float nx[NPL];
#pragma unroll
  for (int u = 0; u < NPL; ++u) nx[u] = i < a.m && lane + 64 * u < n ? a.s[i * n + lane + 64 * u] : 0.f;
  for (; i < a.m; i += stride) {
    float v[NPL];
    int jj[NPL];
#pragma unroll
    for (int u = 0; u < NPL; ++u) {
      const int j = lane + 64 * u;
      v[u] = j < n ? nx[u] - bl[u] : -INFINITY;
      jj[u] = j < n ? j : 0x7FFFFFFF;
    }
    const int64_t i2 = i + stride;   // next row of this wave, loaded while this one is ranked
#pragma unroll
    for (int u = 0; u < NPL; ++u) nx[u] = i2 < a.m && lane + 64 * u < n ? a.s[i2 * n + lane + 64 * u] : 0.f;
    if (NPL == 2) ce_desc<IDX, NPL>(v, jj, 0, 1 % NPL);
    if (NPL == 4) {
      ce_desc<IDX, NPL>(v, jj, 0, 1 % NPL);
      ce_desc<IDX, NPL>(v, jj, 2 % NPL, 3 % NPL);
      ce_desc<IDX, NPL>(v, jj, 0, 2 % NPL);
      ce_desc<IDX, NPL>(v, jj, 1 % NPL, 3 % NPL);
      ce_desc<IDX, NPL>(v, jj, 1 % NPL, 2 % NPL);
    }
    float hi_key = INFINITY, lo_key = INFINITY;
    int my_j = 0;
    for (int r = 0; r < rounds; ++r) {
      const float h = v[0];
      const float mx = wave_max_dpp(h);
      const bool top = h == mx;
      const uint64_t tied = __ballot(top);
      int win = tied ? __ffsll((unsigned long long)tied) - 1 : 0;
      if (IDX && r < k) {
        if (__popcll(tied) > 1) {   // equal heads: the lowest expert goes first
          const int mj = wave_min_i_dpp(top ? jj[0] : 0x7FFFFFFF);
          const uint64_t w = __ballot(top && jj[0] == mj);
          win = w ? __ffsll((unsigned long long)w) - 1 : 0;
        }
        const int bj = __builtin_amdgcn_readlane(jj[0], win);
        if (lane == r) my_j = bj;
        if (lane == 0) atomicAdd(&hist[bj], 1);
      }
      if (r == arank - 1) hi_key = mx;
      if (r == arank) lo_key = mx;
      if (lane == win) {
#pragma unroll
        for (int u = 0; u + 1 < NPL; ++u) {
          v[u] = v[u + 1];
          if (IDX) jj[u] = jj[u + 1];
        }
        v[NPL - 1] = -INFINITY;
        if (IDX) jj[NPL - 1] = 0x7FFFFFFF;
      }
    }
    if (ALPHA && lane == 0) {
      float al = lo_key;
      if (a.quantile) al = lerp_np(lo_key, arank >= 1 ? hi_key : lo_key, a.g_row);
      if (a.bip) al = fmaxf(al, 0.f);
      alpha[i] = al;
    }
    if (IDX && lane < k) a.idx[i * k + lane] = my_j;
  }
  if (!IDX) return;
  __syncthreads();   // this workgroup's count row; k_qb_count_finish folds them
  for (int j = threadIdx.x; j < n; j += kRowsRegThreads) chunks[int64_t(blockIdx.x) * n + j] = pack_chunk(hist[j], 0.f);
}

// n <= 256 (and k <= 32 when counting): two rows per wave, one per 32-lane
// half; lane l of a half holds experts l + 32u (u < NPL) sorted in registers
// (by value, and by index among equal values when the picks are wanted), and
// each round every half pops its best head (half-wave DPP max; among equal
// heads the lowest expert).  Without picks equal values need no order, since
// only the values of the order statistics are kept.
template <bool USEJ, int NPL>
__device__ __forceinline__ void sort_desc(float (&v)[NPL], int (&j)[NPL]) {
  auto ce = [&](int p, int q) { ce_desc<USEJ, NPL>(v, j, p, q); };
  if constexpr (NPL == 2) ce(0, 1);
  if constexpr (NPL == 4) {
    ce(0, 1), ce(2, 3), ce(0, 2), ce(1, 3), ce(1, 2);
  }
  if constexpr (NPL == 8) {   // Batcher's odd-even merge network, 19 exchanges
    ce(0, 1), ce(2, 3), ce(4, 5), ce(6, 7), ce(0, 2), ce(1, 3), ce(4, 6), ce(5, 7), ce(1, 2), ce(5, 6);
    ce(0, 4), ce(1, 5), ce(2, 6), ce(3, 7), ce(2, 4), ce(3, 5), ce(1, 2), ce(3, 4), ce(5, 6);
  }
}

// The same network on order-preserving integer keys (values only): two instructions per exchange.
template <int NPL>
__device__ __forceinline__ void sort_desc_u(uint32_t (&v)[NPL]) {
  auto ce = [&](int p, int q) {
    const uint32_t hi = max(v[p], v[q]), lo = min(v[p], v[q]);
    v[p] = hi;
    v[q] = lo;
  };
  if constexpr (NPL == 2) ce(0, 1);
  if constexpr (NPL == 4) {
    ce(0, 1), ce(2, 3), ce(0, 2), ce(1, 3), ce(1, 2);
  }
  if constexpr (NPL == 8) {
    ce(0, 1), ce(2, 3), ce(4, 5), ce(6, 7), ce(0, 2), ce(1, 3), ce(4, 6), ce(5, 7), ce(1, 2), ce(5, 6);
    ce(0, 4), ce(1, 5), ce(2, 6), ce(3, 7), ce(2, 4), ce(3, 5), ce(1, 2), ce(3, 4), ce(5, 6);
  }
}

template <bool IDX, bool ALPHA, int NPL>
__global__ __launch_bounds__(kRowsRegThreads) void k_qb_rows_half(BalanceArgs a, const float* __restrict__ beta,
                                                                     float* __restrict__ alpha,
                                                                     uint64_t* __restrict__ chunks) {
  extern __shared__ __attribute__((aligned(16))) int hist[];   // [n], then the finishing scratch
  const int n = a.n, k = a.k;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, hl = lane & 31, half = lane >> 5;
  if (IDX) {
    for (int j = threadIdx.x; j < n; j += kRowsRegThreads) hist[j] = 0;
    __syncthreads();
  }
  const int arank = a.quantile ? a.rank_row : k;
  const int rounds = ALPHA ? (IDX ? max(k, arank + 1) : arank + 1) : k;
  constexpr int kWaves = kRowsRegThreads / 64;
  const int64_t stride = int64_t(gridDim.x) * kWaves * 2;
  int64_t i = (int64_t(blockIdx.x) * kWaves + wave) * 2 + half;
  // this half's β row: block 0, or the block of its current row (mini-batch duals)
  int64_t cur_b = a.nblocks > 1 && i < a.m ? i / a.beta_rows : 0;
  float bl[NPL];
#pragma unroll
  for (int u = 0; u < NPL; ++u) bl[u] = hl + 32 * u < n ? beta[cur_b * n + hl + 32 * u] : 0.f;
  // the rows of this half's next PF iterations are loaded ahead (two for the value-only form,
  // whose registers allow it)
  constexpr int PF = IDX ? 1 : 2;
  float nx[PF][NPL];
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    const int64_t ip = i + p * stride;
#pragma unroll
    for (int u = 0; u < NPL; ++u) nx[p][u] = ip < a.m && hl + 32 * u < n ? a.s[ip * n + hl + 32 * u] : 0.f;
  }
  // both halves run the same number of iterations (the wave's first row decides)
  for (int64_t i0 = i - half; i0 < a.m; i0 += stride, i += stride) {
    const bool live = i < a.m;
    if (a.nblocks > 1 && live && i / a.beta_rows != cur_b) {
      cur_b = i / a.beta_rows;
#pragma unroll
      for (int u = 0; u < NPL; ++u) bl[u] = hl + 32 * u < n ? beta[cur_b * n + hl + 32 * u] : 0.f;
    }
    float v[NPL];
    int jj[NPL];
#pragma unroll
    for (int u = 0; u < NPL; ++u) {
      const int j = hl + 32 * u;
      v[u] = j < n && live ? nx[0][u] - bl[u] : -INFINITY;
      jj[u] = j < n ? j : 0x7FFFFFFF;
    }
#pragma unroll
    for (int p = 0; p + 1 < PF; ++p)
#pragma unroll
      for (int u = 0; u < NPL; ++u) nx[p][u] = nx[p + 1][u];
    const int64_t i2 = i + PF * stride;
#pragma unroll
    for (int u = 0; u < NPL; ++u) nx[PF - 1][u] = i2 < a.m && hl + 32 * u < n ? a.s[i2 * n + hl + 32 * u] : 0.f;
    float hi_key = INFINITY, lo_key = INFINITY;
    int my_j = 0;
    if constexpr (!IDX) {
      // values only: order-preserving integer keys, so the sort is integer max/min and each
      // round a fused DPP integer maximum; an absent or popped entry holds the key of -inf
      constexpr uint32_t kNegInf = 0x007FFFFFu;   // f32_key(-inf)
      uint32_t kv[NPL];
#pragma unroll
      for (int u = 0; u < NPL; ++u) kv[u] = f32_key(v[u]);
      sort_desc_u<NPL>(kv);
      uint32_t hk = 0xFF800000u, lk = 0xFF800000u;   // f32_key(+inf)
      for (int r = 0; r < rounds; ++r) {
        const uint32_t mk = half_max_u(kv[0]);
        const uint64_t tied = __ballot(kv[0] == mk);
        const uint32_t tlo = uint32_t(tied), thi = uint32_t(tied >> 32);
        const int win = half ? (thi ? __ffs(thi) + 31 : 32) : (tlo ? __ffs(tlo) - 1 : 0);
        if (r == arank - 1) hk = mk;
        if (r == arank) lk = mk;
        if (lane == win) {
#pragma unroll
          for (int u = 0; u + 1 < NPL; ++u) kv[u] = kv[u + 1];
          kv[NPL - 1] = kNegInf;
        }
      }
      hi_key = key_f32(hk);
      lo_key = key_f32(lk);
    } else {
      sort_desc<IDX, NPL>(v, jj);
      for (int r = 0; r < rounds; ++r) {
        const float mx = half_max(v[0]);
        bool top = v[0] == mx;
        uint64_t tied = __ballot(top);
        if (IDX && r < k && (__popc(uint32_t(tied)) > 1 || __popc(uint32_t(tied >> 32)) > 1)) {
          // equal heads: the lowest expert goes first
          const int mj = half_min_i(top ? jj[0] : 0x7FFFFFFF);
          top = top && jj[0] == mj;
          tied = __ballot(top);
        }
        const uint32_t tlo = uint32_t(tied), thi = uint32_t(tied >> 32);
        const int wlo = tlo ? __ffs(tlo) - 1 : 0, whi = thi ? __ffs(thi) + 31 : 32;
        const int win = half ? whi : wlo;
        if (IDX && r < k) {
          const int bj = __shfl(jj[0], win, 64);
          if (hl == r) my_j = bj;
          if (hl == 0 && live) atomicAdd(&hist[bj], 1);
        }
        if (r == arank - 1) hi_key = mx;
        if (r == arank) lo_key = mx;
        if (lane == win) {
#pragma unroll
          for (int u = 0; u + 1 < NPL; ++u) {
            v[u] = v[u + 1];
            if (IDX) jj[u] = jj[u + 1];
          }
          v[NPL - 1] = -INFINITY;
          if (IDX) jj[NPL - 1] = 0x7FFFFFFF;
        }
      }
    }
    if (ALPHA && hl == 0 && live) {
      float al = lo_key;
      if (a.quantile) al = lerp_np(lo_key, arank >= 1 ? hi_key : lo_key, a.g_row);
      if (a.bip) al = fmaxf(al, 0.f);
      alpha[i] = al;
    }
    if (IDX && hl < k && live) a.idx[i * k + hl] = my_j;
  }
  if (!IDX) return;
  __syncthreads();   // this workgroup's count row; k_qb_count_finish folds them
  for (int j = threadIdx.x; j < n; j += kRowsRegThreads) chunks[int64_t(blockIdx.x) * n + j] = pack_chunk(hist[j], 0.f);
}

// Counts of the final top-k from the register row kernels' count rows, and
// whether every expert holds exactly q tokens.  One 1024-thread workgroup.
__global__ __launch_bounds__(kRowsRegThreads) void k_qb_count_finish(BalanceArgs a, const uint64_t* __restrict__ chunks,
                                                                     int nch) {
  extern __shared__ __attribute__((aligned(16))) int lds[];
  FinalizeArgs f{};
  f.chunks = chunks;
  f.nch = nch;
  f.sup = super_chunk(nch);
  f.n = a.n;
  f.m = a.m;
  f.counts = a.counts;
  f.capacity = -1;
  finalize_chunks(f, lds, a.n + 4096, kRowsRegThreads);
  __shared__ int s_bal;
  if (threadIdx.x == 0) s_bal = 1;
  __syncthreads();
  for (int j = threadIdx.x; j < a.n; j += kRowsRegThreads)
    if (int64_t(lds[j]) != a.q) atomicAnd(&s_bal, 0);
  __syncthreads();
  if (threadIdx.x == 0 && a.info) a.info[2] = s_bal;
}

// One SignSGD step on β ([MoE tour 6] "경사하강" eq. (15)-(17)): the counts of the
// counting top-k (folded from its count rows) against q, β_j ← fl32(β_j + γ·sign(c_j − q)).
__global__ __launch_bounds__(kRowsRegThreads) void k_qb_signsgd_step(BalanceArgs a, const uint64_t* __restrict__ chunks,
                                                                     int nch, float gamma) {
  extern __shared__ __attribute__((aligned(16))) int lds[];
  FinalizeArgs f{};
  f.chunks = chunks;
  f.nch = nch;
  f.sup = super_chunk(nch);
  f.n = a.n;
  f.m = a.m;
  f.capacity = -1;
  finalize_chunks(f, lds, a.n + 4096, kRowsRegThreads);
  __syncthreads();
  for (int j = threadIdx.x; j < a.n; j += kRowsRegThreads) {
    const int64_t c = lds[j];
    const float sg = c > a.q ? 1.f : (c < a.q ? -1.f : 0.f);
    a.beta[j] = a.beta[j] + gamma * sg;
  }
}

// ------------------------------------------------------------------ columns: an order statistic per expert
// One 1024-thread workgroup per expert on the transposed copy of s.  Keys are
// the order-preserving uint32 images of fl32(s_ij - α_i).  Pass 1 histograms
// the top 12 key bits; pass 2 copies the keys of the bin that holds the wanted
// rank into LDS (when they fit), and the remaining 12 + 8 bits are selected
// there; otherwise those two digits take further passes over the column.
// Histogram adds are merged per wave for the lanes that share the first
// active lane's digit (the column's keys crowd into few top-bit bins).
constexpr int kColThreads = 1024;
constexpr int kColBins = 4096;
constexpr int kColCap = 24576;
constexpr int kColWaveSlots = 1024;                       // per-wave window slots (long columns)
constexpr int kColPackOff = kColWaveSlots * (kColThreads / 64);   // packed window keys after them
constexpr size_t kColLds = (size_t(kColBins) + kColCap) * sizeof(int);

__device__ __forceinline__ void hist_add(int* hist, uint32_t d, bool act) {
  const uint64_t am = __ballot(act);
  if (!am) return;
  const uint32_t lead = uint32_t(__builtin_amdgcn_readlane(int(d), __ffsll((unsigned long long)am) - 1));
  const uint64_t peers = __ballot(act && d == lead);
  if (!act) return;
  if (d != lead) {
    atomicAdd(&hist[d], 1);
  } else if ((threadIdx.x & 63) == __ffsll((unsigned long long)peers) - 1) {
    atomicAdd(&hist[lead], __popcll(peers));
  }
}

// The bin of hist[0..nb) (taken in descending digit order) holding descending
// rank `rank`, and the rank within it.
__device__ __forceinline__ void col_select(const int* hist, int nb, int rank, int* s_wsum, int* s_bin,
                                           int* s_rank) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = ceil_div(nb, kColThreads);
  int hv[4], tot = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int b = nb - 1 - (tid * per + u);
    hv[u] = u < per && b >= 0 ? hist[b] : 0;
    tot += hv[u];
  }
  int incl = tot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int cum = incl - tot;
  for (int w = 0; w < wave; ++w) cum += s_wsum[w];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (u < per && cum <= rank && rank < cum + hv[u]) {
      *s_bin = nb - 1 - (tid * per + u);
      *s_rank = rank - cum;
    }
    cum += hv[u];
  }
  __syncthreads();
}

// f(key, active) over the column in no particular order.  A column whose
// length is a multiple of 4, with α 16-byte aligned (the transposed copy starts
// on 256 bytes in an aligned workspace), is read as float4 pairs (8 keys per
// thread per step); otherwise four scalar loads at a time.
template <typename F>
__device__ __forceinline__ void col_scan(const float* __restrict__ col, const float* __restrict__ alpha, int64_t m,
                                         F f) {
  if ((m & 3) == 0 && ((reinterpret_cast<uintptr_t>(col) | reinterpret_cast<uintptr_t>(alpha)) & 15) == 0) {
    const int64_t nv = m >> 2;
    const f32x4* c4 = reinterpret_cast<const f32x4*>(col);
    const f32x4* a4 = reinterpret_cast<const f32x4*>(alpha);
    // the next iteration's vectors are loaded before this one's keys are used, so two
    // iterations of loads are in flight; the loads are unconditional (an index past the
    // column reads its last vector again, whose keys are then inactive), so the waits count
    // only the loads of the keys in use
    if (nv == 0) return;
    auto load = [&](int64_t b, f32x4 (&xx)[2], f32x4 (&aa)[2]) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t v = min(b + int64_t(u) * kColThreads, nv - 1);
        xx[u] = c4[v];
        aa[u] = a4[v];
      }
    };
    f32x4 xc[2], ac[2];
    load(threadIdx.x, xc, ac);
    for (int64_t b = threadIdx.x; b - threadIdx.x < nv; b += 2 * kColThreads) {   // uniform trip count
      f32x4 x[2], al[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        x[u] = xc[u];
        al[u] = ac[u];
      }
      load(b + 2 * kColThreads, xc, ac);
      if (b - threadIdx.x + 2 * kColThreads <= nv) {   // a full step (uniform): every key active
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int c = 0; c < 4; ++c) f(f32_key(x[u][c] - al[u][c]), true);
      } else {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const bool act = b + int64_t(u) * kColThreads < nv;
#pragma unroll
          for (int c = 0; c < 4; ++c) f(f32_key(x[u][c] - al[u][c]), act);
        }
      }
    }
    return;
  }
  for (int64_t b = threadIdx.x; b - threadIdx.x < m; b += 4 * kColThreads) {   // uniform trip count
    float x[4], al[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = b + int64_t(u) * kColThreads;
      x[u] = i < m ? col[i] : 0.f;
      al[u] = i < m ? alpha[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) f(f32_key(x[u] - al[u]), b + int64_t(u) * kColThreads < m);
  }
}

// Radix select of descending rank `rank` over keys[0..nk) in LDS (12 + 12 + 8
// bits): the key, and its rank among the keys equal to it.
__device__ __forceinline__ void lds_select(const uint32_t* keys, int nk, int rank, int* hist, int* s_wsum, int* s_bin,
                                           int* s_rank, uint32_t& key, int& rank_out) {
  const int tid = threadIdx.x;
  for (int b = tid; b < kColBins; b += kColThreads) hist[b] = 0;
  __syncthreads();
  for (int t = tid; t - tid < nk; t += kColThreads) {
    const bool act = t < nk;
    hist_add(hist, act ? keys[t] >> 20 : 0u, act);
  }
  __syncthreads();
  col_select(hist, kColBins, rank, s_wsum, s_bin, s_rank);
  const uint32_t b1 = uint32_t(*s_bin);
  rank = *s_rank;
  __syncthreads();
  for (int b = tid; b < kColBins; b += kColThreads) hist[b] = 0;
  __syncthreads();
  for (int t = tid; t - tid < nk; t += kColThreads) {
    const bool act = t < nk && (keys[t] >> 20) == b1;
    hist_add(hist, act ? (keys[t] >> 8) & 0xFFFu : 0u, act);
  }
  __syncthreads();
  col_select(hist, kColBins, rank, s_wsum, s_bin, s_rank);
  const uint32_t p2 = (b1 << 12) | uint32_t(*s_bin);   // key >> 8
  rank = *s_rank;
  __syncthreads();
  for (int b = tid; b < 256; b += kColThreads) hist[b] = 0;
  __syncthreads();
  for (int t = tid; t - tid < nk; t += kColThreads) {
    const bool act = t < nk && (keys[t] >> 8) == p2;
    hist_add(hist, act ? keys[t] & 0xFFu : 0u, act);
  }
  __syncthreads();
  col_select(hist, 256, rank, s_wsum, s_bin, s_rank);
  key = (p2 << 8) | uint32_t(*s_bin);
  rank_out = *s_rank;
  __syncthreads();
}

// The bins of hist[0..nb) (descending digit order) holding descending ranks ra and rb (-1: not
// wanted), and the ranks within them: out = {bin of ra, rank in it, bin of rb, rank in it}.
__device__ __forceinline__ void col_select2(const int* hist, int nb, int ra, int rb, int* s_wsum, int* out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = ceil_div(nb, kColThreads);
  int hv[4], tot = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int b = nb - 1 - (tid * per + u);
    hv[u] = u < per && b >= 0 ? hist[b] : 0;
    tot += hv[u];
  }
  int incl = tot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int cum = incl - tot;
  for (int w = 0; w < wave; ++w) cum += s_wsum[w];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (u < per) {
      const int bin = nb - 1 - (tid * per + u);
      if (cum <= ra && ra < cum + hv[u]) {
        out[0] = bin;
        out[1] = ra - cum;
      }
      if (cum <= rb && rb < cum + hv[u]) {
        out[2] = bin;
        out[3] = rb - cum;
      }
    }
    cum += hv[u];
  }
  __syncthreads();
}

// Window bounds from the nk sample keys: k_hi at least the key of descending rank rh, k_lo at
// most the key of rank rl (rh or rl -1: that bound stays open), both ranks found together by
// two 12-bit radix passes, so the bounds are the ranks' 24-bit key prefixes widened to whole
// prefixes.  h2 holds two histograms [2][kColBins].
__device__ __forceinline__ void window_bounds(const uint32_t* keys, int nk, int rh, int rl, int* h1, int* h2,
                                              int* s_wsum, int* s_sel, uint32_t& k_hi, uint32_t& k_lo) {
  const int tid = threadIdx.x;
  for (int b = tid; b < kColBins; b += kColThreads) {
    h1[b] = 0;
    h2[b] = 0;
    h2[kColBins + b] = 0;
  }
  __syncthreads();
  for (int t = tid; t - tid < nk; t += kColThreads) {
    const bool act = t < nk;
    hist_add(h1, act ? keys[t] >> 20 : 0u, act);
  }
  __syncthreads();
  col_select2(h1, kColBins, rh, rl, s_wsum, s_sel);
  const uint32_t bh = uint32_t(s_sel[0]), bl = uint32_t(s_sel[2]);
  const int qh = s_sel[1], ql = s_sel[3];
  __syncthreads();   // every thread has read s_sel
  for (int t = tid; t - tid < nk; t += kColThreads) {
    const uint32_t u = t < nk ? keys[t] : 0u;
    const bool ah = t < nk && rh >= 0 && (u >> 20) == bh;
    hist_add(h2, ah ? (u >> 8) & 0xFFFu : 0u, ah);
    const bool al = t < nk && rl >= 0 && (u >> 20) == bl;
    hist_add(h2 + kColBins, al ? (u >> 8) & 0xFFFu : 0u, al);
  }
  __syncthreads();
  if (rh >= 0) {
    col_select2(h2, kColBins, qh, -1, s_wsum, s_sel);
    k_hi = (((bh << 12) | uint32_t(s_sel[0])) << 8) | 0xFFu;
    __syncthreads();
  }
  if (rl >= 0) {
    col_select2(h2 + kColBins, kColBins, ql, -1, s_wsum, s_sel);
    k_lo = ((bl << 12) | uint32_t(s_sel[0])) << 8;
    __syncthreads();
  }
}

// Appends the keys with take == true to keys[] (wave-aggregated slots);
// slots past the capacity set *ovf instead.
__device__ __forceinline__ void lds_append(uint32_t* keys, int* s_nk, int* s_ovf, uint32_t u, bool take) {
  const uint64_t bm = __ballot(take);
  if (!bm) return;
  const int lead = __ffsll((unsigned long long)bm) - 1;
  int base = 0;
  if ((threadIdx.x & 63) == lead) base = atomicAdd(s_nk, __popcll(bm));
  base = __builtin_amdgcn_readlane(base, lead);
  const int at = base + __popcll(bm & lanemask_lt());
  if (take && at < kColCap) keys[at] = u;
  if (take && at >= kColCap) *s_ovf = 1;
}

// Column order statistic.  Columns that fit in LDS are copied there whole.
// Longer ones: a sample of about 4096 keys in 32-key segments (one segment per
// 512 keys or sparser) is copied to LDS and two of its order statistics bound a
// key window expected to hold the wanted rank (4 standard deviations of the
// sample rank plus 8); one pass over the column then counts the keys above the
// window and copies the window's keys to LDS (per-wave slots, then packed),
// and the rank is selected there.
// When the window misses the rank or overflows LDS, the exact radix passes
// over the column run instead.
__global__ __launch_bounds__(kColThreads) void k_qb_cols(const float* __restrict__ sT,
                                                         const float* __restrict__ alpha, float* __restrict__ beta,
                                                         BalanceArgs a) {
  extern __shared__ __attribute__((aligned(16))) int hist[];   // [kColBins], then [kColCap] keys
  uint32_t* keys = reinterpret_cast<uint32_t*>(hist + kColBins);
  __shared__ int s_wsum[kColThreads / 64], s_wcnt[kColThreads / 64], s_bin, s_rank, s_nk, s_ovf, s_above, s_sel[4];
  __shared__ uint32_t s_min;
  const int j = blockIdx.x, tid = threadIdx.x;
  // block blockIdx.y's segment of column j: beta_rows keys from row blockIdx.y * beta_rows
  const int64_t m = a.beta_rows, r0 = int64_t(blockIdx.y) * m;
  const float* col = sT + int64_t(j) * a.m + r0;
  alpha += r0;
  beta += int64_t(blockIdx.y) * a.n;
  const int rank0 = int(a.quantile ? a.rank_col : a.q);   // 0-based rank in descending order
  if (tid == 0) {
    s_nk = 0;
    s_ovf = 0;
    s_above = 0;
    s_min = 0xFFFFFFFFu;
  }
  __syncthreads();
  // ---- key window [k_lo, k_hi]
  uint32_t k_lo = 0, k_hi = 0xFFFFFFFFu;
  if (m > kColCap) {
    // at most 128 segments of 32 keys: 4096 samples, within kColCap
    const int64_t period = 32 * std::max<int64_t>(16, ceil_div64(m, 4096));
    const int64_t nseg = ceil_div64(m, period);
    for (int64_t t = tid; t - tid < nseg * 32; t += kColThreads) {   // uniform trip count
      const int64_t i = (t >> 5) * period + (t & 31);
      const bool act = t < nseg * 32 && i < m;
      const uint32_t u = act ? f32_key(col[i] - alpha[i]) : 0u;
      lds_append(keys, &s_nk, &s_ovf, u, act);
    }
    __syncthreads();
    const int ns = min(s_nk, kColCap);
    const bool sampled = !s_ovf && ns > 0;
    __syncthreads();   // every thread has read the counters
    if (sampled) {
      const double rs = double(rank0) * double(ns) / double(m);
      const int dev = int(4.0 * sqrt(fmax(rs * (1.0 - rs / double(ns)), 0.0))) + 8;
      const int r_hi = int(rs) - dev, r_lo = int(rs) + dev;
      // second-level histograms in the key area above the (at most 4096) samples
      window_bounds(keys, ns, r_hi > 0 ? r_hi : -1, r_lo < ns - 1 ? r_lo : -1, hist,
                    reinterpret_cast<int*>(keys + 4096), s_wsum, s_sel, k_hi, k_lo);
    }
    if (tid == 0) {
      s_nk = 0;
      s_ovf = 0;
    }
    __syncthreads();
  }
  // ---- one pass: keys above the window counted, the window's keys to LDS
  int above = 0;
  uint32_t mn = 0xFFFFFFFFu;   // least key above the window
  uint32_t* wk = keys;         // the window's keys, contiguous
  int nk;
  bool w_ovf;
  if (m <= kColCap) {   // the whole column: one shared append counter
    col_scan(col, alpha, m, [&](uint32_t u, bool act) { lds_append(keys, &s_nk, &s_ovf, u, act); });
    __syncthreads();
    nk = s_nk;
    w_ovf = s_ovf;
  } else {
    // each wave appends to slots of its own (no shared counter in the loop),
    // then the waves' keys are packed after those slots
    const int wave = tid >> 6, lane = tid & 63;
    uint32_t* slots = keys + wave * kColWaveSlots;
    int wcnt = 0;
    const uint32_t span = k_hi - k_lo;   // k_lo <= k_hi: u is in the window iff u - k_lo <= span
    col_scan(col, alpha, m, [&](uint32_t u, bool act) {
      const bool up = act && u > k_hi;
      above += up;
      mn = min(mn, up ? u : 0xFFFFFFFFu);
      const bool take = act && u - k_lo <= span;
      const uint64_t bm = __ballot(take);
      if (!bm) return;
      const int at = wcnt + int(__builtin_amdgcn_mbcnt_hi(uint32_t(bm >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(bm), 0u)));
      if (take && at < kColWaveSlots) slots[at] = u;
      wcnt += __popcll(bm);
    });
    if (lane == 0) s_wcnt[wave] = wcnt;
    __syncthreads();
    int off = 0, tot = 0;
    w_ovf = false;
    for (int v = 0; v < kColThreads / 64; ++v) {
      const int c = s_wcnt[v];
      w_ovf |= c > kColWaveSlots;
      off += v < wave ? c : 0;
      tot += c;
    }
    w_ovf |= tot > kColCap - kColPackOff;
    wk = keys + kColPackOff;
    if (!w_ovf)
      for (int q = lane; q < wcnt; q += 64) wk[off + q] = slots[q];
    nk = tot;
  }
  // per-wave totals first: one LDS atomic per wave, not per thread
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    above += __shfl_xor(above, off, 64);
    mn = min(mn, uint32_t(__shfl_xor(int(mn), off, 64)));
  }
  if ((tid & 63) == 0) atomicAdd(&s_above, above);
  __syncthreads();
  const int nabove = s_above;
  const bool hit = !w_ovf && nabove <= rank0 && rank0 < nabove + nk;
  __syncthreads();   // every thread has read the counters
  uint32_t prefix;
  int rank;
  if (hit) {
    lds_select(wk, nk, rank0 - nabove, hist, s_wsum, &s_bin, &s_rank, prefix, rank);
    if (a.quantile && rank == 0)
      for (int t = tid; t < nk; t += kColThreads)
        if (wk[t] > prefix) mn = min(mn, wk[t]);
  } else {
    // exact radix passes over the column: 12 top bits, then the chosen bin's
    // keys in LDS when they fit, else two more passes (12 and 8 bits)
    mn = 0xFFFFFFFFu;
    for (int b = tid; b < kColBins; b += kColThreads) hist[b] = 0;
    if (tid == 0) s_nk = 0;
    __syncthreads();
    col_scan(col, alpha, m, [&](uint32_t u, bool act) { hist_add(hist, u >> 20, act); });
    __syncthreads();
    col_select(hist, kColBins, rank0, s_wsum, &s_bin, &s_rank);
    const uint32_t b1 = uint32_t(s_bin);
    rank = s_rank;
    const bool in_lds = hist[b1] <= kColCap;
    __syncthreads();
    if (in_lds) {
      col_scan(col, alpha, m, [&](uint32_t u, bool act) {
        if (act && (u >> 20) > b1) mn = min(mn, u);
        lds_append(keys, &s_nk, &s_ovf, u, act && (u >> 20) == b1);
      });
      __syncthreads();
      const int nb = s_nk;
      lds_select(keys, nb, rank, hist, s_wsum, &s_bin, &s_rank, prefix, rank);
      if (a.quantile && rank == 0)
        for (int t = tid; t < nb; t += kColThreads)
          if (keys[t] > prefix) mn = min(mn, keys[t]);
    } else {
      for (int b = tid; b < kColBins; b += kColThreads) hist[b] = 0;
      __syncthreads();
      col_scan(col, alpha, m, [&](uint32_t u, bool act) {
        const bool take = act && (u >> 20) == b1;
        hist_add(hist, take ? (u >> 8) & 0xFFFu : 0u, take);
      });
      __syncthreads();
      col_select(hist, kColBins, rank, s_wsum, &s_bin, &s_rank);
      const uint32_t p2 = (b1 << 12) | uint32_t(s_bin);
      rank = s_rank;
      __syncthreads();
      for (int b = tid; b < 256; b += kColThreads) hist[b] = 0;
      __syncthreads();
      col_scan(col, alpha, m, [&](uint32_t u, bool act) {
        const bool take = act && (u >> 8) == p2;
        hist_add(hist, take ? u & 0xFFu : 0u, take);
      });
      __syncthreads();
      col_select(hist, 256, rank, s_wsum, &s_bin, &s_rank);
      prefix = (p2 << 8) | uint32_t(s_bin);
      rank = s_rank;
      if (a.quantile && rank == 0)
        col_scan(col, alpha, m, [&](uint32_t u, bool act) {
          if (act && u > prefix) mn = min(mn, u);
        });
    }
  }
  float bv = key_f32(prefix);
  if (a.quantile) {
    // descending rank rank0 - 1: the least key above when exactly rank0 keys
    // lie above this one (rank within equal keys is 0), else this key again
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mn = min(mn, uint32_t(__shfl_xor(int(mn), off, 64)));
    if ((tid & 63) == 0) atomicMin(&s_min, mn);
    __syncthreads();
    const float hi = rank0 >= 1 && rank == 0 ? key_f32(s_min) : bv;
    bv = lerp_np(bv, hi, a.g_col);
  }
  if (a.bip) bv = fmaxf(bv, 0.f);
  if (tid == 0) beta[j] = bv;
}

// ------------------------------------------------------------------ exact completion (n <= 64)
__device__ __forceinline__ uint64_t f64_key(double d) {
  const uint64_t u = __double_as_longlong(d);
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}
__device__ __forceinline__ double key_f64(uint64_t k) {
  if (k == ~0ull) return INFINITY;
  return __longlong_as_double((k & 0x8000000000000000ull) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k);
}
__device__ __forceinline__ bool better64(double ka, int ia, double kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}
// Wave-wide minima without the LDS crossbar: DPP within 16-lane rows (xor 1, xor 2,
// the mirrored quad, the mirrored row), the other row of the half
// (v_permlane16_swap), then the two halves (lanes 0 and 32 read as scalars).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  return (uint64_t(dpp32<CTRL>(uint32_t(v >> 32))) << 32) | dpp32<CTRL>(uint32_t(v));
}
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
  uint64_t o = dpp64<0xB1>(v);
  v = o < v ? o : v;
  o = dpp64<0x4E>(v);
  v = o < v ? o : v;
  o = dpp64<0x141>(v);
  v = o < v ? o : v;
  o = dpp64<0x140>(v);
  v = o < v ? o : v;
  const auto lo = __builtin_amdgcn_permlane16_swap(uint32_t(v), uint32_t(v), false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap(uint32_t(v >> 32), uint32_t(v >> 32), false, false);
  const uint64_t p = (uint64_t(hi[0]) << 32) | lo[0], q = (uint64_t(hi[1]) << 32) | lo[1];
  v = p < q ? p : q;
  const uint64_t a = (uint64_t(uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v >> 32)), 0))) << 32) |
                     uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v)), 0));
  const uint64_t b = (uint64_t(uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v >> 32)), 32))) << 32) |
                     uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v)), 32));
  return a < b ? a : b;
}
__device__ __forceinline__ int wave_min_i32(int v) {
  v = min(v, int(dpp32<0xB1>(uint32_t(v))));
  v = min(v, int(dpp32<0x4E>(uint32_t(v))));
  v = min(v, int(dpp32<0x141>(uint32_t(v))));
  v = min(v, int(dpp32<0x140>(uint32_t(v))));
  const auto r = __builtin_amdgcn_permlane16_swap(uint32_t(v), uint32_t(v), false, false);
  v = min(int(r[0]), int(r[1]));
  return min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 32));
}
__device__ __forceinline__ void wave_argbest64(double& key, int& ix) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const double ok = __shfl_xor(key, off, 64);
    const int oi = __shfl_xor(ix, off, 64);
    if (better64(ok, oi, key, ix)) {
      key = ok;
      ix = oi;
    }
  }
}

// Move costs of one source expert e (one row of M): for every target j, the
// cheapest s_te − s_tj over the tokens t that hold e but not j, ties to the
// lower token index.  Thread (slice, j) scans every 16th token of e's list
// (batches of 8 tokens, loads first); slices meet in LDS.
__device__ __forceinline__ void qb_row_costs(const BalanceArgs& a, const int32_t* __restrict__ xi,
                                             const int32_t* __restrict__ lst, int e, int cnt_e,
                                             unsigned long long* Mk, int* arg, unsigned long long* pk, int* pi_) {
  const int n = a.n, k = a.k, tid = threadIdx.x, j = tid & 63, sl = tid >> 6;
  const int64_t m = a.m;
  unsigned long long bk = ~0ull;
  int bt = 0x7FFFFFFF;
  const int32_t* L = lst + int64_t(e) * m;
  for (int b0 = sl * 8; b0 < cnt_e; b0 += 16 * 8) {
    int t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = L[min(b0 + u, cnt_e - 1)];
    float se[8], sj[8];
    bool has[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float* sr = a.s + int64_t(t[u]) * n;
      se[u] = sr[e];
      sj[u] = j < n ? sr[j] : 0.f;
      has[u] = false;
      for (int r = 0; r < k; ++r) has[u] |= xi[int64_t(t[u]) * k + r] == j;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (b0 + u < cnt_e && j < n && !has[u]) {
        const unsigned long long key = f64_key(double(se[u]) - double(sj[u]));
        if (key < bk || (key == bk && t[u] < bt)) {
          bk = key;
          bt = t[u];
        }
      }
    }
  }
  pk[sl * 64 + j] = bk;
  pi_[sl * 64 + j] = bt;
  __syncthreads();
  if (tid < 64) {
    for (int q = 1; q < 16; ++q) {
      const unsigned long long ok = pk[q * 64 + tid];
      const int ot = pi_[q * 64 + tid];
      if (ok < bk || (ok == bk && ot < bt)) {
        bk = ok;
        bt = ot;
      }
    }
    if (tid < n) {
      Mk[e * n + tid] = bk;
      arg[e * n + tid] = bt;
    }
  }
  __syncthreads();
}

// Exact completion by successive shortest paths.  xi: [m][k] assignment,
// pos: [m][k] position of token i in the list of its r-th expert, lst:
// [n][m] token lists.  M is kept in LDS and only the rows of the experts a
// moved token held before or after its move are recomputed.
__global__ __launch_bounds__(1024) void k_qb_complete(BalanceArgs a, int32_t* __restrict__ xi,
                                                      int32_t* __restrict__ pos, int32_t* __restrict__ lst) {
  __shared__ unsigned long long Mk[kCompleteMaxN * kCompleteMaxN];
  __shared__ int arg[kCompleteMaxN * kCompleteMaxN];
  __shared__ unsigned long long pk[1024];
  __shared__ int pt[1024];
  __shared__ double pi[kCompleteMaxN], dist[kCompleteMaxN];
  __shared__ int cnt[kCompleteMaxN], pred[kCompleteMaxN], vis[kCompleteMaxN], dirty[kCompleteMaxN];
  __shared__ int ptok[kCompleteMaxN];
  __shared__ int s_go, s_target, s_fail;
  __shared__ double s_D;
  const int n = a.n, k = a.k;
  const int64_t m = a.m, q = a.q;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const float* s = a.s;

  for (int j = tid; j < n; j += 1024) {
    pi[j] = double(a.beta[j]);
    cnt[j] = 0;
    dirty[j] = 1;
  }
  __syncthreads();
  // initial assignment: top-k of the exact keys s_ij − β_j (lower index on ties),
  // and the per-expert token lists (their order does not matter: every row
  // minimum breaks ties by token index)
  for (int64_t i = wave; i < m; i += 16) {
    double last = INFINITY;
    int lj = -1;
    for (int r = 0; r < k; ++r) {
      double bk = -INFINITY;
      int bj = 0x7FFFFFFF;
      if (lane < n) {
        const double v = double(s[i * n + lane]) - pi[lane];
        if (better64(last, lj, v, lane)) {
          bk = v;
          bj = lane;
        }
      }
      wave_argbest64(bk, bj);
      last = bk;
      lj = bj;
      if (lane == 0) {
        xi[i * k + r] = bj;
        const int slot = atomicAdd(&cnt[bj], 1);
        lst[int64_t(bj) * m + slot] = int(i);
        pos[i * k + r] = slot;
      }
    }
  }
  __threadfence_block();
  __syncthreads();
  int aug = 0;
  const int max_aug = int(min<int64_t>(m * k, 0x7FFFFFFF));
  for (;;) {
    // refresh the rows of M whose source expert changed
    for (int e = 0; e < n; ++e)
      if (dirty[e]) qb_row_costs(a, xi, lst, e, cnt[e], Mk, arg, pk, pt);
    __syncthreads();
    if (tid == 0) {
      int go = 0;
      for (int j = 0; j < n; ++j) {
        go |= cnt[j] > q;
        dirty[j] = 0;
      }
      s_go = go && aug < max_aug;
      s_fail = 0;
    }
    __syncthreads();
    if (!s_go) break;
    // Dijkstra from every over-full expert to the first under-full one reached
    if (wave == 0) {
      double dv = (lane < n && cnt[lane] > q) ? 0.0 : INFINITY;
      int pv = -1;
      bool done = lane >= n;
      int target = -1;
      double D = 0.0;
      // potentials and counts in registers; expert u's read back with readlane
      const double pil = lane < n ? pi[lane] : 0.0;
      const int cntl = lane < n ? cnt[lane] : 0;
      for (int it = 0; it < n; ++it) {
        // the unfinished expert of least distance, the lower index on ties
        // (dist >= 0, so its order-preserving key orders like the distance)
        const uint64_t dk = done ? ~0ull : f64_key(dv);
        const uint64_t mk = wave_min_u64(dk);
        if (mk == ~0ull) break;
        const double du = key_f64(mk);
        if (du == INFINITY) break;
        const int u = wave_min_i32(dk == mk ? lane : 64);
        if (lane == u) done = true;
        if (__builtin_amdgcn_readlane(cntl, u) < q) {
          target = u;
          D = du;
          break;
        }
        if (!done) {
          const uint64_t pb = uint64_t(__double_as_longlong(pil));
          const double piu = __longlong_as_double(
              int64_t((uint64_t(uint32_t(__builtin_amdgcn_readlane(int(uint32_t(pb >> 32)), u))) << 32) |
                      uint32_t(__builtin_amdgcn_readlane(int(uint32_t(pb)), u))));
          double w = key_f64(Mk[u * n + lane]) - piu + pil;
          w = fmax(w, 0.0);
          const double nd = du + w;
          if (nd < dv) {
            dv = nd;
            pv = u;
          }
        }
      }
      if (lane < n) {
        dist[lane] = dv;
        pred[lane] = pv;
        vis[lane] = done;
      }
      if (lane == 0) {
        s_target = target;
        s_D = D;
        s_fail = target < 0;
      }
    }
    __syncthreads();
    if (s_fail) break;
    if (tid < n) {
      const double D = s_D;
      pi[tid] -= vis[tid] ? fmin(dist[tid], D) : D;
    }
    if (wave == 0) {
      // move one token along every edge of the path (target back to source).
      // M stays exact: the source row is rescanned next round; token i joining
      // j adds it as a candidate to row j; for the other experts a of token i,
      // (a -> aa) gains candidate i and (a -> j) loses it (a rescan only if i
      // was its cheapest token).  Every edge moves the token its cost was taken from:
      // the path's tokens are read before any of them moves.
      if (lane == 0) {
        int jj = s_target, len = 0;
        while (pred[jj] >= 0) {
          ptok[len++] = arg[pred[jj] * n + jj];
          jj = pred[jj];
        }
      }
      __builtin_amdgcn_wave_barrier();
      int j = s_target, pe = 0;
      while (pred[j] >= 0) {
        const int aa = pred[j];
        const int i = __builtin_amdgcn_readfirstlane(ptok[pe++]);
        int32_t* xr = xi + int64_t(i) * k;
        int r = 0;
        for (int rr = 0; rr < k; ++rr)
          if (xr[rr] == aa) r = rr;
        const float* si = s + int64_t(i) * n;
        // row j gains candidate i for every l the token will not hold
        if (lane < n) {
          bool held = lane == j;
          for (int rr = 0; rr < k; ++rr) held |= rr != r && xr[rr] == lane;
          if (!held) {
            const unsigned long long key = f64_key(double(si[j]) - double(si[lane]));
            const int o = j * n + lane;
            if (key < Mk[o] || (key == Mk[o] && i < arg[o])) {
              Mk[o] = key;
              arg[o] = i;
            }
          }
        }
        __builtin_amdgcn_wave_barrier();
        if (lane == 0) {
          for (int rr = 0; rr < k; ++rr) {
            const int e = xr[rr];
            if (rr == r) continue;
            const unsigned long long key = f64_key(double(si[e]) - double(si[aa]));
            const int o = e * n + aa;
            if (key < Mk[o] || (key == Mk[o] && i < arg[o])) {
              Mk[o] = key;
              arg[o] = i;
            }
            if (arg[e * n + j] == i) dirty[e] = 1;
          }
          dirty[aa] = 1;
          // leave aa's list (the last entry fills the hole), join j's
          const int p = pos[int64_t(i) * k + r];
          const int last = lst[int64_t(aa) * m + cnt[aa] - 1];
          lst[int64_t(aa) * m + p] = last;
          for (int rr = 0; rr < k; ++rr)
            if (xi[int64_t(last) * k + rr] == aa) pos[int64_t(last) * k + rr] = p;
          cnt[aa] -= 1;
          lst[int64_t(j) * m + cnt[j]] = i;
          pos[int64_t(i) * k + r] = cnt[j];
          cnt[j] += 1;
          xr[r] = j;
        }
        __builtin_amdgcn_wave_barrier();
        j = aa;
      }
    }
    __threadfence_block();
    __syncthreads();
    ++aug;
  }
  __syncthreads();
  // outputs: idx by descending s_ij − π_j (lower index on ties), counts, β, info
  for (int64_t i = wave; i < m; i += 16) {
    const int32_t* xr = xi + i * k;
    double v = -INFINITY;
    int jj = 0x7FFFFFFF;
    if (lane < k) {
      jj = xr[lane];
      v = double(s[i * n + jj]) - pi[jj];
    }
    // rank of lane's element among the k (k <= 64)
    int rank = 0;
    for (int r = 0; r < k; ++r) {
      const double ov = __shfl(v, r, 64);
      const int oj = __shfl(jj, r, 64);
      if (lane < k && better64(ov, oj, v, jj)) ++rank;
    }
    if (lane < k) a.idx[i * k + rank] = jj;
  }
  int bal = 1;
  for (int j = tid; j < n; j += 1024) {
    a.counts[j] = cnt[j];
    a.beta[j] = float(pi[j]);
  }
  __syncthreads();
  if (tid == 0) {
    for (int j = 0; j < n; ++j) bal &= cnt[j] == q;
    if (a.info) {
      a.info[1] = aug;
      a.info[2] = bal && !s_fail;
      a.info[3] = s_fail;
    }
  }
}

// ------------------------------------------------------------------ exact completion, LDS-resident form
// The same successive shortest paths for n <= 128 when the assignment fits in LDS (per token a
// mask of the experts it holds, per expert a 16-bit token list):
//  * k_qbc_init (one wave per token, many workgroups): x = top-k of the exact keys s_ij − β_j;
//  * k_qbc_minit (one workgroup per expert): the initial M;
//  * k_qbc_solve (one workgroup): x, the lists and, for n <= 64, M (fp64 values and tokens) in
//    LDS (for n <= 128 M lives in global memory, two experts per lane).  A token that leaves
//    expert a stales only the entries of row a (and of its other experts' rows, column j) whose
//    cheapest token it was; each round recomputes those (row, column) pairs, one wave per pair
//    with the lanes over the row's tokens, or whole rows (lanes over the columns, the row's
//    tokens split over waves that meet in LDS) when many are stale.  The lists are kept across
//    rounds when every expert's list fits its largest size (an over-full expert only shrinks, an
//    under-full one grows to q), else the stale rows are listed anew each round.  Dijkstra on one
//    wave reads precomputed reduced costs; its minimum is two 32-bit DPP reductions (the
//    distances are >= 0, so their raw bits order like their values) and the arg-min lane a
//    ballot.  The tokens of the path's edges are read before any of them moves, so every edge
//    moves the token its cost was taken from;
//  * k_qbc_out (one wave per token): idx by descending s_ij − π_j.
// Candidates compare as fp64 values with the lower token index on ties.
constexpr int kFastMaxN = 128;
constexpr int kFastLdsLimit = 150 * 1024;   // dynamic LDS the solve kernel may take (static arrays aside)

static int fast_npl(int n) { return n <= 64 ? 1 : 2; }
// n <= 64: M (fp64), its tokens and the reduced costs; n <= 128: the wave partials; then the
// token masks and the 16-bit token lists
static size_t fast_lds_bytes(int npl, int64_t m, int k) {
  const size_t fixed = npl == 1 ? size_t(64 * 64) * 20 : size_t(16 * 128) * 12;
  return fixed + size_t(m) * 8 * npl + size_t(round_up(int(m * k) * 2, 16));
}
static bool fast_complete_ok(int64_t m, int n, int k) {
  return n <= kFastMaxN && m <= 65535 && m * k <= (1 << 20) &&
         fast_lds_bytes(fast_npl(n), m, k) <= size_t(kFastLdsLimit);
}
bool exact_completion_supported(int64_t m, int n, int k) { return n <= kCompleteMaxN || fast_complete_ok(m, n, k); }

__global__ __launch_bounds__(256) void k_qbc_init(BalanceArgs a, int32_t* __restrict__ xi) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t i = int64_t(blockIdx.x) * 4 + wave;
  if (i >= a.m) return;
  const int n = a.n, k = a.k;
  // lane holds experts lane and lane + 64
  double v[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int j = lane + 64 * u;
    v[u] = j < n ? double(a.s[i * n + j]) - double(a.beta[j]) : -INFINITY;
  }
  double last = INFINITY;
  int lj = -1;
  for (int r = 0; r < k; ++r) {
    double bk = -INFINITY;
    int bj = 0x7FFFFFFF;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = lane + 64 * u;
      if (j < n && better64(last, lj, v[u], j) && better64(v[u], j, bk, bj)) {
        bk = v[u];
        bj = j;
      }
    }
    wave_argbest64(bk, bj);
    last = bk;
    lj = bj;
    if (lane == 0) xi[i * k + r] = bj;
  }
}

__global__ __launch_bounds__(256) void k_qbc_out(BalanceArgs a, const int32_t* __restrict__ xi,
                                                 const double* __restrict__ pi) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t i = int64_t(blockIdx.x) * 4 + wave;
  if (i >= a.m) return;
  const int n = a.n, k = a.k;
  double v = -INFINITY;
  int jj = 0x7FFFFFFF;
  if (lane < k) {
    jj = xi[i * k + lane];
    v = double(a.s[i * n + jj]) - pi[jj];
  }
  int rank = 0;   // rank of the lane's expert among the token's k (k <= 64)
  for (int r = 0; r < k; ++r) {
    const double ov = __shfl(v, r, 64);
    const int oj = __shfl(jj, r, 64);
    if (lane < k && better64(ov, oj, v, jj)) ++rank;
  }
  if (lane < k) a.idx[i * k + rank] = jj;
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t b = uint64_t(__double_as_longlong(v));
  return __longlong_as_double(
      int64_t((uint64_t(uint32_t(__builtin_amdgcn_readlane(int(uint32_t(b >> 32)), l))) << 32) |
              uint32_t(__builtin_amdgcn_readlane(int(uint32_t(b)), l))));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const uint64_t b = uint64_t(__double_as_longlong(v));
  const uint32_t lo = uint32_t(__builtin_amdgcn_update_dpp(0, int(uint32_t(b)), CTRL, 0xF, 0xF, false));
  const uint32_t hi = uint32_t(__builtin_amdgcn_update_dpp(0, int(uint32_t(b >> 32)), CTRL, 0xF, 0xF, false));
  return __longlong_as_double(int64_t((uint64_t(hi) << 32) | lo));
}
// Wave-wide fp64 minimum (no NaN inputs): DPP within 16-lane rows, the row swap, the two halves.
__device__ __forceinline__ double wave_min_f64(double v) {
  v = fmin(v, dpp_d<kDppXor1>(v));
  v = fmin(v, dpp_d<kDppXor2>(v));
  v = fmin(v, dpp_d<kDppHalfMirror>(v));
  v = fmin(v, dpp_d<kDppMirror>(v));
  const uint64_t b = uint64_t(__double_as_longlong(v));
  const auto lo = __builtin_amdgcn_permlane16_swap(uint32_t(b), uint32_t(b), false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap(uint32_t(b >> 32), uint32_t(b >> 32), false, false);
  v = fmin(__longlong_as_double(int64_t((uint64_t(hi[0]) << 32) | lo[0])),
           __longlong_as_double(int64_t((uint64_t(hi[1]) << 32) | lo[1])));
  return fmin(readlane_f64(v, 0), readlane_f64(v, 32));
}

// All-lane fp64 minimum (no NaN inputs): DPP within 16-lane rows, then the row and half swaps.
__device__ __forceinline__ double wave_min_f64_all(double v) {
  v = fmin(v, dpp_d<kDppXor1>(v));
  v = fmin(v, dpp_d<kDppXor2>(v));
  v = fmin(v, dpp_d<kDppHalfMirror>(v));
  v = fmin(v, dpp_d<kDppMirror>(v));
  uint64_t b = uint64_t(__double_as_longlong(v));
  auto lo = __builtin_amdgcn_permlane16_swap(uint32_t(b), uint32_t(b), false, false);
  auto hi = __builtin_amdgcn_permlane16_swap(uint32_t(b >> 32), uint32_t(b >> 32), false, false);
  v = fmin(__longlong_as_double(int64_t((uint64_t(hi[0]) << 32) | lo[0])),
           __longlong_as_double(int64_t((uint64_t(hi[1]) << 32) | lo[1])));
  b = uint64_t(__double_as_longlong(v));
  lo = __builtin_amdgcn_permlane32_swap(uint32_t(b), uint32_t(b), false, false);
  hi = __builtin_amdgcn_permlane32_swap(uint32_t(b >> 32), uint32_t(b >> 32), false, false);
  return fmin(__longlong_as_double(int64_t((uint64_t(hi[0]) << 32) | lo[0])),
              __longlong_as_double(int64_t((uint64_t(hi[1]) << 32) | lo[1])));
}

// All-lane u32 minimum: DPP within 16-lane rows, then the row and half swaps.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(int(0xFFFFFFFFu), int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t wave_min_u32_all(uint32_t v) {
  v = min(v, dpp_u<kDppXor1>(v));
  v = min(v, dpp_u<kDppXor2>(v));
  v = min(v, dpp_u<kDppHalfMirror>(v));
  v = min(v, dpp_u<kDppMirror>(v));
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = min(uint32_t(r[0]), uint32_t(r[1]));
  r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return min(uint32_t(r[0]), uint32_t(r[1]));
}

// u32 minimum of the wave in lane 63's result (scalar): DPP within 16-lane rows, then the GFX9
// row broadcasts (row 0's lane 15 into row 1, row 2's into row 3; then lane 31 into rows 2 and 3).
__device__ __forceinline__ uint32_t wave_min_u32_bcast(uint32_t v) {
  v = min(v, dpp_u<kDppXor1>(v));
  v = min(v, dpp_u<kDppXor2>(v));
  v = min(v, dpp_u<kDppHalfMirror>(v));
  v = min(v, dpp_u<kDppMirror>(v));
  v = min(v, uint32_t(__builtin_amdgcn_update_dpp(int(v), int(v), 0x142, 0xA, 0xF, false)));   // row_bcast:15
  v = min(v, uint32_t(__builtin_amdgcn_update_dpp(int(v), int(v), 0x143, 0xC, 0xF, false)));   // row_bcast:31
  return uint32_t(__builtin_amdgcn_readlane(int(v), 63));
}

constexpr int kPairMax = 64;   // stale (row, column) pairs recomputed one by one; more: whole rows

// Experts held by one token: NPL 64-bit words (experts 64 c + bit of word c).
template <int NPL>
struct XMask {
  uint64_t w[NPL];
};
template <int NPL>
__device__ __forceinline__ bool xm_has(const XMask<NPL>& h, int j) {
  if constexpr (NPL == 1) return (h.w[0] >> j) & 1ull;
  else return ((j < 64 ? h.w[0] : h.w[1]) >> (j & 63)) & 1ull;
}
template <int NPL>
__device__ __forceinline__ void xm_flip(XMask<NPL>& h, int j) {
  if constexpr (NPL == 1) h.w[0] ^= 1ull << j;
  else if (j < 64) h.w[0] ^= 1ull << j;
  else h.w[1] ^= 1ull << (j - 64);
}
__device__ __forceinline__ uint64_t col_bits(int c, int n) {   // experts 64 c .. of n present in word c
  const int v = n - 64 * c;
  return v <= 0 ? 0ull : v >= 64 ? ~0ull : (1ull << v) - 1ull;
}
// a lane's value of expert j (uniform), the lane holding experts lane + 64 c
template <int NPL>
__device__ __forceinline__ float lane_of(const float (&v)[NPL], int j) {
  if constexpr (NPL == 1) return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v[0]), j));
  else
    return j < 64 ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v[0]), j))
                  : __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v[1]), j - 64));
}

// The initial M, one workgroup per row e (4 waves): the tokens holding e listed in LDS from x, the
// lanes over the columns j, each wave over a quarter of the tokens, the waves meeting in LDS.
// M[e][j] = min over tokens t holding e and not j of s_te − s_tj (lower token on ties).
template <int NPL>
__global__ __launch_bounds__(256) void k_qbc_minit(BalanceArgs a, const int32_t* __restrict__ xi,
                                                   double* __restrict__ gM, int* __restrict__ gArg) {
  constexpr int NN = 64 * NPL;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  double* pk = reinterpret_cast<double*>(lds_raw);   // [4][NN]
  int* pt = reinterpret_cast<int*>(pk + 4 * NN);      // [4][NN]
  int* toks = pt + 4 * NN;                            // [m] tokens holding e
  __shared__ int s_len;
  const int n = a.n, k = a.k, m = int(a.m), e = blockIdx.x;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  if (tid == 0) s_len = 0;
  __syncthreads();
  // 16 loads of x in flight per thread, then the matches appended
  for (int o0 = tid; o0 < m * k; o0 += 256 * 16) {
    int v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = o0 + 256 * u < m * k ? xi[o0 + 256 * u] : -1;
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (v[u] == e) toks[atomicAdd(&s_len, 1)] = (o0 + 256 * u) / k;
  }
  __syncthreads();
  const int len = s_len, lo = len * wave / 4, hi = len * (wave + 1) / 4;
  double bv[NPL];
  int bt[NPL];
#pragma unroll
  for (int c = 0; c < NPL; ++c) {
    bv[c] = INFINITY;
    bt[c] = 0x7FFFFFFF;
  }
  for (int b = lo; b < hi; b += 8) {
    int t[8];
    float sv[8][NPL];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = toks[min(b + u, hi - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int c = 0; c < NPL; ++c) sv[u][c] = lane + 64 * c < n ? a.s[int64_t(t[u]) * n + lane + 64 * c] : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (b + u < hi) {
        const float se = lane_of<NPL>(sv[u], e);
#pragma unroll
        for (int c = 0; c < NPL; ++c) {
          const int j = lane + 64 * c;
          bool held = false;
          for (int r = 0; r < k; ++r) held |= xi[int64_t(t[u]) * k + r] == j;
          if (j < n && !held) {
            const double v = double(se) - double(sv[u][c]);
            if (v < bv[c] || (v == bv[c] && t[u] < bt[c])) {
              bv[c] = v;
              bt[c] = t[u];
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < NPL; ++c) {
    pk[wave * NN + lane + 64 * c] = bv[c];
    pt[wave * NN + lane + 64 * c] = bt[c];
  }
  __syncthreads();
  if (tid < NN) {
    double cv = INFINITY;
    int ct = 0x7FFFFFFF;
    for (int w = 0; w < 4; ++w) {
      const double ov = pk[w * NN + tid];
      const int ot = pt[w * NN + tid];
      if (ov < cv || (ov == cv && ot < ct)) {
        cv = ov;
        ct = ot;
      }
    }
    gM[e * NN + tid] = cv;
    gArg[e * NN + tid] = ct;
  }
}

// NPL experts per lane (n <= 64 NPL).  NPL = 1: M, its tokens and the reduced costs in LDS;
// NPL = 2: in global memory (gM, gArg, gW), the rest in LDS.
template <int NPL>
__global__ __launch_bounds__(1024) void k_qbc_solve(BalanceArgs a, int32_t* __restrict__ xi,
                                                    double* __restrict__ pi_out, double* __restrict__ gM,
                                                    int* __restrict__ gArg, double* __restrict__ gW, int list_cap) {
  constexpr int NN = 64 * NPL;
  constexpr int TB = 16 / NPL;   // tokens per batch in the whole-row refresh
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  double* Md;     // [NN][NN] M (INFINITY: no token)
  int* arg;       // [NN][NN] its tokens
  double* W;      // [NN][NN] reduced costs (Dijkstra)
  double* pk;     // [16][NN] wave partials (whole-row refresh)
  int* pt;
  unsigned char* rest;
  if constexpr (NPL == 1) {
    Md = reinterpret_cast<double*>(lds_raw);
    arg = reinterpret_cast<int*>(Md + NN * NN);
    W = reinterpret_cast<double*>(arg + NN * NN);
    pk = W;   // the partials live only while the reduced costs are dead
    pt = reinterpret_cast<int*>(pk + 16 * NN);
    rest = reinterpret_cast<unsigned char*>(W + NN * NN);
  } else {
    Md = gM;
    arg = gArg;
    W = gW;
    pk = reinterpret_cast<double*>(lds_raw);
    pt = reinterpret_cast<int*>(pk + 16 * NN);
    rest = reinterpret_cast<unsigned char*>(pt + 16 * NN);
  }
  const int n = a.n, k = a.k, m = int(a.m), q = int(a.q);
  XMask<NPL>* hm = reinterpret_cast<XMask<NPL>*>(rest);    // [m] experts held by each token
  // token lists: per expert, kept across rounds when every list fits its largest size (an
  // over-full expert only shrinks, an under-full one grows to q); else the rows being refreshed,
  // listed anew each round
  uint16_t* lst = reinterpret_cast<uint16_t*>(hm + m);
  __shared__ double pi[NN], dist[NN];
  __shared__ uint64_t dcol[NN * NPL];   // per row of M: the columns whose cheapest token may have left
  __shared__ int cnt[NN], pred[NN], vis[NN], roff[NN], rfill[NN], drow[NN];
  __shared__ int path_a[NN], path_j[NN], path_t[NN];
  __shared__ uint8_t pair_e[kPairMax], pair_j[kPairMax];
  __shared__ uint64_t s_dm[NPL];
  __shared__ int s_nd, s_np, s_go, s_target, s_fail, s_len, s_keep;
  __shared__ double s_D;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const float* __restrict__ s = a.s;

  if (tid < NN) {
    pi[tid] = tid < n ? double(a.beta[tid]) : 0.0;
    cnt[tid] = 0;
#pragma unroll
    for (int c = 0; c < NPL; ++c) dcol[tid * NPL + c] = 0ull;   // M starts exact (k_qbc_minit)
  }
  if constexpr (NPL == 1)
    for (int o = tid; o < NN * NN; o += 1024) {
      Md[o] = gM[o];
      arg[o] = gArg[o];
    }
  __syncthreads();
  for (int t = tid; t < m; t += 1024) {
    XMask<NPL> h{};
    for (int r = 0; r < k; ++r) {
      const int e = xi[int64_t(t) * k + r];
      xm_flip(h, e);
      atomicAdd(&cnt[e], 1);
    }
    hm[t] = h;
  }
  __syncthreads();
  // persistent lists when Σ_e max(c_e, q) fits
  if (wave == 0) {
    int cap[NPL], incl[NPL], tot = 0;
#pragma unroll
    for (int c = 0; c < NPL; ++c) {
      const int r = lane + 64 * c;
      cap[c] = r < n ? max(cnt[r], q) : 0;
      incl[c] = cap[c];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl[c], off, 64);
        if (lane >= off) incl[c] += o;
      }
      roff[r] = tot + incl[c] - cap[c];
      rfill[r] = 0;
      tot += __shfl(incl[c], 63, 64);
    }
    if (lane == 0) s_keep = tot <= list_cap;
  }
  __syncthreads();
  const bool keep = s_keep;
  if (keep) {
    for (int t = tid; t < m; t += 1024) {
      const XMask<NPL> ht = hm[t];
#pragma unroll
      for (int c = 0; c < NPL; ++c)
        for (uint64_t h = ht.w[c]; h; h &= h - 1) {
          const int e = 64 * c + __builtin_ctzll(h);
          lst[roff[e] + atomicAdd(&rfill[e], 1)] = uint16_t(t);
        }
    }
  }
  int aug = 0;
  const int max_aug = m * k;
  auto over_full = [&]() {   // wave 0: any expert over-full (and augmentations left)?
    bool over = false;
#pragma unroll
    for (int c = 0; c < NPL; ++c) over |= lane + 64 * c < n && cnt[lane + 64 * c] > q;
    const uint64_t ov = __ballot(over);
    if (lane == 0) s_go = ov != 0 && aug < max_aug;
  };
  if (wave == 0) over_full();
  if (wave == 0 && lane == 0) s_fail = 0;
  __syncthreads();
  for (;;) {
    if (!s_go) break;
    // ---- refresh the entries of M whose cheapest token may have left
    if (wave == 0) {
      // rows lane + 64 c, in the order c, then lane
      int cc[NPL], pc[NPL], ci[NPL], pi_[NPL];
      bool dj[NPL];
      uint64_t dmk[NPL];
      int tot_c = 0, tot_p = 0;
#pragma unroll
      for (int c = 0; c < NPL; ++c) {
        const int r = lane + 64 * c;
        uint64_t any = 0;
        int pop = 0;
#pragma unroll
        for (int w = 0; w < NPL; ++w) {
          const uint64_t d = r < n ? dcol[r * NPL + w] : 0ull;
          any |= d;
          pop += __popcll(d);
        }
        dj[c] = any != 0ull;
        cc[c] = dj[c] ? cnt[r] : 0;
        pc[c] = pop;
        int incl = cc[c], pincl = pc[c];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int o = __shfl_up(incl, off, 64), po = __shfl_up(pincl, off, 64);
          if (lane >= off) {
            incl += o;
            pincl += po;
          }
        }
        ci[c] = tot_c + incl - cc[c];
        pi_[c] = tot_p + pincl - pc[c];
        tot_c += __shfl(incl, 63, 64);
        tot_p += __shfl(pincl, 63, 64);
        dmk[c] = __ballot(dj[c]);
      }
      int dbase = 0;
#pragma unroll
      for (int c = 0; c < NPL; ++c) {
        const int r = lane + 64 * c;
        if (dj[c]) {
          if (!keep) {
            roff[r] = ci[c];
            rfill[r] = 0;
          }
          drow[dbase + __popcll(dmk[c] & ((1ull << lane) - 1ull))] = r;
          if (tot_p <= kPairMax) {
            int p = pi_[c];
#pragma unroll
            for (int w = 0; w < NPL; ++w)
              for (uint64_t b = dcol[r * NPL + w]; b; b &= b - 1) {
                pair_e[p] = uint8_t(r);
                pair_j[p] = uint8_t(64 * w + __builtin_ctzll(b));
                ++p;
              }
          }
        }
        dbase += __popcll(dmk[c]);
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int c = 0; c < NPL; ++c)
#pragma unroll
        for (int w = 0; w < NPL; ++w) dcol[(lane + 64 * c) * NPL + w] = 0ull;
      if (lane == 0) {
        s_nd = dbase;
        s_np = tot_p;
#pragma unroll
        for (int c = 0; c < NPL; ++c) s_dm[c] = dmk[c];
      }
    }
    __syncthreads();
    const int D = s_nd, P = s_np;
    if (D > 0) {
      uint64_t dm[NPL];
#pragma unroll
      for (int c = 0; c < NPL; ++c) dm[c] = s_dm[c];
      for (int t = keep ? m : tid; t < m; t += 1024) {
        const XMask<NPL> ht = hm[t];
#pragma unroll
        for (int c = 0; c < NPL; ++c) {
          uint64_t h = ht.w[c] & dm[c];
          while (h) {
            const int e = 64 * c + __builtin_ctzll(h);
            h &= h - 1;
            lst[roff[e] + atomicAdd(&rfill[e], 1)] = uint16_t(t);
          }
        }
      }
      __syncthreads();
      if (P <= kPairMax) {
        // one wave per (row, column) pair, lanes over the row's tokens
        for (int p = wave; p < P; p += 16) {
          const int e = pair_e[p], j = pair_j[p];
          const int len = cnt[e], beg = roff[e];
          double bv = INFINITY;
          int bt = 0x7FFFFFFF;
          for (int c0 = 0; c0 < len; c0 += 64 * 8) {
            int t[8];
            float se[8], sj[8];
            bool hj[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) t[u] = lst[beg + min(c0 + 64 * u + lane, len - 1)];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              se[u] = s[int64_t(t[u]) * n + e];
              sj[u] = s[int64_t(t[u]) * n + j];
              hj[u] = xm_has(hm[t[u]], j);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              if (c0 + 64 * u + lane < len && !hj[u]) {
                const double v = double(se[u]) - double(sj[u]);
                if (v < bv || (v == bv && t[u] < bt)) {
                  bv = v;
                  bt = t[u];
                }
              }
            }
          }
          const double mv = wave_min_f64_all(bv);
          const int mt = wave_min_i_dpp(bv == mv ? bt : 0x7FFFFFFF);
          if (lane == 0) {
            Md[e * NN + j] = mv;
            arg[e * NN + j] = mt;
          }
        }
        __syncthreads();
      } else {
        // whole rows, lanes over the columns; rounds of at most 16 rows, a row's tokens split over wpr waves
        for (int o = tid; o < D * NN; o += 1024) {
          const int e = drow[o / NN], j = o % NN;
          Md[e * NN + j] = INFINITY;
          arg[e * NN + j] = 0x7FFFFFFF;
        }
        for (int r0 = 0; r0 < D; r0 += 16) {
          const int R = min(16, D - r0);
          const int wpr = 16 / R;
          const int ri = wave / wpr, sub = wave - ri * wpr;
          double bv[NPL];
          int bt[NPL];
#pragma unroll
          for (int c = 0; c < NPL; ++c) {
            bv[c] = INFINITY;
            bt[c] = 0x7FFFFFFF;
          }
          if (ri < R) {
            const int e = __builtin_amdgcn_readfirstlane(drow[r0 + ri]);
            const int len = cnt[e], beg = roff[e];
            const int lo = beg + len * sub / wpr, hi = beg + len * (sub + 1) / wpr;
            for (int b = lo; b < hi; b += TB) {
              int t[TB];
              float sv[TB][NPL];
              XMask<NPL> hu[TB];
#pragma unroll
              for (int u = 0; u < TB; ++u) t[u] = lst[min(b + u, hi - 1)];
#pragma unroll
              for (int u = 0; u < TB; ++u)
#pragma unroll
                for (int c = 0; c < NPL; ++c)
                  sv[u][c] = lane + 64 * c < n ? s[int64_t(t[u]) * n + lane + 64 * c] : 0.f;
#pragma unroll
              for (int u = 0; u < TB; ++u) hu[u] = hm[t[u]];
#pragma unroll
              for (int u = 0; u < TB; ++u) {
                if (b + u < hi) {
                  const float sev = lane_of<NPL>(sv[u], e);
#pragma unroll
                  for (int c = 0; c < NPL; ++c) {
                    if (lane + 64 * c < n && !((hu[u].w[c] >> lane) & 1ull)) {
                      const double v = double(sev) - double(sv[u][c]);
                      if (v < bv[c] || (v == bv[c] && t[u] < bt[c])) {
                        bv[c] = v;
                        bt[c] = t[u];
                      }
                    }
                  }
                }
              }
            }
          }
#pragma unroll
          for (int c = 0; c < NPL; ++c) {
            pk[wave * NN + lane + 64 * c] = bv[c];
            pt[wave * NN + lane + 64 * c] = bt[c];
          }
          __syncthreads();
          // a row's waves meet: (value, token) minimum over its wpr partials
          for (int o = tid; o < R * NN; o += 1024) {
            const int ri2 = o / NN, j = o % NN, e = drow[r0 + ri2];
            double cv = INFINITY;
            int ct = 0x7FFFFFFF;
            for (int w = ri2 * wpr; w < (ri2 + 1) * wpr; ++w) {
              const double ov = pk[w * NN + j];
              const int ot = pt[w * NN + j];
              if (ov < cv || (ov == cv && ot < ct)) {
                cv = ov;
                ct = ot;
              }
            }
            Md[e * NN + j] = cv;
            arg[e * NN + j] = ct;
          }
          __syncthreads();
        }
      }
    }
    // ---- reduced costs max(M(u, j) − π_u + π_j, 0)
    for (int o = tid; o < NN * NN; o += 1024) {
      const int u = o / NN, j = o % NN;
      W[o] = (u < n && j < n) ? fmax(Md[o] - pi[u] + pi[j], 0.0) : INFINITY;
    }
    __syncthreads();
    // ---- Dijkstra from every over-full expert to the first under-full one reached
    if (wave == 0) {
      uint64_t under[NPL];
      double dv[NPL];
      int pv[NPL];
      bool done[NPL];
#pragma unroll
      for (int c = 0; c < NPL; ++c) {
        const int r = lane + 64 * c;
        under[c] = __ballot(r < n && cnt[r] < q);
        dv[c] = (r < n && cnt[r] > q) ? 0.0 : INFINITY;
        pv[c] = -1;
        done[c] = r >= n;
      }
      int target = -1;
      double Dt = 0.0;
      constexpr uint64_t kInfBits = 0x7FF0000000000000ull;
      for (int it = 0; it < n; ++it) {
        // distances are >= 0, so their raw bits order like their values: the minimum as two
        // 32-bit reductions (high word, then the low word among the lanes holding the high one)
        uint64_t kb[NPL];
#pragma unroll
        for (int c = 0; c < NPL; ++c) kb[c] = done[c] ? kInfBits : uint64_t(__double_as_longlong(dv[c]));
        uint64_t kl = kb[0];
#pragma unroll
        for (int c = 1; c < NPL; ++c) kl = kb[c] < kl ? kb[c] : kl;
        const uint32_t khi = uint32_t(kl >> 32);
        const uint32_t mhi = wave_min_u32_bcast(khi);
        const uint32_t mlo = wave_min_u32_bcast(khi == mhi ? uint32_t(kl) : 0xFFFFFFFFu);
        const uint64_t mkey = (uint64_t(mhi) << 32) | mlo;
        if (mkey >= kInfBits) break;   // every remaining expert unreachable
        const double du = __longlong_as_double(int64_t(mkey));
        // the unfinished expert of least distance, the lower index on ties
        int u = -1;
#pragma unroll
        for (int c = 0; c < NPL; ++c) {
          const uint64_t b = __ballot(kb[c] == mkey);
          if (u < 0 && b) u = 64 * c + int(__builtin_ctzll(b));
        }
        u = __builtin_amdgcn_readfirstlane(u);
        double wrow[NPL];   // u's reduced costs, read before the target test
#pragma unroll
        for (int c = 0; c < NPL; ++c) wrow[c] = W[u * NN + lane + 64 * c];
#pragma unroll
        for (int c = 0; c < NPL; ++c)
          if (lane + 64 * c == u) done[c] = true;
        if ((under[NPL == 1 ? 0 : (u >> 6)] >> (u & 63)) & 1ull) {
          target = u;
          Dt = du;
          break;
        }
#pragma unroll
        for (int c = 0; c < NPL; ++c) {
          if (!done[c]) {
            const double nd = du + wrow[c];
            if (nd < dv[c]) {
              dv[c] = nd;
              pv[c] = u;
            }
          }
        }
      }
#pragma unroll
      for (int c = 0; c < NPL; ++c) {
        const int r = lane + 64 * c;
        if (r < n) {
          dist[r] = dv[c];
          pred[r] = pv[c];
          vis[r] = done[c];
        }
      }
      if (lane == 0) {
        s_target = target;
        s_D = Dt;
        s_fail = target < 0;
      }
    }
    __syncthreads();
    if (s_fail) break;
    if (tid < n) {
      const double Dt = s_D;
      pi[tid] -= vis[tid] ? fmin(dist[tid], Dt) : Dt;
    }
    if (wave == 0) {
      // the path's edges (target back to source) and the token each one's cost came from
      if (lane == 0) {
        int j = s_target, len = 0;
        while (pred[j] >= 0) {
          const int aa = pred[j];
          path_a[len] = aa;
          path_j[len] = j;
          path_t[len] = arg[aa * NN + j];
          ++len;
          j = aa;
        }
        s_len = len;
      }
      __builtin_amdgcn_wave_barrier();
      const int len = __builtin_amdgcn_readfirstlane(s_len);
      for (int p0 = 0; p0 < len; p0 += 8) {
        float rowv[8][NPL];   // the score rows of the next 8 edges' tokens, read together
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int c = 0; c < NPL; ++c)
            rowv[u][c] = (p0 + u < len && lane + 64 * c < n)
                             ? s[int64_t(path_t[min(p0 + u, len - 1)]) * n + lane + 64 * c]
                             : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (p0 + u < len) {
            const int pe = p0 + u;
            const int aa = __builtin_amdgcn_readfirstlane(path_a[pe]), j = __builtin_amdgcn_readfirstlane(path_j[pe]);
            const int i = __builtin_amdgcn_readfirstlane(path_t[pe]);
            XMask<NPL> after = hm[i];
            xm_flip(after, aa);
            xm_flip(after, j);
            const float sij = lane_of<NPL>(rowv[u], j), sia = lane_of<NPL>(rowv[u], aa);
            // row aa loses the token: the columns it was cheapest for
            uint64_t lost[NPL];
#pragma unroll
            for (int c = 0; c < NPL; ++c) lost[c] = __ballot(lane + 64 * c < n && arg[aa * NN + lane + 64 * c] == i);
#pragma unroll
            for (int c = 0; c < NPL; ++c) {
              const int e = lane + 64 * c;
              if (e < n) {
                const float sie = rowv[u][c];
                if (!xm_has(after, e)) {
                  // row j gains candidate i for every expert the token will not hold
                  const double v = double(sij) - double(sie);
                  const int o = j * NN + e;
                  if (v < Md[o] || (v == Md[o] && i < arg[o])) {
                    Md[o] = v;
                    arg[o] = i;
                  }
                } else if (e != j) {
                  // an expert e the token keeps: (e -> aa) gains it, (e -> j) loses it
                  const double v = double(sie) - double(sia);
                  const int o = e * NN + aa;
                  if (v < Md[o] || (v == Md[o] && i < arg[o])) {
                    Md[o] = v;
                    arg[o] = i;
                  }
                  if (arg[e * NN + j] == i) dcol[e * NPL + (NPL == 1 ? 0 : (j >> 6))] |= 1ull << (j & 63);
                }
              }
            }
            __builtin_amdgcn_wave_barrier();
            if (keep) {
              // the token leaves aa's list (the last entry fills its place) and joins j's
              const int ca = cnt[aa], ba = roff[aa];
              int where = -1;
              for (int c0 = 0; c0 < ca && where < 0; c0 += 64) {
                const uint64_t hit = __ballot(c0 + lane < ca && lst[ba + c0 + lane] == i);
                if (hit) where = c0 + int(__builtin_ctzll(hit));
              }
              if (lane == 0) {
                lst[ba + where] = lst[ba + ca - 1];
                lst[roff[j] + cnt[j]] = uint16_t(i);
              }
            }
            __builtin_amdgcn_wave_barrier();
            if (lane == 0) {
#pragma unroll
              for (int c = 0; c < NPL; ++c) dcol[aa * NPL + c] |= lost[c];
              hm[i] = after;
              cnt[aa] -= 1;
              cnt[j] += 1;
            }
            __builtin_amdgcn_wave_barrier();
          }
        }
      }
      ++aug;
      over_full();
    } else {
      ++aug;
    }
    __syncthreads();
  }
  __syncthreads();
  for (int t = tid; t < m; t += 1024) {
    const XMask<NPL> ht = hm[t];
    int r = 0;
#pragma unroll
    for (int c = 0; c < NPL; ++c)
      for (uint64_t h = ht.w[c]; h && r < k; h &= h - 1) xi[int64_t(t) * k + r++] = 64 * c + __builtin_ctzll(h);
  }
  if (tid < n) {
    a.counts[tid] = cnt[tid];
    a.beta[tid] = float(pi[tid]);
    pi_out[tid] = pi[tid];
  }
  if (wave == 0) {
    bool offq = false;
#pragma unroll
    for (int c = 0; c < NPL; ++c) offq |= lane + 64 * c < n && cnt[lane + 64 * c] != q;
    const uint64_t off = __ballot(offq);
    if (lane == 0 && a.info) {
      a.info[1] = aug;
      a.info[2] = off == 0 && !s_fail;
      a.info[3] = s_fail;
    }
  }
}

__global__ void k_qb_info(int32_t* info, int iters) {
  if (threadIdx.x == 0) {
    info[0] = iters;
    info[1] = 0;
    info[2] = 0;
    info[3] = 0;
  }
}

// ------------------------------------------------------------------ launcher
// numpy's linear quantile of N values at 1 - k/n (the level and the index in
// fp32, as numpy computes them for fp32 data): the lower neighbour's 0-based
// descending rank and the interpolation weight
static void quantile_pos(int64_t N, int k, int n, int64_t& rank, float& g) {
  const float lev = float(1.0 - double(k) / double(n));
  const float vi = float(N - 1) * lev;
  const float lo = std::floor(vi);
  rank = N - 1 - int64_t(lo);
  g = vi - lo;
}

// β of every block set to the incoming β (mini-batch solve)
__global__ __launch_bounds__(256) void k_qb_beta_fill(const float* __restrict__ beta, float* __restrict__ blk, int n,
                                                      int nb) {
  for (int64_t o = int64_t(blockIdx.x) * 256 + threadIdx.x; o < int64_t(n) * nb; o += int64_t(gridDim.x) * 256)
    blk[o] = beta[o % n];
}

// β_j = fl32((Σ_b β_b,j) / nb), the sum in fp64 in block order
__global__ __launch_bounds__(256) void k_qb_beta_mean(const float* __restrict__ blk, int n, int nb,
                                                      float* __restrict__ beta) {
  for (int j = blockIdx.x * 256 + threadIdx.x; j < n; j += gridDim.x * 256) {
    double acc = 0.0;
    for (int b = 0; b < nb; ++b) acc += double(blk[int64_t(b) * n + j]);
    beta[j] = float(acc / double(nb));
  }
}

// Row pass: α (al) and / or the top-k with its counts (idx) of fl32(s_i − β) for every
// token, on the kernel that fits n and k; beta is one row, or one row per block of
// a.beta_rows tokens (α only).
static void launch_rows(const BalanceArgs& a, const float* beta, float* alpha, uint64_t* chunks, bool idx, bool al,
                        hipStream_t s) {
  const unsigned rblocks = unsigned(ceil_div64(a.m, kQbRowsPerBlock));
  const size_t rlds = (size_t(a.n) + 4096) * sizeof(int);
  // register rows: grid-stride waves; the counting form keeps at most 512
  // per-workgroup count rows (ceil(m/16) are allocated) for the last workgroup to fold
  const int npl = a.n <= 64 ? 1 : a.n <= 128 ? 2 : a.n <= 256 ? 4 : 0;
  const unsigned gidx = unsigned(std::min<int64_t>(ceil_div64(a.m, 64), 512));
#define MOE_QB_ROWS(NPL)                                                                                      \
  if (al)                                                                                                  \
    hipLaunchKernelGGL((k_qb_rows_reg<true, true, NPL>), dim3(gidx), dim3(kRowsRegThreads), rlds, s, a, beta, alpha, chunks); \
  else                                                                                                     \
    hipLaunchKernelGGL((k_qb_rows_reg<true, false, NPL>), dim3(gidx), dim3(kRowsRegThreads), rlds, s, a, beta, alpha, chunks);
    // (half-wave rows; the counting form needs a lane per pick in each half: k <= 32)
    if (a.n <= 256 && (!idx || a.k <= 32)) {
      const int nh = a.n <= 32 ? 1 : a.n <= 64 ? 2 : a.n <= 128 ? 4 : 8;
      // two rows per wave; the counting form keeps at most 256 count rows (one
      // workgroup per CU: its registers allow no more) for k_qb_count_finish to fold
      // (value-only form: two 1024-thread workgroups per CU, striding over the rows)
      const unsigned gh = unsigned(std::min<int64_t>(ceil_div64(a.m, 128), idx ? 256 : 512));
#define MOE_QB_HALF(NH)                                                                                        \
  if (idx && al)                                                                                            \
    hipLaunchKernelGGL((k_qb_rows_half<true, true, NH>), dim3(gh), dim3(kRowsRegThreads), rlds, s, a, beta, alpha, chunks); \
  else if (idx)                                                                                             \
    hipLaunchKernelGGL((k_qb_rows_half<true, false, NH>), dim3(gh), dim3(kRowsRegThreads), rlds, s, a, beta, alpha, chunks); \
  else                                                                                                      \
    hipLaunchKernelGGL((k_qb_rows_half<false, true, NH>), dim3(gh), dim3(kRowsRegThreads), 0, s, a, beta, alpha, chunks);
      if (nh == 1) {
        MOE_QB_HALF(1)
      } else if (nh == 2) {
        MOE_QB_HALF(2)
      } else if (nh == 4) {
        MOE_QB_HALF(4)
      } else {
        MOE_QB_HALF(8)
      }
#undef MOE_QB_HALF
      if (idx) hipLaunchKernelGGL(k_qb_count_finish, dim3(1), dim3(kRowsRegThreads), rlds, s, a, chunks, int(gh));
    } else if (npl == 1) {
      MOE_QB_ROWS(1)
      hipLaunchKernelGGL(k_qb_count_finish, dim3(1), dim3(kRowsRegThreads), rlds, s, a, chunks, int(gidx));
    } else if (npl == 2) {
      MOE_QB_ROWS(2)
      hipLaunchKernelGGL(k_qb_count_finish, dim3(1), dim3(kRowsRegThreads), rlds, s, a, chunks, int(gidx));
    } else if (npl == 4) {
      MOE_QB_ROWS(4)
      hipLaunchKernelGGL(k_qb_count_finish, dim3(1), dim3(kRowsRegThreads), rlds, s, a, chunks, int(gidx));
    } else if (idx && al) {
      hipLaunchKernelGGL((k_qb_rows<true, true>), dim3(rblocks), dim3(256), rlds, s, a, beta, alpha, chunks);
    } else if (idx) {
      hipLaunchKernelGGL((k_qb_rows<true, false>), dim3(rblocks), dim3(256), rlds, s, a, beta, alpha, chunks);
    } else {
      hipLaunchKernelGGL((k_qb_rows<false, true>), dim3(rblocks), dim3(256), 0, s, a, beta, alpha, chunks);
    }
#undef MOE_QB_ROWS
}

hipError_t launch_balance(const BalanceArgs& a_in, hipStream_t s) {
  BalanceArgs a = a_in;
  a.nblocks = 1;
  a.beta_rows = a.m;
  if (a.quantile) {
    int64_t rr = 0;
    quantile_pos(a.n, a.k, a.n, rr, a.g_row);
    a.rank_row = int(rr);
    quantile_pos(a.m, a.k, a.n, a.rank_col, a.g_col);
  }
  char* ws = static_cast<char*>(a.ws);
  float* sT = reinterpret_cast<float*>(ws);
  ws += al256(size_t(a.m) * a.n * sizeof(float));
  float* alpha_int = reinterpret_cast<float*>(ws);
  ws += al256(size_t(a.m) * sizeof(float));
  uint64_t* chunks = reinterpret_cast<uint64_t*>(ws);
  ws += al256(size_t(ceil_div64(a.m, kQbRowsPerBlock)) * a.n * sizeof(uint64_t));
  int32_t* xi = reinterpret_cast<int32_t*>(ws);
  ws += al256(size_t(a.m) * a.k * sizeof(int32_t));
  int32_t* pos = reinterpret_cast<int32_t*>(ws);
  ws += al256(size_t(a.m) * a.k * sizeof(int32_t));
  int32_t* lst = reinterpret_cast<int32_t*>(ws);
  ws += al256(size_t(a.n) * a.m * sizeof(int32_t));
  double* pi_fin = reinterpret_cast<double*>(ws);
  ws += al256(size_t(a.n) * sizeof(double));
  double* gM = reinterpret_cast<double*>(ws);   // M, its tokens and the reduced costs for 64 < n <= 128
  ws += al256(size_t(kFastMaxN) * kFastMaxN * sizeof(double));
  int* gArg = reinterpret_cast<int*>(ws);
  ws += al256(size_t(kFastMaxN) * kFastMaxN * sizeof(int));
  double* gW = reinterpret_cast<double*>(ws);
  float* alpha = a.alpha_out ? a.alpha_out : alpha_int;

  if (a.info) hipLaunchKernelGGL(k_qb_info, dim3(1), dim3(64), 0, s, a.info, a.iters);
  auto rows = [&](bool idx, bool al) { launch_rows(a, a.beta, alpha, chunks, idx, al, s); };
  auto cols = [&]() {
    hipLaunchKernelGGL(k_qb_cols, dim3(a.n, 1), dim3(kColThreads), kColLds, s, sT, alpha, a.beta, a);
  };
  hipLaunchKernelGGL(k_qb_transpose, dim3(unsigned(ceil_div64(a.m, 64)), ceil_div(a.n, 64)), dim3(256), 0, s, a.s,
                     sT, a.m, a.n);
  if (a.mode == 1) {  // online: route with the old β, then one α and one β step
    rows(true, true);
    cols();
    return hipGetLastError();
  }
  for (int it = 0; it < a.iters; ++it) {
    rows(false, true);
    cols();
  }
  if (a.exact && fast_complete_ok(a.m, a.n, a.k)) {
    const unsigned tok_blocks = unsigned(ceil_div64(a.m, 4));
    hipLaunchKernelGGL(k_qbc_init, dim3(tok_blocks), dim3(256), 0, s, a, xi);
    const size_t minit_lds = size_t(8) * 128 * 12 + size_t(a.m) * sizeof(int);
    if (fast_npl(a.n) == 1)
      hipLaunchKernelGGL(k_qbc_minit<1>, dim3(a.n), dim3(256), minit_lds, s, a, xi, gM, gArg);
    else
      hipLaunchKernelGGL(k_qbc_minit<2>, dim3(a.n), dim3(256), minit_lds, s, a, xi, gM, gArg);
    // the token lists take all the LDS left (at least m·k entries)
    const int npl = fast_npl(a.n);
    const size_t fixed = fast_lds_bytes(npl, a.m, a.k) - size_t(round_up(int(a.m * a.k) * 2, 16));
    const int list_cap = int((size_t(kFastLdsLimit) - fixed) / 2) & ~7;
    if (npl == 1)
      hipLaunchKernelGGL(k_qbc_solve<1>, dim3(1), dim3(1024), kFastLdsLimit, s, a, xi, pi_fin, gM, gArg, gW, list_cap);
    else
      hipLaunchKernelGGL(k_qbc_solve<2>, dim3(1), dim3(1024), kFastLdsLimit, s, a, xi, pi_fin, gM, gArg, gW, list_cap);
    hipLaunchKernelGGL(k_qbc_out, dim3(tok_blocks), dim3(256), 0, s, a, xi, pi_fin);
  } else if (a.exact)
    hipLaunchKernelGGL(k_qb_complete, dim3(1), dim3(1024), 0, s, a, xi, pos, lst);
  else
    rows(true, false);
  return hipGetLastError();
}

// Mini-batch duals ([MoE tour 6] "함정에 주의", last paragraph): the tokens are
// cut into blocks of a.beta_rows rows, each block runs the QB steps with its own
// quota q_b = beta_rows·k/n and its own β row (all blocks in the same launches:
// α rows read their block's β, the column kernel takes one segment per block),
// and the blocks' β are averaged into a.beta.  SOLVE: every block starts from
// the incoming β, then idx = top-k of fl32(s − mean β).  ONLINE: idx = top-k
// of fl32(s − β_old) first, then one step per block from β_old.
hipError_t launch_balance_minibatch(const BalanceArgs& a_in, hipStream_t s) {
  BalanceArgs a = a_in;                 // global view: rows, final top-k, info
  BalanceArgs b = a_in;                 // block view: α rows and column segments
  a.nblocks = 1;
  a.beta_rows = a.m;
  b.q = b.beta_rows * b.k / b.n;
  if (a.quantile) {
    int64_t rr = 0;
    quantile_pos(a.n, a.k, a.n, rr, a.g_row);
    a.rank_row = int(rr);
    b.rank_row = a.rank_row;
    b.g_row = a.g_row;
    quantile_pos(b.beta_rows, b.k, b.n, b.rank_col, b.g_col);
  }
  char* ws = static_cast<char*>(a.ws);
  float* sT = reinterpret_cast<float*>(ws);
  ws += al256(size_t(a.m) * a.n * sizeof(float));
  float* alpha_int = reinterpret_cast<float*>(ws);
  ws += al256(size_t(a.m) * sizeof(float));
  uint64_t* chunks = reinterpret_cast<uint64_t*>(ws);
  ws += al256(size_t(ceil_div64(a.m, kQbRowsPerBlock)) * a.n * sizeof(uint64_t));
  float* blk = reinterpret_cast<float*>(ws);   // [nblocks, n] β rows
  float* alpha = a.alpha_out ? a.alpha_out : alpha_int;
  const unsigned fill_grid = unsigned(std::min<int64_t>(ceil_div64(int64_t(b.nblocks) * a.n, 256), 1024));

  if (a.info) hipLaunchKernelGGL(k_qb_info, dim3(1), dim3(64), 0, s, a.info, a.iters);
  hipLaunchKernelGGL(k_qb_transpose, dim3(unsigned(ceil_div64(a.m, 64)), ceil_div(a.n, 64)), dim3(256), 0, s, a.s,
                     sT, a.m, a.n);
  auto cols = [&]() {
    hipLaunchKernelGGL(k_qb_cols, dim3(a.n, b.nblocks), dim3(kColThreads), kColLds, s, sT, alpha, blk, b);
  };
  if (a.mode == 1) {
    launch_rows(a, a.beta, alpha, chunks, true, true, s);   // route with β_old; α from β_old
    cols();
  } else {
    hipLaunchKernelGGL(k_qb_beta_fill, dim3(fill_grid), dim3(256), 0, s, a.beta, blk, a.n, b.nblocks);
    for (int it = 0; it < a.iters; ++it) {
      launch_rows(b, blk, alpha, chunks, false, true, s);
      cols();
    }
  }
  if (a.mode == 1 || a.iters > 0)
    hipLaunchKernelGGL(k_qb_beta_mean, dim3(unsigned(ceil_div(a.n, 256))), dim3(256), 0, s, blk, a.n, b.nblocks,
                       a.beta);
  if (a.mode != 1) launch_rows(a, a.beta, alpha, chunks, true, false, s);
  return hipGetLastError();
}

hipError_t launch_signsgd(const BalanceArgs& a, float gamma, hipStream_t s) {
  // the counting top-k of launch_balance's register paths (n <= 256) and its count rows
  char* ws = static_cast<char*>(a.ws);
  ws += al256(size_t(a.m) * a.n * sizeof(float));
  ws += al256(size_t(a.m) * sizeof(float));
  uint64_t* chunks = reinterpret_cast<uint64_t*>(ws);
  const size_t rlds = (size_t(a.n) + 4096) * sizeof(int);
  float* alpha = nullptr;
  const bool half = a.k <= 32;
  const int nh = a.n <= 32 ? 1 : a.n <= 64 ? 2 : a.n <= 128 ? 4 : 8;
  const int npl = a.n <= 64 ? 1 : a.n <= 128 ? 2 : 4;
  const unsigned grid = half ? unsigned(std::min<int64_t>(ceil_div64(a.m, 128), 256))
                             : unsigned(std::min<int64_t>(ceil_div64(a.m, 64), 512));
  auto count = [&]() {
    if (half) {
      if (nh == 1) hipLaunchKernelGGL((k_qb_rows_half<true, false, 1>), dim3(grid), dim3(kRowsRegThreads), rlds, s, a, a.beta, alpha, chunks);
      if (nh == 2) hipLaunchKernelGGL((k_qb_rows_half<true, false, 2>), dim3(grid), dim3(kRowsRegThreads), rlds, s, a, a.beta, alpha, chunks);
      if (nh == 4) hipLaunchKernelGGL((k_qb_rows_half<true, false, 4>), dim3(grid), dim3(kRowsRegThreads), rlds, s, a, a.beta, alpha, chunks);
      if (nh == 8) hipLaunchKernelGGL((k_qb_rows_half<true, false, 8>), dim3(grid), dim3(kRowsRegThreads), rlds, s, a, a.beta, alpha, chunks);
    } else {
      if (npl == 1) hipLaunchKernelGGL((k_qb_rows_reg<true, false, 1>), dim3(grid), dim3(kRowsRegThreads), rlds, s, a, a.beta, alpha, chunks);
      if (npl == 2) hipLaunchKernelGGL((k_qb_rows_reg<true, false, 2>), dim3(grid), dim3(kRowsRegThreads), rlds, s, a, a.beta, alpha, chunks);
      if (npl == 4) hipLaunchKernelGGL((k_qb_rows_reg<true, false, 4>), dim3(grid), dim3(kRowsRegThreads), rlds, s, a, a.beta, alpha, chunks);
    }
  };
  for (int it = 0; it < a.iters; ++it) {
    count();
    hipLaunchKernelGGL(k_qb_signsgd_step, dim3(1), dim3(kRowsRegThreads), rlds, s, a, chunks, int(grid), gamma);
  }
  count();
  hipLaunchKernelGGL(k_qb_count_finish, dim3(1), dim3(kRowsRegThreads), rlds, s, a, chunks, int(grid));
  return hipGetLastError();
}

}  // namespace moe
