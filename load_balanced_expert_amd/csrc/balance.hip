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
//    s_ia − s_ij over tokens holding a but not j, kept in LDS; Dijkstra runs
//    on one wave with one expert per lane) until every expert has q tokens.
//    Requires n <= 64.
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
  float nx[NPL];
#pragma unroll
  for (int u = 0; u < NPL; ++u) nx[u] = i < a.m && hl + 32 * u < n ? a.s[i * n + hl + 32 * u] : 0.f;
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
      v[u] = j < n && live ? nx[u] - bl[u] : -INFINITY;
      jj[u] = j < n ? j : 0x7FFFFFFF;
    }
    const int64_t i2 = i + stride;
#pragma unroll
    for (int u = 0; u < NPL; ++u) nx[u] = i2 < a.m && hl + 32 * u < n ? a.s[i2 * n + hl + 32 * u] : 0.f;
    sort_desc<IDX, NPL>(v, jj);
    float hi_key = INFINITY, lo_key = INFINITY;
    int my_j = 0;
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
    for (int64_t b = threadIdx.x; b - threadIdx.x < nv; b += 2 * kColThreads) {   // uniform trip count
      f32x4 x[2], al[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t v = b + int64_t(u) * kColThreads;
        x[u] = v < nv ? c4[v] : f32x4{0.f, 0.f, 0.f, 0.f};
        al[u] = v < nv ? a4[v] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bool act = b + int64_t(u) * kColThreads < nv;
        f(f32_key(x[u][0] - al[u][0]), act);
        f(f32_key(x[u][1] - al[u][1]), act);
        f(f32_key(x[u][2] - al[u][2]), act);
        f(f32_key(x[u][3] - al[u][3]), act);
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
  __shared__ int s_wsum[kColThreads / 64], s_wcnt[kColThreads / 64], s_bin, s_rank, s_nk, s_ovf, s_above;
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
      int rr;
      if (r_hi > 0) lds_select(keys, ns, r_hi, hist, s_wsum, &s_bin, &s_rank, k_hi, rr);
      if (r_lo < ns - 1) lds_select(keys, ns, r_lo, hist, s_wsum, &s_bin, &s_rank, k_lo, rr);
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
    col_scan(col, alpha, m, [&](uint32_t u, bool act) {
      if (act && u > k_hi) {
        ++above;
        mn = min(mn, u);
      }
      const bool take = act && u >= k_lo && u <= k_hi;
      const uint64_t bm = __ballot(take);
      if (!bm) return;
      const int at = wcnt + __popcll(bm & lanemask_lt());
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
  atomicAdd(&s_above, above);
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
    atomicMin(&s_min, mn);
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
      // was its cheapest token).
      int j = s_target;
      while (pred[j] >= 0) {
        const int aa = pred[j];
        const int i = arg[aa * n + j];
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
      const unsigned gh = unsigned(std::min<int64_t>(ceil_div64(a.m, 128), idx ? 256 : 1024));
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
  if (a.exact)
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
