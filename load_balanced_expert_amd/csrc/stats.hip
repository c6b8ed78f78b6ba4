// Load statistics, Switch aux loss, global-batch accumulation and the
// Loss-Free bias update (one small workgroup; n <= 4096).
//
// [Switch review] "로드 밸런싱 손실": f_i = c_i / T, P_i = (1/T) Σ p_i(x),
// L_aux = α·N·Σ f_i P_i.  [Qwen global] "글로벌-배치 로드 밸런스 구현": f is
// gathered over all micro-batches of the global batch, each micro-batch's
// loss uses that f, and the losses are aggregated (mean).  [MoE tour 6]
// "방법 회고" eq. (2): b ← b − γ·sign(F − 1/n), after routing with the old b.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kStatsThreads = 1024;

// Fixed-order block sum of fp64 values: per-thread partials, then wave
// butterflies, then the 16 wave results in wave order.
__device__ double block_sum_f64(double v, double* red) {
  v = wave_sum_f64(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0) {
    for (int w = 0; w < int(blockDim.x >> 6); ++w) t += red[w];
    red[0] = t;
  }
  __syncthreads();
  t = red[0];
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(kStatsThreads) void k_stats(int64_t m, int n, int k, const int32_t* __restrict__ counts,
                                                          const float* __restrict__ prob_sum, float alpha,
                                                          float* __restrict__ f, float* __restrict__ P,
                                                          float* __restrict__ aux, int64_t* __restrict__ gcounts,
                                                          int64_t* __restrict__ gtokens, float* __restrict__ bias,
                                                          float gamma) {
  __shared__ double red[kStatsThreads / 64];
  const float fm = float(m);
  double part = 0.0;
  for (int j = threadIdx.x; j < n; j += blockDim.x) {
    const int64_t c = counts[j];
    const double fj = double(c) / double(m);
    if (f) f[j] = float(c) / fm;
    if (prob_sum) {
      const double Pj = double(prob_sum[j]) / double(m);
      if (P) P[j] = prob_sum[j] / fm;
      part += fj * Pj;
    }
    if (gcounts) gcounts[j] += c;
    if (bias) {
      const int64_t diff = c * int64_t(n) - m * int64_t(k);
      const float sgn = diff > 0 ? 1.f : (diff < 0 ? -1.f : 0.f);
      bias[j] = bias[j] - gamma * sgn;
    }
  }
  if (prob_sum && aux) {
    const double tot = block_sum_f64(part, red);
    if (threadIdx.x == 0) aux[0] = float(double(alpha) * double(n) * tot);
  }
  if (gtokens && threadIdx.x == 0) gtokens[0] += m;
}

hipError_t launch_stats(int64_t m, int n, int k, const int32_t* counts, const float* prob_sum, float alpha,
                        float* f, float* P, float* aux, int64_t* gcounts, int64_t* gtokens, float* bias,
                        float gamma, hipStream_t s) {
  hipLaunchKernelGGL(k_stats, dim3(1), dim3(kStatsThreads), 0, s, m, n, k, counts, prob_sum, alpha, f, P, aux,
                     gcounts, gtokens, bias, gamma);
  return hipGetLastError();
}

// One workgroup per micro-batch row of P, plus the shared global f.
__global__ __launch_bounds__(kStatsThreads) void k_global_aux(int n, const int64_t* __restrict__ gcounts,
                                                               const int64_t* __restrict__ gtokens,
                                                               const float* __restrict__ P, int nb, float alpha,
                                                               float* __restrict__ fg, float* __restrict__ losses,
                                                               float* __restrict__ loss_mean,
                                                               const float* __restrict__ micro_aux, float global_weight,
                                                               float micro_weight,
                                                               float* __restrict__ hybrid,
                                                               float* __restrict__ hybrid_mean) {
  __shared__ double red[kStatsThreads / 64];
  const double T = double(gtokens[0]);
  double mean = 0.0, hmean = 0.0;
  for (int t = 0; t < nb; ++t) {
    double part = 0.0;
    for (int j = threadIdx.x; j < n; j += blockDim.x) {
      const double f = double(gcounts[j]) / T;
      if (t == 0 && fg) fg[j] = float(f);
      part += f * double(P[int64_t(t) * n + j]);
    }
    const double L = double(alpha) * double(n) * block_sum_f64(part, red);
    if (threadIdx.x == 0 && losses) losses[t] = float(L);
    mean += L;
    if (micro_aux) {   // hybrid: the global-batch and the micro-batch losses, each with a constant weight
      const double H = double(global_weight) * L + double(micro_weight) * double(micro_aux[t]);
      if (threadIdx.x == 0 && hybrid) hybrid[t] = float(H);
      hmean += H;
    }
  }
  if (threadIdx.x == 0 && loss_mean) loss_mean[0] = float(mean / double(nb));
  if (threadIdx.x == 0 && hybrid_mean && micro_aux) hybrid_mean[0] = float(hmean / double(nb));
  if (nb == 0 && fg)
    for (int j = threadIdx.x; j < n; j += blockDim.x) fg[j] = float(double(gcounts[j]) / T);
}

hipError_t launch_global_aux(int n, const int64_t* gcounts, const int64_t* gtokens, const float* P, int nb,
                             float alpha, float* fg, float* losses, float* loss_mean, const float* micro_aux,
                             float global_weight, float micro_weight, float* hybrid, float* hybrid_mean,
                             hipStream_t s) {
  hipLaunchKernelGGL(k_global_aux, dim3(1), dim3(kStatsThreads), 0, s, n, gcounts, gtokens, P, nb, alpha, fg,
                     losses, loss_mean, micro_aux, global_weight, micro_weight, hybrid, hybrid_mean);
  return hipGetLastError();
}

}  // namespace moe
