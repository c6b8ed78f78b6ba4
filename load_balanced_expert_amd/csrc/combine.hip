// Combine: inverse permute, gate scaling and residual.
//   out[t] = residual[t] + Σ_{r kept} gate[t, r] · y[token_to_row[t, r]]
// ([Switch review] "Switch Routing 메커니즘" Step 3: the expert output is scaled
// by the router probability; [Switch impl] pipeline list: restore the token
// order, multiply by the gate and join the residual path; dropped tokens take
// the residual path alone.)  fp32 arithmetic, r in increasing order, one
// rounding to the output dtype; HBM-bound, so every thread moves 8 elements
// with 16-byte (bf16) or 2x16-byte (fp32) accesses.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// Every element is read once and written once, so the loads and stores are
// non-temporal: they do not displace cached lines (with the caches full of
// another kernel's dirty lines this measured 16.3 -> 11.4 us at T = 8192,
// d = 768, and the same with warm caches).
template <bool BF16>
__device__ __forceinline__ void load_vec(const void* p, int64_t i, float (&v)[8]) {
  if constexpr (BF16) {
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + i);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(w[q] << 16);
      v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
    }
  } else {
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 2 * i);
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 2 * i + 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = a[q];
      v[4 + q] = b[q];
    }
  }
}

template <bool BF16>
__device__ __forceinline__ void store_vec(void* p, int64_t i, const float (&v)[8]) {
  if constexpr (BF16) {
    u32x4 w;
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = uint32_t(f32_to_bf16(v[2 * q])) | (uint32_t(f32_to_bf16(v[2 * q + 1])) << 16);
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p) + i);
  } else {
    f32x4 a, b;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a[q] = v[q];
      b[q] = v[4 + q];
    }
    __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(p) + 2 * i);
    __builtin_nontemporal_store(b, reinterpret_cast<f32x4*>(p) + 2 * i + 1);
  }
}

// One wave per token: the token's (row, gate) pairs are wave-uniform, so the
// expert rows it gathers are addressed right after one scalar load; lanes
// stream the d/8 16-byte vectors of the row.
constexpr int kCombineWaves = 16;   // tokens (waves) per workgroup
template <bool XB, bool YB>
__global__ __launch_bounds__(64 * kCombineWaves) void k_combine_vec(int64_t m, int d, int k, const void* __restrict__ y,
                                                     const float* __restrict__ gate,
                                                     const int32_t* __restrict__ t2r, const void* __restrict__ res,
                                                     void* __restrict__ out, u32x4* clear, int clear_vecs) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < clear_vecs; i += 64 * kCombineWaves) clear[i] = u32x4{0u, 0u, 0u, 0u};
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * kCombineWaves + wave;
  if (t >= m) return;
  const int vpr = d / 8;
  for (int v0 = 0; v0 < vpr; v0 += 128) {
    float acc[2][8];
    const int vv[2] = {v0 + lane, v0 + 64 + lane};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (res && vv[u] < vpr) {
        load_vec<XB>(res, t * vpr + vv[u], acc[u]);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[u][q] = 0.f;
      }
    }
    for (int r = 0; r < k; ++r) {
      const int32_t row = t2r[t * k + r];
      if (row >= 0) {
        const float g = gate[t * k + r];
        float yv[2][8];
#pragma unroll
        for (int u = 0; u < 2; ++u)
          if (vv[u] < vpr) load_vec<YB>(y, int64_t(row) * vpr + vv[u], yv[u]);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[u][q] = fmaf(g, yv[u][q], acc[u][q]);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (vv[u] < vpr) store_vec<XB>(out, t * vpr + vv[u], acc[u]);
  }
}

// Any d: one element per thread.
__global__ __launch_bounds__(256) void k_combine_scalar(int64_t m, int d, int k, const void* __restrict__ y, int yb,
                                                        const float* __restrict__ gate,
                                                        const int32_t* __restrict__ t2r,
                                                        const void* __restrict__ res, void* __restrict__ out, int xb,
                                                        u32x4* clear, int clear_vecs) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < clear_vecs; i += 256) clear[i] = u32x4{0u, 0u, 0u, 0u};
  const int64_t items = m * d;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < items; i += int64_t(gridDim.x) * 256) {
    const int64_t t = i / d, c = i - t * d;
    float acc = 0.f;
    if (res) acc = xb ? bf16_to_f32(static_cast<const uint16_t*>(res)[i]) : static_cast<const float*>(res)[i];
    for (int r = 0; r < k; ++r) {
      const int32_t row = t2r[t * k + r];
      if (row >= 0) {
        const int64_t o = int64_t(row) * d + c;
        const float yv = yb ? bf16_to_f32(static_cast<const uint16_t*>(y)[o]) : static_cast<const float*>(y)[o];
        acc = fmaf(gate[t * k + r], yv, acc);
      }
    }
    if (xb)
      static_cast<uint16_t*>(out)[i] = f32_to_bf16(acc);
    else
      static_cast<float*>(out)[i] = acc;
  }
}

hipError_t launch_combine(int64_t m, int d, int k, const void* y, bool y_bf16, const float* gate,
                          const int32_t* t2r, const void* residual, void* out, bool x_bf16, hipStream_t s,
                          void* clear, size_t clear_bytes) {
  u32x4* cv = static_cast<u32x4*>(clear);
  const int cn = clear ? int(clear_bytes / sizeof(u32x4)) : 0;
  const uintptr_t al = reinterpret_cast<uintptr_t>(y) | reinterpret_cast<uintptr_t>(out) |
                       reinterpret_cast<uintptr_t>(residual);
  if (d % 8 == 0 && (al % 16) == 0) {
    const unsigned blocks = unsigned(ceil_div64(m, kCombineWaves));
    const dim3 tb(64 * kCombineWaves);
    if (x_bf16 && y_bf16)
      hipLaunchKernelGGL((k_combine_vec<true, true>), dim3(blocks), tb, 0, s, m, d, k, y, gate, t2r, residual, out,
                         cv, cn);
    else if (x_bf16)
      hipLaunchKernelGGL((k_combine_vec<true, false>), dim3(blocks), tb, 0, s, m, d, k, y, gate, t2r, residual,
                         out, cv, cn);
    else if (y_bf16)
      hipLaunchKernelGGL((k_combine_vec<false, true>), dim3(blocks), tb, 0, s, m, d, k, y, gate, t2r, residual,
                         out, cv, cn);
    else
      hipLaunchKernelGGL((k_combine_vec<false, false>), dim3(blocks), tb, 0, s, m, d, k, y, gate, t2r, residual,
                         out, cv, cn);
  } else {
    const unsigned blocks = unsigned(std::min<int64_t>(ceil_div64(m * d, 256), 65536));
    hipLaunchKernelGGL(k_combine_scalar, dim3(blocks), dim3(256), 0, s, m, d, k, y, int(y_bf16), gate, t2r, residual,
                       out, int(x_bf16), cv, cn);
  }
  return hipGetLastError();
}

}  // namespace moe
