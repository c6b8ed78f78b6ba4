// Grouped expert FFN on bf16 matrix cores: for every expert e,
//   H_e = bf16(max(0, D_e · W1_e)),  Y_e = bf16(H_e · W2_e)
// ([Switch review] "Switch Layer의 구조": FFN(x) = max(0, x·W1 + b1)·W2 + b2, one
// weight set per expert; no biases here).  D_e are the rows of expert e in the
// dispatched buffer (expert_offsets), weights in Linear layout
// (w1: [n][d_ff][d], w2: [n][d][d_ff]), fp32 accumulation.
//
// At the routing capacities of interest an expert holds <= ~100 rows, so the
// FFN is bound by streaming the weights from HBM.  One workgroup owns
// (expert, 128 output columns) and reads that weight slab exactly once per
// 128 rows; each wave owns 32 columns and keeps up to 4 row tiles of 32 in
// v_mfma_f32_32x32x16_bf16 accumulators.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

size_t ffn_ws_bytes(int64_t rows_bound, int d_ff) { return size_t(rows_bound) * d_ff * sizeof(uint16_t); }

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// One wave: MT row tiles of 32 x its 32 output columns of one expert, full K.
// Branch-free K loop with ping-pong operand buffers: the next K block's
// weight and activation fragments are in flight while the current block is
// multiplied (scheduling barriers keep the loads ahead of the MFMAs).
template <int MT, bool RELU>
__device__ __forceinline__ void ffn_tile(const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bw,
                                         uint16_t* __restrict__ C, int mb, int r_end, int K, int N, int col0,
                                         int lane) {
  const int h = lane >> 5, r32 = lane & 31;
  const uint16_t* Ar[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) Ar[mt] = A + size_t(min(mb + 32 * mt + r32, r_end - 1)) * K;
  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;
  const int nkb = K / 32;
  auto load = [&](int kb, bf16x8 (&aa)[MT][2], bf16x8 (&bb)[2]) {
    const int k0 = kb * 32 + 16 * h;
    bb[0] = ld8(Bw + k0);
    bb[1] = ld8(Bw + k0 + 8);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      aa[mt][0] = ld8(Ar[mt] + k0);
      aa[mt][1] = ld8(Ar[mt] + k0 + 8);
    }
  };
  auto mma = [&](const bf16x8 (&aa)[MT][2], const bf16x8 (&bb)[2]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aa[mt][0], bb[0], acc[mt], 0, 0, 0);
      acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aa[mt][1], bb[1], acc[mt], 0, 0, 0);
    }
  };
  bf16x8 a0[MT][2], b0[2], a1[MT][2], b1[2];
  load(0, a0, b0);
  for (int kb = 0; kb < nkb; kb += 2) {
    load(min(kb + 1, nkb - 1), a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    mma(a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    if (kb + 1 < nkb) {
      load(min(kb + 2, nkb - 1), a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      mma(a1, b1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = mb + 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
      if (row < r_end) {
        float v = acc[mt][i];
        if (RELU) v = fmaxf(v, 0.f);
        C[size_t(row) * N + col0 + r32] = f32_to_bf16(v);
      }
    }
  }
}

template <bool RELU>
__global__ __launch_bounds__(256) void k_grouped_gemm(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                      uint16_t* __restrict__ C, const int32_t* __restrict__ offsets,
                                                      int K, int N, int row_limit) {
  const int e = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col0 = blockIdx.x * 128 + wave * 32;
  if (col0 >= N) return;
  // rows at or past row_limit (the hidden buffer's size) are never touched
  const int r_begin = min(offsets[e], row_limit), r_end = min(offsets[e + 1], row_limit);
  const uint16_t* Bw = B + (size_t(e) * N + col0 + (lane & 31)) * K;
  for (int mb = r_begin; mb < r_end; mb += 128) {
    switch (ceil_div(min(128, r_end - mb), 32)) {
      case 1: ffn_tile<1, RELU>(A, Bw, C, mb, r_end, K, N, col0, lane); break;
      case 2: ffn_tile<2, RELU>(A, Bw, C, mb, r_end, K, N, col0, lane); break;
      case 3: ffn_tile<3, RELU>(A, Bw, C, mb, r_end, K, N, col0, lane); break;
      default: ffn_tile<4, RELU>(A, Bw, C, mb, r_end, K, N, col0, lane); break;
    }
  }
}

hipError_t launch_expert_ffn(int n, int d, int d_ff, int rows_max, const int32_t* offsets, const uint16_t* D,
                             const uint16_t* w1, const uint16_t* w2, uint16_t* hidden, uint16_t* y,
                             hipStream_t s) {
  const int row_limit = int(std::min<int64_t>(int64_t(n) * rows_max, 0x7FFFFFFF));
  hipLaunchKernelGGL(k_grouped_gemm<true>, dim3(ceil_div(d_ff, 128), n), dim3(256), 0, s, D, w1, hidden, offsets,
                     d, d_ff, row_limit);
  hipLaunchKernelGGL(k_grouped_gemm<false>, dim3(ceil_div(d, 128), n), dim3(256), 0, s, hidden, w2, y, offsets,
                     d_ff, d, row_limit);
  return hipGetLastError();
}

}  // namespace moe
