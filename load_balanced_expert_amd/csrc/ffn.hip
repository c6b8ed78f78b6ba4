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

// End row of expert e: offsets[e] + rows[e] (capacity-padded layout) or offsets[e + 1].
__device__ __forceinline__ int expert_end(const int32_t* offsets, const int32_t* rows, int e) {
  return rows ? offsets[e] + rows[e] : offsets[e + 1];
}

template <bool RELU>
__global__ __launch_bounds__(256) void k_grouped_gemm(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                      uint16_t* __restrict__ C, const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ rows, int K, int N, int row_limit) {
  const int e = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col0 = blockIdx.x * 128 + wave * 32;
  if (col0 >= N) return;
  // rows at or past row_limit (the hidden buffer's size) are never touched
  const int r_begin = min(offsets[e], row_limit), r_end = min(expert_end(offsets, rows, e), row_limit);
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

// ------------------------------------------------------------------ streaming path
// For K % 256 == 0 and N % 128 == 0.  One workgroup (W = 4 or 8 waves) owns
// one expert and 32 W output columns; wave w owns 32 of them.  The expert's rows (up to
// 128 per pass) are staged through LDS in K chunks of 128 (register
// prefetch of the next chunk, one LDS buffer) and shared by the W waves.
// Each wave streams its 32 weight rows with coalesced 16-byte loads (eight
// lanes per 128-byte line), kFfnRing - 1 K steps of 64 ahead, and turns each
// step into MFMA fragments through its own LDS slab; the A fragments use the
// same K order.  The workgroup order puts all column blocks of an expert on
// one XCD, so the expert's rows are fetched into that XCD's L2 once.
constexpr int kFfnKA = 128;            // K per staged A chunk
constexpr int kFfnLdA = kFfnKA + 8;    // LDS row stride (bf16), 16 bytes of padding
constexpr int kFfnLdB = 72;            // per-wave weight slab row stride (bf16): 64 + 16 bytes of padding
constexpr int kFfnRing = 4;            // weight K steps in flight + 1 (even)

// Packed weights (PACKED): an expert's [N][K] matrix stored as the MFMA B fragments this kernel
// feeds, in the order it reads them: for 32-row block rb, K step s (64 inputs) and fragment q,
// the 64 lanes' 8 bf16 are contiguous (1 KiB), lane l = r + 32 h holding row 32 rb + r, inputs
// 64 s + 32 h + 8 q + [0, 8).  A wave's weight step is then four contiguous 1 KiB loads that are
// already fragments, and its 32 rows stream as one contiguous run (moe_expert_weights_pack).
__host__ __device__ inline size_t packed_frag_off(int64_t e, int rb, int s, int q, int N, int K) {
  return ((((size_t(e) * (N / 32) + rb) * size_t(K / 64) + s) * 4 + q) * 64) * 8;
}

template <int W, int MT, bool RELU, bool PACKED>   // W waves per workgroup, 32 output columns each
__device__ __forceinline__ void ffn_stream_rows(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                uint16_t* __restrict__ C, uint16_t* As, uint16_t* Bs, int r0, int r_end, int K,
                                                int N, int col0, int tid) {
  const int lane = tid & 63, h = lane >> 5, r32 = lane & 31;
  const int nks = K / 64, nch = K / kFfnKA;
  // A chunk: 32 MT rows x 16 segments of 16 bytes over the workgroup
  constexpr int AL = 8 * MT / W;
  // thread's A items: rows row0 + 16 u (clamped to the last row), 16-byte segment seg
  const int row0 = tid >> 4, seg = tid & 15;
  static_assert(W == 4 || W == 8, "A item mapping");
  constexpr int kRowStep = 64 * W / 16;
  const int lo0 = row0 * kFfnLdA + seg * 8;
  u32x4 areg[AL];
  auto a_fetch = [&](int c) {
    c = min(c, nch - 1);
#pragma unroll
    for (int u = 0; u < AL; ++u) {
      const uint32_t off = uint32_t(min(r0 + row0 + kRowStep * u, r_end - 1)) * uint32_t(K) + c * kFfnKA + seg * 8;
      areg[u] = *reinterpret_cast<const u32x4*>(A + off);
    }
  };
  auto a_store = [&]() {
#pragma unroll
    for (int u = 0; u < AL; ++u) *reinterpret_cast<u32x4*>(As + lo0 + u * kRowStep * kFfnLdA) = areg[u];
  };
  // weight K step s: load q brings rows 8q + lane / 8 of the wave's 32, 16 bytes each
  // (eight lanes cover one 128-byte line), coalesced; the wave then transposes
  // the step through its own LDS slab into MFMA fragments.
  // (PACKED: B is the expert's packed matrix; the wave's run starts at its 32-row block)
  const uint16_t* bp = PACKED ? B + packed_frag_off(0, col0 / 32, 0, 0, N, K) + lane * 8
                              : B + size_t(col0 + (lane >> 3)) * K + 8 * (lane & 7);
  const size_t bq = size_t(8) * K;
  auto b_fetch = [&](bf16x8 (&b)[4], int s) {
    s = min(s, nks - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) b[q] = PACKED ? ld8(bp + (size_t(s) * 4 + q) * 512) : ld8(bp + q * bq + 64 * s);
  };
  uint16_t* bw = Bs + (tid >> 6) * (32 * kFfnLdB);
  auto b_stage = [&](const bf16x8 (&b)[4]) {   // same-wave LDS accesses stay in order
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<bf16x8*>(bw + (8 * q + (lane >> 3)) * kFfnLdB + 8 * (lane & 7)) = b[q];
  };
  const uint16_t* brow = bw + r32 * kFfnLdB + 32 * h;
  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;
  const uint16_t* arow = As + r32 * kFfnLdA + 32 * h;
  auto step = [&](const bf16x8 (&b)[4], int t) {
    if constexpr (!PACKED) b_stage(b);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x8 bf = PACKED ? b[q] : *reinterpret_cast<const bf16x8*>(brow + 8 * q);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(arow + 32 * mt * kFfnLdA + 64 * t + 8 * q);
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bf, acc[mt], 0, 0, 0);
      }
    }
  };
  // weight ring: step s lives in slot s % kFfnRing and is fetched kFfnRing - 1 steps ahead
  bf16x8 ring[kFfnRing][4];
  a_fetch(0);
  a_store();
  a_fetch(1);
#pragma unroll
  for (int u = 0; u < kFfnRing - 1; ++u) b_fetch(ring[u], u);
  lds_barrier();
  // K % 256 == 0 (the launcher's condition): whole groups of kFfnRing steps, so the loop body has
  // no early exit and the waits for the weight ring keep their steady-state counts
  for (int s0 = 0; s0 < nks; s0 += kFfnRing) {
#pragma unroll
    for (int u = 0; u < kFfnRing; ++u) {
      b_fetch(ring[(u + kFfnRing - 1) % kFfnRing], s0 + u + kFfnRing - 1);
      step(ring[u], u & 1);
      if (u & 1) {  // chunk (s0 + u) / 2 consumed: stage the next one, prefetch the one after
        lds_barrier();
        a_store();
        a_fetch((s0 + u) / 2 + 2);
        lds_barrier();
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = r0 + 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
      if (row < r_end) {
        float v = acc[mt][i];
        if (RELU) v = fmaxf(v, 0.f);
        C[size_t(row) * N + col0 + r32] = f32_to_bf16(v);
      }
    }
  }
}

template <int W, bool RELU, bool PACKED = false>
__global__ __launch_bounds__(64 * W) void k_grouped_gemm_stream(const uint16_t* __restrict__ A,
                                                             const uint16_t* __restrict__ B, uint16_t* __restrict__ C,
                                                             const int32_t* __restrict__ offsets,
                                                             const int32_t* __restrict__ rows, int n, int K, int N,
                                                             int row_limit) {
  __shared__ __align__(16) uint16_t As[128 * kFfnLdA];
  __shared__ __align__(16) uint16_t Bs[W * 32 * kFfnLdB];
  const int ncb = N / (32 * W);
  const unsigned G = unsigned(n) * ncb, b = blockIdx.x;
  // XCD-major order: workgroup b runs on XCD b % 8; give each XCD a contiguous range of (expert, block)
  const unsigned L = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
  const int e = int(L / ncb), cb = int(L % ncb);
  const int r_begin = min(offsets[e], row_limit), r_end = min(expert_end(offsets, rows, e), row_limit);
  const int wave = threadIdx.x >> 6;
  const int col0 = cb * (32 * W) + wave * 32;
  const uint16_t* Be = B + size_t(e) * N * K;   // plain and packed matrices have the same size
  for (int r0 = r_begin; r0 < r_end; r0 += 128) {
    switch (ceil_div(min(128, r_end - r0), 32)) {
      case 1: ffn_stream_rows<W, 1, RELU, PACKED>(A, Be, C, As, Bs, r0, r_end, K, N, col0, threadIdx.x); break;
      case 2: ffn_stream_rows<W, 2, RELU, PACKED>(A, Be, C, As, Bs, r0, r_end, K, N, col0, threadIdx.x); break;
      case 3: ffn_stream_rows<W, 3, RELU, PACKED>(A, Be, C, As, Bs, r0, r_end, K, N, col0, threadIdx.x); break;
      default: ffn_stream_rows<W, 4, RELU, PACKED>(A, Be, C, As, Bs, r0, r_end, K, N, col0, threadIdx.x); break;
    }
  }
}

// Packs [n][N][K] bf16 weights into the fragment order above: one thread per 16-byte fragment
// slice, in the packed order, so the writes are contiguous.
__global__ __launch_bounds__(256) void k_pack_weights(const uint16_t* __restrict__ w, uint16_t* __restrict__ p,
                                                      int64_t n, int N, int K) {
  const int64_t items = n * N * (K / 8);
  for (int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x; t < items; t += int64_t(gridDim.x) * 256) {
    const int l = int(t & 63), q = int((t >> 6) & 3);
    const int64_t u = t >> 8;   // (e, rb, s)
    const int nks = K / 64, nrb = N / 32;
    const int s = int(u % nks);
    const int64_t v = u / nks;
    const int rb = int(v % nrb);
    const int64_t e = v / nrb;
    const size_t src = (size_t(e) * N + size_t(rb) * 32 + (l & 31)) * K + size_t(s) * 64 + 32 * (l >> 5) + 8 * q;
    *reinterpret_cast<u32x4*>(p + size_t(t) * 8) = *reinterpret_cast<const u32x4*>(w + src);
  }
}

hipError_t launch_pack_weights(int64_t n, int N, int K, const uint16_t* w, uint16_t* p, hipStream_t s) {
  const int64_t items = n * N * (K / 8);
  const unsigned blocks = unsigned(std::min<int64_t>(ceil_div64(items, 256), 1 << 20));
  hipLaunchKernelGGL(k_pack_weights, dim3(blocks), dim3(256), 0, s, w, p, n, N, K);
  return hipGetLastError();
}

// the streaming kernel addresses the activations with 32-bit element offsets
static bool ffn_streams(int K, int N, int row_limit) {
  return K % 256 == 0 && N % 128 == 0 && int64_t(row_limit) * K < (int64_t(1) << 32);
}

// 8-wave workgroups (256 columns: twice the reuse of each staged row chunk)
// where N allows, else 4-wave workgroups (128 columns).
template <bool RELU, bool PACKED>
static void launch_stream(int n, int K, int N, int row_limit, const int32_t* offsets, const int32_t* rows,
                          const uint16_t* A, const uint16_t* B, uint16_t* C, hipStream_t s) {
  if (N % 256 == 0)
    hipLaunchKernelGGL((k_grouped_gemm_stream<8, RELU, PACKED>), dim3(unsigned(n) * (N / 256)), dim3(512), 0, s, A, B,
                       C, offsets, rows, n, K, N, row_limit);
  else
    hipLaunchKernelGGL((k_grouped_gemm_stream<4, RELU, PACKED>), dim3(unsigned(n) * (N / 128)), dim3(256), 0, s, A, B,
                       C, offsets, rows, n, K, N, row_limit);
}

bool ffn_packed_ok(int d, int d_ff, int rows_max, int n) {
  const int row_limit = int(std::min<int64_t>(int64_t(n) * rows_max, 0x7FFFFFFF));
  return ffn_streams(d, d_ff, row_limit) && ffn_streams(d_ff, d, row_limit);
}

hipError_t launch_expert_ffn(int n, int d, int d_ff, int rows_max, const int32_t* offsets, const int32_t* rows,
                             const uint16_t* D, const uint16_t* w1, const uint16_t* w2, uint16_t* hidden, uint16_t* y,
                             hipStream_t s, bool packed) {
  const int row_limit = int(std::min<int64_t>(int64_t(n) * rows_max, 0x7FFFFFFF));
  if (packed) {   // the caller checked ffn_packed_ok
    launch_stream<true, true>(n, d, d_ff, row_limit, offsets, rows, D, w1, hidden, s);
    launch_stream<false, true>(n, d_ff, d, row_limit, offsets, rows, hidden, w2, y, s);
    return hipGetLastError();
  }
  if (ffn_streams(d, d_ff, row_limit))
    launch_stream<true, false>(n, d, d_ff, row_limit, offsets, rows, D, w1, hidden, s);
  else
    hipLaunchKernelGGL(k_grouped_gemm<true>, dim3(ceil_div(d_ff, 128), n), dim3(256), 0, s, D, w1, hidden, offsets,
                       rows, d, d_ff, row_limit);
  if (ffn_streams(d_ff, d, row_limit))
    launch_stream<false, false>(n, d_ff, d, row_limit, offsets, rows, hidden, w2, y, s);
  else
    hipLaunchKernelGGL(k_grouped_gemm<false>, dim3(ceil_div(d, 128), n), dim3(256), 0, s, hidden, w2, y, offsets,
                       rows, d_ff, d, row_limit);
  return hipGetLastError();
}

}  // namespace moe
