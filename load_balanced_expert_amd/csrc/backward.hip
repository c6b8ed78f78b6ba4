// Backward pass of the Switch layer: gradients of L = Σ out ⊙ dout + L_aux with respect to x,
// W_r, W1 and W2, at one forward's saved values (selection, gates, dispatch maps, the
// dispatched rows D, the hidden activation H and the expert outputs Y).
//
// [Switch review] "Switch Routing 메커니즘" Step 3: the output is scaled by the chosen
// expert's router probability, which carries the gradient to W_r; [Switch impl] "argmax가
// 있어도 Router를 학습할 수 있는 이유": the expert id itself gets no gradient.  [Switch review]
// "로드 밸런싱 손실": f_i (from the argmax) is constant, P_i (mean softmax) is differentiable.
//
//   dY[row] = g·dout[t],  dg = <dout[t], Y[row]>              (combine transpose)  k_bwd_gate
//   dA = (dY·W2_e) ⊙ [H > 0],  dD = dA·W1_e                    (expert data gradients)
//   dW2_e = dYᵀ·H,  dW1_e = dAᵀ·D                              (expert weight gradients)
//   h = x·W_r,  p = softmax(h),  c_j = α·N·f_j/T
//   dh = Σ_r dg_r·g_r·(e_{i_r} − p) + p ⊙ (c − <p, c>)          (softmax Jacobian)  k_bwd_dh
//   dW_r = xᵀ·dh,  dx = dout + Σ_r dD[row_r] + dh·W_rᵀ         (dispatch transpose) k_bwd_dx
//
// Every product is one launch of a grouped MFMA GEMM (64 x 64 output tiles, 4 waves of
// 32 x 32, K in steps of 32 staged through LDS): bf16 operands with fp32 accumulation for the
// expert GEMMs (v_mfma_f32_32x32x16_bf16), fp32 operands for the router's (v_mfma_f32_32x32x2_f32:
// the router runs in fp32, [Switch review] "선택적 정밀도 캐스팅").  dW_r's long reduction over
// the tokens is split into token ranges whose partial products are summed in a fixed order.

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kBwdTile = 64;
constexpr int kBwdK = 32;
constexpr int kBwdThreads = 256;

// ------------------------------------------------------------------ grouped GEMM
// C_g[M, N] = A_g[M, K] · B_g[K, N] for groups g (experts or split-K ranges).  Element (m, k) of
// A sits at A + m·sAm + k·sAk, element (k, n) of B at B + k·sBk + n·sBn, element (m, n) of C at
// C + m·ldc + n.  Per group: rows_dim 0 — M is the group's row count (rows of the dispatched
// buffer from offsets[g]: A's and C's row index is offsets[g] + m); rows_dim 1 — K is the group's
// row count (A's and B's k index is offsets[g] + k); rows_dim 2 — fixed sizes.  gA, gB, gC move
// A, B, C by group (per-expert weights and gradients); with splits > 1 each group is a range of
// K (split s covers [s·K/splits, (s+1)·K/splits)) and writes its own C at C + s·gC.
struct GemmArgs {
  const void* A;
  const void* B;
  void* C;
  int64_t sAm, sAk, sBk, sBn, ldc;
  int64_t gA, gB, gC;
  int M, N, K;
  const int32_t* offsets;
  const int32_t* rows;      // rows of each group (nullptr: offsets[g + 1] - offsets[g])
  int rows_dim;
  int splits;
  const uint16_t* mask;     // out = bf16(acc · [mask > 0]) when set (C then bf16, same indexing)
};

__device__ __forceinline__ float ld_elem(const void* p, int64_t i, bool f32) {
  return f32 ? static_cast<const float*>(p)[i] : bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}

// fp32 MFMA form: operands of type TA / TB (0 bf16, 1 fp32) converted to fp32 in LDS.  VEC: every
// operand's contiguous dimension (and K when k is contiguous) a multiple of 8, the tile staged
// with 16-byte loads (the next K step's issued before the current step's products); else each
// element is loaded and range-checked alone.
template <int TA, int TB, bool VEC>
__global__ __launch_bounds__(kBwdThreads) void k_bwd_gemm_f32(GemmArgs a) {
  __shared__ float As[kBwdTile][kBwdK + 1];   // [m][k]
  __shared__ float Bs[kBwdTile][kBwdK + 1];   // [n][k]
  const int g = blockIdx.z;
  const int e = a.splits > 1 ? 0 : g;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int M = a.M, K = a.K;
  int64_t row0 = 0;
  if (a.rows_dim < 2) {
    row0 = a.offsets[e];
    const int cnt = a.rows ? a.rows[e] : a.offsets[e + 1] - a.offsets[e];
    if (a.rows_dim == 0) M = cnt; else K = cnt;
  }
  const int m0 = blockIdx.y * kBwdTile, n0 = blockIdx.x * kBwdTile;
  if (m0 >= M && a.rows_dim == 0) return;   // this expert has no rows here
  int k_begin = 0, k_end = K;
  if (a.splits > 1) {
    k_begin = int(int64_t(g) * K / a.splits);
    k_end = int(int64_t(g + 1) * K / a.splits);
  }
  const char* Ab = static_cast<const char*>(a.A) + int64_t(e) * a.gA * (TA ? 4 : 2);
  const char* Bb = static_cast<const char*>(a.B) + int64_t(e) * a.gB * (TB ? 4 : 2);
  // A / B index of (m, k) / (k, n) with the group's row offset applied
  auto a_idx = [&](int m, int k) {
    const int64_t mm = a.rows_dim == 0 ? row0 + m : m, kk = a.rows_dim == 1 ? row0 + k : k;
    return mm * a.sAm + kk * a.sAk;
  };
  auto b_idx = [&](int k, int n) {
    const int64_t kk = a.rows_dim == 1 ? row0 + k : k;
    return kk * a.sBk + int64_t(n) * a.sBn;
  };
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32, r32 = lane & 31, h = lane >> 5;
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  if constexpr (VEC) {
    // the thread's 8 elements of one operand tile [64 outer][32 k]: fp32 as two 16-byte vectors,
    // bf16 as one; along k when k is contiguous, else along the outer dimension
    auto fetch = [&](const char* base, bool fp32, bool kc, bool is_a, int lim, int o0, int k0, u32x4 (&r)[2],
                     int& o, int& kk) {
      const int per = fp32 ? 4 : 8;   // elements per vector
      r[0] = r[1] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (!fp32 && u == 1) break;
        const int v = fp32 ? tid + kBwdThreads * u : tid;
        int oo, kq;
        if (kc) { oo = v / (32 / per); kq = (v % (32 / per)) * per; } else { kq = v / (64 / per); oo = (v % (64 / per)) * per; }
        if (u == 0) { o = oo; kk = kq; }
        const int go = o0 + oo, gk = k0 + kq;
        if (go < lim && gk < k_end) {
          const int64_t ix = is_a ? a_idx(go, gk) : b_idx(gk, go);
          r[u] = *reinterpret_cast<const u32x4*>(base + ix * (fp32 ? 4 : 2));
        }
      }
    };
    auto put = [&](float (*S)[kBwdK + 1], bool fp32, bool kc, const u32x4 (&r)[2], int o, int kk) {
      if (fp32) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int v = tid + kBwdThreads * u;
          int oo, kq;
          if (kc) { oo = v / 8; kq = (v % 8) * 4; } else { kq = v / 16; oo = (v % 16) * 4; }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float f = __uint_as_float(r[u][j]);
            if (kc) S[oo][kq + j] = f; else S[oo + j][kq] = f;
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float f = bf16_to_f32(uint16_t(r[0][j >> 1] >> (16 * (j & 1))));
          if (kc) S[o][kk + j] = f; else S[o + j][kk] = f;
        }
      }
    };
    const bool akc = a.sAk == 1, bkc = a.sBk == 1;
    u32x4 ra[2], rb[2];
    int ao, ak, bo, bk;
    fetch(Ab, TA == 1, akc, true, M, m0, k_begin, ra, ao, ak);
    fetch(Bb, TB == 1, bkc, false, a.N, n0, k_begin, rb, bo, bk);
    for (int k0 = k_begin; k0 < k_end; k0 += kBwdK) {
      put(As, TA == 1, akc, ra, ao, ak);
      put(Bs, TB == 1, bkc, rb, bo, bk);
      lds_barrier();
      if (k0 + kBwdK < k_end) {
        fetch(Ab, TA == 1, akc, true, M, m0, k0 + kBwdK, ra, ao, ak);
        fetch(Bb, TB == 1, bkc, false, a.N, n0, k0 + kBwdK, rb, bo, bk);
      }
#pragma unroll
      for (int s = 0; s < kBwdK / 2; ++s) {
        const float av = As[wm + r32][2 * s + h], bv = Bs[wn + r32][2 * s + h];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
      }
      lds_barrier();
    }
  } else {
    for (int k0 = k_begin; k0 < k_end; k0 += kBwdK) {
      // stage A [64 m][32 k] and B [64 n][32 k]: 2048 elements each, 8 per thread, every element
      // range-checked (zeros outside)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = tid + u * kBwdThreads;
        // A: k fastest when A is k-contiguous, else m fastest (coalesced either way)
        int am, ak;
        if (a.sAk == 1) { am = i >> 5; ak = i & 31; } else { ak = i >> 6; am = i & 63; }
        const int gm = m0 + am, gk = k0 + ak;
        float av = 0.f;
        if (gm < M && gk < k_end) av = ld_elem(Ab, a_idx(gm, gk), TA == 1);
        int bn, bk;
        if (a.sBk == 1) { bn = i >> 5; bk = i & 31; } else { bk = i >> 6; bn = i & 63; }
        const int gn = n0 + bn, gk2 = k0 + bk;
        float bv = 0.f;
        if (gn < a.N && gk2 < k_end) bv = ld_elem(Bb, b_idx(gk2, gn), TB == 1);
        As[am][ak] = av;
        Bs[bn][bk] = bv;
      }
      __syncthreads();
#pragma unroll
      for (int s = 0; s < kBwdK / 2; ++s) {
        const float av = As[wm + r32][2 * s + h], bv = Bs[wn + r32][2 * s + h];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
      }
      __syncthreads();
    }
  }
  // store: element i of the accumulator is row 8 (i / 4) + 4 h + i % 4, column r32 of the 32 x 32 tile
  const int64_t cg = int64_t(g) * a.gC;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = m0 + wm + 8 * (i >> 2) + 4 * h + (i & 3), n = n0 + wn + r32;
    if (m < M && n < a.N) {
      const int64_t mm = a.rows_dim == 0 ? row0 + m : m;
      static_cast<float*>(a.C)[cg + mm * a.ldc + n] = acc[i];
    }
  }
}

// bf16 MFMA form (v_mfma_f32_32x32x16_bf16), both operands bf16.  Each K step of 32 puts the
// operand tiles [64 outer][32 k] in LDS with k contiguous; each operand arrives as one 16-byte
// vector per thread (256 vectors per tile), along k when k is contiguous in memory (written to
// LDS whole), along the outer dimension otherwise (written element by element, transposed).  The
// contiguous dimension of each operand is a multiple of 8; a vector past the tile's valid range
// is zeros.  The next step's loads are issued before the current step's products.
__global__ __launch_bounds__(kBwdThreads) void k_bwd_gemm_bf16(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kBwdTile][kBwdK + 8];   // [m][k]
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kBwdTile][kBwdK + 8];   // [n][k]
  const int g = blockIdx.z;
  const int e = a.splits > 1 ? 0 : g;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int M = a.M, K = a.K;
  int64_t row0 = 0;
  if (a.rows_dim < 2) {
    row0 = a.offsets[e];
    const int cnt = a.rows ? a.rows[e] : a.offsets[e + 1] - a.offsets[e];
    if (a.rows_dim == 0) M = cnt; else K = cnt;
  }
  const int m0 = blockIdx.y * kBwdTile, n0 = blockIdx.x * kBwdTile;
  if (m0 >= M && a.rows_dim == 0) return;   // this expert has no rows here
  int k_begin = 0, k_end = K;
  if (a.splits > 1) {
    k_begin = int(int64_t(g) * K / a.splits);
    k_end = int(int64_t(g + 1) * K / a.splits);
  }
  const uint16_t* Ab = static_cast<const uint16_t*>(a.A) + int64_t(e) * a.gA;
  const uint16_t* Bb = static_cast<const uint16_t*>(a.B) + int64_t(e) * a.gB;
  auto a_idx = [&](int m, int k) {
    const int64_t mm = a.rows_dim == 0 ? row0 + m : m, kk = a.rows_dim == 1 ? row0 + k : k;
    return mm * a.sAm + kk * a.sAk;
  };
  auto b_idx = [&](int k, int n) {
    const int64_t kk = a.rows_dim == 1 ? row0 + k : k;
    return kk * a.sBk + int64_t(n) * a.sBn;
  };
  const bool a_kc = a.sAk == 1, b_kc = a.sBk == 1;
  // the thread's vector of one operand at step k0: (outer, k .. k + 7) or (outer .. outer + 7, k)
  auto fetch = [&](const uint16_t* base, bool kc, bool is_a, int lim, int o0, int k0) {
    u32x4 w = u32x4{0u, 0u, 0u, 0u};
    if (kc) {
      const int go = o0 + (tid >> 2), gk = k0 + (tid & 3) * 8;
      if (go < lim && gk < k_end)
        w = *reinterpret_cast<const u32x4*>(base + (is_a ? a_idx(go, gk) : b_idx(gk, go)));
    } else {
      const int go = o0 + (tid & 7) * 8, gk = k0 + (tid >> 3);
      if (go < lim && gk < k_end)
        w = *reinterpret_cast<const u32x4*>(base + (is_a ? a_idx(go, gk) : b_idx(gk, go)));
    }
    return w;
  };
  auto put = [&](uint16_t (*S)[kBwdK + 8], bool kc, const u32x4& w) {
    if (kc) {
      *reinterpret_cast<u32x4*>(&S[tid >> 2][(tid & 3) * 8]) = w;
    } else {
      const int o = (tid & 7) * 8, kk = tid >> 3;
#pragma unroll
      for (int j = 0; j < 8; ++j) S[o + j][kk] = uint16_t(w[j >> 1] >> (16 * (j & 1)));
    }
  };
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32, r32 = lane & 31, h = lane >> 5;
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  u32x4 ra = fetch(Ab, a_kc, true, M, m0, k_begin);
  u32x4 rb = fetch(Bb, b_kc, false, a.N, n0, k_begin);
  for (int k0 = k_begin; k0 < k_end; k0 += kBwdK) {
    put(As, a_kc, ra);
    put(Bs, b_kc, rb);
    lds_barrier();
    if (k0 + kBwdK < k_end) {
      ra = fetch(Ab, a_kc, true, M, m0, k0 + kBwdK);
      rb = fetch(Bb, b_kc, false, a.N, n0, k0 + kBwdK);
    }
#pragma unroll
    for (int s = 0; s < kBwdK / 16; ++s) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(&As[wm + r32][16 * s + 8 * h]);
      const bf16x8 bf = *reinterpret_cast<const bf16x8*>(&Bs[wn + r32][16 * s + 8 * h]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc, 0, 0, 0);
    }
    lds_barrier();
  }
  const int64_t cg = int64_t(g) * a.gC;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = m0 + wm + 8 * (i >> 2) + 4 * h + (i & 3), n = n0 + wn + r32;
    if (m < M && n < a.N) {
      const int64_t mm = a.rows_dim == 0 ? row0 + m : m;
      const int64_t o = cg + mm * a.ldc + n;
      if (a.mask) {
        const float v = a.mask[o] > 0 && (a.mask[o] & 0x8000u) == 0 ? acc[i] : 0.f;   // H > 0 (bf16 bits)
        static_cast<uint16_t*>(a.C)[o] = f32_to_bf16(v);
      } else {
        static_cast<float*>(a.C)[o] = acc[i];
      }
    }
  }
}

// ------------------------------------------------------------------ data gradients: weight stream
// dA = (dY · W2_e) ⊙ [H > 0] and dD = dA · W1_e read the weights as stored, [K][N] with N
// contiguous (W2 [d][d_ff], W1 [d_ff][d]).  As in the forward FFN, one workgroup (W waves) owns an
// expert and 32 W output columns and reads that weight slab once per 128 rows: the expert's rows
// are staged through LDS in K chunks of 128 (register prefetch of the next chunk), each wave
// streams its 64 x 32 weight block per K step of 64 (four 16-byte loads per lane, kNnRing - 1
// steps ahead) into its own LDS slab in the stored [k][n] layout, and takes its MFMA B fragments
// with the gfx950 LDS transpose read ds_read_b64_tr_b16: in each 16-lane group, lane L names row
// L / 4 and columns 4 (L % 4) .. + 3 of a 4 x 16 block, and lane i receives column i's 4 values.
// Requires K % 256 == 0 and N % (32 W) == 0.
constexpr int kNnKA = 128;           // K per staged A chunk
constexpr int kNnLdA = kNnKA + 8;    // LDS row stride of the A chunk (bf16)
constexpr int kNnLdB = 40;           // per-wave slab row stride (bf16): 32 columns + 16 bytes
constexpr int kNnRing = 4;           // weight K steps in flight + 1 (even)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((__attribute__((address_space(3))) uint16_t*)(p)));
}

// BF16OUT: bf16 output times [H > 0] (omask = H, indexed as the output), else fp32 output
template <int W, int MT, bool BF16OUT>
__device__ __forceinline__ void nn_rows(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                        void* __restrict__ C, const uint16_t* __restrict__ omask, uint16_t* As,
                                        uint16_t* Bs, int r0, int r_end, int K, int N, int col0, int tid) {
  const int lane = tid & 63, h = lane >> 5, r32 = lane & 31;
  const int nks = K / 64, nch = K / kNnKA;
  constexpr int AL = 8 * MT / W;       // A chunk: 32 MT rows x 16 segments of 16 bytes over the workgroup
  const int row0 = tid >> 4, seg = tid & 15;
  constexpr int kRowStep = 64 * W / 16;
  const int lo0 = row0 * kNnLdA + seg * 8;
  u32x4 areg[AL];
  auto a_fetch = [&](int c) {
    c = min(c, nch - 1);
#pragma unroll
    for (int u = 0; u < AL; ++u) {
      const uint32_t off = uint32_t(min(r0 + row0 + kRowStep * u, r_end - 1)) * uint32_t(K) + c * kNnKA + seg * 8;
      areg[u] = *reinterpret_cast<const u32x4*>(A + off);
    }
  };
  auto a_store = [&]() {
#pragma unroll
    for (int u = 0; u < AL; ++u)
      *reinterpret_cast<u32x4*>(As + lo0 + u * kRowStep * kNnLdA) = areg[u];
  };
  // weight K step s: load q brings row 16 q + lane / 4 of the step's 64, columns 8 (lane % 4) .. + 7
  const uint16_t* bp = B + size_t(lane >> 2) * N + col0 + 8 * (lane & 3);
  auto b_fetch = [&](u32x4 (&b)[4], int s) {
    s = min(s, nks - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) b[q] = *reinterpret_cast<const u32x4*>(bp + size_t(64 * s + 16 * q) * N);
  };
  uint16_t* bw = Bs + (tid >> 6) * (64 * kNnLdB);
  auto b_stage = [&](const u32x4 (&b)[4]) {   // same-wave LDS accesses stay in order
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<u32x4*>(bw + (16 * q + (lane >> 2)) * kNnLdB + 8 * (lane & 3)) = b[q];
  };
  // B fragment of substep q: k = 32 h + 8 q + [0, 8) of column r32, two transposed 4 x 16 reads;
  // 16-lane group g covers columns 16 (g % 2) + [0, 16) and the k rows of h = g / 2
  const int g = lane >> 4, L = lane & 15;
  const uint16_t* bt0 = bw + (32 * (g >> 1) + (L >> 2)) * kNnLdB + 16 * (g & 1) + 4 * (L & 3);
  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;
  const uint16_t* arow = As + r32 * kNnLdA + 32 * h;
  auto step = [&](const u32x4 (&b)[4], int t) {
    b_stage(b);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const s16x4 lo = lds_read_tr16(bt0 + (8 * q) * kNnLdB);
      const s16x4 hi = lds_read_tr16(bt0 + (8 * q + 4) * kNnLdB);
      const bf16x8 bf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(arow + 32 * mt * kNnLdA + 64 * t + 8 * q);
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bf, acc[mt], 0, 0, 0);
      }
    }
  };
  u32x4 ring[kNnRing][4];
  a_fetch(0);
  a_store();
  a_fetch(1);
#pragma unroll
  for (int u = 0; u < kNnRing - 1; ++u) b_fetch(ring[u], u);
  lds_barrier();
  for (int s0 = 0; s0 < nks; s0 += kNnRing) {
#pragma unroll
    for (int u = 0; u < kNnRing; ++u) {
      if (s0 + u < nks) {
        b_fetch(ring[(u + kNnRing - 1) % kNnRing], s0 + u + kNnRing - 1);
        step(ring[u], u & 1);
        if (u & 1) {   // chunk (s0 + u) / 2 consumed: stage the next one, prefetch the one after
          lds_barrier();
          a_store();
          a_fetch((s0 + u) / 2 + 2);
          lds_barrier();
        }
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    // the tile's 16 mask values read together, then its 16 outputs
    uint16_t hv[16];
    if constexpr (BF16OUT) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = min(r0 + 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3), r_end - 1);
        hv[i] = omask[size_t(row) * N + col0 + r32];
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = r0 + 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
      if (row < r_end) {
        const size_t o = size_t(row) * N + col0 + r32;
        if constexpr (BF16OUT) {
          static_cast<uint16_t*>(C)[o] = f32_to_bf16(int16_t(hv[i]) > 0 ? acc[mt][i] : 0.f);
        } else {
          static_cast<float*>(C)[o] = acc[mt][i];
        }
      }
    }
  }
}

template <int W, bool BF16OUT>
__global__ __launch_bounds__(64 * W) void k_bwd_nn_stream(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                          void* __restrict__ C, const uint16_t* __restrict__ omask,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ rows, int n, int K, int N) {
  __shared__ __attribute__((aligned(16))) uint16_t As[128 * kNnLdA];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[W * 64 * kNnLdB];
  const int ncb = N / (32 * W);
  const unsigned G = unsigned(n) * ncb, b = blockIdx.x;
  // XCD-major order: workgroup b runs on XCD b % 8; give each XCD a contiguous range of (expert, block)
  const unsigned Lx = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
  const int e = int(Lx / ncb), cb = int(Lx % ncb);
  const int r_begin = offsets[e], r_end = rows ? offsets[e] + rows[e] : offsets[e + 1];
  const int col0 = cb * (32 * W) + (threadIdx.x >> 6) * 32;
  const uint16_t* Be = B + size_t(e) * K * N;
  for (int r0 = r_begin; r0 < r_end; r0 += 128) {
    switch (ceil_div(min(128, r_end - r0), 32)) {
      case 1: nn_rows<W, 1, BF16OUT>(A, Be, C, omask, As, Bs, r0, r_end, K, N, col0, threadIdx.x); break;
      case 2: nn_rows<W, 2, BF16OUT>(A, Be, C, omask, As, Bs, r0, r_end, K, N, col0, threadIdx.x); break;
      case 3: nn_rows<W, 3, BF16OUT>(A, Be, C, omask, As, Bs, r0, r_end, K, N, col0, threadIdx.x); break;
      default: nn_rows<W, 4, BF16OUT>(A, Be, C, omask, As, Bs, r0, r_end, K, N, col0, threadIdx.x); break;
    }
  }
}

// ------------------------------------------------------------------ weight gradients
// C_e[M][N] (fp32) = Σ_r A[r][m] · B[r][n] over the rows r of expert e: dW2_e = dYᵀ·H (A = dY
// [rows][d], B = H [rows][d_ff]) and dW1_e = dAᵀ·D (A = dA [rows][d_ff], B = D [rows][d]).  Both
// operands are stored k-major (a row per token), so both are staged in that layout and read into
// MFMA fragments by LDS transpose reads.  Workgroup: 128 x 256 outputs of one expert, 8 waves of
// 64 x 64 (2 x 2 accumulators); the expert's rows in passes of 64 (the next pass's loads issued
// before the current pass's products), rows past the expert's zero-filled.  The workgroup order
// keeps an expert's blocks on one XCD.  Requires M % 128 == 0 and N % 256 == 0; an expert without
// rows gets zeros.
constexpr int kWgBM = 128, kWgBN = 256, kWgK = 64;
constexpr int kWgLdA = kWgBM + 16, kWgLdB = kWgBN + 16;   // bf16 strides: 4 rows of a transposed read on distinct banks

__global__ __launch_bounds__(512, 4) void k_bwd_wgrad(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                   float* __restrict__ C, const int32_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ rows, int n, int M, int N) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kWgK * kWgLdA];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kWgK * kWgLdB];
  const int nbm = M / kWgBM, nbn = N / kWgBN, per = nbm * nbn;
  const unsigned G = unsigned(n) * per, b = blockIdx.x;
  const unsigned Lx = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;   // XCD-major
  const int e = int(Lx / per), bi = int(Lx % per), bm = bi / nbn, bn = bi % nbn;
  const int r0 = offsets[e], K = rows ? rows[e] : offsets[e + 1] - offsets[e];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r32 = lane & 31, h = lane >> 5;
  const int m0 = bm * kWgBM, n0 = bn * kWgBN;
  const int wm = (wave >> 2) * 64, wn = (wave & 3) * 64;
  // staging: A pass [64 k][128 m] = 1024 vectors of 8, B pass [64 k][256 n] = 2048: 2 + 4 per thread
  u32x4 ra[2], rb[4];
  // the workgroup's operand bases (uniform) and 32-bit element offsets per lane (K <= rows of one
  // expert, so (k0 + k) · N stays far below 2^32)
  const uint16_t* Ab = A + size_t(r0) * M + m0;
  const uint16_t* Bb = B + size_t(r0) * N + n0;
  auto fetch = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int v = tid + 512 * u, k = v >> 4, mm = (v & 15) * 8;
      ra[u] = k0 + k < K ? *reinterpret_cast<const u32x4*>(Ab + uint32_t((k0 + k) * M + mm)) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = tid + 512 * u, k = v >> 5, nn = (v & 31) * 8;
      rb[u] = k0 + k < K ? *reinterpret_cast<const u32x4*>(Bb + uint32_t((k0 + k) * N + nn)) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto put = [&]() {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int v = tid + 512 * u;
      *reinterpret_cast<u32x4*>(As + (v >> 4) * kWgLdA + (v & 15) * 8) = ra[u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = tid + 512 * u;
      *reinterpret_cast<u32x4*>(Bs + (v >> 5) * kWgLdB + (v & 31) * 8) = rb[u];
    }
  };
  // transposed fragment reads: 16-lane group g covers outer 16 (g % 2) + [0, 16) and the k rows of h = g / 2
  const int g = lane >> 4, L = lane & 15;
  const uint16_t* at0 = As + (8 * (g >> 1) + (L >> 2)) * kWgLdA + wm + 16 * (g & 1) + 4 * (L & 3);
  const uint16_t* bt0 = Bs + (8 * (g >> 1) + (L >> 2)) * kWgLdB + wn + 16 * (g & 1) + 4 * (L & 3);
  auto frag = [&](const uint16_t* p, int ld) -> bf16x8 {
    const s16x4 lo = lds_read_tr16(p);
    const s16x4 hi = lds_read_tr16(p + 4 * ld);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[u][v][i] = 0.f;
  if (K > 0) fetch(0);
  for (int k0 = 0; k0 < K; k0 += kWgK) {
    put();
    lds_barrier();
    if (k0 + kWgK < K) fetch(k0 + kWgK);
#pragma unroll
    for (int st = 0; st < kWgK / 16; ++st) {
      bf16x8 af[2], bf[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) af[u] = frag(at0 + 16 * st * kWgLdA + 32 * u, kWgLdA);
#pragma unroll
      for (int v = 0; v < 2; ++v) bf[v] = frag(bt0 + 16 * st * kWgLdB + 32 * v, kWgLdB);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 2; ++v) acc[u][v] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[u], bf[v], acc[u][v], 0, 0, 0);
    }
    lds_barrier();
  }
  float* Cw = C + size_t(e) * M * N + size_t(m0 + wm) * N + n0 + wn;   // this wave's 64 x 64 block
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int mr = 32 * u + 8 * (i >> 2) + 4 * h + (i & 3), nc = 32 * v + r32;
        __builtin_nontemporal_store(acc[u][v][i], Cw + uint32_t(mr * N + nc));   // written once, read by the caller
      }
}

// Fixed-order sum of split-K partials: out[i] = Σ_s part[s][i].
__global__ __launch_bounds__(256) void k_bwd_sum_splits(const float* __restrict__ part, int splits, int64_t count,
                                                        float* __restrict__ out) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < count; i += int64_t(gridDim.x) * 256) {
    float v = 0.f;
    for (int s = 0; s < splits; ++s) v += part[int64_t(s) * count + i];
    out[i] = v;
  }
}

// ------------------------------------------------------------------ combine transpose
// One wave per token: for each kept pair, dg = <dout[t], Y[row]> (lane partials, then a butterfly
// sum: a fixed order) and dY[row] = bf16(g · dout[t]); dropped pairs get dg = 0.
__global__ __launch_bounds__(256) void k_bwd_gate(int64_t m, int d, int k, const float* __restrict__ dout,
                                                  const uint16_t* __restrict__ y, const float* __restrict__ gate,
                                                  const int32_t* __restrict__ t2r, uint16_t* __restrict__ dy,
                                                  float* __restrict__ dgate) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * 4 + wave;
  if (t >= m) return;
  for (int r = 0; r < k; ++r) {
    const int32_t row = t2r[t * k + r];
    float part = 0.f;
    if (row >= 0) {
      const float g = gate[t * k + r];
      for (int c = lane; c < d; c += 64) {
        const float go = dout[t * d + c];
        part += go * bf16_to_f32(y[int64_t(row) * d + c]);
        dy[int64_t(row) * d + c] = f32_to_bf16(g * go);
      }
    }
    const float dg = wave_sum(part);
    if (lane == 0) dgate[t * k + r] = row >= 0 ? dg : 0.f;
  }
}

// ------------------------------------------------------------------ router: softmax Jacobian
// One wave per token over its logits row h (fp32, in place): p = softmax(h),
// dh = Σ_r dg_r·g_r·(e_{i_r} − p) + p ⊙ (c − <p, c>), c_j = α·N·counts_j / T².  g_r is the
// chosen expert's probability recomputed here.
__global__ __launch_bounds__(256) void k_bwd_dh(int64_t m, int n, int k, float* __restrict__ hrow,
                                                const int32_t* __restrict__ idx, const float* __restrict__ dgate,
                                                const int32_t* __restrict__ counts, float alpha) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * 4 + wave;
  if (t >= m) return;
  float* h = hrow + t * n;
  const double cs = double(alpha) * double(n) / (double(m) * double(m));
  float mx = -INFINITY;
  for (int j = lane; j < n; j += 64) mx = fmaxf(mx, h[j]);
  mx = wave_max(mx);
  float s = 0.f;
  for (int j = lane; j < n; j += 64) s += expf(h[j] - mx);
  const float inv = 1.0f / wave_sum(s);
  float pc = 0.f;   // <p, c>
  for (int j = lane; j < n; j += 64) pc += expf(h[j] - mx) * inv * float(cs * double(counts[j]));
  pc = wave_sum(pc);
  // lane r < k holds pick r: its expert and dg_r·g_r, with g_r the chosen expert's probability
  // (k <= 64, one lane per pick); Σ_r dg_r g_r over the wave
  const int my_j = lane < k ? idx[t * k + lane] : -1;
  const float my_coef = lane < k ? dgate[t * k + lane] * (expf(h[my_j] - mx) * inv) : 0.f;
  const float csum = wave_sum(my_coef);
  __builtin_amdgcn_wave_barrier();   // every lane has read the logits it needs before any is overwritten
  // whole-wave passes (the shuffles read every pick's lane), the stores guarded
  for (int j0 = 0; j0 < n; j0 += 64) {
    const int j = j0 + lane;
    float add = 0.f;
    for (int r = 0; r < k; ++r) {
      const int jr = __shfl(my_j, r);
      const float cr = __shfl(my_coef, r);
      if (jr == j) add += cr;
    }
    if (j < n) {
      const float p = expf(h[j] - mx) * inv;
      h[j] = p * (float(cs * double(counts[j])) - pc) - csum * p + add;
    }
  }
}

// ------------------------------------------------------------------ dx assembly
// dx[t] = dout[t] + Σ_r dD[row(t, r)] (kept pairs, r in order) + dxr[t].
__global__ __launch_bounds__(256) void k_bwd_dx(int64_t m, int d, int k, const float* __restrict__ dout,
                                                const float* __restrict__ dD, const int32_t* __restrict__ t2r,
                                                const float* __restrict__ dxr, float* __restrict__ dx) {
  const int64_t items = m * d;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < items; i += int64_t(gridDim.x) * 256) {
    const int64_t t = i / d, c = i - t * d;
    float v = dout[i];
    for (int r = 0; r < k; ++r) {
      const int32_t row = t2r[t * k + r];
      if (row >= 0) v += dD[int64_t(row) * d + c];
    }
    dx[i] = v + dxr[i];
  }
}

// ------------------------------------------------------------------ launcher
static size_t al256b(size_t b) { return (b + 255) / 256 * 256; }
constexpr int kBwdRouterSplits = 32;

size_t backward_ws_bytes(int64_t m, int d, int n, int k, int64_t rows_bound, int d_ff) {
  size_t b = 0;
  b += al256b(size_t(rows_bound) * d * sizeof(uint16_t));       // dY
  b += al256b(size_t(m) * k * sizeof(float));                    // dgate
  b += al256b(size_t(rows_bound) * d_ff * sizeof(uint16_t));    // dA
  b += al256b(size_t(rows_bound) * d * sizeof(float));          // dD
  b += al256b(size_t(m) * n * sizeof(float));                   // h, then dh
  b += al256b(size_t(m) * d * sizeof(float));                   // dh · W_rᵀ
  b += al256b(size_t(kBwdRouterSplits) * d * n * sizeof(float));  // dW_r partials
  return b;
}

static dim3 gemm_grid(const GemmArgs& a, int groups, int m_max) {
  return dim3(unsigned(ceil_div(a.N, kBwdTile)), unsigned(ceil_div(std::max(m_max, 1), kBwdTile)), unsigned(groups));
}

static void gemm_bf16(const GemmArgs& a, int groups, int m_max, hipStream_t s) {
  hipLaunchKernelGGL(k_bwd_gemm_bf16, gemm_grid(a, groups, m_max), dim3(kBwdThreads), 0, s, a);
}

// the vector form needs every operand's contiguous dimension, and K when k is contiguous (and
// every split range's start), to be multiples of 8
template <int TA, int TB>
static void gemm_f32(const GemmArgs& a, int groups, int m_max, hipStream_t s) {
  auto contig = [](int64_t s_outer, int64_t s_k, int outer) {
    return s_k == 1 ? (s_outer % 8 == 0) : (s_outer == 1 && s_k % 8 == 0 && outer % 8 == 0);
  };
  const bool k_ok = (a.sAk != 1 && a.sBk != 1) || (a.K % 8 == 0 && (a.splits <= 1 || a.K % (8 * a.splits) == 0));
  const bool vec = a.rows_dim == 2 && k_ok && contig(a.sAm, a.sAk, a.M) && contig(a.sBn, a.sBk, a.N);
  if (vec)
    hipLaunchKernelGGL((k_bwd_gemm_f32<TA, TB, true>), gemm_grid(a, groups, m_max), dim3(kBwdThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k_bwd_gemm_f32<TA, TB, false>), gemm_grid(a, groups, m_max), dim3(kBwdThreads), 0, s, a);
}

hipError_t launch_backward(const BackwardArgs& b, hipStream_t s) {
  char* ws = static_cast<char*>(b.ws);
  uint16_t* dY = reinterpret_cast<uint16_t*>(ws);
  ws += al256b(size_t(b.rows_bound) * b.d * sizeof(uint16_t));
  float* dgate = reinterpret_cast<float*>(ws);
  ws += al256b(size_t(b.m) * b.k * sizeof(float));
  uint16_t* dA = reinterpret_cast<uint16_t*>(ws);
  ws += al256b(size_t(b.rows_bound) * b.d_ff * sizeof(uint16_t));
  float* dD = reinterpret_cast<float*>(ws);
  ws += al256b(size_t(b.rows_bound) * b.d * sizeof(float));
  float* hbuf = reinterpret_cast<float*>(ws);
  ws += al256b(size_t(b.m) * b.n * sizeof(float));
  float* dxr = reinterpret_cast<float*>(ws);
  ws += al256b(size_t(b.m) * b.d * sizeof(float));
  float* dwr_part = reinterpret_cast<float*>(ws);

  const int n = b.n, d = b.d, d_ff = b.d_ff, k = b.k;
  const unsigned tok_blocks = unsigned(ceil_div64(b.m, 4));
  // 1. combine transpose: dY and the gate gradients
  hipLaunchKernelGGL(k_bwd_gate, dim3(tok_blocks), dim3(256), 0, s, b.m, d, k, b.dout, b.y, b.gate, b.t2r, dY, dgate);
  // 2. expert gradients, grouped by expert
  // the weight-stream form where the shapes allow it (and the row offsets fit 32 bits)
  auto nn_ok = [&](int K, int N) {
    return K % 256 == 0 && N % 256 == 0 && b.rows_bound * int64_t(K) < (int64_t(1) << 32);
  };
  const bool stream = nn_ok(d, d_ff) && nn_ok(d_ff, d);
  if (stream) {   // dA = (dY · W2_e) ⊙ [H > 0]: K = d, N = d_ff
    hipLaunchKernelGGL((k_bwd_nn_stream<8, true>), dim3(unsigned(n) * (d_ff / 256)), dim3(512), 0, s, dY,
                       static_cast<const uint16_t*>(b.w2), dA, b.hidden, b.offsets, b.rows, n, d, d_ff);
  } else {
    GemmArgs g{};   // dA = (dY · W2_e) ⊙ [H > 0]: M = rows, K = d, N = d_ff
    g.A = dY; g.sAm = d; g.sAk = 1;
    g.B = b.w2; g.sBk = d_ff; g.sBn = 1; g.gB = int64_t(d) * d_ff;
    g.C = dA; g.ldc = d_ff; g.mask = b.hidden;
    g.N = d_ff; g.K = d; g.offsets = b.offsets; g.rows = b.rows; g.rows_dim = 0; g.splits = 1;
    gemm_bf16(g, n, b.rows_max, s);
  }
  if (stream) {   // dD = dA · W1_e: K = d_ff, N = d
    hipLaunchKernelGGL((k_bwd_nn_stream<8, false>), dim3(unsigned(n) * (d / 256)), dim3(512), 0, s, dA,
                       static_cast<const uint16_t*>(b.w1), dD, nullptr, b.offsets, b.rows, n, d_ff, d);
  } else {
    GemmArgs g{};   // dD = dA · W1_e: M = rows, K = d_ff, N = d
    g.A = dA; g.sAm = d_ff; g.sAk = 1;
    g.B = b.w1; g.sBk = d; g.sBn = 1; g.gB = int64_t(d_ff) * d;
    g.C = dD; g.ldc = d;
    g.N = d; g.K = d_ff; g.offsets = b.offsets; g.rows = b.rows; g.rows_dim = 0; g.splits = 1;
    gemm_bf16(g, n, b.rows_max, s);
  }
  if (d % kWgBM == 0 && d_ff % kWgBN == 0) {   // dW2_e = dYᵀ · H: M = d, N = d_ff
    hipLaunchKernelGGL(k_bwd_wgrad, dim3(unsigned(n) * (d / kWgBM) * (d_ff / kWgBN)), dim3(512), 0, s, dY, b.hidden,
                       b.dw2, b.offsets, b.rows, n, d, d_ff);
  } else {
    GemmArgs g{};   // dW2_e = dYᵀ · H: M = d, K = rows, N = d_ff
    g.A = dY; g.sAm = 1; g.sAk = d;
    g.B = b.hidden; g.sBk = d_ff; g.sBn = 1;
    g.C = b.dw2; g.ldc = d_ff; g.gC = int64_t(d) * d_ff;
    g.M = d; g.N = d_ff; g.offsets = b.offsets; g.rows = b.rows; g.rows_dim = 1; g.splits = 1;
    gemm_bf16(g, n, d, s);
  }
  if (d_ff % kWgBM == 0 && d % kWgBN == 0) {   // dW1_e = dAᵀ · D: M = d_ff, N = d
    hipLaunchKernelGGL(k_bwd_wgrad, dim3(unsigned(n) * (d_ff / kWgBM) * (d / kWgBN)), dim3(512), 0, s, dA,
                       static_cast<const uint16_t*>(b.dispatched), b.dw1, b.offsets, b.rows, n, d_ff, d);
  } else {
    GemmArgs g{};   // dW1_e = dAᵀ · D: M = d_ff, K = rows, N = d
    g.A = dA; g.sAm = 1; g.sAk = d_ff;
    g.B = b.dispatched; g.sBk = d; g.sBn = 1;
    g.C = b.dw1; g.ldc = d; g.gC = int64_t(d_ff) * d;
    g.M = d_ff; g.N = d; g.offsets = b.offsets; g.rows = b.rows; g.rows_dim = 1; g.splits = 1;
    gemm_bf16(g, n, d_ff, s);
  }
  // 3. router: h = x · W_r in fp32, then dh in place
  {
    GemmArgs g{};
    g.A = b.x; g.sAm = d; g.sAk = 1;
    g.B = b.w_r; g.sBk = n; g.sBn = 1;
    g.C = hbuf; g.ldc = n;
    g.M = int(b.m); g.N = n; g.K = d; g.rows_dim = 2; g.splits = 1;
    if (b.x_bf16) gemm_f32<0, 1>(g, 1, int(b.m), s);
    else gemm_f32<1, 1>(g, 1, int(b.m), s);
  }
  hipLaunchKernelGGL(k_bwd_dh, dim3(tok_blocks), dim3(256), 0, s, b.m, n, k, hbuf, b.idx, dgate, b.counts, b.alpha);
  {
    GemmArgs g{};   // dh · W_rᵀ: M = m, K = n, N = d; B(k = j, n = c) = W_r[c][j]
    g.A = hbuf; g.sAm = n; g.sAk = 1;
    g.B = b.w_r; g.sBk = 1; g.sBn = n;
    g.C = dxr; g.ldc = d;
    g.M = int(b.m); g.N = d; g.K = n; g.rows_dim = 2; g.splits = 1;
    gemm_f32<1, 1>(g, 1, int(b.m), s);
  }
  {
    GemmArgs g{};   // dW_r = xᵀ · dh: M = d, K = m (split in token ranges), N = n
    g.A = b.x; g.sAm = 1; g.sAk = d;
    g.B = hbuf; g.sBk = n; g.sBn = 1;
    g.C = dwr_part; g.ldc = n; g.gC = int64_t(d) * n;
    g.M = d; g.N = n; g.K = int(b.m); g.rows_dim = 2; g.splits = kBwdRouterSplits;
    if (b.x_bf16) gemm_f32<0, 1>(g, kBwdRouterSplits, d, s);
    else gemm_f32<1, 1>(g, kBwdRouterSplits, d, s);
    const int64_t cnt = int64_t(d) * n;
    hipLaunchKernelGGL(k_bwd_sum_splits, dim3(unsigned(std::min<int64_t>(ceil_div64(cnt, 256), 4096))), dim3(256), 0,
                       s, dwr_part, kBwdRouterSplits, cnt, b.dw_r);
  }
  // 4. dx = dout + dispatch transpose + router path
  hipLaunchKernelGGL(k_bwd_dx, dim3(unsigned(std::min<int64_t>(ceil_div64(b.m * d, 256), 65536))), dim3(256), 0, s,
                     b.m, d, k, b.dout, dD, b.t2r, dxr, b.dx);
  return hipGetLastError();
}

}  // namespace moe
