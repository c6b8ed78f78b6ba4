// Router: h = x · W_r, softmax / sigmoid score, top-k selection, gates, the
// expert histogram and Σ_t score_j(t).
//
// [Switch review] "Switch Routing 메커니즘" Step 1-3 (h = x·W_r, p = softmax(h),
// i* = argmax p, gate = p_{i*}); "선택적 정밀도 캐스팅" (router in fp32 on bf16
// hidden states); [MoE tour 6] "방법 회고" eq. (1) (Loss-Free: top-k of ρ + b,
// gate ρ); [Switch review] "로드 밸런싱 손실" (counts for f_i, Σ p for P_i).
//
// gfx950 design
//  * bf16 x: W_r is split once into three bf16 planes hi + mid + lo that sum
//    exactly to the fp32 weight; three bf16 MFMAs with fp32 accumulation give
//    an fp32-accurate product (every bf16 x bf16 product is exact in fp32).
//    v_mfma_f32_32x32x16_bf16 on 64-lane waves.
//  * n <= 256: one 16-wave workgroup owns 32 tokens x all experts.  The K
//    dimension is split across waves, operands for the next K block are
//    loaded (branch-free) while the current one is multiplied, partial tiles
//    meet in LDS in a fixed order, and the epilogue (softmax statistics,
//    top-k, gates, histogram, per-expert score sums) runs in the same kernel.
//  * n > 256: a tiled MFMA GEMM writes fp32 logits to the workspace, then a
//    row kernel reads them once through LDS sub-tiles and runs the same
//    epilogue (one wave per token).
//  * Each workgroup stores its per-expert counts and score sums as a chunk
//    row; the workgroup that finishes last sums the rows in a fixed order
//    (prefix.hpp), so every output is bit-reproducible.  In the Switch layer
//    the route stops after its chunk rows and per-super-chunk sums, and the
//    dispatch derives the rest.
#include "common.hpp"
#include "dpp.hpp"
#include "kernels.hpp"
#include "prefix.hpp"

namespace moe {

constexpr int kRouteBM = 32;      // tokens per route workgroup (n <= 256)
constexpr int kRowsBM = 256;      // tokens per route-epilogue workgroup (n > 256)
constexpr int kRouteThreads = 1024;  // 16 waves

// LDS ints of the region each route kernel reserves.  Fused: the x tile (if
// staged, at most 128 KiB: the workgroup's K range of 32 rows) and the partial
// logit tiles [KS][32][npad + 8] (one per K group; the first becomes the
// logits tile), which either follow the x tile or, when both do not fit,
// reuse its region once the product is done; the last workgroup's finishing
// scratch reuses the tiles.  Rows kernel: the logit sub-tiles, then the
// scratch.  The padding of 8 columns puts the two lane halves of an
// accumulator store on different banks.
constexpr int kXStageMaxInts = 32768;
static int fused_parts(const RoutePlan& plan) {
  const int nt = plan.npad / 32;
  return plan.mfma ? 16 / (nt <= 1 ? 1 : nt <= 2 ? 2 : nt <= 4 ? 4 : 8) : 1;
}
static int fused_partial_ints(const RoutePlan& plan, int n) {
  return std::max(fused_parts(plan) * kRouteBM * (plan.npad + 8), n + 2 * kMaxSuperChunks * 16);
}
// width of the staged x tile: the K range of one workgroup (the whole of d
// unless the tile's K range is split over kg workgroups)
static int x_tile_cols(const RoutePlan& plan) {
  const int nkb = plan.dpad / 32;
  return (plan.kg > 1 ? (nkb + plan.kg - 1) / plan.kg : nkb) * 32;
}
static int x_tile_ints(const RoutePlan& plan) { return kRouteBM * (x_tile_cols(plan) + 8) / 2; }
static bool stage_x(const RoutePlan& plan, int) { return x_tile_ints(plan) + plan.npad <= kXStageMaxInts + 256; }
// whether the partial tiles get a region of their own after the x tile (it
// fits in LDS), so that each wave stores its partial tile as soon as its
// product is done instead of waiting until every wave has read the x tile
static bool partials_apart(const RoutePlan& plan, int n) {
  return plan.fused && plan.mfma && stage_x(plan, n) &&
         x_tile_ints(plan) + fused_partial_ints(plan, n) + 2 * plan.npad + 1024 <= 40960;   // + histogram, bias
}
static int route_region_ints(const RoutePlan& plan, int n) {
  if (!plan.fused) return n + 4096;
  const int part = fused_partial_ints(plan, n);
  if (partials_apart(plan, n)) return x_tile_ints(plan) + part;
  return plan.mfma && stage_x(plan, n) ? std::max(part, x_tile_ints(plan)) : part;
}

// Reading fp32 W_r (4 bytes per weight per workgroup) and splitting it in
// registers measured faster than loading prepared planes (6 bytes per weight)
// both at d x n = 768 x 128 and at 2048 x 256, and it needs no preparation
// kernel.
bool route_direct(const RoutePlan& plan, int d, int n) {
  return plan.fused && plan.mfma && d % 32 == 0 && (n == 32 || n == 64 || n == 128 || n == 256);
}

RoutePlan route_plan(int64_t m, int d, int n, bool x_bf16) {
  RoutePlan p{};
  p.fused = n <= kFusedMaxN;
  // matrix cores need d % 8 == 0 (16-byte rows); without the LDS x tile also d % 32 == 0
  p.mfma = x_bf16 && (d % 8 == 0);
  // fused: 32, 64, 128 or 256 columns, one 32-expert tile per wave column and
  // npad / 32 experts per lane in the epilogue; big n: 128-column GEMM tiles
  p.npad = p.fused ? (n <= 32 ? 32 : n <= 64 ? 64 : n <= 128 ? 128 : 256) : round_up(n, 128);
  p.dpad = round_up(d, 32);
  if (p.fused && p.mfma && p.dpad != d && !stage_x(p, n)) p.mfma = false;   // global x rows need d % 32 == 0
  p.planes_bytes = p.mfma ? size_t(3) * p.npad * p.dpad * sizeof(uint16_t) : 0;
  p.logits_bytes = p.fused ? 0 : size_t(m) * p.npad * sizeof(float);
  // Few token tiles (small batches): split each tile's K range over 2 or 4
  // workgroups so that the whole chip works; the last of them adds the parts.
  p.kg = 1;
  const int64_t tiles = ceil_div64(m, kRouteBM);
  if (route_direct(p, d, n) && tiles <= kMaxKgTiles) {
    const int nt = p.npad / 32, ks = 16 / (nt <= 1 ? 1 : nt <= 2 ? 2 : nt <= 4 ? 4 : 8);
    p.kg = tiles <= 64 ? 4 : 2;
    while (p.kg > 1 && p.dpad / 32 < p.kg * ks) p.kg /= 2;
  }
  p.kpart_bytes = p.kg > 1 ? size_t(tiles) * p.kg * kRouteBM * (p.npad + 8) * sizeof(float) : 0;
  return p;
}

// ------------------------------------------------------------------ W_r split
// The three planes are stored fragment-major: for expert tile t (32 experts),
// K block kb (32 inputs), plane p and MFMA substep s, the 64 lanes' 8-element
// B fragments are contiguous (1 KiB), so every fragment load of the GEMM is
// one fully coalesced 16-byte-per-lane access.  Lane l = r + 32h holds expert
// t*32 + r and inputs kb*32 + 16h + 8s + [0, 8).
__host__ __device__ inline size_t frag_off(int t, int kb, int p, int s, int nkb) {
  return ((((size_t(t) * nkb + kb) * 3 + p) * 2 + s) * 64) * 8;
}

// One workgroup per (expert tile, K block): transpose through LDS, split each
// fp32 weight into hi + mid + lo bf16 (exact), write the fragments.
__global__ __launch_bounds__(256) void k_router_split(const float* __restrict__ w,
                                                       uint16_t* __restrict__ planes, int d, int n,
                                                       int npad, int dpad) {
  __shared__ float tile[32][33];
  const int t = blockIdx.x, kb = blockIdx.y, nkb = dpad / 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int r = ty; r < 32; r += 8) {
    const int k = kb * 32 + r, j = t * 32 + tx;
    tile[r][tx] = (k < d && j < n) ? w[size_t(k) * n + j] : 0.f;
  }
  __syncthreads();
  // 1024 (s, lane, e) slots per plane, 4 consecutive per thread
  uint16_t out[3][4];
  const int o0 = threadIdx.x * 4;
  const int s = o0 >> 9, lane = (o0 >> 3) & 63, e0 = o0 & 7;
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float v = tile[16 * h + 8 * s + e0 + q][r];
    const uint16_t hi = f32_to_bf16(v);
    const float r1 = v - bf16_to_f32(hi);     // exact: |r1| <= half a bf16 ulp of v
    const uint16_t mid = f32_to_bf16(r1);
    const float r2 = r1 - bf16_to_f32(mid);   // exact, at most 8 significant bits
    out[0][q] = hi;
    out[1][q] = mid;
    out[2][q] = f32_to_bf16(r2);               // exact
  }
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    uint16_t* dst = planes + frag_off(t, kb, p, s, nkb) + lane * 8 + e0;
    const uint64_t v = uint64_t(out[p][0]) | (uint64_t(out[p][1]) << 16) | (uint64_t(out[p][2]) << 32) |
                       (uint64_t(out[p][3]) << 48);
    *reinterpret_cast<uint64_t*>(dst) = v;
  }
}

__device__ __forceinline__ bf16x8 load8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
  return z;
}

// Block product of 32 tokens x npad experts on bf16 MFMA, split over the 16
// waves of the workgroup: wave w owns expert tile (w % NT) and the K-block
// range ks = w / NT of KS = 16 / NT equal ranges.  Lane l = r + 32h holds
// token row r and, in substep s of K block kb, inputs kb*32 + 16h + 8s +
// [0, 8) — the same lane -> k mapping as the W_r fragments, so every k meets
// itself exactly once.  arow points at lane (r, h)'s row r, input 16h, in an
// LDS copy of the x tile or in global memory; B fragments are one coalesced
// 1 KiB load each.  The loop body is branch-free with ping-pong
// operand buffers: the next K block's fragments are in flight while the
// current block is multiplied (scheduling barriers keep the loads ahead of
// the MFMAs).  Each workgroup starts its K range at a different block (rot)
// to spread the shared W_r reads over the L2 channels.
template <int NT>
__device__ __forceinline__ f32x16 gemm_ksplit_bf16x3(const uint16_t* __restrict__ arow,
                                                     const uint16_t* __restrict__ planes, int dpad, int wave,
                                                     int lane, int rot) {
  constexpr int KS = 16 / NT;
  const int tile = wave % NT, ks = wave / NT;
  const int nkb = dpad / 32;
  const int kb0 = ks * nkb / KS, cnt = (ks + 1) * nkb / KS - kb0;
  const uint16_t* bt = planes + frag_off(tile, 0, 0, 0, nkb) + lane * 8;
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  if (cnt <= 0) return acc;
  rot %= cnt;
  auto load = [&](int i, bf16x8 (&aa)[2], bf16x8 (&bb)[3][2]) {
    int r = i + rot;
    r = r >= cnt ? r - cnt : r;
    const int kb = kb0 + r;
    aa[0] = load8(arow + kb * 32);
    aa[1] = load8(arow + kb * 32 + 8);
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      bb[p][0] = load8(bt + (size_t(kb) * 3 + p) * 1024);
      bb[p][1] = load8(bt + (size_t(kb) * 3 + p) * 1024 + 512);
    }
  };
  auto mma = [&](const bf16x8 (&aa)[2], const bf16x8 (&bb)[3][2]) {
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aa[0], bb[p][0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aa[1], bb[p][1], acc, 0, 0, 0);
    }
  };
  // ping-pong buffers; the scheduling barriers keep each block's loads ahead
  // of the previous block's MFMAs instead of letting them sink to their uses
  bf16x8 a0[2], b0[3][2], a1[2], b1[3][2];
  load(0, a0, b0);
  for (int i = 0; i < cnt; i += 2) {
    load(min(i + 1, cnt - 1), a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    mma(a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    if (i + 1 < cnt) {
      load(min(i + 2, cnt - 1), a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      mma(a1, b1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  return acc;
}

// Exact three-way split of 8 fp32 weights into bf16 fragments: hi = w with
// the low 16 bits cleared, mid = (w - hi) likewise, lo = w - hi - mid (at
// most 8 significant bits, so exact in bf16); hi + mid + lo == w.
__device__ __forceinline__ void split3(const float* v, bf16x8& hi, bf16x8& mid, bf16x8& lo) {
  u32x4 wh, wm, wl;
  constexpr uint32_t kHigh = 0x07060302u;   // v_perm selector: high halves of (src1, src0) -> (lo, hi)
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t u0 = __float_as_uint(v[2 * p]), u1 = __float_as_uint(v[2 * p + 1]);
    const float r0 = v[2 * p] - __uint_as_float(u0 & 0xFFFF0000u);
    const float r1 = v[2 * p + 1] - __uint_as_float(u1 & 0xFFFF0000u);
    const uint32_t s0 = __float_as_uint(r0), s1 = __float_as_uint(r1);
    const float q0 = r0 - __uint_as_float(s0 & 0xFFFF0000u);
    const float q1 = r1 - __uint_as_float(s1 & 0xFFFF0000u);
    wh[p] = __builtin_amdgcn_perm(u1, u0, kHigh);
    wm[p] = __builtin_amdgcn_perm(s1, s0, kHigh);
    wl[p] = __builtin_amdgcn_perm(__float_as_uint(q1), __float_as_uint(q0), kHigh);
  }
  hi = __builtin_bit_cast(bf16x8, wh);
  mid = __builtin_bit_cast(bf16x8, wm);
  lo = __builtin_bit_cast(bf16x8, wl);
}

// Exact three-way split of 8 fp32 weights (raw bits) into bf16 fragments, as above.
__device__ __forceinline__ void split8(const uint32_t* u, bf16x8 (&f)[3]) {
  u32x4 wh, wm, wl;
  constexpr uint32_t kHigh = 0x07060302u;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t u0 = u[2 * p], u1 = u[2 * p + 1];
    const float r0 = __uint_as_float(u0) - __uint_as_float(u0 & 0xFFFF0000u);
    const float r1 = __uint_as_float(u1) - __uint_as_float(u1 & 0xFFFF0000u);
    const uint32_t s0 = __float_as_uint(r0), s1 = __float_as_uint(r1);
    const float q0 = r0 - __uint_as_float(s0 & 0xFFFF0000u);
    const float q1 = r1 - __uint_as_float(s1 & 0xFFFF0000u);
    wh[p] = __builtin_amdgcn_perm(u1, u0, kHigh);
    wm[p] = __builtin_amdgcn_perm(s1, s0, kHigh);
    wl[p] = __builtin_amdgcn_perm(__float_as_uint(q1), __float_as_uint(q0), kHigh);
  }
  f[0] = __builtin_bit_cast(bf16x8, wh);
  f[1] = __builtin_bit_cast(bf16x8, wm);
  f[2] = __builtin_bit_cast(bf16x8, wl);
}

// The same block product taking W_r [d, n] fp32 straight from global memory:
// lane (r, h) loads the 16 weights of expert 32 tile + r it needs per K block
// (each load instruction reads two 128-byte rows of W_r) and splits them in
// registers, so no prepared planes are needed.  Used when d % 32 == 0 and
// n == 32 NT (compile-time row stride).
//
// Software pipeline in half blocks (8 weights per lane, three MFMAs): while
// the matrix core runs the three products of one half, the vector ALUs split
// the next half, so the split and the products overlap inside every wave.
// Raw weights are loaded two K blocks ahead through a buffer resource: a load
// for a block past the wave's range is given an offset past the end of W_r,
// which returns zero without reading memory, so the load sequence has no
// branches and every wait counts exactly the loads it needs.
template <int NT>
struct DirectGemm {
  static constexpr int kRow = 4 * 32 * NT;          // bytes per W_r row
  static constexpr uint32_t kOut = 0x7FFF0000u;      // beyond num_records
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t vbase;                                    // lane's byte offset inside a K block
  int kb0, cnt, rot;
  uint32_t ra[16], rb[16];
  bf16x8 g0[3], g1[3];

  // K blocks [kbA, kbB) of the workgroup, split over its KS wave groups
  __device__ __forceinline__ void init(const float* w, int d, int kbA, int kbB, int wave, int lane, int rot_) {
    constexpr int KS = 16 / NT;
    const int tile = wave % NT, ks = wave / NT;
    const int nkb = kbB - kbA;
    kb0 = kbA + ks * nkb / KS;
    cnt = kbA + (ks + 1) * nkb / KS - kb0;
    rot = cnt > 0 ? rot_ % cnt : 0;
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(w), 0, d * kRow, 0x00020000);
    vbase = uint32_t((tile * 32 + (lane & 31)) * 4 + 16 * (lane >> 5) * kRow);
    load(ra, 0);
    load(rb, 1);
  }
  __device__ __forceinline__ int kb(int i) const {   // i < cnt
    const int r = i + rot;
    return kb0 + (r >= cnt ? r - cnt : r);
  }
  __device__ __forceinline__ void load(uint32_t (&b)[16], int i) {
    const uint32_t o = i < cnt ? vbase + uint32_t(kb(i)) * uint32_t(32 * kRow) : kOut;
#pragma unroll
    for (int q = 0; q < 16; ++q) b[q] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, int(o + q * kRow), 0, 0);
  }
  // first half of block 0, split while the x tile is still being staged
  __device__ __forceinline__ void prime() {
    if (cnt > 0) split8(ra, g0);
  }
  // three products of one half (fragments g, A operand a) with the split of
  // the next half (raw u -> gn) interleaved: MFMA, then a share of the split
  __device__ __forceinline__ static void half(f32x16& acc, const bf16x8& a, const bf16x8 (&g)[3],
                                              const uint32_t* u, bf16x8 (&gn)[3]) {
    split8(u, gn);
#pragma unroll
    for (int p = 0; p < 3; ++p) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, g[p], acc, 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // the next half's A operand read first
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 15, 0);   // then vector ALU work
    }
  }
  __device__ __forceinline__ f32x16 run(const uint16_t* arow) {
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    if (cnt == 0) return acc;
    int i = 0;
    bf16x8 a0 = load8(arow + kb(0) * 32), a1;
    // blocks i (raw in ra) and i + 1 (rb) per pass; block i + 2 exists, so its
    // first half is split in the pass and its load is always in range
    for (; i + 2 < cnt; i += 2) {
      a1 = load8(arow + kb(i) * 32 + 8);
      half(acc, a0, g0, ra + 8, g1);
      load(ra, i + 2);
      __builtin_amdgcn_sched_barrier(0);
      a0 = load8(arow + kb(i + 1) * 32);
      half(acc, a1, g1, rb, g0);
      __builtin_amdgcn_sched_barrier(0);
      a1 = load8(arow + kb(i + 1) * 32 + 8);
      half(acc, a0, g0, rb + 8, g1);
      load(rb, i + 3);
      __builtin_amdgcn_sched_barrier(0);
      a0 = load8(arow + kb(i + 2) * 32);
      half(acc, a1, g1, ra, g0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // one or two blocks left: i (ra) and possibly i + 1 (rb)
    a1 = load8(arow + kb(i) * 32 + 8);
    half(acc, a0, g0, ra + 8, g1);
    __builtin_amdgcn_sched_barrier(0);
    if (i + 1 < cnt) {
      a0 = load8(arow + kb(i + 1) * 32);
      half(acc, a1, g1, rb, g0);
      __builtin_amdgcn_sched_barrier(0);
      a1 = load8(arow + kb(i + 1) * 32 + 8);
      half(acc, a0, g0, rb + 8, g1);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int p = 0; p < 3; ++p) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, g1[p], acc, 0, 0, 0);
    return acc;
  }
};

// 32x32 accumulator layout: lane l, element i -> row 8*(i/4) + 4*(l/32) + (i%4), col l%32.
__device__ __forceinline__ int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// ------------------------------------------------------------------ epilogue
struct EpiArgs {
  int n, k, score, gate;
  const float* bias;
  const float* bias_lds;   // the bias staged in LDS (fused kernel), or nullptr
};

// Logistic score; the reciprocal is the hardware one (within 1 ulp; 1 + e^-h >= 1).
__device__ __forceinline__ float sigm(float h) { return __builtin_amdgcn_rcpf(1.0f + expf(-h)); }

// Order-preserving integer image of a selection key: a > b as floats iff ord_key(a) >
// ord_key(b) as unsigned integers, with -0 taken as +0 (equal keys stay equal) and NaN as
// -inf.  Every key maps above 0, which is left to mark absent or already picked experts.
__device__ __forceinline__ uint32_t ord_key(float f) { return f32_key(f == f ? f + 0.0f : -INFINITY); }

// Score of expert j for a token with softmax statistics (mx, sum); the softmax
// exponential is the hardware exp2 of the scaled argument (about 1e-6 relative).
__device__ __forceinline__ float score_of(int score, float h, float mx, float sum) {
  return score == 0 ? __expf(h - mx) / sum : sigm(h);
}

// Per-token selection for the `rows` tokens of one block, wave w taking
// tokens w, w+16, ...; writes idx/gate, per-token softmax statistics to
// tok_mx/tok_sum (shared) and counts selections into hist (shared).
__device__ __forceinline__ void route_rows(const float* lg, int64_t ld, int rows, int64_t t0,
                                           const EpiArgs& e, int32_t* __restrict__ idx,
                                           float* __restrict__ gate_out, float* tok_mx,
                                           float* tok_sum, int* hist) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = e.n;
  for (int tl = wave; tl < rows; tl += kRouteThreads / 64) {
    const float* row = lg + int64_t(tl) * ld;
    float mx = -INFINITY, sum = 1.0f;
    if (e.score == 0) {
      for (int j = lane; j < n; j += 64) mx = fmaxf(mx, row[j]);
      mx = wave_max(mx);
      float s = 0.f;
      for (int j = lane; j < n; j += 64) s += __expf(row[j] - mx);
      sum = wave_sum(s);
    }
    if (lane == 0) {
      tok_mx[tl] = mx;
      tok_sum[tl] = sum;
    }
    // k rounds: each picks the best (key, j) strictly after the previous pick
    float last_key = INFINITY;
    int last_j = -1;
    int my_j = 0;
    float my_score = 0.f, score_total = 0.f;
    for (int r = 0; r < e.k; ++r) {
      float bk = -INFINITY;
      int bj = 0x7FFFFFFF;
      for (int j = lane; j < n; j += 64) {
        const float h = row[j];
        const float k0 = e.bias ? score_of(e.score, h, mx, sum) + e.bias[j] : h;
        const float key = k0 == k0 ? k0 : -INFINITY;   // NaN ranks as -inf (the order of the integer keys)
        if (better(last_key, last_j, key, j) && better(key, j, bk, bj)) {
          bk = key;
          bj = j;
        }
      }
      wave_argbest(bk, bj);
      last_key = bk;
      last_j = bj;
      const float sc = score_of(e.score, row[bj], mx, sum);
      score_total += sc;
      if (lane == r) {
        my_j = bj;
        my_score = sc;
      }
      if (lane == 0) atomicAdd(&hist[bj], 1);
    }
    if (lane < e.k) {
      const int64_t o = (t0 + tl) * e.k + lane;
      idx[o] = my_j;
      gate_out[o] = e.gate == 1 ? my_score / score_total : my_score;
    }
  }
}

// Fused-route epilogue for k <= 32: one half-wave per token, NV = npad/32
// logits per lane in registers (expert j = lane + 32u).  Computes the scores
// (softmax or sigmoid), the top-k by key (logit, or score + bias), the gates
// and the histogram, then overwrites the token's LDS row with its scores so
// that the per-expert score sums are plain column sums.  Top-1 softmax
// without bias (the Switch router) takes a shorter path: a max reduction
// gives the softmax maximum, a min reduction over the lanes holding it the
// pick (the lowest such expert), whose score is exp(0) / sum = 1 / sum; the
// exponentials and that reciprocal use the hardware exp2 (argument scaled by
// log2 e) and reciprocal, about 1e-6 relative, well inside the fp32 tolerance
// the scores are checked to.
template <int NV>
__device__ __forceinline__ void route_rows_half(float* lg, int ld, int rows, int64_t t0, const EpiArgs& e,
                                                int32_t* __restrict__ idx, float* __restrict__ gate_out,
                                                int* hist) {
  const int half = threadIdx.x >> 5, l = threadIdx.x & 31;
  const int nhalf = kRouteThreads / 32;
  const bool fast = e.k == 1 && e.score == 0 && !e.bias;
  for (int tl = half; tl < rows; tl += nhalf) {
    float* row = lg + tl * ld;
    float h[NV], sc[NV], bv[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int j = l + 32 * u;
      h[u] = j < e.n ? row[j] : -INFINITY;
    }
    if (fast) {
      // the maximum, then the lowest expert attaining it (ties to the lower index)
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < NV; ++u) mx = fmaxf(mx, h[u]);
      mx = half_max(mx);
      int cand = 0x7FFFFFFF;
#pragma unroll
      for (int u = NV - 1; u >= 0; --u)
        if (l + 32 * u < e.n && h[u] == mx) cand = l + 32 * u;
      // no expert holds the maximum only when every logit is NaN: NaN ranks as -inf, so all
      // tie and the lowest expert is picked (indices stay in [0, n) for any input)
      int bj = half_min_i(cand);
      bj = bj < e.n ? bj : 0;
      float sum = 0.f;
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        sc[u] = l + 32 * u < e.n ? __expf(h[u] - mx) : 0.f;   // hardware exp2 of the scaled argument
        sum += sc[u];
      }
      const float inv = __builtin_amdgcn_rcpf(half_sum(sum));   // sum >= 1 (the maximum's term is 1)
      if (l == 0) {
        atomicAdd(&hist[bj], 1);
        idx[t0 + tl] = bj;
        gate_out[t0 + tl] = e.gate == 1 ? 1.0f : inv;
      }
#pragma unroll
      for (int u = 0; u < NV; ++u) row[l + 32 * u] = sc[u] * inv;
      continue;
    }
#pragma unroll
    for (int u = 0; u < NV; ++u)
      bv[u] = (e.bias && l + 32 * u < e.n) ? (e.bias_lds ? e.bias_lds[l + 32 * u] : e.bias[l + 32 * u]) : 0.f;
    if (e.score == 0) {
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < NV; ++u) mx = fmaxf(mx, h[u]);
      mx = half_max(mx);
      float sum = 0.f;
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        sc[u] = l + 32 * u < e.n ? expf(h[u] - mx) : 0.f;
        sum += sc[u];
      }
      const float inv = 1.0f / half_sum(sum);
#pragma unroll
      for (int u = 0; u < NV; ++u) sc[u] *= inv;
    } else {
#pragma unroll
      for (int u = 0; u < NV; ++u) sc[u] = l + 32 * u < e.n ? sigm(h[u]) : 0.f;
    }
    // k rounds: each picks the largest key not picked yet, the lowest expert among equal keys: a
    // half-wave maximum of the integer keys, then a half-wave minimum of the experts holding it;
    // a pick's key becomes 0, below every expert's (k <= n, so a round always finds one)
    uint32_t key[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) key[u] = l + 32 * u < e.n ? ord_key(e.bias ? sc[u] + bv[u] : h[u]) : 0u;
    int my_j = 0;
    for (int r = 0; r < e.k; ++r) {
      uint32_t mk = key[0];
#pragma unroll
      for (int u = 1; u < NV; ++u) mk = max(mk, key[u]);
      mk = half_max_u(mk);
      int cand = 0x7FFFFFFF;
#pragma unroll
      for (int u = NV - 1; u >= 0; --u)
        if (key[u] == mk) cand = l + 32 * u;
      const int bj = half_min_i(cand);
#pragma unroll
      for (int u = 0; u < NV; ++u)
        if (l + 32 * u == bj) key[u] = 0u;
      if (l == r) my_j = bj;
    }
    if (l < e.k) atomicAdd(&hist[my_j], 1);   // the k picks are distinct experts
    // the picks' scores, after the rounds: lane r < k reads its pick's score from the lane holding it
    float my_score = 0.f;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const float v = __shfl(sc[u], my_j & 31, 32);
      if ((my_j >> 5) == u) my_score = v;
    }
    const float total = half_sum(l < e.k ? my_score : 0.f);
    if (l < e.k) {
      const int64_t o = (t0 + tl) * e.k + l;
      idx[o] = my_j;
      gate_out[o] = e.gate == 1 ? my_score / total : my_score;
    }
#pragma unroll
    for (int u = 0; u < NV; ++u)
      if (l + 32 * u < ld) row[l + 32 * u] = sc[u];
  }
}

// Chunk row of this workgroup: per expert, its count and (if wanted) Σ over
// its tokens of score_j(t) in token order, packed into one 64-bit word; the
// last workgroup publishes the totals, the optional load statistics and the
// capacity prefix sums.  SCORES: lg rows already hold the scores (fused
// epilogue); otherwise they hold logits and the scores are recomputed.
// Expert j's entry of this chunk's row: count and score sum.
__device__ __forceinline__ void chunk_row_out(const RouteArgs& a, const EpiArgs& e, int chunk, int j, int count,
                                              float acc) {
  const int64_t row0 = int64_t(chunk) * e.n;
  if (a.finish && !a.fin_super) {
    store_agent(a.chunks + row0 + j, pack_chunk(count, acc));
  } else {
    // this chunk's share of its super chunk's totals: integer adds, so their order does not
    // matter; and (layer) count rows [chunks][n] int32 for the next kernel
    const int64_t so = int64_t(chunk / a.sup) * e.n + j;
    if (!a.finish) reinterpret_cast<int32_t*>(a.chunks)[row0 + j] = count;
    if (count) atomicAdd(a.sup_counts + so, count);
    if (a.want_psum) atomicAdd(a.sup_psum + so, __float2ull_rn(acc * kPsumScale));
  }
}
template <bool SUPER>
__device__ __forceinline__ void route_finish(const RouteArgs& a, const EpiArgs& e, int* scratch, int scratch_ints,
                                             int nchunks);

template <bool SCORES>
__device__ __forceinline__ void route_tail(const float* lg, int64_t ld, int rows, const EpiArgs& e,
                                           const float* tok_mx, const float* tok_sum, const int* hist,
                                           const RouteArgs& a, int* scratch, int scratch_ints, int chunk,
                                           int nchunks) {
  for (int j = threadIdx.x; j < e.n; j += kRouteThreads) {
    float acc = 0.f;
    if (a.want_psum) {
      // token order; 32 reads in flight
      for (int tl0 = 0; tl0 < rows; tl0 += 32) {
        float v[32];
#pragma unroll
        for (int u = 0; u < 32; ++u) v[u] = tl0 + u < rows ? lg[int64_t(tl0 + u) * ld + j] : 0.f;
#pragma unroll
        for (int u = 0; u < 32; ++u)
          if (tl0 + u < rows) acc += SCORES ? v[u] : score_of(e.score, v[u], tok_mx[tl0 + u], tok_sum[tl0 + u]);
      }
    }
    chunk_row_out(a, e, chunk, j, hist[j], acc);
  }
  route_finish<true>(a, e, scratch, scratch_ints, nchunks);
}

// The workgroup that finishes last (stand-alone route) sums the per-super-chunk
// rows (SUPER: the fused kernel, n <= 256, whose launch always sets fin_super)
// or the chunk rows (the n > 256 path).  Only one of the two finishes is
// compiled into a kernel: the chunk-row one alone holds about as many
// registers as the fused kernel's product, and both together made it spill.
template <bool SUPER>
__device__ __forceinline__ void route_finish(const RouteArgs& a, const EpiArgs& e, int* scratch, int scratch_ints,
                                             int nchunks) {
  if (!a.finish) return;
  __shared__ int s_flag;
  if (!last_workgroup(a.done, unsigned(nchunks), &s_flag)) return;
  FinalizeArgs f{};
  f.chunks = a.chunks;
  f.nch = nchunks;
  f.sup = a.sup;
  f.n = e.n;
  f.m = a.m;
  f.counts = a.counts;
  f.prob_sum = a.prob_sum;
  f.f = a.f;
  f.P = a.P;
  f.aux = a.aux;
  f.alpha = a.alpha;
  f.capacity = a.capacity;
  f.expert_offsets = a.expert_offsets;
  f.super_prefix = a.super_prefix;
  f.expert_rows = a.expert_rows;
  f.padded = a.padded;
  f.k = e.k;
  f.gcounts = a.gcounts;
  f.gtokens = a.gtokens;
  f.lf_bias = a.lf_bias;
  f.gamma = a.gamma;
  if constexpr (SUPER)
    finalize_super(f, a.sup_counts, a.sup_psum, a.want_psum, scratch, kRouteThreads);
  else
    finalize_chunks(f, scratch, scratch_ints, kRouteThreads);
}

// The epilogue above with NV = npad / 32 chosen at run time (vector-ALU product path).
__device__ __forceinline__ void route_rows_half_nv(int nv, float* lg, int ld, int rows, int64_t t0, const EpiArgs& e,
                                                   int32_t* idx, float* gate_out, int* hist) {
  if (nv == 1) route_rows_half<1>(lg, ld, rows, t0, e, idx, gate_out, hist);
  else if (nv == 2) route_rows_half<2>(lg, ld, rows, t0, e, idx, gate_out, hist);
  else if (nv == 4) route_rows_half<4>(lg, ld, rows, t0, e, idx, gate_out, hist);
  else route_rows_half<8>(lg, ld, rows, t0, e, idx, gate_out, hist);
}

__device__ __forceinline__ float load_x(const void* x, bool bf16, int64_t i) {
  return bf16 ? bf16_to_f32(static_cast<const uint16_t*>(x)[i]) : static_cast<const float*>(x)[i];
}

// ------------------------------------------------------------------ fused route (n <= 256)
// LDS region (lds_region_ints): first the bf16 x tile [32][dpad + 8] (XLDS),
// then, after the product, the KS-1 partial tiles [32][npad]; the first of
// them becomes the logits tile and, in the last workgroup, the finishing
// scratch.  The histogram follows the region.
template <int NT, bool MFMA, bool XLDS, bool DIRECT>
__global__ __launch_bounds__(kRouteThreads) void k_route_fused(RouteArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem[];   // 16-byte LDS vectors need a 16-byte base
  __shared__ float tok_mx[kRouteBM], tok_sum[kRouteBM];   // softmax statistics (k > 32 epilogue)
  const int ldl = a.npad + 8;   // logit and partial tile row stride
  // the staged x tile holds one workgroup's K range: xcols columns, row stride xcols + 8
  // (x_tile_cols on the host); partials apart: the partial (and logit) tiles follow it
  const int xcols = ((a.dpad / 32 + a.kg - 1) / a.kg) * 32;
  const int lg_off = XLDS && a.parts_apart ? kRouteBM * (xcols + 8) / 2 : 0;
  float* lg = smem + lg_off;
  int* hist = reinterpret_cast<int*>(smem) + a.lds_region_ints;
  float* bias_l = reinterpret_cast<float*>(hist + a.npad);   // the Loss-Free bias, staged once
  // the wave index is uniform: keep it (and every K-block index derived from it) in scalar registers
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  // a token tile may be split over a.kg workgroups by K range (direct path only)
  const int tile = int(blockIdx.x) / a.kg, g = int(blockIdx.x) % a.kg, ntiles = int(gridDim.x) / a.kg;
  const int nkb = a.dpad / 32, kbA = g * nkb / a.kg, kbB = (g + 1) * nkb / a.kg;
  const int64_t t0 = int64_t(tile) * kRouteBM;
  const int rows = int(min<int64_t>(kRouteBM, a.m - t0));
  for (int j = tid; j < a.npad; j += kRouteThreads) {
    hist[j] = 0;
    if (a.bias) bias_l[j] = j < a.n ? a.bias[j] : 0.f;
  }

  if constexpr (MFMA) {
    constexpr int KS = 16 / NT;
    const uint16_t* x = static_cast<const uint16_t*>(a.x);
    const uint16_t* arow;
    DirectGemm<NT> dg;
    if constexpr (XLDS) {
      // stage the 32 x rows in LDS with coalesced 16-byte loads (zero padding past the end)
      uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
      // only this workgroup's K range [32 kbA, 32 kbB) of the tile is staged
      // columns [kx, kx + 32 (kbB - kbA)) of x land at tile columns from 0 (row stride ldx)
      const int ldx = xcols + 8, cpr = (kbB - kbA) * 4, kx = kbA * 32, items = kRouteBM * cpr;
      // The first pass (all of it for d <= 1024): four unconditional 16-byte loads per
      // thread through a buffer resource over the tile's rows (an item past the tile reads
      // zeros without touching memory), then the W_r loads of the product's first blocks,
      // so the LDS stores wait for the x loads alone and the weights stay in flight.
      const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(x + t0 * a.d), 0, rows * a.d * int(sizeof(uint16_t)), 0x00020000);
      {
        u32x4 v[4];
        int dst[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = tid + u * kRouteThreads;
          const int r = c / cpr, k = kx + (c - r * cpr) * 8;
          const bool in = c < items && r < rows && k < a.d;
          v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               xr, in ? (r * a.d + k) * int(sizeof(uint16_t)) : int(0x7FFF0000), 0, 0));
          dst[u] = c < items ? r * ldx + (k - kx) : -1;
        }
        if constexpr (DIRECT) dg.init(a.w_r, a.d, kbA, kbB, wave, lane, tile);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (dst[u] >= 0) *reinterpret_cast<u32x4*>(xs + dst[u]) = v[u];
        if constexpr (DIRECT) dg.prime();   // split the first weights
      }
      // further passes (d > 1024 without a K split)
      for (int c0 = tid + 4 * kRouteThreads; c0 < items; c0 += 4 * kRouteThreads) {
        u32x4 v[4];
        int dst[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = c0 + u * kRouteThreads;
          const int r = c / cpr, k = kx + (c - r * cpr) * 8;
          v[u] = u32x4{0u, 0u, 0u, 0u};
          dst[u] = c < items ? r * ldx + (k - kx) : -1;
          if (c < items && r < rows && k < a.d) v[u] = *reinterpret_cast<const u32x4*>(x + (t0 + r) * a.d + k);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (dst[u] >= 0) *reinterpret_cast<u32x4*>(xs + dst[u]) = v[u];
      }
      lds_barrier();   // the tile is in LDS; the weight loads stay in flight
      // the product indexes x by absolute K block: shift the row start back by kx
      arow = xs + (lane & 31) * ldx + 16 * (lane >> 5) - kx;
    } else {
      if constexpr (DIRECT) dg.init(a.w_r, a.d, kbA, kbB, wave, lane, tile);
      arow = x + (t0 + min(lane & 31, rows - 1)) * a.d + 16 * (lane >> 5);  // requires d == dpad
      if constexpr (DIRECT) dg.prime();
    }
    const f32x16 acc = DIRECT ? dg.run(arow) : gemm_ksplit_bf16x3<NT>(arow, a.planes, a.dpad, wave, lane, int(blockIdx.x));
    const int col = (wave % NT) * 32 + (lane & 31), ks = wave / NT;
    if (XLDS && !a.parts_apart) __syncthreads();   // the x tile is dead before partials overwrite it
    {
      float* buf = lg + ks * kRouteBM * ldl;
#pragma unroll
      for (int i = 0; i < 16; ++i) buf[acc_row(i, lane) * ldl + col] = acc[i];
    }
    __syncthreads();
    // the KS partial tiles added in K-range order, every thread owning npad / 32 elements
    // (the sum lands in the first tile, element by element)
    constexpr int NPAD = 32 * NT;   // = npad on the matrix-core path
    for (int o = tid; o < kRouteBM * NPAD; o += kRouteThreads) {
      const int li = (o / NPAD) * ldl + o % NPAD;
      float p[KS];
#pragma unroll
      for (int q = 0; q < KS; ++q) p[q] = lg[q * kRouteBM * ldl + li];
      float v = p[0];
#pragma unroll
      for (int q = 1; q < KS; ++q) v += p[q];
      lg[li] = v;
    }
    __syncthreads();
    if (a.kg > 1) {
      // publish this K group's tile; the group that arrives last adds all of
      // them in K-group order and goes on with the epilogue
      const int tsz = kRouteBM * ldl;
      float* mine = a.kpart + (int64_t(tile) * a.kg + g) * tsz;
      for (int o = tid; o < tsz; o += kRouteThreads) store_agent(mine + o, lg[o]);
      __shared__ int s_last;
      if (!last_workgroup(a.tile_tickets + tile, unsigned(a.kg), &s_last)) return;
      // every other group's elements of this thread loaded first (no serial round trips),
      // then added in K-group order
      constexpr int kBatch = 8;
      for (int o0 = tid; o0 < tsz; o0 += kBatch * kRouteThreads) {
        float w[kBatch][4];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int o = o0 + u * kRouteThreads;
            w[u][q] = q < a.kg && q != g && o < tsz ? load_agent(a.kpart + (int64_t(tile) * a.kg + q) * tsz + o) : 0.f;
          }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int o = o0 + u * kRouteThreads;
          if (o < tsz) {
            float v = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (q < a.kg) v += q == g ? lg[o] : w[u][q];
            lg[o] = v;
          }
        }
      }
      __syncthreads();
    }
  } else {
    // fp32 product on the vector ALUs: thread (token, expert group), fma over k in order.
    const int tl = tid >> 5, jg = tid & 31;
    if (tl < rows) {
      const int64_t xo = (t0 + tl) * a.d;
      for (int j = jg; j < a.npad; j += 32) {
        float h = 0.f;
        if (j < a.n)
          for (int kk = 0; kk < a.d; ++kk) h = fmaf(load_x(a.x, a.x_bf16, xo + kk), a.w_r[int64_t(kk) * a.n + j], h);
        lg[tl * ldl + j] = h;
      }
    }
    __syncthreads();
  }
  EpiArgs e{a.n, a.k, a.score, a.gate, a.bias, a.bias ? bias_l : nullptr};
  if (a.k <= 32) {
    if constexpr (MFMA) route_rows_half<NT>(lg, ldl, rows, t0, e, a.idx, a.gate_out, hist);
    else route_rows_half_nv(a.npad / 32, lg, ldl, rows, t0, e, a.idx, a.gate_out, hist);
    lds_barrier();   // scores and histogram in LDS (the idx / gate stores need not land first)
    route_tail<true>(lg, ldl, rows, e, tok_mx, tok_sum, hist, a, reinterpret_cast<int*>(lg), a.lds_region_ints - lg_off,
                     tile, ntiles);
  } else {
    route_rows(lg, ldl, rows, t0, e, a.idx, a.gate_out, tok_mx, tok_sum, hist);
    lds_barrier();
    route_tail<false>(lg, ldl, rows, e, tok_mx, tok_sum, hist, a, reinterpret_cast<int*>(lg), a.lds_region_ints - lg_off,
                      tile, ntiles);
  }
}

// ------------------------------------------------------------------ big-n route: logits GEMM
// Workgroup: 128 tokens x 128 experts; wave (wm, wn) owns 64 x 64 = 2 x 2 MFMA tiles.
__global__ __launch_bounds__(256) void k_route_logits_mfma(RouteArgs a) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5, r32 = lane & 31;
  // expert tiles fastest: the tiles of one token block run together (its x rows read once)
  const int64_t tb = int64_t(blockIdx.y) * 128 + 64 * wm;
  const int jb = blockIdx.x * 128 + 64 * wn;
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* xr[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) xr[mt] = x + min<int64_t>(tb + 32 * mt + r32, a.m - 1) * a.d;
  const int nkb = a.dpad / 32;
  const uint16_t* br[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) br[nt] = a.planes + frag_off((jb + 32 * nt) / 32, 0, 0, 0, nkb) + lane * 8;
  f32x16 acc[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.f;
  for (int kb = 0; kb < nkb; ++kb) {
    const int k0 = kb * 32 + 16 * h;
    bf16x8 av[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      av[mt][0] = (k0 + 8 <= a.d) ? load8(xr[mt] + k0) : zero8();
      av[mt][1] = (k0 + 16 <= a.d) ? load8(xr[mt] + k0 + 8) : zero8();
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        const uint16_t* f = br[nt] + (size_t(kb) * 3 + p) * 1024;
        const bf16x8 b0 = load8(f), b1 = load8(f + 512);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[mt][0], b0, acc[mt][nt], 0, 0, 0);
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[mt][1], b1, acc[mt][nt], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int col = jb + 32 * nt + r32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t t = tb + 32 * mt + acc_row(i, lane);
        if (t < a.m) a.logits[t * a.npad + col] = acc[mt][nt][i];
      }
    }
}

// fp32 vector-ALU logits for the big-n path (fp32 x, or bf16 x with d % 8 != 0).
// Workgroup: 32 tokens x 64 experts.
__global__ __launch_bounds__(256) void k_route_logits_valu(RouteArgs a) {
  const int tid = threadIdx.x, tl = tid >> 3, jg = tid & 7;
  const int64_t t = int64_t(blockIdx.x) * 32 + tl;
  const int jb = blockIdx.y * 64;
  if (t >= a.m) return;
  for (int u = 0; u < 8; ++u) {
    const int j = jb + jg + 8 * u;
    float h = 0.f;
    if (j < a.n)
      for (int kk = 0; kk < a.d; ++kk) h = fmaf(load_x(a.x, a.x_bf16, t * a.d + kk), a.w_r[int64_t(kk) * a.n + j], h);
    a.logits[t * a.npad + j] = h;
  }
}

// Top-1 softmax without bias (the Switch router) for n > 256: one wave per
// token, lane l taking experts l + 64 u; a max reduction, a min
// reduction over the lanes holding the maximum (the lowest such expert), and
// the sum of the exponentials; the pick's score is exp(0) / sum.  Writes what
// route_rows writes.
__device__ __forceinline__ void route_rows_top1(float* lg, int ld, int rows, int64_t t0, const EpiArgs& e,
                                                int32_t* __restrict__ idx, float* __restrict__ gate_out,
                                                float* tok_mx, float* tok_sum, int* hist) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nv = ld / 64;   // ld = npad, a multiple of 128: every lane reads nv in-row values
  for (int tl = wave; tl < rows; tl += kRouteThreads / 64) {
    float* row = lg + tl * ld;
    // three passes over the LDS row (padded experts hold -inf in the tile, so
    // nothing is masked; few registers: the prefetch of the next sub-tile stays live):
    // maximum, lowest expert holding it, then the exponentials, which replace
    // the logits in the row for the score column sums
    float mx = -INFINITY;
#pragma unroll 8
    for (int u = 0; u < nv; ++u) mx = fmaxf(mx, row[lane + 64 * u]);
    mx = wave_max_dpp(mx);
    int cand = 0x7FFFFFFF;
#pragma unroll 8
    for (int u = 0; u < nv; ++u) cand = min(cand, row[lane + 64 * u] == mx ? lane + 64 * u : 0x7FFFFFFF);
    // a padded expert or none holds the maximum only when every logit is NaN: NaN ranks as
    // -inf, so all tie and the lowest expert is picked
    int bj = wave_min_i_dpp(cand);
    bj = bj < e.n ? bj : 0;
    float s = 0.f;
#pragma unroll 8
    for (int u = 0; u < nv; ++u) {
      const float ex = __expf(row[lane + 64 * u] - mx);
      row[lane + 64 * u] = ex;
      s += ex;
    }
    const float sum = wave_sum_dpp(s);
    if (lane == 0) {
      tok_mx[tl] = mx;
      tok_sum[tl] = sum;
      atomicAdd(&hist[bj], 1);
      idx[t0 + tl] = bj;
      gate_out[t0 + tl] = e.gate == 1 ? 1.0f : __builtin_amdgcn_rcpf(sum);   // sum >= 1
    }
  }
}

// big-n route epilogue: kRowsBM tokens per workgroup (one chunk) from the
// logits in global memory, read once: sub-tiles of `rows_sub` tokens are staged
// in LDS (the next one loaded into registers while the current one is routed),
// each routed one wave per token, then its scores added into per-thread
// column sums in token order.  The barriers order LDS only, so the prefetch
// stays in flight while a sub-tile is routed.  NV = logits per lane of the top-1 path (npad <= 64 NV).
constexpr int kRowsLdsFloats = 32768;   // LDS floats for a staged sub-tile (128 KiB)
constexpr int kRowsMaxSub = 16;
constexpr int kRowsLoadItems = 8;       // 16-byte loads per thread and sub-tile (at most)
template <int NV>
__global__ __launch_bounds__(kRouteThreads) void k_route_rows(RouteArgs a) {
  constexpr int NQ = NV * 64 > kRouteThreads ? NV * 64 / kRouteThreads : 1;   // experts per thread
  extern __shared__ __attribute__((aligned(16))) int lds_i[];   // 16-byte LDS vectors need a 16-byte base
  __shared__ float tok_mx[kRowsMaxSub], tok_sum[kRowsMaxSub], tok_inv[kRowsMaxSub];
  int* hist = lds_i;                                             // [npad]
  float* tile = reinterpret_cast<float*>(lds_i + a.npad);        // [rows_sub][npad]
  int* scratch = lds_i + a.npad;                                 // finishing scratch, after the last sub-tile
  const int tid = threadIdx.x, npad = a.npad, sub = a.rows_sub;
  const int64_t t0 = int64_t(blockIdx.x) * kRowsBM;
  const int rows = int(min<int64_t>(kRowsBM, a.m - t0));
  const int nsub = (rows + sub - 1) / sub;
  const int vpr = npad / 4, items = sub * vpr;                   // 16-byte items per sub-tile
  const f32x4* lg4 = reinterpret_cast<const f32x4*>(a.logits + t0 * npad);
  for (int j = tid; j < npad; j += kRouteThreads) hist[j] = 0;
  EpiArgs e{a.n, a.k, a.score, a.gate, a.bias, nullptr};
  f32x4 v[kRowsLoadItems];
  auto load = [&](int s) {
#pragma unroll
    for (int u = 0; u < kRowsLoadItems; ++u) {
      const int i = tid + u * kRouteThreads;
      v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (i < items && s * sub + i / vpr < rows) v[u] = lg4[int64_t(s) * items + i];
    }
  };
  float acc[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) acc[q] = 0.f;
  load(0);
  for (int s = 0; s < nsub; ++s) {
    lds_barrier();   // the previous sub-tile is read (and hist zeroed)
#pragma unroll
    for (int u = 0; u < kRowsLoadItems; ++u) {
      const int i = tid + u * kRouteThreads;
      if (i < items) {
        if (a.n < npad) {   // padded experts become -inf in the LDS tile
          const int c = (i % vpr) * 4;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (c + q >= a.n) v[u][q] = -INFINITY;
        }
        reinterpret_cast<f32x4*>(tile)[i] = v[u];
      }
    }
    lds_barrier();
    if (s + 1 < nsub) load(s + 1);
    const int r = min(sub, rows - s * sub);
    const bool top1 = e.k == 1 && e.score == 0 && !e.bias;
    if (top1)
      route_rows_top1(tile, npad, r, t0 + int64_t(s) * sub, e, a.idx, a.gate_out, tok_mx, tok_sum, hist);
    else
      route_rows(tile, npad, r, t0 + int64_t(s) * sub, e, a.idx, a.gate_out, tok_mx, tok_sum, hist);
    lds_barrier();
    if (a.want_psum) {
      if (tid < r) tok_inv[tid] = 1.0f / tok_sum[tid];
      lds_barrier();
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int j = tid + q * kRouteThreads;
        if (j < a.n) {
          if (top1)   // the row holds exp(h - max) already
            for (int tl = 0; tl < r; ++tl) acc[q] += tile[tl * npad + j] * tok_inv[tl];
          else if (e.score == 0)
            for (int tl = 0; tl < r; ++tl) acc[q] += __expf(tile[tl * npad + j] - tok_mx[tl]) * tok_inv[tl];
          else
            for (int tl = 0; tl < r; ++tl) acc[q] += sigm(tile[tl * npad + j]);
        }
      }
    }
  }
  lds_barrier();
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int j = tid + q * kRouteThreads;
    if (j < a.n) chunk_row_out(a, e, int(blockIdx.x), j, hist[j], acc[q]);
  }
  route_finish<false>(a, e, scratch, a.lds_region_ints, int(gridDim.x));
}

// ------------------------------------------------------------------ launchers
hipError_t launch_router_prepare(const RoutePlan& plan, int d, int n, const float* w_r, uint16_t* planes,
                                 hipStream_t s) {
  if (!plan.mfma) return hipSuccess;   // the vector-ALU product reads W_r directly
  const dim3 g(plan.npad / 32, plan.dpad / 32);   // (expert tile, K block)
  hipLaunchKernelGGL(k_router_split, g, dim3(256), 0, s, w_r, planes, d, n, plan.npad, plan.dpad);
  return hipGetLastError();
}

int route_chunk_tokens(const RoutePlan& plan) { return plan.fused ? kRouteBM : kRowsBM; }


// The fused kernel splits W_r in registers whenever route_direct allows it
// (prepared planes are then not needed); otherwise it reads the planes.
template <int NT>
static void launch_fused(const RoutePlan& plan, const RouteArgs& a, dim3 g, size_t lds, hipStream_t s) {
  const bool x_lds = stage_x(plan, a.n);
  if (!route_direct(plan, a.d, a.n)) {
    if (x_lds)
      hipLaunchKernelGGL((k_route_fused<NT, true, true, false>), g, dim3(kRouteThreads), lds, s, a);
    else
      hipLaunchKernelGGL((k_route_fused<NT, true, false, false>), g, dim3(kRouteThreads), lds, s, a);
  } else {
    if (x_lds)
      hipLaunchKernelGGL((k_route_fused<NT, true, true, true>), g, dim3(kRouteThreads), lds, s, a);
    else
      hipLaunchKernelGGL((k_route_fused<NT, true, false, true>), g, dim3(kRouteThreads), lds, s, a);
  }
}

hipError_t launch_route(const RoutePlan& plan, const RouteArgs& a_in, hipStream_t s) {
  RouteArgs a = a_in;
  a.lds_region_ints = route_region_ints(plan, a.n);
  a.parts_apart = partials_apart(plan, a.n);
  if (plan.mfma && !a.planes_ready && !route_direct(plan, a.d, a.n)) {
    const hipError_t err = launch_router_prepare(plan, a.d, a.n, a.w_r, const_cast<uint16_t*>(a.planes), s);
    if (err != hipSuccess) return err;
  }
  a.kg = plan.kg;
  if (plan.fused) {
    if (a.finish && !a.fin_super) return hipErrorInvalidValue;   // the fused kernel finishes from super-chunk sums only
    const dim3 g(unsigned(ceil_div64(a.m, kRouteBM) * plan.kg));
    const size_t lds = (size_t(a.lds_region_ints) + 2 * size_t(plan.npad)) * sizeof(float);   // + histogram, bias
    const int nt = plan.npad / 32;
    if (!plan.mfma)
      hipLaunchKernelGGL((k_route_fused<1, false, false, false>), g, dim3(kRouteThreads), lds, s, a);
    else if (nt == 1)
      launch_fused<1>(plan, a, g, lds, s);
    else if (nt == 2)
      launch_fused<2>(plan, a, g, lds, s);
    else if (nt <= 4)
      launch_fused<4>(plan, a, g, lds, s);
    else
      launch_fused<8>(plan, a, g, lds, s);
  } else {
    if (plan.mfma)
      hipLaunchKernelGGL(k_route_logits_mfma, dim3(plan.npad / 128, unsigned(ceil_div64(a.m, 128))), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(k_route_logits_valu, dim3(unsigned(ceil_div64(a.m, 32)), plan.npad / 64), dim3(256), 0, s, a);
    // sub-tiles of the logits staged in LDS; the finishing scratch reuses that region
    a.rows_sub = std::min(kRowsMaxSub, kRowsLdsFloats / plan.npad);
    a.lds_region_ints = std::max(a.lds_region_ints, a.rows_sub * plan.npad);
    const size_t lds = (size_t(plan.npad) + a.lds_region_ints) * sizeof(int);
    const dim3 g(unsigned(ceil_div64(a.m, kRowsBM)));
    if (plan.npad <= 512)
      hipLaunchKernelGGL(k_route_rows<8>, g, dim3(kRouteThreads), lds, s, a);
    else if (plan.npad <= 1024)
      hipLaunchKernelGGL(k_route_rows<16>, g, dim3(kRouteThreads), lds, s, a);
    else if (plan.npad <= 2048)
      hipLaunchKernelGGL(k_route_rows<32>, g, dim3(kRouteThreads), lds, s, a);
    else
      hipLaunchKernelGGL(k_route_rows<64>, g, dim3(kRouteThreads), lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace moe
