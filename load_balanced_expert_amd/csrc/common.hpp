// Device helpers shared by the gfx950 kernels of libmoe.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxExperts = 4096;
constexpr int kMaxK = 64;   // picks per token (one wave lane per pick in the epilogues)

// Control region at the start of every workspace: completion tickets of the
// last-workgroup pattern (zero before first use; each kernel that takes a
// ticket leaves it zero again).
constexpr int kMaxSuperChunks = 16;
constexpr int kMaxD = 65536;   // keeps per-chunk copy item counts within 32 bits
// Control region: tickets in the first 4096 bytes, then the per-super-chunk
// expert counts [16][256] int32 and fixed-point score sums [16][256] uint64
// that the Switch layer's route kernel accumulates and its combine clears.
constexpr size_t kSupCountsOff = 4096;
constexpr size_t kSupPsumOff = kSupCountsOff + size_t(kMaxSuperChunks) * 256 * sizeof(int32_t);
constexpr size_t kControlBytes = kSupPsumOff + size_t(kMaxSuperChunks) * 256 * sizeof(uint64_t);
constexpr int kSelfPrefixMaxN = 256;
constexpr float kPsumScale = 4294967296.0f;   // 2^32: fixed-point score sums
enum CtlTicket { kTicketRoute = 0, kTicketDispatch = 1, kTicketBalance = 2 };
constexpr int kTileTicketsOff = 1024;   // bytes: per-token-tile tickets of the K-split route
constexpr int kMaxKgTiles = 128;        // token tiles up to which the route splits K over workgroups
inline uint32_t* ctl_ticket(void* ws, int which) { return static_cast<uint32_t*>(ws) + which; }

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads it does
// not wait for the wave's global loads and stores, so loads issued before it
// (a prefetch) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Order-preserving map of fp32 onto uint32 (larger float <-> larger key).
__device__ __forceinline__ uint32_t f32_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return u ^ (uint32_t(int32_t(u) >> 31) | 0x80000000u);   // negative: all bits flipped; else the sign bit set
}
__device__ __forceinline__ float key_f32(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// (key, index) ordering used by every top-k: larger key first, lower index on ties.
__device__ __forceinline__ bool better(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// Wave-wide arg-best of (key, index) by the order above; every lane gets the result.
__device__ __forceinline__ void wave_argbest(float& key, int& ix) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float ok = __shfl_xor(key, off, kWave);
    int oi = __shfl_xor(ix, off, kWave);
    if (better(ok, oi, key, ix)) { key = ok; ix = oi; }
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// Butterfly sum: every lane ends with the same value, and the association order
// depends only on lane positions, so the result is reproducible.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (kWave - 1);
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Lanes of the wave whose `key` equals this lane's (a "match any" built from
// one ballot per key bit), restricted to `active`.
__device__ __forceinline__ uint64_t match_any(uint32_t key, int nbits, uint64_t active) {
  uint64_t peers = active;
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1u;
    const uint64_t bal = __ballot(bit);
    peers &= bit ? bal : ~bal;
  }
  return peers;
}

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ constexpr int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ constexpr int round_up(int a, int b) { return ceil_div(a, b) * b; }

inline int bits_for(int n) {  // bits needed for values 0..n-1
  int b = 0;
  while ((1 << b) < n) ++b;
  return b;
}

}  // namespace moe
