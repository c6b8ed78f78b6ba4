// Wave-wide all-reductions on gfx950 through DPP row permutes, the 16-lane
// row swap and lane reads (no LDS crossbar traffic).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Half-wave (32 lanes) all-reductions without the LDS crossbar: partners at
// lane xor 1 and xor 2 (quad permutes), the mirrored quad and the mirrored
// half-row (row_half_mirror, row_mirror DPP), then the other 16-lane row of
// the half (gfx950 v_permlane16_swap).  Each step combines a lane with a
// partner that already holds the same partial, so every lane of the half ends
// with the same bits.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppMirror = 0x140, kDppHalfMirror = 0x141;
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
// (value of the even row, value of the odd row) of this lane's 32-lane half
__device__ __forceinline__ void row_pair(uint32_t v, uint32_t& even, uint32_t& odd) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  even = r[0];
  odd = r[1];
}
__device__ __forceinline__ float half_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  uint32_t a, b;
  row_pair(__float_as_uint(v), a, b);
  return fmaxf(__uint_as_float(a), __uint_as_float(b));
}
__device__ __forceinline__ float half_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  uint32_t a, b;
  row_pair(__float_as_uint(v), a, b);
  return __uint_as_float(a) + __uint_as_float(b);
}
__device__ __forceinline__ uint32_t half_max_u(uint32_t v) {
  v = max(v, uint32_t(dpp_i<kDppXor1>(int(v))));
  v = max(v, uint32_t(dpp_i<kDppXor2>(int(v))));
  v = max(v, uint32_t(dpp_i<kDppHalfMirror>(int(v))));
  v = max(v, uint32_t(dpp_i<kDppMirror>(int(v))));
  uint32_t a, b;
  row_pair(v, a, b);
  return max(a, b);
}
__device__ __forceinline__ int half_min_i(int v) {
  v = min(v, dpp_i<kDppXor1>(v));
  v = min(v, dpp_i<kDppXor2>(v));
  v = min(v, dpp_i<kDppHalfMirror>(v));
  v = min(v, dpp_i<kDppMirror>(v));
  uint32_t a, b;
  row_pair(uint32_t(v), a, b);
  return min(int(a), int(b));
}
// Whole-wave forms: the two halves meet through lane reads (scalar results).
__device__ __forceinline__ float lane_value(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = half_max(v);
  return fmaxf(lane_value(v, 0), lane_value(v, 32));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = half_sum(v);
  return lane_value(v, 0) + lane_value(v, 32);
}
__device__ __forceinline__ int wave_min_i_dpp(int v) {
  v = half_min_i(v);
  return min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 32));
}
}  // namespace moe
