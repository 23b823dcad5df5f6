// bw_lanes.h - cross-lane sums and maxima of a wave without the LDS crossbar (gfx950).
#pragma once

#include "bw_common.h"

namespace bw {

// ---- cross-lane steps without the LDS crossbar -------------------------------------------------
// DPP moves within a row of 16 lanes and the row / half-wave swaps of gfx950. Each reduction
// combines (lane, partner) in the same order on both lanes, so all lanes of a group agree.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
// sum over each aligned group of 8 lanes (xor 1, xor 2, then the mirror within the half row)
__device__ __forceinline__ float sum8(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  return v + dpp_mov<0x141>(v);  // row_half_mirror
}
// the value of lane ^ 8 (rotation by 8 within the row of 16)
__device__ __forceinline__ float xor8(float v) { return dpp_mov<0x128>(v); }
// rotations within each row of 16 lanes (DPP row_ror: lane i receives lane (i - n) mod 16)
template <int N>
__device__ __forceinline__ float row_to(float v) {  // lane i gets lane i - N (mod 16)
  static_assert(N > 0 && N < 16, "rotation by 1..15");
  return dpp_mov<0x120 + N>(v);
}
template <int N>
__device__ __forceinline__ float row_from(float v) {  // lane i gets lane i + N (mod 16)
  static_assert(N > 0 && N < 16, "rotation by 1..15");
  return dpp_mov<0x120 + 16 - N>(v);
}
// (v of the even row, v of the odd row) of each pair of 16-lane rows (0, 1), (2, 3)
__device__ __forceinline__ float2 pair16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// (v of lanes 0..31, v of lanes 32..63), paired lane by lane
__device__ __forceinline__ float2 pair32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) { const float2 t = pair16(v); return t.x + t.y; }
__device__ __forceinline__ float sum_xor32(float v) { const float2 t = pair32(v); return t.x + t.y; }
__device__ __forceinline__ float max_xor16(float v) { const float2 t = pair16(v); return fmaxf(t.x, t.y); }
__device__ __forceinline__ float max_xor32(float v) { const float2 t = pair32(v); return fmaxf(t.x, t.y); }
// whole-wave sum / max (every lane active)
__device__ __forceinline__ float wsum(float v) {
  v = sum8(v);
  v += xor8(v);
  return sum_xor32(sum_xor16(v));
}
__device__ __forceinline__ float wmax(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));
  v = fmaxf(v, dpp_mov<0x4E>(v));
  v = fmaxf(v, dpp_mov<0x141>(v));
  v = fmaxf(v, xor8(v));
  return max_xor32(max_xor16(v));
}
// maximum of an unsigned 64-bit value over each aligned row of 16 lanes (every lane active)
__device__ __forceinline__ uint64_t max16_u64(uint64_t v) {
  auto step = [](uint64_t a, uint64_t o) { return o > a ? o : a; };
#define BW_MAX16_STEP(CTRL)                                                                                       \
  v = step(v, ((uint64_t)(uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false) << 32) | \
                  (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, false))
  BW_MAX16_STEP(0xB1);   // quad_perm [1, 0, 3, 2]
  BW_MAX16_STEP(0x4E);   // quad_perm [2, 3, 0, 1]
  BW_MAX16_STEP(0x141);  // row_half_mirror
  BW_MAX16_STEP(0x128);  // row_ror:8
#undef BW_MAX16_STEP
  return v;
}
// sum over aligned groups of n lanes, n a power of two up to 64 (wave-uniform)
__device__ __forceinline__ float sum_lanes(float v, int n) {
  if (n >= 2) v += dpp_mov<0xB1>(v);
  if (n >= 4) v += dpp_mov<0x4E>(v);
  if (n >= 8) v += dpp_mov<0x141>(v);
  if (n >= 16) v += xor8(v);
  if (n >= 32) v = sum_xor16(v);
  if (n >= 64) v = sum_xor32(v);
  return v;
}

}  // namespace bw
