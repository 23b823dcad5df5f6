// bw_dot.h - the int4 block dot product shared by the batch-1 GEMV kernels (gfx950).
#pragma once

#include "bw_common.h"

namespace bw {

// dot product of one 32-element block: sum_i (q_i - 8) x_i
// Two codes (w >> s) & 0x000F000F read as two fp16 subnormals q * 2^-24 (exact), so one shift and
// one and unpack two codes; each feeds an fp32 FMA directly from its half of the register
// (v_fma_mix_f32 converts the fp16 operand exactly), so every product and sum is fp32. For code
// dword k of a block (bytes 4k..4k+3: low nibbles are elements 4k..4k+3, high nibbles elements
// 16+4k..16+4k+3) the x values come from chunks k and 4+k of the block. With D = sum q 2^-24 x
// and S = sum x over the block: sum (q - 8) x = 2^24 D - 8 S.
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float mix2(uint32_t pair, float x_even, float x_odd, float acc) {
  const h2_t h = __builtin_bit_cast(h2_t, pair);
  acc = fmaf((float)h[0], x_even, acc);
  return fmaf((float)h[1], x_odd, acc);
}

__device__ __forceinline__ float block_dot(u32x4 q, const float4* xv, float bsum) {
  float d = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w = q[k];
    const float4 lo = xv[k], hi = xv[4 + k];
    d = mix2(w & 0x000F000Fu, lo.x, lo.z, d);           // elements 4k, 4k+2
    d = mix2((w >> 8) & 0x000F000Fu, lo.y, lo.w, d);    // elements 4k+1, 4k+3
    d = mix2((w >> 4) & 0x000F000Fu, hi.x, hi.z, d);    // elements 16+4k, 16+4k+2
    d = mix2((w >> 12) & 0x000F000Fu, hi.y, hi.w, d);   // elements 16+4k+1, 16+4k+3
  }
  return fmaf(16777216.0f, d, -8.0f * bsum);
}

}  // namespace bw
