// bw_mfma.h - 16x16 matrix-core products on 16-bit cache elements, shared by the attention kernels
// (gfx950).
#pragma once

#include "bw_common.h"

namespace bw {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int KVDT>
struct MfmaT;
template <>
struct MfmaT<1> {  // fp16 cache
  typedef _Float16 e8 __attribute__((ext_vector_type(8)));
  typedef _Float16 e4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ f32x4 mm32(e8 a, e8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mm16(e4 a, e4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
};
template <>
struct MfmaT<2> {  // bf16 cache
  typedef __bf16 e8 __attribute__((ext_vector_type(8)));
  typedef short e4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ f32x4 mm32(e8 a, e8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mm16(e4 a, e4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
};

// Round to the cache dtype, nearest even, with the hardware conversion (v_cvt_pk_bf16_f32 for
// bf16); used for the query and probability parts, which no stored value depends on.
template <int KVDT>
__device__ __forceinline__ uint16_t part_bits(float x) {
  if constexpr (KVDT == 1) return f32_to_f16(x);
  else return __builtin_bit_cast(uint16_t, (__bf16)x);
}

}  // namespace bw
