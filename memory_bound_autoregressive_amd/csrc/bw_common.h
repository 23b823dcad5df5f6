// bw_common.h - device helpers and shared parameter structs of libbw (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bw {

constexpr int kWave = 64;   // CDNA wavefront
constexpr int kBlock = 256; // threads per workgroup of the streaming kernels (4 waves)
constexpr int kPageTokens = 16;

// ---- number formats -------------------------------------------------------------------------

// fp16 bits -> fp32 (v_cvt_f32_f16: exact, subnormal inputs kept)
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}
// fp32 -> bf16 bits, round to nearest, ties to even (NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
// fp32 -> fp16 bits, round to nearest even (hardware conversion in the default mode)
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
// OCP FP8 E4M3 bits (low byte) -> fp32, exact (v_cvt_f32_fp8 decodes the OCP format on gfx950)
__device__ __forceinline__ float fp8_to_f32(uint32_t b) {
  return __builtin_amdgcn_cvt_f32_fp8((int)b, 0);
}
// fp32 -> OCP FP8 E4M3 bits, round to nearest even (hardware), saturating: the value is first
// clamped to [-448, 448], so magnitudes beyond the largest finite E4M3 value (and infinities)
// store +-448
__device__ __forceinline__ uint16_t f32_to_fp8(float f) {
  f = __builtin_amdgcn_fmed3f(f, -448.f, 448.f);
  return (uint16_t)(__builtin_amdgcn_cvt_pk_fp8_f32(f, f, 0, false) & 0xFF);
}
// cache dtypes: 1 = fp16, 2 = bf16 (16-bit elements), 3 = FP8 E4M3 (8-bit elements); bits are
// passed around in the low bits of a uint16_t
template <int KVDT>
__device__ __forceinline__ float kv_to_f32(uint16_t v) {
  if constexpr (KVDT == 1) return f16_to_f32(v);
  else if constexpr (KVDT == 3) return fp8_to_f32(v);
  else return bf16_to_f32(v);
}
template <int KVDT>
__device__ __forceinline__ uint16_t f32_to_kv(float f) {
  if constexpr (KVDT == 1) return f32_to_f16(f);
  else if constexpr (KVDT == 3) return f32_to_fp8(f);
  else return f32_to_bf16(f);
}

// ---- loads ------------------------------------------------------------------------------------

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Storage of a cache dtype: E is one element; C8 holds 8 consecutive elements (one load).
template <int KVDT>
struct KvT {
  typedef uint16_t E;
  typedef u32x4 C8;
  static constexpr int ES = 2;
};
template <>
struct KvT<3> {
  typedef uint8_t E;
  typedef u32x2 C8;
  static constexpr int ES = 1;
};

// 8 cache elements -> fp32
template <int KVDT>
__device__ __forceinline__ void kv_unpack8(typename KvT<KVDT>::C8 v, float* out) {
  if constexpr (KVDT == 3) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[i], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[i], true);
      out[4 * i] = lo[0];
      out[4 * i + 1] = lo[1];
      out[4 * i + 2] = hi[0];
      out[4 * i + 3] = hi[1];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = kv_to_f32<KVDT>((uint16_t)(v[i] & 0xFFFFu));
      out[2 * i + 1] = kv_to_f32<KVDT>((uint16_t)(v[i] >> 16));
    }
  }
}

// 8 FP8 E4M3 elements -> 8 bf16 (exact: every E4M3 value is a bf16 value), as the matrix-core
// operand of a bf16 product: gfx950's scaled conversion with scale 1, two elements per instruction
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(u32x2 v) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    r[2 * i] = __builtin_bit_cast(uint32_t, (b2)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[i], 1.0f, false));
    r[2 * i + 1] = __builtin_bit_cast(uint32_t, (b2)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[i], 1.0f, true));
  }
  return r;
}

// 16-byte streaming load that does not displace cached data (weights are read once per step)
__device__ __forceinline__ u32x4 load_stream16(const void* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

// ---- LDS layout of the input vector ---------------------------------------------------------
// Each 32-element block of the input occupies 128 bytes = eight 16-byte chunks. Chunk c of block b
// is stored in slot (c + b) & 7 of the block's row, so eight lanes reading chunk c of eight
// consecutive blocks touch eight different slots (all banks).
__device__ __forceinline__ float* xs_chunk(float* xs, int b, int c) {
  return xs + b * 32 + (((c + b) & 7) << 2);
}
__device__ __forceinline__ const float* xs_chunk(const float* xs, int b, int c) {
  return xs + b * 32 + (((c + b) & 7) << 2);
}

// ---- reductions -------------------------------------------------------------------------------

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Sum over a 256-thread block; every thread gets the result. `red` holds >= 4 floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

}  // namespace bw
