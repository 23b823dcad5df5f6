// bw_mx.hip - MXFP4 weights on gfx950: batch-1 GEMV on the vector units and the batched GEMM on
// the scaled matrix cores.
//
// Weight format (OCP Microscaling MXFP4; the 4-bit floating-point weights of the bw24 deep-dive
// page, section 1 quantisation formats and the section 7 table): blocks of 32 E2M1 elements
// along K share one E8M0 scale byte, w = 2^(e - 127) * element. Row n of an [N][K] matrix holds
// K/2 code bytes (element 2i in bits 0-3 of byte i, element 2i+1 in bits 4-7) and K/32 scale
// bytes in a separate [N][K/32] array.
//
// GEMV (y = W x, x fp32). A row is shared by 16 lanes; lane j takes blocks j, j + 16, ... of
// the row, one 16-byte load each, so the 16 lanes of a row read 256 contiguous bytes per load
// instruction. Each wave handles 4 rows at a time. The input vector is staged once per workgroup
// in LDS (fp32). Each 32-element block is decoded in registers by v_cvt_scalef32_pk_f32_fp4 (two
// elements per instruction, the block's E8M0 scale applied by the conversion, exact) and
// multiplied into fp32 FMAs.
//
// GEMM (Y = X W^T, X fp32 [M][K]). The matrix cores take the weights as they are stored: E2M1
// codes with their E8M0 block scales are the fp4 operand of v_mfma_scale_f32_32x32x64_f8f6f4.
// The other operand must also be a scaled 8/6/4-bit format, so X is first written as the sum
// of three MXFP8 (E4M3, one E8M0 scale per 32) terms: term t quantises the residual left by
// terms 1..t-1, each residual exact in fp32. Each term leaves at most 2^-4 of its block's
// largest magnitude, so the three-term expansion is within 2^-12 of each block's maximum. One
// fp4 weight fragment then feeds three scaled products.
#include <algorithm>

#include "bw_common.h"
#include "bw_internal.h"

namespace bw {

// ---- E8M0 and E2M1 ------------------------------------------------------------------------------

// 2^(e - 127) as fp32 (e = 0 is the subnormal 2^-127; 255 is NaN)
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  e &= 0xFFu;
  if (e == 255u) return __uint_as_float(0x7FC00000u);
  if (e == 0u) return __uint_as_float(0x00400000u);
  return __uint_as_float(e << 23);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// sum over the 32 elements of one block (codes in q, element 2i+h in nibble h of byte i) of
// scale * element * x. The conversion applies the block's E8M0 scale itself (it reads only the
// exponent field of its fp32 scale operand: field e means 2^(e - 127), 255 is NaN), so each
// weight comes out exact in fp32. x sits in LDS chunk-major: chunk c (elements 4c..4c+3) of
// block b at xc + c * cstride, with xc the block's first chunk.
__device__ __forceinline__ float mx_block_dot(u32x4 q, float scale, const float* xc, int cstride) {
  float d0 = 0.f, d1 = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float4 xa = *(const float4*)(xc + (2 * w) * cstride);
    const float4 xb = *(const float4*)(xc + (2 * w + 1) * cstride);
    const f32x2 e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[w], scale, 0);
    const f32x2 e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[w], scale, 1);
    const f32x2 e2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[w], scale, 2);
    const f32x2 e3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[w], scale, 3);
    d0 = fmaf(e0[0], xa.x, d0);
    d1 = fmaf(e0[1], xa.y, d1);
    d0 = fmaf(e1[0], xa.z, d0);
    d1 = fmaf(e1[1], xa.w, d1);
    d0 = fmaf(e2[0], xb.x, d0);
    d1 = fmaf(e2[1], xb.y, d1);
    d0 = fmaf(e3[0], xb.z, d0);
    d1 = fmaf(e3[1], xb.w, d1);
  }
  return d0 + d1;
}

// ---- GEMV ---------------------------------------------------------------------------------------

constexpr int kMxLpr = 16;                  // lanes per row
constexpr int kMxRpw = kWave / kMxLpr;      // rows per wave step
constexpr int kMxNbc = 8;                   // blocks per lane per chunk (16 lanes x 8 = 128 blocks)
static_assert(kMxGemvMaxK * 4 <= 65536, "input vector in LDS");

struct MxGemvParams {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* x;
  float* y;
  int64_t N;
  int K;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mx_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, 0, (int)bytes, 0x00020000);
}

// Work: wave gw takes row steps gw, gw + W, ... (W = all waves of the grid). Per row step it
// walks the row in chunks of 16 x 8 blocks; the next chunk's codes and scales are loaded before
// the current one is computed.
__global__ __launch_bounds__(kBlock) void k_mx_gemv(MxGemvParams p) {
  extern __shared__ __align__(16) float xs[];  // K floats
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: descriptors built from it stay scalar
  const int K = p.K, nb = K / 32;
  // stage x chunk-major: chunk c of block b at float (c * nb + b) * 4, so the 16 lanes of a row,
  // reading chunk c of 16 consecutive blocks, touch 256 consecutive bytes (every bank once), and
  // a lane's addresses differ only by constants
  for (int i = tid; i < K / 4; i += kBlock) {
    const int b = i >> 3, c = i & 7;
    *(float4*)(xs + (c * nb + b) * 4) = ((const float4*)p.x)[i];
  }
  __syncthreads();
  const int j = lane % kMxLpr, rsub = lane / kMxLpr;
  const int nch = (nb + kMxLpr * kMxNbc - 1) / (kMxLpr * kMxNbc);
  const int64_t steps = (p.N + kMxRpw - 1) / kMxRpw;
  const int64_t nw = (int64_t)gridDim.x * (kBlock / kWave);
  const int64_t gw = (int64_t)blockIdx.x * (kBlock / kWave) + wave;
  const int64_t units = steps > gw ? ((steps - gw + nw - 1) / nw) * nch : 0;
  // each descriptor covers one row (K/2 code bytes, K/32 scale bytes), so matrices of any size
  // take 32-bit offsets
  struct Unit {
    u32x4 q[kMxNbc];
    uint32_t sc[kMxNbc];
  };
  auto load = [&](int64_t u, Unit& f) {
    const int64_t rs = gw + (u / nch) * nw;
    const int ch = (int)(u % nch);
    // descriptors on the row step's first row (wave-uniform), covering its rows below N; this
    // lane's row is an offset, and rows past N read zeros
    const int64_t n0 = rs * kMxRpw;
    const int rows = (int)std::max<int64_t>(0, std::min<int64_t>(kMxRpw, p.N - n0));
    const int64_t nbase = rows ? n0 : 0;
    const __amdgpu_buffer_rsrc_t rc = mx_rsrc(p.codes + nbase * (int64_t)(K / 2), rows * (K / 2));
    const __amdgpu_buffer_rsrc_t rsc = mx_rsrc(p.scales + nbase * (int64_t)nb, rows * nb);
#pragma unroll
    for (int i = 0; i < kMxNbc; ++i) {
      // blocks past the row end are skipped by compute (their loads read the next row or zeros)
      const int b = min(j + kMxLpr * (ch * kMxNbc + i), nb - 1);
      f.q[i] = __builtin_amdgcn_raw_buffer_load_b128(rc, rsub * (K / 2) + b * 16, 0, 2);
      f.sc[i] = __builtin_amdgcn_raw_buffer_load_b8(rsc, rsub * nb + b, 0, 2);
    }
  };
  float acc = 0.f;
  auto compute = [&](int64_t u, const Unit& f) {
    const int ch = (int)(u % nch);
#pragma unroll
    for (int i = 0; i < kMxNbc; ++i) {
      const int b = j + kMxLpr * (ch * kMxNbc + i);
      if (b < nb) acc += mx_block_dot(f.q[i], __uint_as_float(f.sc[i] << 23), xs + b * 4, nb * 4);
    }
    if (ch == nch - 1) {
      // the 16 lanes of a row
      acc += __shfl_xor(acc, 8);
      acc += __shfl_xor(acc, 4);
      acc += __shfl_xor(acc, 2);
      acc += __shfl_xor(acc, 1);
      const int64_t rs = gw + (u / nch) * nw;
      const int64_t n = rs * kMxRpw + rsub;
      if (j == 0 && n < p.N) p.y[n] = acc;
      acc = 0.f;
    }
  };
  // two register sets, each unit's loads issued one unit ahead (static indexing: no scratch)
  // every load is issued unconditionally (past the last unit it re-reads that unit), so the wait
  // before each unit's products counts exactly the next unit's loads
  Unit fa, fb;
  const int64_t ul = units > 0 ? units - 1 : 0;
  if (units > 0) load(0, fa);
  for (int64_t u = 0; u < units; u += 2) {
    load(std::min(u + 1, ul), fb);
    __builtin_amdgcn_sched_barrier(0);
    compute(u, fa);
    if (u + 1 >= units) break;
    load(std::min(u + 2, ul), fa);
    __builtin_amdgcn_sched_barrier(0);
    compute(u + 1, fb);
  }
}

int launch_mx_gemv(const uint8_t* codes, const uint8_t* scales, const float* x, float* y, int64_t N, int K,
                   hipStream_t st) {
  MxGemvParams p{codes, scales, x, y, N, K};
  const int64_t steps = (N + kMxRpw - 1) / kMxRpw;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  // up to 4 resident workgroups per CU, never more waves than row steps
  const int64_t want = (steps + (kBlock / kWave) - 1) / (kBlock / kWave);
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(want, (int64_t)cus * 4));
  hipLaunchKernelGGL(k_mx_gemv, dim3(grid), dim3(kBlock), (size_t)K * sizeof(float), st, p);
  return hipGetLastError() != hipSuccess;
}

// ---- X as three MXFP8 terms --------------------------------------------------------------------

// Workspace layout for M rows and Kp = K rounded up to 64:
//   xq: [M][Kp/32][3][32] E4M3 bytes (term t of block b of row m: 32 bytes)
//   xs: [M][Kp/32] uint32, byte t = E8M0 scale of term t (byte 3 zero)
// Blocks at or past K (when K is an odd number of blocks) are zero with scale byte 0.
struct MxQuantParams {
  const float* X;
  uint8_t* xq;
  uint32_t* xs;
  int64_t M;
  int K, Kp;
  float* Y;        // zeroed here when the GEMM accumulates split partials in place (else null)
  int64_t y_elems;
};

__device__ __forceinline__ uint32_t e8m0_for(float amax) {
  // the largest magnitude maps into [128, 256): scale 2^(E - 7), E = floor(log2 amax)
  if (!(amax > 0.f)) return 0u;
  const int E = (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 127;
  return (uint32_t)min(max(E + 120, 0), 254);
}

// One thread per (row, block).
__global__ __launch_bounds__(kBlock) void k_mx_quant(MxQuantParams p) {
  const int nbp = p.Kp / 32, nb = p.K / 32;
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (p.Y) {
    for (int64_t e = i; e < p.y_elems; e += (int64_t)gridDim.x * kBlock) p.Y[e] = 0.f;
  }
  if (i >= p.M * nbp) return;
  const int64_t m = i / nbp;
  const int b = (int)(i % nbp);
  float v[32];
  if (b < nb) {
    const float4* src = (const float4*)(p.X + m * p.K + (int64_t)b * 32);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float4 t = src[c];
      v[4 * c] = t.x;
      v[4 * c + 1] = t.y;
      v[4 * c + 2] = t.z;
      v[4 * c + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) v[e] = 0.f;
  }
  uint32_t scales = 0;
  u32x4* dst = (u32x4*)(p.xq + (i * 3) * 32);
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(v[e]));
    const uint32_t eb = e8m0_for(amax);
    scales |= eb << (8 * t);
    // v / s and s * q are exact powers-of-two scalings; q is v / s rounded to E4M3 (nearest even,
    // |v / s| < 256 so never saturated), and v - s * q is exact
    const float inv = __uint_as_float((254u - eb) << 23);  // 2^(127 - eb), eb in [0, 254]
    const float s = e8m0_to_f32(eb);
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      uint32_t word = 0;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int e = 4 * k + h;
        const float a = v[e] * inv;
        const uint32_t byte = __builtin_amdgcn_cvt_pk_fp8_f32(a, a, 0, false) & 0xFFu;
        word |= byte << (8 * h);
        v[e] = v[e] - s * __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
      }
      w[k] = word;
    }
    dst[2 * t] = u32x4{w[0], w[1], w[2], w[3]};
    dst[2 * t + 1] = u32x4{w[4], w[5], w[6], w[7]};
  }
  p.xs[i] = scales;
}

int launch_mx_quant(const float* X, uint8_t* xq, uint32_t* xs, int64_t M, int K, int Kp, float* Y_zero,
                    int64_t y_elems, hipStream_t st) {
  MxQuantParams p{X, xq, xs, M, K, Kp, Y_zero, y_elems};
  const int64_t n = M * (Kp / 32);
  const int grid = (int)std::max<int64_t>(1, (n + kBlock - 1) / kBlock);
  hipLaunchKernelGGL(k_mx_quant, dim3(grid), dim3(kBlock), 0, st, p);
  return hipGetLastError() != hipSuccess;
}

// ---- GEMM on the scaled matrix cores -----------------------------------------------------------

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMxTm = 128, kMxTn = 128;  // workgroup tile: 4 waves x 32 rows, 4 column tiles of 32

struct MxGemmParams {
  const uint8_t* xq;
  const uint32_t* xs;
  const uint8_t* codes;
  const uint8_t* scales;
  float* out;        // Y [M][N], or partials [ksplit][M][N]
  int64_t M, N;
  int K, Kp;
  int steps_per_split;  // k-steps of 64
};

// One k-step's operands of one lane: three E4M3 terms of its X row (32 bytes each) with their
// scale word, and the fp4 codes and scale of its column in each of the four column tiles.
typedef int i32x4 __attribute__((ext_vector_type(4)));
struct MxFrag {
  i32x8 a[3];  // the two 16-byte halves of each term, already in operand order
  uint32_t as;
  i32x4 b[4];
  uint32_t bs[4];
};

// Operand layout of v_mfma_scale_f32_32x32x64_f8f6f4 (measured on gfx950 with one-hot operands):
// lane l supplies row l % 32 of A and column l % 32 of B. With h = l / 32, the E2M1 B operand
// holds k = 32h + i in nibble i (the whole block h of the k-step), while the E4M3 A operand holds
// k = 16h + i in byte i and k = 32 + 16h + i in byte 16 + i (half h of each of the two blocks).
// The scale of block h, for A and for B, is the scale byte of lane half h. The 32 x 32 result has
// column l % 32 in lane l and rows (r % 4) + 8 (r / 4) + 4h in accumulator r.
__global__ __launch_bounds__(kBlock, 2) void k_mx_gemm(MxGemmParams p) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: descriptors built from it stay scalar
  const int l32 = lane & 31, kh = lane >> 5;
  const int nbp = p.Kp / 32, nb = p.K / 32;
  const int64_t n0 = (int64_t)blockIdx.x * kMxTn;
  const int64_t m0 = (int64_t)blockIdx.y * kMxTm + 32 * wave;
  const int s0 = blockIdx.z * p.steps_per_split;
  const int s1 = min(p.Kp / 64, s0 + p.steps_per_split);
  // A: descriptors on the wave's first X row (wave-uniform) covering its rows below M; this
  // lane's row is an offset, and rows at or past M read zeros
  const int arows = (int)std::max<int64_t>(0, std::min<int64_t>(32, p.M - m0));
  const int64_t abase = arows ? m0 : 0;
  const __amdgpu_buffer_rsrc_t ra = mx_rsrc(p.xq + abase * (int64_t)nbp * 96, arows * nbp * 96);
  const __amdgpu_buffer_rsrc_t ras = mx_rsrc(p.xs + abase * (int64_t)nbp, arows * nbp * 4);
  const int arow_q = l32 * nbp * 96, arow_s = l32 * nbp * 4;
  // B: one descriptor per column tile covering its valid rows
  __amdgpu_buffer_rsrc_t rb[4], rbs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t nt = n0 + 32 * j;
    const int64_t rows = nt < p.N ? min((int64_t)32, p.N - nt) : 0;
    rb[j] = mx_rsrc(p.codes + (rows ? nt : 0) * (int64_t)(p.K / 2), rows * (p.K / 2));
    rbs[j] = mx_rsrc(p.scales + (rows ? nt : 0) * (int64_t)nb, rows * nb);
  }
  auto load = [&](int s, MxFrag& f) {
    const int kb = 2 * s + kh;
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const i32x4 lo = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, arow_q + ((2 * s) * 3 + t) * 32 + 16 * kh, 0, 0));
      const i32x4 hi = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, arow_q + ((2 * s + 1) * 3 + t) * 32 + 16 * kh, 0, 0));
      f.a[t] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    f.as = __builtin_amdgcn_raw_buffer_load_b32(ras, arow_s + kb * 4, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f.b[j] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rb[j], l32 * (p.K / 2) + kb * 16, 0, 2));
      f.bs[j] = __builtin_amdgcn_raw_buffer_load_b8(rbs[j], l32 * nb + kb, 0, 2);
    }
  };
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  auto compute = [&](int s, const MxFrag& f) {
    // the E2M1 operand uses the first four registers of the eight
    i32x8 bv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bv[j] = __builtin_shufflevector(f.b[j], f.b[j], 0, 1, 2, 3, -1, -1, -1, -1);
    const i32x8* a = f.a;
    // past an odd number of blocks, X is zero (every term) and the weights read there are finite
    // codes of the next row; their scale is replaced by 1 so that a NaN scale byte there cannot
    // reach the sum
    const bool pad = 2 * s + kh >= nb;
    uint32_t bs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bs[j] = pad ? 127u : f.bs[j];
    // A format 0 = E4M3, B format 4 = E2M1; the A scale of term t is byte t of the scale word.
    // Term-major order: four independent accumulators between two products into the same one.
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[0], bv[j], acc[j], 0, 4, 0, (int)f.as, 0, (int)bs[j]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[1], bv[j], acc[j], 0, 4, 1, (int)f.as, 0, (int)bs[j]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[2], bv[j], acc[j], 0, 4, 2, (int)f.as, 0, (int)bs[j]);
  };
  // two register sets, each k-step's loads issued one step ahead (static indexing: no scratch);
  // every load is issued unconditionally (past the split it re-reads the split's last step), so
  // the wait before each step's products counts exactly the next step's loads
  MxFrag f0, f1;
  const int sl = max(s0, s1 - 1);
  load(min(s0, sl), f0);
  // (a scheduling barrier after each step's loads keeps them ahead of the products)
  for (int s = s0; s < s1; s += 2) {
    load(min(s + 1, sl), f1);
    __builtin_amdgcn_sched_barrier(0);
    compute(s, f0);
    if (s + 1 >= s1) break;
    load(min(s + 2, sl), f0);
    __builtin_amdgcn_sched_barrier(0);
    compute(s + 1, f1);
  }
  float* dst = p.out + (int64_t)blockIdx.z * p.M * p.N;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = n0 + 32 * j + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t mr = m0 + (r % 4) + 8 * (r / 4) + 4 * kh;
      if (mr < p.M && n < p.N) dst[mr * p.N + n] = acc[j][r];
    }
  }
}

// Y = sum over the splits, in split order
__global__ __launch_bounds__(kBlock) void k_mx_reduce(const float* part, float* Y, int64_t n, int splits) {
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += (int64_t)gridDim.x * kBlock) {
    float a = part[i];
    for (int z = 1; z < splits; ++z) a += part[(int64_t)z * n + i];
    Y[i] = a;
  }
}

int64_t mx_gemm_workspace_bytes(int64_t M, int64_t N, int K, int splits) {
  const int64_t Kp = (K + 63) / 64 * 64;
  const int64_t q = M * (Kp / 32) * 96, sc = M * (Kp / 32) * 4;
  const int64_t part = splits > 1 ? (int64_t)splits * M * N * 4 : 0;
  return ((q + 255) / 256) * 256 + ((sc + 255) / 256) * 256 + part;
}

int mx_gemm_splits(int64_t M, int64_t N, int K) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int64_t tiles = ((N + kMxTn - 1) / kMxTn) * ((M + kMxTm - 1) / kMxTm);
  const int steps = (K + 63) / 64;
  int64_t sp = (2 * (int64_t)cus + tiles - 1) / tiles;  // about two workgroups per CU
  sp = std::min<int64_t>(sp, std::max(1, steps / 8));  // at least 8 k-steps per split
  return (int)std::max<int64_t>(1, std::min<int64_t>(sp, 16));
}

int launch_mx_gemm(const uint8_t* codes, const uint8_t* scales, const float* X, float* Y, int64_t M, int64_t N,
                   int K, void* ws, int splits, hipStream_t st) {
  const int Kp = (K + 63) / 64 * 64;
  uint8_t* w = (uint8_t*)ws;
  uint8_t* xq = w;
  const int64_t q = M * (Kp / 32) * 96, sc = M * (Kp / 32) * 4;
  uint32_t* xs = (uint32_t*)(w + ((q + 255) / 256) * 256);
  float* part = (float*)(w + ((q + 255) / 256) * 256 + ((sc + 255) / 256) * 256);
  if (launch_mx_quant(X, xq, xs, M, K, Kp, nullptr, 0, st)) return 1;
  const int steps = Kp / 64;
  const int per = (steps + splits - 1) / splits;
  const int z = (steps + per - 1) / per;
  MxGemmParams p{xq, xs, codes, scales, z > 1 ? part : Y, M, N, K, Kp, per};
  hipLaunchKernelGGL(k_mx_gemm, dim3((unsigned)((N + kMxTn - 1) / kMxTn), (unsigned)((M + kMxTm - 1) / kMxTm), z),
                     dim3(kBlock), 0, st, p);
  if (hipGetLastError() != hipSuccess) return 1;
  if (z > 1) {
    const int64_t n = M * N;
    const int grid = (int)std::min<int64_t>(4096, (n + kBlock - 1) / kBlock);
    hipLaunchKernelGGL(k_mx_reduce, dim3(grid), dim3(kBlock), 0, st, part, Y, n, z);
    if (hipGetLastError() != hipSuccess) return 1;
  }
  return 0;
}

}  // namespace bw
