// bw_gemm.hip - int4 block-quantised GEMM on the matrix cores for the batched / verify step.
//
// Operation: Y[m][n] = sum_k W[n][k] X[m][k] for all M = batch * t rows of a step at once, W int4 in
// blocks of 32 along K with one fp16 scale per block (w = scale * (q - 8)). With many rows every
// weight is used by all of them, so the product is a dense contraction (bw24 deep-dive page,
// section 5, stage 4: the verify kernel takes the drafted tokens as extra rows that share one pass
// over the weights).
//
// Numerics, exact up to fp32 summation order:
//  - a code q becomes the fp16 value (q - 8) exactly: the nibble goes into the mantissa of 1024
//    (bits 0x6400 | q) and one packed subtract of 1032 follows;
//  - X is staged as an fp16 pair x_hi = fp16(x), x_lo = fp16(x - x_hi), so a 32-wide block costs
//    two v_mfma_f32_16x16x32_f16 whose products are exact and whose sums are fp32;
//  - the fp16 block scale multiplies each block's 16x16 fp32 result, so no weight is rounded.
//
// MFMA operand layout (16x16x32 f16): lane l supplies row l % 16 of A and column l % 16 of B, eight
// K slots each, lane group l / 16 taking slots 8 (l / 16) .. +7; the result lane l holds rows
// 4 (l / 16) .. +3 of column l % 16. The sum over K does not depend on which element sits in which
// slot as long as A and B agree, so lane group g takes bytes 4g..4g+3 of a block (elements 4g..4g+3
// in the low nibbles, 16+4g..16+4g+3 in the high nibbles) with one 4-byte load, and X is staged in
// the matching order.
//
// Work split: workgroup = (tile of 128 weight rows, k-split, group of up to 128 X rows); 4 waves,
// wave w owns rows [32w, 32w + 32) of the tile as two 16-column B tiles and every m-tile. X is
// staged through LDS 64 columns at a time. Each k-split writes fp32 partials; k_gemm_epilogue sums
// them in split order and applies the step's epilogue (RoPE + KV append, residual, SwiGLU, logits).
//
// Products of more than 64 rows (verify steps, prefill chunks) take k_gemm_w32 instead: 32x32
// tiles, 256 weight rows per workgroup, and the block scales applied once per block to exact block
// sums (described at the kernel). The two forms write the same partials.
#include <algorithm>

#include "bw_common.h"
#include "bw_internal.h"

namespace bw {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr int kNS = 2;              // 16-column B tiles per wave
constexpr int kNT = 4 * 16 * kNS;   // weight rows per workgroup
constexpr int kKC = 64;             // K columns staged per round (two blocks)
constexpr int kXP = kKC + 8;        // staged row pitch in fp16 elements (16-byte aligned, skews banks)
constexpr int kMaxRowsWG = 128;     // X rows per workgroup (8 m-tiles)

// 1 / sqrt(mean(x^2) + eps) of each row of x (the RMSNorm factor of the batched path)
__global__ __launch_bounds__(kBlock) void k_rowrms(const float* __restrict__ x, int64_t stride, int K,
                                                   float eps, float* __restrict__ r) {
  __shared__ float red[4];
  const float* xr = x + (int64_t)blockIdx.x * stride;
  float ss = 0.f;
  for (int k = threadIdx.x; k < K; k += kBlock) ss = fmaf(xr[k], xr[k], ss);
  ss = block_sum(ss, red);
  if (threadIdx.x == 0) r[blockIdx.x] = 1.0f / sqrtf(ss / (float)K + eps);
}

// Bytes 4g..4g+3 of a block as eight fp16 (q - 8): low nibbles of the four bytes, then high nibbles.
__device__ __forceinline__ h8_t codes_to_h8(uint32_t c) {
  const uint32_t lo = c & 0x0F0F0F0Fu, hi = (c >> 4) & 0x0F0F0F0Fu;
  u32x4 r;
  r[0] = ((lo & 0xFFu) | ((lo & 0xFF00u) << 8)) | 0x64006400u;
  r[1] = (((lo >> 16) & 0xFFu) | ((lo >> 8) & 0xFF0000u)) | 0x64006400u;
  r[2] = ((hi & 0xFFu) | ((hi & 0xFF00u) << 8)) | 0x64006400u;
  r[3] = (((hi >> 16) & 0xFFu) | ((hi >> 8) & 0xFF0000u)) | 0x64006400u;
  const h8_t off = {(_Float16)1032.0f, (_Float16)1032.0f, (_Float16)1032.0f, (_Float16)1032.0f,
                    (_Float16)1032.0f, (_Float16)1032.0f, (_Float16)1032.0f, (_Float16)1032.0f};
  return __builtin_bit_cast(h8_t, r) - off;  // (1024 + q) - 1032 = q - 8, exact
}

// Staged position of element kb (0..31, kb % 4 == 0) of a block: lane group (kb % 16) / 4, low half
// for kb < 16, high half otherwise.
__device__ __forceinline__ int staged_pos(int kb) { return 8 * ((kb & 15) >> 2) + 4 * (kb >> 4); }

// X as fp16 pairs once per product: xh = fp16(x), xl = fp16(x - xh), with x times the row's
// RMSNorm factor and the gain for IN_RMSNORM, each 32-wide block in the staged order above.
// Every workgroup of the product then copies 16-byte chunks into LDS with no conversion.
template <int IN>
__global__ __launch_bounds__(kBlock) void k_stage_x(const float* __restrict__ x, int64_t stride, int K, int M,
                                                   const float* __restrict__ rms, const uint16_t* __restrict__ gamma,
                                                   uint16_t* __restrict__ xh, uint16_t* __restrict__ xl) {
  const int n4 = K >> 2;
  const int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (e >= (int64_t)M * n4) return;
  const int m = (int)(e / n4), c4 = (int)(e - (int64_t)m * n4) * 4;
  float4 v = *(const float4*)(x + (int64_t)m * stride + c4);
  if constexpr (IN == IN_RMSNORM) {
    const float r = rms[m];
    const uint2 gh = *(const uint2*)(gamma + c4);
    v.x *= r * f16_to_f32((uint16_t)(gh.x & 0xFFFFu));
    v.y *= r * f16_to_f32((uint16_t)(gh.x >> 16));
    v.z *= r * f16_to_f32((uint16_t)(gh.y & 0xFFFFu));
    v.w *= r * f16_to_f32((uint16_t)(gh.y >> 16));
  }
  const float vv[4] = {v.x, v.y, v.z, v.w};
  uint16_t hh[4], ll[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const _Float16 h = (_Float16)vv[j];
    hh[j] = __builtin_bit_cast(uint16_t, h);
    ll[j] = __builtin_bit_cast(uint16_t, (_Float16)(vv[j] - (float)h));
  }
  const int64_t at = (int64_t)m * K + (c4 & ~31) + staged_pos(c4 & 31);
  *(uint2*)(xh + at) = make_uint2(hh[0] | ((uint32_t)hh[1] << 16), hh[2] | ((uint32_t)hh[3] << 16));
  *(uint2*)(xl + at) = make_uint2(ll[0] | ((uint32_t)ll[1] << 16), ll[2] | ((uint32_t)ll[3] << 16));
}

// element (m, n) of k-split ks goes to out[ks * ks_stride + m * ldo + n]
// Rounds of kKC columns are software-pipelined: round r + 1's codes, scales and X values are
// loaded into registers before round r's products, and its X is converted and staged into the
// other LDS buffer after them, so one barrier per round separates the buffers and the memory
// latency of a round overlaps the previous round's matrix-core work. Every load is issued
// unconditionally (rows past N or M are clamped and their values zeroed by selection), so the
// compiler's wait counts are exact.
template <int MT>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm(GemvParams p, int M, int ksplit, const uint16_t* __restrict__ gxh,
                                                const uint16_t* __restrict__ gxl, float* __restrict__ out, int64_t ldo,
                                                int64_t ks_stride) {
  constexpr int XB = MT * 16 * kXP;  // one staged buffer (fp16 elements)
  __shared__ __attribute__((aligned(16))) _Float16 xh[2][XB];
  __shared__ __attribute__((aligned(16))) _Float16 xl[2][XB];
  constexpr int XCH = MT * 16 * (kKC / 8);            // 16-byte chunks of one round's X (each of hi, lo)
  constexpr int NX = (XCH + kBlock - 1) / kBlock;     // per thread
  const int K = p.w.K, N = p.w.N;
  const int nblk = K >> 5;
  const int n0 = blockIdx.x * kNT;
  const int ks = blockIdx.y;
  const int m0 = blockIdx.z * kMaxRowsWG;
  const int kc = K / ksplit;
  const int k_begin = ks * kc, k_end = k_begin + kc;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ln = lane & 15, g = lane >> 4;

  int nrow[kNS];
  bool nok[kNS];
#pragma unroll
  for (int s = 0; s < kNS; ++s) {
    nrow[s] = n0 + wave * 16 * kNS + s * 16 + ln;
    nok[s] = nrow[s] < N;
  }

  f4_t tot[kNS][MT];
#pragma unroll
  for (int s = 0; s < kNS; ++s)
#pragma unroll
    for (int t = 0; t < MT; ++t) tot[s][t] = f4_t{0.f, 0.f, 0.f, 0.f};

  struct Round {
    uint32_t cw[kNS][kKC / 32];
    uint16_t sc[kNS][kKC / 32];
    u32x4 xv[NX][2];  // hi, lo chunks
  };
  auto load_round = [&](int k0, Round& r) {
#pragma unroll
    for (int s = 0; s < kNS; ++s)
#pragma unroll
      for (int bb = 0; bb < kKC / 32; ++bb) {
        const int b = (k0 >> 5) + bb;
        const int64_t n = min(nrow[s], N - 1);
        r.cw[s][bb] = __builtin_nontemporal_load((const uint32_t*)(p.w.codes + n * (K >> 1) + b * 16 + 4 * g));
        r.sc[s][bb] = p.w.scales[n * nblk + (b % p.w.lpr) * p.w.nb + b / p.w.lpr];
      }
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int e = min((int)threadIdx.x + i * kBlock, XCH - 1);
      const int row = e / (kKC / 8), ch = e - row * (kKC / 8);
      const int64_t at = (int64_t)min(m0 + row, M - 1) * K + k0 + 8 * ch;
      r.xv[i][0] = *(const u32x4*)(gxh + at);
      r.xv[i][1] = *(const u32x4*)(gxl + at);
    }
  };
  auto stage_round = [&](const Round& r, int buf) {
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int e = threadIdx.x + i * kBlock;
      if (e >= XCH) continue;
      const int row = e / (kKC / 8), ch = e - row * (kKC / 8);
      const bool in = m0 + row < M;
      const u32x4 z = {0u, 0u, 0u, 0u};
      *(u32x4*)(xh[buf] + row * kXP + 8 * ch) = in ? r.xv[i][0] : z;
      *(u32x4*)(xl[buf] + row * kXP + 8 * ch) = in ? r.xv[i][1] : z;
    }
  };
  auto compute_round = [&](const Round& r, int buf) {
#pragma unroll
    for (int bb = 0; bb < kKC / 32; ++bb) {
      h8_t bf[kNS];
      float scf[kNS];
#pragma unroll
      for (int s = 0; s < kNS; ++s) {
        bf[s] = codes_to_h8(nok[s] ? r.cw[s][bb] : 0x88888888u);  // rows past N: codes 8, value 0
        scf[s] = nok[s] ? f16_to_f32(r.sc[s][bb]) : 0.f;
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int at = (t * 16 + ln) * kXP + bb * 32 + 8 * g;
        const h8_t ah = *(const h8_t*)(xh[buf] + at);
        const h8_t al = *(const h8_t*)(xl[buf] + at);
#pragma unroll
        for (int s = 0; s < kNS; ++s) {
          f4_t acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bf[s], f4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bf[s], acc, 0, 0, 0);
          tot[s][t] += scf[s] * acc;
        }
      }
    }
  };

  Round ra, rb;
  load_round(k_begin, ra);
  stage_round(ra, 0);
  __syncthreads();
  int buf = 0;
  for (int k0 = k_begin; k0 < k_end; k0 += 2 * kKC) {
    const bool more1 = k0 + kKC < k_end;
    if (more1) load_round(k0 + kKC, rb);
    compute_round(ra, buf);
    if (!more1) break;
    stage_round(rb, buf ^ 1);
    __syncthreads();
    buf ^= 1;
    const bool more2 = k0 + 2 * kKC < k_end;
    if (more2) load_round(k0 + 2 * kKC, ra);
    compute_round(rb, buf);
    if (!more2) break;
    stage_round(ra, buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
#pragma unroll
  for (int s = 0; s < kNS; ++s) {
    if (!nok[s]) continue;
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + t * 16 + 4 * g + v;
        if (m < M) out[(int64_t)ks * ks_stride + (int64_t)m * ldo + nrow[s]] = tot[s][t][v];
      }
  }
}

// ---- the wide form: 32x32 tiles, block sums scaled once per block --------------------------------
// For products of more than 64 rows. A workgroup of 8 waves covers 256 weight rows x 128 X rows:
// wave w owns weight rows [32 w, +32) against all 128 X rows as 4 tiles of
// v_mfma_f32_32x32x16_f16 (lane l gives A row / B column l % 32 with K slots 8 (l / 32) .. +7; the
// result's slot r of lane l is row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32), so each
// unpacked weight fragment feeds 8 matrix instructions.
// Weights: lane l reads bytes 8h..8h+7 of a block (h = l / 32); its 4-byte group g = 2h + s feeds
// K-step s of the block, in the staged X order. The codes enter the products as q - 8, exact in
// fp16, against x_hi and x_lo (x = x_hi + x_lo in fp16, so every product is exact in fp32): each
// block's sums d = sum (q - 8)(x_hi + x_lo) over its 32 columns start from zero, and the block
// scale is applied once, acc += s d (one fused multiply-add per output per block, with the fp16
// scale read by v_fma_mix_f32). Rows past N or M read clamped addresses; their results are never
// stored.
// Pipelining: a chunk's X (from L2) is loaded one chunk ahead and staged into the other LDS buffer
// after the current chunk's products; its codes and scales (from HBM) are loaded two chunks ahead
// into one of three register sets.
constexpr int kW32Threads = 512;
constexpr int kW32N = 256;          // weight rows per workgroup
constexpr int kW32M = 128;          // X rows per workgroup
constexpr int kW32KC = 64;          // K columns per chunk (two blocks)
constexpr int kW32XP = kW32KC + 8;  // LDS row pitch in fp16 elements (16-byte aligned, skews banks)
constexpr int kW32MinRows = 65;     // products with fewer rows use k_gemm

typedef float f16x_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// codes_to_h8 with byte permutes: each half is byte 0x64 over a code nibble, 1024 + q
__device__ __forceinline__ h8_t codes_to_h8_perm(uint32_t c) {
  const uint32_t lo = c & 0x0F0F0F0Fu, hi = (c >> 4) & 0x0F0F0F0Fu;
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u);
  r[1] = __builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u);
  r[2] = __builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u);
  r[3] = __builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u);
  const h8_t off = {(_Float16)1032.0f, (_Float16)1032.0f, (_Float16)1032.0f, (_Float16)1032.0f,
                    (_Float16)1032.0f, (_Float16)1032.0f, (_Float16)1032.0f, (_Float16)1032.0f};
  return __builtin_bit_cast(h8_t, r) - off;  // (1024 + q) - 1032 = q - 8, exact
}

// (X without __restrict__: restrict-qualified loads could be moved across the compiler barriers)
__global__ __launch_bounds__(kW32Threads, 2) void k_gemm_w32(GemvParams p, int M, int ksplit, const uint16_t* gxh,
                                                             const uint16_t* gxl, float* __restrict__ out, int64_t ldo,
                                                             int64_t ks_stride) {
  __shared__ __attribute__((aligned(16))) _Float16 xs[2][2][kW32M * kW32XP];  // [buffer][hi, lo]
  const int K = p.w.K, N = p.w.N, nblk = K >> 5;
  // the scale of block b sits at (b % lpr) nb + b / lpr of its row (lpr a power of two)
  const int lpr_mask = p.w.lpr - 1, lpr_log = __builtin_ctz(p.w.lpr), nb = p.w.nb;
  const int n0 = blockIdx.x * kW32N, ks = blockIdx.y, m0 = blockIdx.z * kW32M;
  const int kc = K / ksplit;
  const int k_begin = ks * kc, k_end = k_begin + kc;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;

  // this wave's first weight row and this lane's (both clamped): the descriptors start at the
  // wave's row, so they are uniform, and the lane's row is an offset
  const int wrow = min(n0 + 32 * wave, N - 1);
  const int nrow = min(n0 + 32 * wave + l32, N - 1);
  const int crow = (nrow - wrow) * (K >> 1) + 8 * h, srow = (nrow - wrow) * nblk * 2;
  // this thread's two 16-byte X chunks per round: row e / 8, columns 8 (e % 8) .. +7
  int xrow[2];
  int64_t xat[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = tid + i * kW32Threads;
    xrow[i] = e >> 3;
    xat[i] = (int64_t)min(m0 + xrow[i], M - 1) * K + 8 * (e & 7);
  }

  struct XChunk {
    u32x4 v[2][2];  // [hi, lo][chunk]
  };
  struct WChunk {
    u32x2_t cw[2];     // [block]
    uint32_t sc[2];    // [block] fp16 bits (whole registers: no sub-word arrays to demote to memory)
  };
  auto next = [&](int k0) { return k0 < k_end ? k0 : k_begin; };  // loads past the split re-read its start
  // buffer loads on this wave's weight rows (codes, scales); X through global pointers, whose loads
  // the compiler memory barriers below keep in place
  const __amdgpu_buffer_rsrc_t rcw =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.w.codes + (int64_t)wrow * (K >> 1)), 0, 32 * (K >> 1), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.w.scales + (int64_t)wrow * nblk), 0, 32 * nblk * 2, 0x00020000);
  auto load_x = [&](int k0, XChunk& c) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      c.v[0][i] = *(const u32x4*)(gxh + xat[i] + k0);
      c.v[1][i] = *(const u32x4*)(gxl + xat[i] + k0);
    }
  };
  auto load_w = [&](int k0, WChunk& c) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int b = (k0 >> 5) + bb;
      c.cw[bb] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rcw, crow + b * 16, 0, 2));
      c.sc[bb] = __builtin_amdgcn_raw_buffer_load_b16(rsc, srow + ((b & lpr_mask) * nb + (b >> lpr_log)) * 2, 0, 0);
    }
  };
  auto stage = [&](const XChunk& c, int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int at = xrow[i] * kW32XP + 8 * ((tid + i * kW32Threads) & 7);
      *(u32x4*)(xs[buf][0] + at) = c.v[0][i];
      *(u32x4*)(xs[buf][1] + at) = c.v[1][i];
    }
  };
  f16x_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  auto compute = [&](const WChunk& c, int buf) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      // the block's sums of (q - 8) x over its 32 columns (q - 8 exact in fp16, x as hi + lo), then
      // scaled once: acc += s * sum
      f16x_t d[4];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const h8_t q = codes_to_h8_perm(c.cw[bb][st]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int at = (32 * i + l32) * kW32XP + 32 * bb + 8 * (2 * h + st);
          const h8_t ah = *(const h8_t*)(xs[buf][0] + at);
          const h8_t al = *(const h8_t*)(xs[buf][1] + at);
          d[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, q, st == 0 ? f16x_t{} : d[i], 0, 0, 0);
          d[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, q, d[i], 0, 0, 0);
        }
      }
      const float sv = (float)__builtin_bit_cast(_Float16, (uint16_t)c.sc[bb]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = fmaf(sv, d[i][r], acc[i][r]);
    }
  };

  // every load is issued unconditionally, so the wait counts stay exact
  XChunk x;
  WChunk w0, w1, w2;
  load_x(k_begin, x);
  load_w(k_begin, w0);
  load_w(next(k_begin + kW32KC), w1);
  stage(x, 0);
  __syncthreads();
  int buf = 0;
  for (int k0 = k_begin;; k0 += 3 * kW32KC) {
    load_x(next(k0 + kW32KC), x);
    load_w(next(k0 + 2 * kW32KC), w2);
    // the loads stay ahead of the products: a compiler memory barrier keeps them from being sunk
    // to their uses past the loop's exit test
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    compute(w0, buf);
    if (k0 + kW32KC >= k_end) break;
    stage(x, buf ^ 1);
    __syncthreads();
    buf ^= 1;
    load_x(next(k0 + 2 * kW32KC), x);
    load_w(next(k0 + 3 * kW32KC), w0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    compute(w1, buf);
    if (k0 + 2 * kW32KC >= k_end) break;
    stage(x, buf ^ 1);
    __syncthreads();
    buf ^= 1;
    load_x(next(k0 + 3 * kW32KC), x);
    load_w(next(k0 + 4 * kW32KC), w1);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    compute(w2, buf);
    if (k0 + 3 * kW32KC >= k_end) break;
    stage(x, buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  const int n = n0 + 32 * wave + l32;
  if (n < N) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m < M) out[(int64_t)ks * ks_stride + (int64_t)m * ldo + n] = acc[i][r];
      }
  }
}

// Sum of the k-split partials part[ks][m][n] (in split order) and the step's epilogue; one thread
// per pair of device rows (2i, 2i + 1), which is a RoPE pair for q / k and a (gate, up) pair for
// the SwiGLU matrix.
template <int EPI>
__global__ __launch_bounds__(kBlock) void k_gemm_epilogue(GemvParams p, int M, int ksplit,
                                                         const float* __restrict__ part) {
  const int N = p.w.N;
  const int64_t pairs = (int64_t)M * (N >> 1);
  for (int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x; t < pairs; t += (int64_t)gridDim.x * kBlock) {
    const int m = (int)(t / (N >> 1));
    const int dr = 2 * (int)(t - (int64_t)m * (N >> 1));
    float v0 = 0.f, v1 = 0.f;
    for (int s = 0; s < ksplit; ++s) {
      const float2 pv = *(const float2*)(part + ((int64_t)s * M + m) * N + dr);
      v0 += pv.x;
      v1 += pv.y;
    }
    float* yr = p.y + (int64_t)m * p.y_stride;
    if constexpr (EPI == EPI_STORE_CANON) {
      const int c0 = (p.row_map ? p.row_map[dr] : dr) - p.map_lo;
      const int c1 = (p.row_map ? p.row_map[dr + 1] : dr + 1) - p.map_lo;
      if (c0 >= 0 && c0 < p.map_n) yr[c0] = v0;
      if (c1 >= 0 && c1 < p.map_n) yr[c1] = v1;
    } else if constexpr (EPI == EPI_RESID) {
      yr[dr] += v0;
      yr[dr + 1] += v1;
    } else if constexpr (EPI == EPI_SWIGLU) {
      yr[dr >> 1] = silu(v0) * v1;
    } else if constexpr (EPI == EPI_LOGITS) {
      yr[dr] = v0;
      yr[dr + 1] = v1;
    } else if constexpr (EPI == EPI_QKV) {
      const int D = p.D, HD = p.H * p.D, GD = p.G * p.D;
      const int b = m / p.t, ti = m - b * p.t;
      const int pos = p.seq_lens[b] + ti;
      if (pos < 0 || pos >= p.max_pos) {
        atomicOr(p.err, 4);
        continue;
      }
      float o0 = v0, o1 = v1;
      int head, d0, d1;
      if (dr < HD + GD) {  // device rows (2i, 2i + 1) hold head dims (i, i + D/2)
        const int local = dr < HD ? dr : dr - HD;
        head = local / D;
        const int i = (local - head * D) >> 1;
        const float2 cs = p.rope[(int64_t)pos * (D >> 1) + i];
        o0 = v0 * cs.x - v1 * cs.y;
        o1 = v0 * cs.y + v1 * cs.x;
        d0 = i;
        d1 = i + (D >> 1);
        if (dr < HD) {
          p.qout[((int64_t)m * p.H + head) * D + d0] = o0;
          p.qout[((int64_t)m * p.H + head) * D + d1] = o1;
          continue;
        }
      } else {
        const int local = dr - HD - GD;
        head = local / D;
        d0 = local - head * D;
        d1 = d0 + 1;
      }
      const int which = dr < HD + GD ? 0 : 1;
      const int page = pos / kPageTokens < p.max_pages ? p.page_table[(int64_t)b * p.max_pages + pos / kPageTokens] : -1;
      if (page < 0 || page >= p.n_pages) {
        atomicOr(p.err, 1);
        continue;
      }
      const int64_t e = (int64_t)page * p.pool_page_stride +
                        ((int64_t)(head * 2 + which) * kPageTokens + (pos % kPageTokens)) * D;
      if (p.kv_dtype == 3) {
        uint8_t* base = (uint8_t*)p.pool + e;
        base[d0] = (uint8_t)f32_to_fp8(o0);
        base[d1] = (uint8_t)f32_to_fp8(o1);
      } else {
        uint16_t* base = p.pool + e;
        base[d0] = (p.kv_dtype == 1) ? f32_to_f16(o0) : f32_to_bf16(o0);
        base[d1] = (p.kv_dtype == 1) ? f32_to_f16(o1) : f32_to_bf16(o1);
      }
    }
  }
}

// argmax of each row of logits [M][N] (lowest index on ties; NaN never wins)
// Per-row argmax of the batched logits in two passes: workgroup (c, m) scans chunk c of row m
// (coalesced, ascending, so the first maximum of a thread is its lowest index) and writes its
// (value, index) partial to val / idx [m][chunks]; k_argmax_final then reduces each row's partials
// (lowest index on ties). NaN never wins; a row without a winner gives index 0.
__global__ __launch_bounds__(kBlock) void k_argmax_rows(const float* __restrict__ logits, int64_t ld, int N,
                                                       int chunk, float* __restrict__ val, int32_t* __restrict__ idx) {
  const int m = blockIdx.y, c = blockIdx.x, chunks = gridDim.x;
  const float* row = logits + (int64_t)m * ld;
  const int i0 = c * chunk, i1 = min(N, i0 + chunk);
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = i0 + (int)threadIdx.x; i < i1; i += kBlock) {
    const float v = row[i];
    if (v > bv) { bv = v; bi = i; }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(bv, o);
    const int oi = __shfl_xor(bi, o);
    if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
  }
  __shared__ float wv[4];
  __shared__ int wi[4];
  if ((threadIdx.x & 63) == 0) { wv[threadIdx.x >> 6] = bv; wi[threadIdx.x >> 6] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w)
      if (wv[w] > wv[0] || (wv[w] == wv[0] && wi[w] < wi[0])) { wv[0] = wv[w]; wi[0] = wi[w]; }
    val[(int64_t)m * chunks + c] = wv[0];
    idx[(int64_t)m * chunks + c] = wi[0];
  }
}

// ---- launch -----------------------------------------------------------------------------------

int launch_rowrms(const float* x, int64_t stride, int K, float eps, int M, float* r, hipStream_t s) {
  hipLaunchKernelGGL(k_rowrms, dim3(M), dim3(kBlock), 0, s, x, stride, K, eps, r);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// k-splits: enough workgroups for 256 CUs while each split keeps >= 4 rounds of 64 columns. A
// wide-form workgroup (one per CU) carries a large fixed cost next to its per-chunk cost (about
// 16 us and 2 us at the 9B shapes), so where the doubling overshoots one round of workgroups the
// last doubling is undone: one round of longer splits beats two rounds of shorter ones.
int gemm_ksplit(int N, int K, int M) {
  const bool wide = M >= kW32MinRows;
  const int tiles = (N + (wide ? kW32N : kNT) - 1) / (wide ? kW32N : kNT);
  const int mg = (M + kMaxRowsWG - 1) / kMaxRowsWG;
  int ks = 1;
  while (tiles * ks * mg < 256 && K % (ks * 2 * kKC) == 0 && K / (ks * 2) >= 4 * kKC) ks *= 2;
  if (wide && ks > 1 && tiles * ks * mg > 256) ks /= 2;
  return ks;
}

int64_t gemm_part_elems(int N, int K, int M) { return (int64_t)gemm_ksplit(N, K, M) * M * N; }

bool gemm_supported(int N, int K) { return K % kKC == 0 && N % 2 == 0 && K >= kKC; }

int launch_gemm(int in_mode, int epi, const GemvParams& p, int M, const float* rms, float* part, uint16_t* xs,
                hipStream_t s) {
  if (M < 1 || !gemm_supported(p.w.N, p.w.K) || xs == nullptr) return -2;
  if (in_mode != IN_PLAIN && in_mode != IN_RMSNORM) return -2;
  if (in_mode == IN_RMSNORM && rms == nullptr) return -2;
  // X once as staged fp16 pairs (xs: [2][M][K])
  uint16_t* gxh = xs;
  uint16_t* gxl = xs + (int64_t)M * p.w.K;
  {
    const int64_t n4 = (int64_t)M * (p.w.K >> 2);
    const dim3 sg((unsigned)((n4 + kBlock - 1) / kBlock));
    if (in_mode == IN_RMSNORM)
      hipLaunchKernelGGL(k_stage_x<IN_RMSNORM>, sg, dim3(kBlock), 0, s, p.x, p.x_stride, p.w.K, M, rms, p.gamma, gxh, gxl);
    else
      hipLaunchKernelGGL(k_stage_x<IN_PLAIN>, sg, dim3(kBlock), 0, s, p.x, p.x_stride, p.w.K, M, rms, p.gamma, gxh, gxl);
  }
  const int ks = gemm_ksplit(p.w.N, p.w.K, M);
  const int mg = (M + kMaxRowsWG - 1) / kMaxRowsWG;
  const int mt = std::min(4, (M + 15) / 16);
  // a single split of the logits goes straight to its destination
  const bool direct = ks == 1 && epi == EPI_LOGITS;
  float* out = direct ? p.y : part;
  const int64_t ldo = direct ? p.y_stride : p.w.N;
  const int64_t ks_stride = (int64_t)M * p.w.N;
  if (out == nullptr) return -2;
  if (M >= kW32MinRows) {
    static_assert(kW32M == kMaxRowsWG, "row groups of the two forms agree");
    hipLaunchKernelGGL(k_gemm_w32, dim3((p.w.N + kW32N - 1) / kW32N, ks, mg), dim3(kW32Threads), 0, s, p, M, ks, gxh,
                       gxl, out, ldo, ks_stride);
  } else {
  const dim3 grid((p.w.N + kNT - 1) / kNT, ks, mg);
#define BW_G(MT_)                                                                                     \
  if (mt <= MT_) {                                                                                    \
    hipLaunchKernelGGL((k_gemm<MT_>), grid, dim3(kBlock), 0, s, p, M, ks, gxh, gxl, out, ldo, ks_stride); \
  } else
  BW_G(1) BW_G(2) BW_G(4) {}  // fewer than kW32MinRows rows: at most 4 m-tiles
#undef BW_G
  }
  if (hipGetLastError() != hipSuccess) return -1;
  if (direct) return 0;
  const int64_t pairs = (int64_t)M * (p.w.N >> 1);
  const int eg = (int)std::min<int64_t>(8192, (pairs + kBlock - 1) / kBlock);
  const float* cpart = part;
  switch (epi) {
    case EPI_STORE_CANON: hipLaunchKernelGGL(k_gemm_epilogue<EPI_STORE_CANON>, dim3(eg), dim3(kBlock), 0, s, p, M, ks, cpart); break;
    case EPI_RESID: hipLaunchKernelGGL(k_gemm_epilogue<EPI_RESID>, dim3(eg), dim3(kBlock), 0, s, p, M, ks, cpart); break;
    case EPI_SWIGLU: hipLaunchKernelGGL(k_gemm_epilogue<EPI_SWIGLU>, dim3(eg), dim3(kBlock), 0, s, p, M, ks, cpart); break;
    case EPI_LOGITS: hipLaunchKernelGGL(k_gemm_epilogue<EPI_LOGITS>, dim3(eg), dim3(kBlock), 0, s, p, M, ks, cpart); break;
    case EPI_QKV: hipLaunchKernelGGL(k_gemm_epilogue<EPI_QKV>, dim3(eg), dim3(kBlock), 0, s, p, M, ks, cpart); break;
    default: return -2;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_argmax_rows(const float* logits, int64_t ld, int N, int M, float* val, int32_t* idx, int max_parts,
                       int32_t* out, hipStream_t s) {
  // about 2048 workgroups over all rows, chunks of at least 2048 columns
  int chunks = std::max(1, std::min((2048 + M - 1) / M, (N + 2047) / 2048));
  chunks = std::min(chunks, max_parts);
  const int chunk = (N + chunks - 1) / chunks;
  hipLaunchKernelGGL(k_argmax_rows, dim3(chunks, M), dim3(kBlock), 0, s, logits, ld, N, chunk, val, idx);
  if (hipGetLastError() != hipSuccess) return -1;
  return launch_argmax_final(val, idx, chunks, M, out, s);
}

}  // namespace bw
