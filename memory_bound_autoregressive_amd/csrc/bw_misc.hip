// bw_misc.hip - the small kernels of the decode step (gfx950): embedding gather, final argmax,
// MoE router GEMV and top-k, plus the dequantisation and fill kernels used by the parity tests.
#include "bw_common.h"
#include "bw_internal.h"

namespace bw {

// x[m][:] = fp32(E[token[m]][:]); out-of-range ids set the error word and read row 0
__global__ __launch_bounds__(kBlock) void k_embed(const uint16_t* __restrict__ E, int32_t vocab,
                                                  int32_t d, const int32_t* __restrict__ tokens,
                                                  float* __restrict__ x, int32_t* err) {
  const int m = blockIdx.x;
  int tok = tokens[m];
  if (tok < 0 || tok >= vocab) {
    if (threadIdx.x == 0) atomicOr(err, 2);
    tok = 0;
  }
  const uint16_t* row = E + (int64_t)tok * d;
  for (int i = threadIdx.x; i < d; i += kBlock) x[(int64_t)m * d + i] = f16_to_f32(row[i]);
}

int launch_embed(const uint16_t* embed, int32_t vocab, int32_t d, const int32_t* tokens, int M,
                 float* x, int32_t* err, hipStream_t s) {
  hipLaunchKernelGGL(k_embed, dim3(M), dim3(kBlock), 0, s, embed, vocab, d, tokens, x, err);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// out[m] = index of the largest of the per-workgroup partials (lowest index on ties)
__global__ __launch_bounds__(kBlock) void k_argmax_final(const float* __restrict__ val,
                                                         const int32_t* __restrict__ idx, int parts,
                                                         int32_t* __restrict__ out) {
  const int m = blockIdx.x;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = threadIdx.x; i < parts; i += kBlock) {
    float v = val[(int64_t)m * parts + i];
    int k = idx[(int64_t)m * parts + i];
    if (v > bv || (v == bv && k < bi)) { bv = v; bi = k; }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    float ov = __shfl_xor(bv, o);
    int oi = __shfl_xor(bi, o);
    if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
  }
  __shared__ float wv[4];
  __shared__ int wi[4];
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { wv[w] = bv; wi[w] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < 4; ++k)
      if (wv[k] > wv[0] || (wv[k] == wv[0] && wi[k] < wi[0])) { wv[0] = wv[k]; wi[0] = wi[k]; }
    out[m] = wi[0] == 0x7fffffff ? 0 : wi[0];
  }
}

int launch_argmax_final(const float* val, const int32_t* idx, int parts, int M, int32_t* out,
                        hipStream_t s) {
  hipLaunchKernelGGL(k_argmax_final, dim3(M), dim3(kBlock), 0, s, val, idx, parts, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Router logits r = W_r h with h = RMSNorm(x) * gamma, W_r fp16 [E][d]. One row per wave: its
// 16-byte weight loads (8 fp16 per lane per step, at most 8 steps) go out first, as buffer loads
// (past the row end they read zeros), so they are in flight during the RMSNorm reduction.
constexpr int kRouterMaxSteps = 8;  // d <= 4096
__global__ __launch_bounds__(kBlock) void k_router(const uint16_t* __restrict__ wr, int E, int d,
                                                   const float* __restrict__ x,
                                                   const uint16_t* __restrict__ gamma, float eps,
                                                   float* __restrict__ logits) {
  extern __shared__ float h[];
  __shared__ float red[16];
  const int m = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + wave);
  const bool row_ok = e < E;
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc((void*)(wr + (int64_t)(row_ok ? e : 0) * d), 0, d * 2, 0x00020000);
  u32x4 raw[kRouterMaxSteps];
#pragma unroll
  for (int st = 0; st < kRouterMaxSteps; ++st) {
    const int k = lane * 8 + st * kWave * 8;
    raw[st] = __builtin_amdgcn_raw_buffer_load_b128(rw, k < d ? k * 2 : 0x7FFFFFF0, 0, 2);
  }
  const float* xr = x + (int64_t)m * d;
  float ss = 0.f;
  for (int k = threadIdx.x; k < d; k += kBlock) ss = fmaf(xr[k], xr[k], ss);
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)d + eps);
  for (int k = threadIdx.x; k < d; k += kBlock) h[k] = xr[k] * r * f16_to_f32(gamma[k]);
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int st = 0; st < kRouterMaxSteps; ++st) {
    const int k = lane * 8 + st * kWave * 8;
    if (k < d) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc = fmaf(f16_to_f32((uint16_t)(raw[st][i] & 0xFFFFu)), h[k + 2 * i], acc);
        acc = fmaf(f16_to_f32((uint16_t)(raw[st][i] >> 16)), h[k + 2 * i + 1], acc);
      }
    }
  }
  acc = wave_sum(acc);
  if (lane == 0 && row_ok) logits[(int64_t)m * E + e] = acc;
}

int launch_router(const uint16_t* wr, int E, int d, const float* x, const uint16_t* gamma,
                  float eps, int M, float* logits, hipStream_t s) {
  if (d > kRouterMaxSteps * kWave * 8 || d % 8 != 0) return -2;
  hipLaunchKernelGGL(k_router, dim3((E + 3) / 4, M), dim3(kBlock), sizeof(float) * d, s, wr, E, d, x, gamma, eps,
                     logits);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// top-k of the router logits (descending, ties to the lower expert index; a NaN logit ranks as
// -inf) and the renormalised gates softmax(r)_e / sum_{e' in top-k} softmax(r)_e'
// = exp(r_e - r_max) / sum_sel exp(r - r_max). One pass: the rank of logit e is the number of
// logits ahead of it, and e is chosen when its rank is below k.
// (The float4 reads cover indices below E rounded down to 4; the rest are read one by one.)
__global__ __launch_bounds__(kBlock) void k_topk(const float* __restrict__ logits, int E, int k,
                                                 int32_t* __restrict__ sel, float* __restrict__ gates) {
  extern __shared__ float r[];
  __shared__ int chosen[64];
  const int m = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += kBlock) {
    const float v = logits[(int64_t)m * E + e];
    r[e] = v != v ? -INFINITY : v;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kBlock) {
    const float v = r[e];
    int rank = 0;
    int j = 0;
    // 16-byte LDS reads, four in flight per step
#pragma unroll 4
    for (; j + 4 <= E; j += 4) {
      const float4 u = *(const float4*)(r + j);
      rank += (u.x > v || (u.x == v && j < e)) + (u.y > v || (u.y == v && j + 1 < e)) +
              (u.z > v || (u.z == v && j + 2 < e)) + (u.w > v || (u.w == v && j + 3 < e));
    }
    for (; j < E; ++j) rank += (r[j] > v || (r[j] == v && j < e)) ? 1 : 0;
    if (rank < k) chosen[rank] = e;
  }
  __syncthreads();
  if (threadIdx.x < k) {
    const float mx = r[chosen[0]];
    float z = 0.f;
    for (int q = 0; q < k; ++q) z += __expf(r[chosen[q]] - mx);
    const int q = threadIdx.x;
    sel[(int64_t)m * k + q] = chosen[q];
    gates[(int64_t)m * k + q] = __expf(r[chosen[q]] - mx) / z;
  }
}

int launch_topk(const float* logits, int E, int k, int M, int32_t* sel, float* gates,
                hipStream_t s) {
  if (k > 64 || k > E) return -2;
  hipLaunchKernelGGL(k_topk, dim3(M), dim3(kBlock), sizeof(float) * ((E + 3) & ~3), s, logits, E, k, sel, gates);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Dequantise with the step's nibble extraction: element i < 16 of a block is the low nibble of
// byte i, element 16 + i the high nibble; w = fp32(scale) * (q - 8), written in canonical order.
__global__ __launch_bounds__(kBlock) void k_dequant(Mat w, const int32_t* __restrict__ row_map,
                                                    int map_lo, int map_n, float* __restrict__ dst) {
  const int nblk = w.K >> 5;
  const int64_t total = (int64_t)w.N * nblk;
  for (int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x; t < total; t += (int64_t)gridDim.x * kBlock) {
    const int row = (int)(t / nblk), b = (int)(t - (int64_t)row * nblk);
    const int cr = (row_map ? row_map[row] : row) - map_lo;
    if (cr < 0 || cr >= map_n) continue;
    const int j = b % w.lpr, c = b / w.lpr;
    const float s = f16_to_f32(w.scales[(int64_t)row * nblk + j * w.nb + c]);
    const u32x4 q = *(const u32x4*)(w.codes + (int64_t)row * (w.K >> 1) + b * 16);
    float* out = dst + (int64_t)cr * w.K + b * 32;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t lo = q[d] & 0x0F0F0F0Fu, hi = (q[d] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        out[4 * d + i] = s * ((float)((lo >> (8 * i)) & 0xFFu) - 8.0f);
        out[16 + 4 * d + i] = s * ((float)((hi >> (8 * i)) & 0xFFu) - 8.0f);
      }
    }
  }
}

int launch_dequant(const Mat& w, const int32_t* row_map, int map_lo, int map_n, float* dst, hipStream_t s) {
  const int64_t total = (int64_t)w.N * (w.K >> 5);
  int grid = (int)((total + kBlock - 1) / kBlock);
  if (grid > 65535) grid = 65535;
  hipLaunchKernelGGL(k_dequant, dim3(grid), dim3(kBlock), 0, s, w, row_map, map_lo, map_n, dst);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

__global__ void k_fill16(uint16_t* __restrict__ dst, size_t n, uint16_t bits) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = bits;
}

int launch_fill16(uint16_t* dst, size_t n, uint16_t bits, hipStream_t s) {
  hipLaunchKernelGGL(k_fill16, dim3(4096), dim3(kBlock), 0, s, dst, n, bits);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// cache-dtype rounding of n values with the device conversions the kernels use: bits (in the
// low bits of a uint16) and the value read back
template <int KVDT>
__global__ void k_kv_round(const float* __restrict__ x, int64_t n, uint16_t* __restrict__ bits,
                           float* __restrict__ back) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint16_t b = f32_to_kv<KVDT>(x[i]);
  bits[i] = b;
  back[i] = kv_to_f32<KVDT>(b);
}

int launch_kv_round(int kv_dtype, const float* x, int64_t n, uint16_t* bits, float* back, hipStream_t s) {
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (kv_dtype == 1) hipLaunchKernelGGL(k_kv_round<1>, dim3(blocks), dim3(256), 0, s, x, n, bits, back);
  else if (kv_dtype == 2) hipLaunchKernelGGL(k_kv_round<2>, dim3(blocks), dim3(256), 0, s, x, n, bits, back);
  else if (kv_dtype == 3) hipLaunchKernelGGL(k_kv_round<3>, dim3(blocks), dim3(256), 0, s, x, n, bits, back);
  else return -2;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// KV host tier: pages (every layer's slice of a physical page id) packed into / unpacked from a
// contiguous staging buffer [i][layer][page_bytes], so that the PCIe transfer is one DMA copy.
// Block (i, l) moves the slice of page ids.id[i] in layer l with 16-byte loads and stores.
__global__ __launch_bounds__(256) void k_page_pack(uint8_t* __restrict__ pool, int64_t layer_bytes, int64_t page_bytes,
                                                   PageList ids, uint8_t* __restrict__ stage, int to_stage) {
  const int i = blockIdx.x, l = blockIdx.y, L = gridDim.y;
  u32x4* dev = (u32x4*)(pool + l * layer_bytes + (int64_t)ids.id[i] * page_bytes);
  u32x4* st = (u32x4*)(stage + ((int64_t)i * L + l) * page_bytes);
  const int64_t n = page_bytes / 16;
  if (to_stage) {
    for (int64_t e = threadIdx.x; e < n; e += blockDim.x) st[e] = dev[e];
  } else {
    for (int64_t e = threadIdx.x; e < n; e += blockDim.x) dev[e] = st[e];
  }
}

int launch_page_pack(uint8_t* pool, int64_t layer_bytes, int64_t page_bytes, int L, const PageList& ids, int n,
                     uint8_t* stage, bool to_stage, hipStream_t s) {
  if (n < 1 || n > PageList::kMax || page_bytes % 16) return -2;
  hipLaunchKernelGGL(k_page_pack, dim3(n, L), dim3(256), 0, s, pool, layer_bytes, page_bytes, ids, stage,
                     to_stage ? 1 : 0);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Expert host tier: repoint routed expert e of one layer's tables at new (gate/up codes, gate/up
// scales, down codes, down scales) addresses, in stream order after the copies that moved it.
__global__ void k_set_expert(ExpertTab tab, int e, const void* gc, const void* gs, const void* dc, const void* ds) {
  if (threadIdx.x == 0) {
    const_cast<const uint8_t**>(tab.gu_codes)[e] = (const uint8_t*)gc;
    const_cast<const uint16_t**>(tab.gu_scales)[e] = (const uint16_t*)gs;
    const_cast<const uint8_t**>(tab.dn_codes)[e] = (const uint8_t*)dc;
    const_cast<const uint16_t**>(tab.dn_scales)[e] = (const uint16_t*)ds;
  }
}

int launch_set_expert(const ExpertTab& tab, int e, const void* gc, const void* gs, const void* dc, const void* ds,
                      hipStream_t s) {
  hipLaunchKernelGGL(k_set_expert, dim3(1), dim3(64), 0, s, tab, e, gc, gs, dc, ds);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace bw
