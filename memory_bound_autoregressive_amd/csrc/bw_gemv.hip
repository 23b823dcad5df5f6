// bw_gemv.hip - fused int4 dequantise-and-GEMV for the batch-1 decode step (gfx950).
//
// Operation (bw24 vs llama.cpp page, section 2.2: the linear layer and its activation run in one
// kernel with intermediates kept on chip): y = W x for one input row per grid.y, where W is int4
// in blocks of 32 along K with one fp16 scale per block and w = scale * (q - 8). Each block is
// dequantised in registers; nothing but the 4-bit codes and fp16 scales is read from HBM.
//
// Work split. A wave computes RW "row steps" of RPW = 64 / LPR rows each: LPR lanes share one
// row and split its K/32 blocks, lane j taking blocks j, j + LPR, ... (NB blocks). Each lane loads
// whole 16-byte blocks (32 codes) with one non-temporal dwordx4 load; the LPR lanes of a row
// read LPR consecutive blocks, i.e. contiguous 16*LPR bytes. The input vector sits in LDS in a
// bank-swizzled layout; each 32-element x block is read once and reused for the RW rows.
// Per block the dot product uses sum_k s (q_k - 8) x_k = s (sum_k q_k x_k - 8 sum_k x_k), with
// the per-block sums of x computed once when the vector is staged.
//
// Prologues: plain vector, RMSNorm of the residual row, or the gated concatenation of the
// selected experts' SwiGLU outputs (MoE down projection). Epilogues: store, residual add, RoPE
// + KV append, SwiGLU, logits with an argmax partial, MoE SwiGLU.
#include <algorithm>

#include "bw_common.h"
#include "bw_dot.h"
#include "bw_internal.h"

namespace bw {

// ---------------------------------------------------------------------------------------------
// input staging
// ---------------------------------------------------------------------------------------------

// ---------------------------------------------------------------------------------------------
// row addressing
// ---------------------------------------------------------------------------------------------

struct RowPtr {
  const uint8_t* codes;    // start of the row's codes
  const uint16_t* scales;  // this lane's NB scales of the row (retiled layout)
};

// ordinary matrix (device row order)
template <int LPR, int NB>
__device__ __forceinline__ RowPtr row_ptr(const Mat& w, int row, int j) {
  const int nblk = w.K >> 5;
  return RowPtr{w.codes + (int64_t)row * (w.K >> 1), w.scales + (int64_t)row * nblk + j * NB};
}

// MoE gate/up virtual row: routed slots first (2*Fe rows each), then shared experts (2*Fs rows)
template <int LPR, int NB>
__device__ __forceinline__ RowPtr moe_gu_row_ptr(const GemvParams& p, int m, int row, int j, int K,
                                                 int* out_off, int* local) {
  const int nblk = K >> 5;
  const int routed_rows = p.top_k * 2 * p.Fe;
  int e, lr, off;
  if (row < routed_rows) {
    int slot = row / (2 * p.Fe);
    lr = row - slot * 2 * p.Fe;
    e = min(max(p.sel[m * p.top_k + slot], 0), p.n_experts - 1);
    off = slot * p.Fe;
  } else {
    int s = (row - routed_rows) / (2 * p.Fs);
    lr = row - routed_rows - s * 2 * p.Fs;
    e = p.n_experts + s;
    off = p.top_k * p.Fe + s * p.Fs;
  }
  *out_off = off;
  *local = lr;
  return RowPtr{p.ex.gu_codes[e] + (int64_t)lr * (K >> 1), p.ex.gu_scales[e] + (int64_t)lr * nblk + j * NB};
}


// MoE down projection: lane block c of output row n covers virtual block b = j + LPR*c of the
// concatenated [routed slots x Fe | shared x Fs] input; returns the 16-byte code address and the
// scale (canonical per-expert layout, valid because each expert's K/32 gives lpr or nb of 1).
__device__ __forceinline__ void moe_dn_block(const GemvParams& p, int m, int n, int b,
                                             const uint8_t** codes, const uint16_t** scale) {
  const int fe_blk = p.Fe >> 5, fs_blk = p.Fs >> 5;
  const int routed_blk = p.top_k * fe_blk;
  int e, lb, F;
  if (b < routed_blk) {
    int slot = b / fe_blk;
    lb = b - slot * fe_blk;
    e = min(max(p.sel[m * p.top_k + slot], 0), p.n_experts - 1);
    F = p.Fe;
  } else {
    int s = (b - routed_blk) / fs_blk;
    lb = b - routed_blk - s * fs_blk;
    e = p.n_experts + s;
    F = p.Fs;
  }
  *codes = p.ex.dn_codes[e] + (int64_t)n * (F >> 1) + lb * 16;
  *scale = p.ex.dn_scales[e] + (int64_t)n * (F >> 5) + lb;
}

// ---------------------------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------------------------

// The codes and scales of one group of rows (RW row steps of RPW rows) for one lane.
template <int LPR, int NB, int RW>
struct Group {
  u32x4 q[RW][NB];
  uint16_t sc[RW][NB];
  int row[RW];
  int moe_off[RW], moe_lr[RW];
  float2 cs[RW];  // RoPE (cos, sin) of each row's pair (QKV epilogue)
};

// RoPE factors of a group's q/k rows at position pos (issued right after the group's weights)
template <int LPR, int NB, int RW>
__device__ __forceinline__ void load_rope(const GemvParams& p, int pos, Group<LPR, NB, RW>& g) {
  const int D = p.D, HD = p.H * p.D, GD = p.G * p.D;
  const bool pos_ok = pos >= 0 && pos < p.max_pos;
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int dr = g.row[r];
    g.cs[r] = make_float2(1.f, 0.f);
    if (pos_ok && dr < HD + GD) {
      const int local = dr < HD ? dr : dr - HD;
      const int i = (local % D) >> 1;
      g.cs[r] = p.rope[(int64_t)pos * (D >> 1) + i];
    }
  }
}

template <int LPR, int NB, int RW, int IN, int EPI>
__device__ __forceinline__ void load_group(const GemvParams& p, int m, int K, int gi, int j, int rsub,
                                           Group<LPR, NB, RW>& g) {
  constexpr int RPW = kWave / LPR;
  constexpr int GROUP = RPW * RW;
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    g.row[r] = gi * GROUP + r * RPW + rsub;
    const bool ok = g.row[r] < p.n_rows;
    if constexpr (IN == IN_MOE_DOWN) {
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        const uint8_t* cp;
        const uint16_t* sp;
        moe_dn_block(p, m, ok ? g.row[r] : 0, j + LPR * c, &cp, &sp);
        g.q[r][c] = ok ? load_stream16(cp) : u32x4{0, 0, 0, 0};
        g.sc[r][c] = ok ? *sp : (uint16_t)0;
      }
    } else {
      RowPtr rp;
      if constexpr (EPI == EPI_MOE_SWIGLU)
        rp = moe_gu_row_ptr<LPR, NB>(p, m, ok ? g.row[r] : 0, j, K, &g.moe_off[r], &g.moe_lr[r]);
      else
        rp = row_ptr<LPR, NB>(p.w, ok ? g.row[r] : 0, j);
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        g.q[r][c] = ok ? load_stream16(rp.codes + (j + LPR * c) * 16) : u32x4{0, 0, 0, 0};
        g.sc[r][c] = ok ? rp.scales[c] : (uint16_t)0;
      }
    }
  }
}

// Work split: wave w of workgroup b takes groups b*4 + w, then every 4*gridDim.x-th group. The
// launcher sizes the grid so that every workgroup is resident at once.
// Latency plan: the input-vector loads are issued first, the first group's weight loads second
// (so the input can be staged while the weights are in flight), the next group's weights are
// loaded before the current group is computed, and the epilogue's own inputs (position, page id,
// RoPE factors) are fetched before any of that completes.
template <int LPR, int NB, int RW, int IN, int EPI>
__global__ __launch_bounds__(kBlock) void k_gemv(GemvParams p) {
  extern __shared__ float lds[];
  constexpr int RPW = kWave / LPR;
  constexpr int GROUP = RPW * RW;
  constexpr int KC = LPR * NB * 32;                   // K of this instantiation
  constexpr int XV = (KC / 4 + kBlock - 1) / kBlock;  // float4 input loads per thread
  const int K = KC;
  const int nblk = K >> 5;
  float* xs = lds;
  float* bs = lds + K;
  float* red = bs + nblk;  // 16 floats
  float* csum = red + 16;  // nblk * 8 chunk sums
  const int m = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane % LPR, rsub = lane / LPR;
  const int n_groups = (p.n_rows + GROUP - 1) / GROUP;

  // ---- 1. input loads (global -> registers)
  float4 xv[XV];
  {
    const bool emb = (IN == IN_RMSNORM) && p.embed != nullptr;
    int tok = 0;
    if (emb) {
      tok = p.tokens[m];
      if (tok < 0 || tok >= p.vocab) {
        if (threadIdx.x == 0 && blockIdx.x == 0) atomicOr(p.err, 2);
        tok = 0;
      }
    }
    const float* xr = p.x + (int64_t)m * p.x_stride;
#pragma unroll
    for (int i = 0; i < XV; ++i) {
      const int k4 = threadIdx.x + i * kBlock;
      xv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (k4 < KC / 4) {
        if (emb) {
          const uint2 h = *(const uint2*)(p.embed + (int64_t)tok * K + 4 * k4);
          xv[i] = make_float4(f16_to_f32((uint16_t)(h.x & 0xFFFFu)), f16_to_f32((uint16_t)(h.x >> 16)),
                              f16_to_f32((uint16_t)(h.y & 0xFFFFu)), f16_to_f32((uint16_t)(h.y >> 16)));
        } else {
          xv[i] = *(const float4*)(xr + 4 * k4);
        }
      }
    }
  }

  // ---- 2. first group's weights
  int gi = blockIdx.x * 4 + wave;
  Group<LPR, NB, RW> cur;
  if (gi < n_groups) load_group<LPR, NB, RW, IN, EPI>(p, m, K, gi, j, rsub, cur);

  // ---- 3. epilogue inputs of the QKV step (uniform per row m), after the weights are in flight
  int pos = 0, page = -1;
  if constexpr (EPI == EPI_QKV) {
    const int b = m / p.t, ti = m - b * p.t;
    pos = p.seq_lens[b] + ti;
    if (pos >= 0 && pos < p.max_pos && pos / kPageTokens < p.max_pages)
      page = p.page_table[(int64_t)b * p.max_pages + pos / kPageTokens];
    if (gi < n_groups) load_rope<LPR, NB, RW>(p, pos, cur);
  }

  // ---- 4. stage the input vector (RMSNorm / gate scaling) into LDS, block sums
  {
    float scale = 1.0f;
    if constexpr (IN == IN_RMSNORM) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < XV; ++i) ss += (xv[i].x * xv[i].x + xv[i].y * xv[i].y) + (xv[i].z * xv[i].z + xv[i].w * xv[i].w);
      ss = block_sum(ss, red);
      scale = 1.0f / sqrtf(ss / (float)K + p.eps);
    }
#pragma unroll
    for (int i = 0; i < XV; ++i) {
      const int k4 = threadIdx.x + i * kBlock;
      if (k4 >= KC / 4) continue;
      const int k = 4 * k4;
      float4 v = xv[i];
      if constexpr (IN == IN_RMSNORM) {
        if (p.embed != nullptr && blockIdx.x == 0) *(float4*)(p.x_out + (int64_t)m * p.x_stride + k) = v;
        const uint2 gh = *(const uint2*)(p.gamma + k);
        v.x *= scale * f16_to_f32((uint16_t)(gh.x & 0xFFFFu));
        v.y *= scale * f16_to_f32((uint16_t)(gh.x >> 16));
        v.z *= scale * f16_to_f32((uint16_t)(gh.y & 0xFFFFu));
        v.w *= scale * f16_to_f32((uint16_t)(gh.y >> 16));
      } else if constexpr (IN == IN_MOE_DOWN) {
        const float g = k < p.top_k * p.Fe ? p.gates[m * p.top_k + k / p.Fe] : 1.0f;
        v.x *= g; v.y *= g; v.z *= g; v.w *= g;
      }
      // 4 consecutive elements of a block form one 16-byte chunk of the swizzled layout
      *(float4*)xs_chunk(xs, k >> 5, (k & 31) >> 2) = v;
      csum[(k >> 5) * 8 + ((k & 31) >> 2)] = (v.x + v.y) + (v.z + v.w);
    }
    __syncthreads();
    for (int b = threadIdx.x; b < nblk; b += kBlock) {
      float sacc = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) sacc += csum[b * 8 + c];
      bs[b] = sacc;
    }
    __syncthreads();
  }

  float best_v = -INFINITY;
  int best_i = 0x7fffffff;

  // ---- 5. groups, double-buffered (A/B alternate so that no registers are copied)
  auto compute = [&](const Group<LPR, NB, RW>& g) {
      float acc[RW];
  #pragma unroll
      for (int r = 0; r < RW; ++r) acc[r] = 0.f;
  #pragma unroll
      for (int c = 0; c < NB; ++c) {
        // keep one x block live at a time (the code loads above are already in flight)
        __builtin_amdgcn_sched_barrier(0);
        const int b = j + LPR * c;
        float4 xb[8];
  #pragma unroll
        for (int k = 0; k < 8; ++k) xb[k] = *(const float4*)xs_chunk(xs, b, k);
        const float sb = bs[b];
  #pragma unroll
        for (int r = 0; r < RW; ++r) acc[r] = fmaf(f16_to_f32(g.sc[r][c]), block_dot(g.q[r][c], xb, sb), acc[r]);
      }
      // reduce over the LPR lanes of each row
  #pragma unroll
      for (int r = 0; r < RW; ++r) {
  #pragma unroll
        for (int o = LPR / 2; o >= 1; o >>= 1) acc[r] += __shfl_xor(acc[r], o);
      }
      // partner row (row ^ 1) for the paired epilogues
      float pv[RW];
  #pragma unroll
      for (int r = 0; r < RW; ++r) {
        if constexpr (RPW >= 2) pv[r] = __shfl_xor(acc[r], LPR);
        else pv[r] = acc[r ^ (RW > 1 ? 1 : 0)];
      }
      if (j == 0) {
  #pragma unroll
        for (int r = 0; r < RW; ++r) {
          const int dr = g.row[r];
          if (dr >= p.n_rows) continue;
          const float v = acc[r];
          float* yr = p.y + (int64_t)m * p.y_stride;
          if constexpr (EPI == EPI_STORE) {
            yr[dr] = v;
          } else if constexpr (EPI == EPI_STORE_CANON) {
            const int cr = (p.row_map ? p.row_map[dr] : dr) - p.map_lo;
            if (cr >= 0 && cr < p.map_n) yr[cr] = v;
          } else if constexpr (EPI == EPI_RESID) {
            yr[dr] += v;
          } else if constexpr (EPI == EPI_LOGITS) {
            yr[dr] = v;
            if (v > best_v) { best_v = v; best_i = dr; }
          } else if constexpr (EPI == EPI_SWIGLU) {
            if ((dr & 1) == 0) yr[dr >> 1] = silu(v) * pv[r];
          } else if constexpr (EPI == EPI_MOE_SWIGLU) {
            if ((g.moe_lr[r] & 1) == 0) yr[g.moe_off[r] + (g.moe_lr[r] >> 1)] = silu(v) * pv[r];
          } else if constexpr (EPI == EPI_QKV) {
            const int D = p.D, HD = p.H * p.D, GD = p.G * p.D;
            if (pos < 0 || pos >= p.max_pos) { atomicOr(p.err, 4); continue; }
            float out;
            int head, d;
            if (dr < HD + GD) {
              const int local = dr < HD ? dr : dr - HD;
              head = local / D;
              const int i = (local - head * D) >> 1;
              const float2 cs = g.cs[r];
              if ((dr & 1) == 0) { out = v * cs.x - pv[r] * cs.y; d = i; }
              else { out = pv[r] * cs.y + v * cs.x; d = i + (D >> 1); }
              if (dr < HD) {
                p.qout[((int64_t)m * p.H + head) * D + d] = out;
                continue;
              }
            } else {
              const int local = dr - HD - GD;
              head = local / D;
              d = local - head * D;
              out = v;
            }
            const int which = dr < HD + GD ? 0 : 1;
            if (page < 0 || page >= p.n_pages) { atomicOr(p.err, 1); continue; }
            const int64_t e = (int64_t)page * p.pool_page_stride +
                              ((int64_t)(head * 2 + which) * kPageTokens + (pos % kPageTokens)) * D + d;
            if (p.kv_dtype == 3) ((uint8_t*)p.pool)[e] = (uint8_t)f32_to_fp8(out);
            else p.pool[e] = (p.kv_dtype == 1) ? f32_to_f16(out) : f32_to_bf16(out);
          }
        }
      }
  };
  Group<LPR, NB, RW> alt;
  while (gi < n_groups) {
    int gn = gi + gridDim.x * 4;
    if (gn < n_groups) {
      load_group<LPR, NB, RW, IN, EPI>(p, m, K, gn, j, rsub, alt);
      if constexpr (EPI == EPI_QKV) load_rope<LPR, NB, RW>(p, pos, alt);
    }
    compute(cur);
    gi = gn;
    if (gi >= n_groups) break;
    gn = gi + gridDim.x * 4;
    if (gn < n_groups) {
      load_group<LPR, NB, RW, IN, EPI>(p, m, K, gn, j, rsub, cur);
      if constexpr (EPI == EPI_QKV) load_rope<LPR, NB, RW>(p, pos, cur);
    }
    compute(alt);
    gi = gn;
  }
  if constexpr (EPI == EPI_LOGITS) {
    // workgroup argmax partial (ties -> lowest index)
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      float ov = __shfl_xor(best_v, o);
      int oi = __shfl_xor(best_i, o);
      if (ov > best_v || (ov == best_v && oi < best_i)) { best_v = ov; best_i = oi; }
    }
    __shared__ float wv[4];
    __shared__ int wi[4];
    if (lane == 0) { wv[wave] = best_v; wi[wave] = best_i; }
    __syncthreads();
    if (threadIdx.x == 0) {
      float bv = wv[0];
      int bi = wi[0];
      for (int w = 1; w < 4; ++w)
        if (wv[w] > bv || (wv[w] == bv && wi[w] < bi)) { bv = wv[w]; bi = wi[w]; }
      p.amax_val[(int64_t)m * gridDim.x + blockIdx.x] = bv;
      p.amax_idx[(int64_t)m * gridDim.x + blockIdx.x] = bi;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------------------------

static int gcd_pow2_64(int nblk) {
  int l = 64;
  while (l > 1 && (nblk % l) != 0) l >>= 1;
  return l;
}

template <int LPR, int NB, int RW, int IN, int EPI>
static int launch_one(const GemvParams& p, int K, int M, hipStream_t s, int* grid_out) {
  constexpr int GROUP = (kWave / LPR) * RW;
  auto kern = k_gemv<LPR, NB, RW, IN, EPI>;
  const size_t lds = sizeof(float) * ((size_t)K + (size_t)(K >> 5) * 9 + 16);
  // resident workgroups of this instantiation (queried once)
  static int resident = 0;
  if (resident == 0) {
    if (lds > 65536 &&
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return -1;
    int per_cu = 0, dev = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kBlock, lds) != hipSuccess || per_cu < 1) per_cu = 1;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
    resident = per_cu * cus;
  }
  const int n_groups = (p.n_rows + GROUP - 1) / GROUP;
  // fewest groups per wave that keeps every workgroup resident (M rows share the grid)
  const int cap = std::max(1, resident / std::max(1, M));
  const int waves_needed = (n_groups + 3) / 4;
  const int per_wave = std::max(1, (waves_needed + cap - 1) / cap);
  int grid = (n_groups + 4 * per_wave - 1) / (4 * per_wave);
  if (grid > 4096) grid = 4096;
  if (grid < 1) grid = 1;
  if (grid_out) *grid_out = grid;
  hipLaunchKernelGGL(kern, dim3(grid, M), dim3(kBlock), lds, s, p);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int IN, int EPI>
static int dispatch_shape(const GemvParams& p, int K, int M, hipStream_t s, int* grid_out) {
  const int nblk = K >> 5;
  const int lpr = gcd_pow2_64(nblk);
  const int nb = nblk / lpr;
#define BW_CASE(L, N, R) \
  if (lpr == L && nb == N) return launch_one<L, N, R, IN, EPI>(p, K, M, s, grid_out);
  BW_CASE(64, 1, 8)
  BW_CASE(64, 2, 4)
  BW_CASE(64, 6, 2)
  BW_CASE(32, 5, 2)
  BW_CASE(32, 17, 1)
  BW_CASE(32, 1, 4)
  BW_CASE(16, 1, 4)
  BW_CASE(16, 9, 1)
  BW_CASE(8, 1, 2)
  BW_CASE(4, 1, 2)
#undef BW_CASE
  return -2;  // unsupported K
}

int launch_gemv(int in_mode, int epi, const GemvParams& p, int M, hipStream_t s, int* grid_out) {
  const int K = (in_mode == IN_MOE_DOWN) ? (p.top_k * p.Fe + p.n_shared * p.Fs) : p.w.K;
#define BW_IE(I, E) \
  if (in_mode == I && epi == E) return dispatch_shape<I, E>(p, K, M, s, grid_out);
  BW_IE(IN_PLAIN, EPI_STORE)
  BW_IE(IN_PLAIN, EPI_STORE_CANON)
  BW_IE(IN_PLAIN, EPI_RESID)
  BW_IE(IN_PLAIN, EPI_SWIGLU)
  BW_IE(IN_RMSNORM, EPI_QKV)
  BW_IE(IN_RMSNORM, EPI_SWIGLU)
  BW_IE(IN_RMSNORM, EPI_LOGITS)
  BW_IE(IN_RMSNORM, EPI_MOE_SWIGLU)
  BW_IE(IN_MOE_DOWN, EPI_RESID)
#undef BW_IE
  return -3;
}

// the same shape rule as the kernels, for the host-side weight layout
int gemv_lane_split(int K, int* lpr, int* nb) {
  const int nblk = K >> 5;
  *lpr = gcd_pow2_64(nblk);
  *nb = nblk / *lpr;
  return 0;
}

}  // namespace bw
