// bw_attn.hip - grouped-query decode attention over a paged KV cache, split along the context
// with an online-softmax merge (gfx950).
//
// Operation: for each new token i of sequence b at position p = seq_lens[b] + i and each query
// head h (KV head g = h / (Hq/Hkv)), o = softmax(q . K^T / sqrt(D)) V over positions 0..p. Keys
// and values are read through the page table: logical position j is slot j % 16 of physical
// page page_table[b][j / 16] (bw24 deep-dive page, section 6 item 2: logical positions map to
// fixed physical pages; section 5 stage 4: the t new tokens of a verify step are unrolled along
// the sequence and share one cache, with causal masking among them). Every new token reads the
// whole cache of its sequence (bw24 vs llama.cpp page, section 2.1).
//
// Split: workgroup (split s, KV head g, sequence b) covers logical pages [s*PPS, (s+1)*PPS) and
// all t * (Hq/Hkv) query rows that use KV head g, so each K/V page is read once per step for all
// heads of its group. Each of the 4 waves takes every 4th page (its K and V loaded together) and
// keeps a running (max, sum, acc) per query row; the waves merge in LDS and write one partial per
// split. A merge kernel combines the splits of each (row, KV group) in split order, so the result
// depends only on logical page order and contents: permuting the physical pool changes nothing,
// bit for bit.
//
// Lane layout per page (D = 128): scores use 8 tokens x 8 lanes per pass (each lane a 16-dim
// slice, 2 loads of 8 elements, 2 passes); values use 4 token groups x 16 lanes (each lane an
// 8-dim slice of 4 tokens). A load of 8 elements is 16 bytes for the 16-bit caches and 8 bytes for
// an FP8 E4M3 cache, which is widened to fp32 by the hardware conversion. Slots past the sequence end are masked by selection, so stale
// or NaN contents there never reach the result.
#include "bw_common.h"
#include "bw_internal.h"
#include "bw_lanes.h"
#include "bw_mfma.h"

#include <type_traits>

namespace bw {

template <int KVDT, int D, int QR>
__global__ __launch_bounds__(kBlock) void k_attn_split(AttnParams p) {
  constexpr int DL = D / 8;             // score dims per lane (8 lanes per token)
  constexpr int NV = D / 8;             // lanes per token row for values (8 dims each)
  constexpr int TG = kWave / NV;        // token groups for values
  constexpr int TPL = kPageTokens / TG; // tokens per lane for values
  constexpr bool QREG = (QR * DL <= 96);
  constexpr int NCH = DL / 8;           // 8-element chunks per lane per token for scores
  typedef typename KvT<KVDT>::E E;
  typedef typename KvT<KVDT>::C8 C8;

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int rep = p.H / p.G;
  const int base_pos = p.seq_lens[b];
  const int kv_len = base_pos + p.t;
  int n_pg = (kv_len + kPageTokens - 1) / kPageTokens;
  const int pg_cap = min(p.max_pages, p.max_splits * p.pages_per_split);
  if (n_pg > pg_cap) {
    if (threadIdx.x == 0 && s == 0) atomicOr(p.err, 1);
    n_pg = pg_cap;
  }
  const int pg0 = s * p.pages_per_split;
  if (pg0 >= n_pg) return;
  const int pg1 = min(n_pg, pg0 + p.pages_per_split);

  __shared__ float q_lds[QR * D];
  __shared__ float p_lds[4][QR][kPageTokens];
  __shared__ float m_lds[4][QR], l_lds[4][QR];
  __shared__ float acc_lds[4][QR * D];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sc_tok = lane >> 3, sc_c = lane & 7;     // scores: token within pass, dim slice
  const int v_c = lane % NV, v_tg = lane / NV;       // values: dim chunk, token group

  // this wave's first page id goes out before anything else
  int pg = pg0 + wave;
  int page = pg < pg1 ? p.page_table[(int64_t)b * p.max_pages + pg] : -1;

  // query rows: qr = ti * rep + r  ->  token ti, head g * rep + r
  for (int e = threadIdx.x; e < QR * D; e += kBlock) {
    const int qr = e / D, d = e - qr * D;
    const int ti = qr / rep, r = qr - ti * rep;
    q_lds[e] = p.q[((int64_t)(b * p.t + ti) * p.H + g * rep + r) * D + d] * p.scale;
  }
  __syncthreads();

  float qreg[QREG ? QR : 1][QREG ? DL : 1];
  if constexpr (QREG) {
#pragma unroll
    for (int qr = 0; qr < QR; ++qr)
#pragma unroll
      for (int e = 0; e < DL; ++e) qreg[qr][e] = q_lds[qr * D + sc_c * DL + e];
  }
  int qpos[QR];
#pragma unroll
  for (int qr = 0; qr < QR; ++qr) qpos[qr] = base_pos + qr / rep;

  float mrun[QR], lrun[QR], acc[QR][8];
#pragma unroll
  for (int qr = 0; qr < QR; ++qr) {
    mrun[qr] = -INFINITY;
    lrun[qr] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[qr][e] = 0.f;
  }

  for (; pg < pg1; pg += 4) {
    const bool valid = page >= 0 && page < p.n_pages;
    if (!valid && lane == 0) atomicOr(p.err, 1);
    // K (for the scores) and V (for the values) of this page, loaded together
    C8 kraw[2][NCH], vraw[TPL];
    if (valid) {
      const E* kbase = (const E*)p.pool + (int64_t)page * p.pool_page_stride + (int64_t)(g * 2) * kPageTokens * D;
      const E* vbase = kbase + kPageTokens * D;
#pragma unroll
      for (int pass = 0; pass < 2; ++pass)
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch)
          kraw[pass][ch] = *(const C8*)(kbase + (pass * 8 + sc_tok) * D + sc_c * DL + ch * 8);
#pragma unroll
      for (int u = 0; u < TPL; ++u) vraw[u] = *(const C8*)(vbase + (v_tg + u * TG) * D + v_c * 8);
    }
    // the next page's id
    const int pgn = pg + 4;
    const int page_n = pgn < pg1 ? p.page_table[(int64_t)b * p.max_pages + pgn] : -1;
    if (valid) {
      // ---- scores for the 16 tokens (2 passes of 8)
      float sc[2][QR];
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        const int j = pg * kPageTokens + pass * 8 + sc_tok;
        float kf[DL];
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) kv_unpack8<KVDT>(kraw[pass][ch], kf + ch * 8);
#pragma unroll
        for (int qr = 0; qr < QR; ++qr) {
          float dot = 0.f;
          if constexpr (QREG) {
#pragma unroll
            for (int e = 0; e < DL; ++e) dot = fmaf(qreg[qr][e], kf[e], dot);
          } else {
#pragma unroll
            for (int e = 0; e < DL; ++e) dot = fmaf(q_lds[qr * D + sc_c * DL + e], kf[e], dot);
          }
          dot += __shfl_xor(dot, 1);
          dot += __shfl_xor(dot, 2);
          dot += __shfl_xor(dot, 4);
          sc[pass][qr] = (j < kv_len && j <= qpos[qr]) ? dot : -INFINITY;
        }
      }
      // ---- online softmax update per query row
#pragma unroll
      for (int qr = 0; qr < QR; ++qr) {
        float pm = fmaxf(sc[0][qr], sc[1][qr]);
        pm = fmaxf(pm, __shfl_xor(pm, 8));
        pm = fmaxf(pm, __shfl_xor(pm, 16));
        pm = fmaxf(pm, __shfl_xor(pm, 32));
        const float mnew = fmaxf(mrun[qr], pm);
        float p0 = 0.f, p1 = 0.f, alpha = 1.f;
        if (mnew != -INFINITY) {
          p0 = __expf(sc[0][qr] - mnew);
          p1 = __expf(sc[1][qr] - mnew);
          alpha = __expf(mrun[qr] - mnew);
        }
        float ps = p0 + p1;
        ps += __shfl_xor(ps, 8);
        ps += __shfl_xor(ps, 16);
        ps += __shfl_xor(ps, 32);
        lrun[qr] = lrun[qr] * alpha + ps;
        mrun[qr] = mnew;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[qr][e] *= alpha;
        if (sc_c == 0) {
          p_lds[wave][qr][sc_tok] = p0;
          p_lds[wave][qr][8 + sc_tok] = p1;
        }
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // ---- values: lane covers 8 dims of TPL tokens
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        const int tok = v_tg + u * TG;
        const int j = pg * kPageTokens + tok;
        float vf[8];
        kv_unpack8<KVDT>(vraw[u], vf);
        const bool live = j < kv_len;
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[e] = live ? vf[e] : 0.f;
#pragma unroll
        for (int qr = 0; qr < QR; ++qr) {
          const float pw = p_lds[wave][qr][tok];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[qr][e] = fmaf(pw, vf[e], acc[qr][e]);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    page = page_n;
  }
  // ---- reduce the value partials over the token groups of the wave
#pragma unroll
  for (int qr = 0; qr < QR; ++qr)
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int o = NV; o < kWave; o <<= 1) acc[qr][e] += __shfl_xor(acc[qr][e], o);
  if (v_tg == 0) {
#pragma unroll
    for (int qr = 0; qr < QR; ++qr)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc_lds[wave][qr * D + v_c * 8 + e] = acc[qr][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int qr = 0; qr < QR; ++qr) {
      m_lds[wave][qr] = mrun[qr];
      l_lds[wave][qr] = lrun[qr];
    }
  }
  __syncthreads();
  // ---- merge the 4 waves and write this split's partial (acc, m, l)
  for (int e = threadIdx.x; e < QR * D; e += kBlock) {
    const int qr = e / D, d = e - qr * D;
    const float M = fmaxf(fmaxf(m_lds[0][qr], m_lds[1][qr]), fmaxf(m_lds[2][qr], m_lds[3][qr]));
    float a = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = __expf(m_lds[w][qr] - M);
        a = fmaf(acc_lds[w][e], f, a);
        l = fmaf(l_lds[w][qr], f, l);
      }
    }
    const int ti = qr / rep, r = qr - ti * rep;
    float* dst = p.part + (((int64_t)(b * p.t + ti) * p.H + g * rep + r) * p.max_splits + s) * (D + 2);
    dst[d] = a;
    if (d == 0) {
      dst[D] = M;
      dst[D + 1] = l;
    }
  }
}

// ---- matrix-core split attention (verify steps: QR query rows per KV head, up to 16) ----------
// The same split and partial format as k_attn_split, with both contractions on the matrix cores.
// Per page (16 tokens) a wave computes
//   scores^T [16 tokens][16 rows] = K [16][D] . Q^T   as D/32 steps of a 16x16x32 product, and
//   O [16 rows][D] += P [16][16 tokens] . V [16][D]    as D/16 steps of a 16x16x16 product.
// The first product's output layout (lane l: tokens 4(l/16)..+3 of row l%16) is the second one's
// A-operand layout, so P never moves between lanes. K rows load directly as A operands (16-byte
// loads, token l%16, dims 8(l/16)..+7 of each 32-dim chunk). V is staged in LDS and read back with
// tokens along K: B[token 4(l/16)+i][dim l%16]. Q and P are split into sums of cache-dtype parts,
// so each product term is exact in fp32 and only the summation order differs from the VALU
// kernel: Q in three bf16 parts (residual below 2^-26 of |q|; a score scales q by up to a few
// hundred) or two fp16 parts (2^-22), P in two parts (2^-17 for bf16). Rows past QR are padding.
constexpr int kVStride = 136;  // LDS row of a staged V page, in 16-bit elements (272 B: conflict-free reads)
constexpr int kMfmaMaxPps = 128;  // most pages of one split of the matrix-core kernel

// Grid (split, KV head x row tile, sequence): a workgroup takes 16 of the QR query rows of its KV
// head (a verify step has one tile; a prefill chunk of t tokens has ceil(QR / 16)), over the pages
// of its split that the tile's last position reaches.
template <int KVDT, int D>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void k_attn_split_mfma(AttnParams p, int QR) {
  // an FP8 cache is widened to bf16 on load (exact) and takes the bf16 products
  constexpr int MT = KVDT == 3 ? 2 : KVDT;
  using M = MfmaT<MT>;
  typedef typename M::e8 e8;
  typedef typename M::e4 e4;
  constexpr int NC = D / 32;  // 32-dim chunks (scores)
  constexpr int NV = D / 16;  // 16-dim chunks (values)

  const int n_tiles = (QR + 15) >> 4;
  const int s = blockIdx.x, g = blockIdx.y / n_tiles, tile = blockIdx.y - g * n_tiles, b = blockIdx.z;
  const int rep = p.H / p.G;
  const int base_pos = p.seq_lens[b];
  const int r_last = min(QR, 16 * tile + 16) - 1;   // last real row of the tile
  const int kv_len = base_pos + r_last / rep + 1;   // positions the tile's rows reach
  int n_pg = (kv_len + kPageTokens - 1) / kPageTokens;
  const int pg_cap = min(p.max_pages, p.max_splits * p.pages_per_split);
  if (n_pg > pg_cap) {
    if (threadIdx.x == 0 && s == 0) atomicOr(p.err, 1);
    n_pg = pg_cap;
  }
  const int pg0 = s * p.pages_per_split;
  if (pg0 >= n_pg) return;
  const int pg1 = min(n_pg, pg0 + p.pages_per_split);

  __shared__ __attribute__((aligned(16))) uint16_t v_lds[4][kPageTokens * kVStride];
  __shared__ float acc_lds[4][16 * D];
  __shared__ float m_lds[4][16], l_lds[4][16];
  __shared__ int pid_lds[kMfmaMaxPps];  // this split's page ids (read once; LDS reads do not wait for memory loads)

  // the wave index through readfirstlane: page ids and buffer descriptors derived from it are
  // then known to be uniform, so no load needs a per-lane loop
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15, grp = lane >> 4;  // column / row-block of the 16x16 tiles
  // query row 16 tile + c16 (padding rows past QR: zero query, no causal limit, never written)
  const int qr = 16 * tile + c16;
  const bool real = qr < QR;
  const int ti = real ? qr / rep : 0, hr = real ? qr - ti * rep : 0;
  const int qpos = real ? base_pos + ti : 0x7fffffff;
  constexpr int NQ = MT == 2 ? 3 : 2;  // parts of the query
  // head dims of the 8 K slots of lane group grp in 32-dim chunk c of the score product. A score
  // sums over all dims, so any order that K and Q share is the same sum: 16-bit caches take dims
  // 32 c + 8 grp ..+7 (one 16-byte load each); an FP8 cache takes 64 (c / 2) + 16 grp + 8 (c % 2)
  // ..+7, so that one 16-byte load brings a lane the dims of two chunks
  auto kdim = [&](int c) { return KVDT == 3 ? 64 * (c >> 1) + 16 * grp + 8 * (c & 1) : 32 * c + 8 * grp; };
  typedef typename std::remove_reference<decltype(e8{}[0])>::type el8;
  typedef typename std::remove_reference<decltype(e4{}[0])>::type el4;
  e8 qp[NQ][NC];
  {
    // unconditional 16-byte loads (a padding row reads row 0 and is zeroed), all issued first
    const float4* qsrc = (const float4*)(p.q + ((int64_t)(b * p.t + ti) * p.H + g * rep + hr) * D);
    float4 qv[NC][2];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h) qv[c][h] = qsrc[kdim(c) / 4 + h];
    const float qs = real ? p.scale : 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float4 v4 = qv[c][e >> 2];
        float x = ((e & 3) == 0 ? v4.x : (e & 3) == 1 ? v4.y : (e & 3) == 2 ? v4.z : v4.w) * qs;
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
          const uint16_t bits = part_bits<MT>(x);
          qp[k][c][e] = __builtin_bit_cast(el8, bits);
          x -= kv_to_f32<MT>(bits);
        }
      }
  }
  float mrun = -INFINITY, lrun = 0.f;  // of row c16
  f32x4 o[NV];
#pragma unroll
  for (int c = 0; c < NV; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint16_t* vl = v_lds[wave];

  // K and V of one page of this KV head as buffer loads on that page (an invalid page id reads
  // zeros from past the buffer), issued one page ahead of the page being computed
  {
    const int32_t* ptab = p.page_table + (int64_t)b * p.max_pages;
    if ((int)threadIdx.x < pg1 - pg0) pid_lds[threadIdx.x] = ptab[pg0 + threadIdx.x];
    __syncthreads();
  }
  // An invalid page id gives a descriptor of zero bytes, so every load through it reads zeros: the
  // offsets need no selection, which the compiler would turn into a branch around each load
  // (and then wait for all loads in flight at the join).
  auto load_kv = [&](int page, u32x4 (&kr)[NC], u32x4 (&vr)[D / 32]) {
    constexpr int ES = KvT<KVDT>::ES;
    const bool ok = page >= 0 && page < p.n_pages;
    const typename KvT<KVDT>::E* base =
        (const typename KvT<KVDT>::E*)p.pool +
        (ok ? (int64_t)page * p.pool_page_stride + (int64_t)(g * 2) * kPageTokens * D : 0);
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, ok ? 2 * kPageTokens * D * ES : 0, 0x00020000);
    if constexpr (KVDT == 3) {
      // 16-byte loads of 16 FP8 elements, widened to bf16 when the page is used: K in kr[0 .. NC/2)
      // (kr[u] holds dims 64 u + 16 grp ..+15 of token c16: chunks 2u and 2u + 1), V in
      // vr[0 .. D/64) (16-byte piece k = lane + 64 u: token k / (D/16), dims 16 (k % (D/16)) ..+15)
#pragma unroll
      for (int u = 0; u < NC / 2; ++u) kr[u] = __builtin_amdgcn_raw_buffer_load_b128(r, c16 * D + 64 * u + 16 * grp, 0, 0);
#pragma unroll
      for (int u = 0; u < D / 64; ++u) {
        const int k = lane + 64 * u;
        vr[u] = __builtin_amdgcn_raw_buffer_load_b128(r, kPageTokens * D + (k / (D / 16)) * D + 16 * (k % (D / 16)), 0, 0);
      }
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        kr[c] = __builtin_amdgcn_raw_buffer_load_b128(r, (c16 * D + 32 * c + 8 * grp) * 2, 0, 0);
#pragma unroll
      for (int q4 = 0; q4 < D / 32; ++q4) {  // 16-byte chunk k = lane + 64 q4: token k / (D/8), dims 8 (k % (D/8))
        const int k = lane + 64 * q4;
        vr[q4] = __builtin_amdgcn_raw_buffer_load_b128(r, (kPageTokens * D + (k / (D / 8)) * D + 8 * (k % (D / 8))) * 2, 0, 0);
      }
    }
  };
  // one page: scores, online softmax, values (kr, vr hold its K and V)
  auto compute = [&](int pg, int page, const u32x4 (&kin)[NC], const u32x4 (&vin)[D / 32]) {
    if (page < 0 || page >= p.n_pages) {
      if (lane == 0) atomicOr(p.err, 1);
      return;
    }
    u32x4 kraw[NC];  // bf16 / fp16 operands
    const u32x4 z = {0u, 0u, 0u, 0u};
    // stage V (this wave's buffer; the LDS operations of one wave run in order); slots past the
    // sequence end are written as zeros, so stale or NaN contents never meet a zero probability
    if constexpr (KVDT == 3) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        kraw[c] = fp8x8_to_bf16x8((c & 1) ? u32x2{kin[c >> 1][2], kin[c >> 1][3]} : u32x2{kin[c >> 1][0], kin[c >> 1][1]});
#pragma unroll
      for (int u = 0; u < D / 64; ++u) {
        const int k = lane + 64 * u;
        const int tk = k / (D / 16);
        const bool live = pg * kPageTokens + tk < kv_len;
        uint16_t* dst = vl + tk * kVStride + 16 * (k % (D / 16));
        *(u32x4*)dst = live ? fp8x8_to_bf16x8(u32x2{vin[u][0], vin[u][1]}) : z;
        *(u32x4*)(dst + 8) = live ? fp8x8_to_bf16x8(u32x2{vin[u][2], vin[u][3]}) : z;
      }
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c) kraw[c] = kin[c];
#pragma unroll
      for (int q4 = 0; q4 < D / 32; ++q4) {
        const int k = lane + 64 * q4;
        const int tk = k / (D / 8);
        *(u32x4*)(vl + tk * kVStride + 8 * (k % (D / 8))) = pg * kPageTokens + tk < kv_len ? vin[q4] : z;
      }
    }
    // scores^T: lane holds tokens 4 grp + i of row c16
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const e8 kop = __builtin_bit_cast(e8, kraw[c]);
#pragma unroll
      for (int k = 0; k < NQ; ++k) sc = M::mm32(kop, qp[k][c], sc);
    }
    float sv[4];
    float pm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = pg * kPageTokens + 4 * grp + i;
      sv[i] = (j < kv_len && j <= qpos) ? sc[i] : -INFINITY;
      pm = fmaxf(pm, sv[i]);
    }
    pm = max_xor32(max_xor16(pm));
    const float mnew = fmaxf(mrun, pm);
    float pv[4], alpha = 1.f, psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = mnew == -INFINITY ? 0.f : __expf(sv[i] - mnew);
      psum += pv[i];
    }
    if (mnew != -INFINITY) alpha = __expf(mrun - mnew);
    psum = sum_xor32(sum_xor16(psum));
    lrun = lrun * alpha + psum;
    mrun = mnew;
    // P as the A operand (row c16, tokens 4 grp + i), hi + lo
    e4 ph, pl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint16_t hb = part_bits<MT>(pv[i]);
      const uint16_t lb = part_bits<MT>(pv[i] - kv_to_f32<MT>(hb));
      ph[i] = __builtin_bit_cast(el4, hb);
      pl[i] = __builtin_bit_cast(el4, lb);
    }
    // rescale the accumulators (lane holds rows 4 grp + i, whose factors sit in lanes 4 grp + i),
    // only when some row's running max moved (rare after the first pages)
    if (__ballot(alpha != 1.f) != 0) {
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * grp + i);
#pragma unroll
      for (int c = 0; c < NV; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[c][i] *= al[i];
    }
    // values: B [token 4 grp + i][dim 16 c + c16] from the staged page by one transpose read per
    // 16-dim chunk: within each 16-lane group, lanes 4r..4r+3 read row r (token 4 grp + r, 16
    // dims) and every lane receives its column, i.e. its four tokens of dim 16 c + c16
    typedef short s4 __attribute__((ext_vector_type(4)));
    const uint16_t* vrow = vl + (4 * grp + (c16 >> 2)) * kVStride + 4 * (c16 & 3);
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      const s4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(vrow + 16 * c));
      const e4 vb = __builtin_bit_cast(e4, t);
      o[c] = M::mm16(ph, vb, o[c]);
      o[c] = M::mm16(pl, vb, o[c]);
    }
  };
  // two register sets alternate: the next page's loads are in flight while a page is computed,
  // and no register moves between them (a move would wait for the loads)
  int pg = pg0 + wave;
  int page = pg < pg1 ? __builtin_amdgcn_readfirstlane(pid_lds[pg - pg0]) : -1;
  u32x4 ka[NC], va[D / 32], kb[NC], vb2[D / 32];
  load_kv(page, ka, va);
  while (pg < pg1) {
    int pgn = pg + 4;
    int page_n = pgn < pg1 ? __builtin_amdgcn_readfirstlane(pid_lds[pgn - pg0]) : -1;
    load_kv(page_n, kb, vb2);
    compute(pg, page, ka, va);
    pg = pgn;
    page = page_n;
    if (pg >= pg1) break;
    pgn = pg + 4;
    page_n = pgn < pg1 ? __builtin_amdgcn_readfirstlane(pid_lds[pgn - pg0]) : -1;
    load_kv(page_n, ka, va);
    compute(pg, page, kb, vb2);
    pg = pgn;
    page = page_n;
  }
  // ---- merge the 4 waves (rows 4 grp + i, dims 16 c + c16) and write this split's partials
#pragma unroll
  for (int c = 0; c < NV; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc_lds[wave][(4 * grp + i) * D + 16 * c + c16] = o[c][i];
  if (grp == 0) {
    m_lds[wave][c16] = mrun;
    l_lds[wave][c16] = lrun;
  }
  __syncthreads();
  const int rows = min(16, QR - 16 * tile);
  for (int e = threadIdx.x; e < rows * D; e += kBlock) {
    const int rl = e / D, d = e - rl * D, r = 16 * tile + rl;
    const float Mx = fmaxf(fmaxf(m_lds[0][rl], m_lds[1][rl]), fmaxf(m_lds[2][rl], m_lds[3][rl]));
    float a = 0.f, l = 0.f;
    if (Mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = __expf(m_lds[w][rl] - Mx);
        a = fmaf(acc_lds[w][rl * D + d], f, a);
        l = fmaf(l_lds[w][rl], f, l);
      }
    }
    const int rt = r / rep, rh = r - rt * rep;
    float* dst = p.part + (((int64_t)(b * p.t + rt) * p.H + g * rep + rh) * p.max_splits + s) * (D + 2);
    dst[d] = a;
    if (d == 0) {
      dst[D] = Mx;
      dst[D + 1] = l;
    }
  }
}

// Merge of the split partials of one (row, query head): o = sum_s acc_s exp(m_s - M) / sum_s l_s
// exp(m_s - M), M = max_s m_s, in split order. The (m, l) of every split are loaded in parallel
// (one split per thread) and the per-split factors staged in LDS, so only the value sums loop.
template <int D>
__global__ __launch_bounds__(kBlock) void k_attn_merge(AttnParams p) {
  __shared__ float fac[1024];
  __shared__ float red[16];
  const int h = blockIdx.x, row = blockIdx.y;
  const int b = row / p.t;
  // the splits this row's own position reaches (later splits of a longer step were written fully
  // masked for it, or, for a prefill tile that ends earlier, not at all)
  const int kv_len = p.seq_lens[b] + (row - b * p.t) + 1;
  const int n_pg = min((kv_len + kPageTokens - 1) / kPageTokens, min(p.max_pages, p.max_splits * p.pages_per_split));
  const int n_split = min((n_pg + p.pages_per_split - 1) / p.pages_per_split, 1024);
  {
    const float* part = p.part + ((int64_t)row * p.H + h) * p.max_splits * (D + 2);
    // 1. M = max over splits (parallel loads)
    float mloc = -INFINITY;
    for (int sp = threadIdx.x; sp < n_split; sp += kBlock) mloc = fmaxf(mloc, part[sp * (D + 2) + D]);
    mloc = wave_max(mloc);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mloc;
    __syncthreads();
    const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    // 2. factors and the denominator
    float lloc = 0.f;
    for (int sp = threadIdx.x; sp < n_split; sp += kBlock) {
      const float f = M == -INFINITY ? 0.f : __expf(part[sp * (D + 2) + D] - M);
      fac[sp] = f;
      lloc = fmaf(part[sp * (D + 2) + D + 1], f, lloc);
    }
    __syncthreads();
    // denominator: fixed per-thread split sets and a fixed reduction tree (deterministic)
    const float L = block_sum(lloc, red + 4);
    // 3. values: thread (d, quarter) sums a quarter of the splits, quarters combined in order
    const int d = threadIdx.x % D, qq = threadIdx.x / D;  // kBlock / D quarters
    constexpr int NQ = kBlock / D;
    // loads in batches of 8 (one wait per batch), sums in the same split order
    float a = 0.f;
    int sp = qq;
    for (; sp + 7 * NQ < n_split; sp += 8 * NQ) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(sp + u * NQ) * (D + 2) + d];
#pragma unroll
      for (int u = 0; u < 8; ++u) a = fmaf(v[u], fac[sp + u * NQ], a);
    }
    for (; sp < n_split; sp += NQ) a = fmaf(part[sp * (D + 2) + d], fac[sp], a);
    __shared__ float asum[kBlock];
    asum[threadIdx.x] = a;
    __syncthreads();
    if (qq == 0) {
      float t = 0.f;
      for (int k = 0; k < NQ; ++k) t += asum[k * D + d];
      p.out[((int64_t)row * p.H + h) * D + d] = L > 0.f ? t / L : 0.f;
    }
  }
}

template <int KVDT, int D, int QR>
static int launch_split(const AttnParams& p, int batch, hipStream_t s) {
  hipLaunchKernelGGL((k_attn_split<KVDT, D, QR>), dim3(p.max_splits, p.G, batch), dim3(kBlock), 0, s, p);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int KVDT, int D>
static int dispatch_qr(const AttnParams& p, int batch, hipStream_t s) {
  const int qr = p.t * (p.H / p.G);
  switch (qr) {
    case 1: return launch_split<KVDT, D, 1>(p, batch, s);
    case 2: return launch_split<KVDT, D, 2>(p, batch, s);
    case 4: return launch_split<KVDT, D, 4>(p, batch, s);
    case 5: return launch_split<KVDT, D, 5>(p, batch, s);
    case 8: return launch_split<KVDT, D, 8>(p, batch, s);
    case 16: return launch_split<KVDT, D, 16>(p, batch, s);
    default: return -2;
  }
}

// pages per split of the matrix-core kernel: 8 pages per wave keep the partials (one per split,
// row and head) small next to the KV read of verify steps over long contexts
// Pages per split: long splits amortise a workgroup's fixed work (the query split, the page ids,
// the wave merge, the partials) and leave fewer partials to merge, so the longest split that
// still gives about four workgroups per CU slot (2048 at two per CU) is taken.
static int mfma_pages_per_split(const AttnParams& p, int batch, int tiles) {
  for (int pps = kMfmaMaxPps; pps > 32; pps /= 2) {
    const int64_t wgs = (int64_t)batch * p.G * tiles * ((p.max_pages + pps - 1) / pps);
    if (wgs >= 2048) return pps;
  }
  return 32;
}

template <int D>
static int launch_mfma(const AttnParams& p, int kv_dtype, int batch, int qr, hipStream_t s) {
  AttnParams m = p;
  const int tiles = (qr + 15) / 16;
  m.pages_per_split = mfma_pages_per_split(p, batch, tiles);
  m.max_splits = min((p.max_pages + m.pages_per_split - 1) / m.pages_per_split, p.max_splits);
  if ((int64_t)m.G * tiles > 65535) return -2;
  if (kv_dtype == 1)
    hipLaunchKernelGGL((k_attn_split_mfma<1, D>), dim3(m.max_splits, m.G * tiles, batch), dim3(kBlock), 0, s, m, qr);
  else if (kv_dtype == 3)
    hipLaunchKernelGGL((k_attn_split_mfma<3, D>), dim3(m.max_splits, m.G * tiles, batch), dim3(kBlock), 0, s, m, qr);
  else
    hipLaunchKernelGGL((k_attn_split_mfma<2, D>), dim3(m.max_splits, m.G * tiles, batch), dim3(kBlock), 0, s, m, qr);
  hipLaunchKernelGGL(k_attn_merge<D>, dim3(m.H, batch * m.t), dim3(kBlock), 0, s, m);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_attention(const AttnParams& p, int kv_dtype, int batch, hipStream_t s) {
  int rc;
  const int qr = p.t * (p.H / p.G);
  if (p.mfma && qr >= 8) {  // verify steps and prefill chunks: both products on the matrix cores
    if (p.D == 128) return launch_mfma<128>(p, kv_dtype, batch, qr, s);
    if (p.D == 64) return launch_mfma<64>(p, kv_dtype, batch, qr, s);
  }
  if (p.D == 128)
    rc = kv_dtype == 1 ? dispatch_qr<1, 128>(p, batch, s)
                       : (kv_dtype == 3 ? dispatch_qr<3, 128>(p, batch, s) : dispatch_qr<2, 128>(p, batch, s));
  else if (p.D == 64)
    rc = kv_dtype == 1 ? dispatch_qr<1, 64>(p, batch, s)
                       : (kv_dtype == 3 ? dispatch_qr<3, 64>(p, batch, s) : dispatch_qr<2, 64>(p, batch, s));
  else
    return -2;
  if (rc) return rc;
  if (p.D == 128) hipLaunchKernelGGL(k_attn_merge<128>, dim3(p.H, batch * p.t), dim3(kBlock), 0, s, p);
  else hipLaunchKernelGGL(k_attn_merge<64>, dim3(p.H, batch * p.t), dim3(kBlock), 0, s, p);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace bw
