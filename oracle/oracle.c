/*
 * oracle.c - plain, slow fp64 CPU oracle of the int4 paged-KV decode step.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call this file:
 * only the tests, the smoke check and the benchmark's CPU-baseline leg use it. It shares no
 * code with the HIP library; the only common piece is the seeded input generator
 * (synth/bw_synth.c), which holds none of the decode step's arithmetic.
 *
 * Every quantity is computed in fp64 with plain loops in the order the definition states. The
 * only rounding the oracle applies is the one the method defines: new keys and values are
 * rounded to the cache dtype (bf16, fp16 or FP8 E4M3, round-to-nearest-even) before they are
 * stored.
 *
 * Sources. The pages ("Deep dive: bw24, a Rust + hand-written CUDA engine for Blackwell RTX 50",
 * 10100.com) describe a decode engine whose KV cache maps logical sequence positions to fixed
 * physical pages (section 6, item 2, "paged cache"), whose verify kernel unrolls the K draft
 * tokens along the sequence dimension over one shared KV cache (section 5, stage 4), whose
 * output must equal token-by-token argmax decoding (section 1 and the comparison table of
 * section 7), and which handles MoE routing (closing summary). The first page ("Rust+CUDA LLM
 * inference: how bw24 beats llama.cpp", devpress.csdn.net) states that each new token reads
 * the whole KV cache (section 2.1) and that linear layers fuse with their activation (section
 * 2.2). The workload fixes the rest: int4 blocks of 32 weights with one fp16 scale each and
 * w = scale * (q - 8); RMSNorm with eps 1e-6; RoPE with base 1e6; SwiGLU FFN; GQA; softmax
 * top-k routing with renormalised gates plus an ungated shared expert; greedy argmax.
 *
 * Readings where the sources are silent (each is listed in the design notes): pre-norm decoder
 * without biases; x * rsqrt(mean(x^2) + eps) * gamma; rotate-half RoPE on pairs (i, i + D/2)
 * with angle pos * base^(-2i/D), applied to q and k before k is cached; attention scale
 * 1/sqrt(D); KV head of query head h is h / (Hq/Hkv); untied lm_head; top-k on router logits
 * with ties to the lower expert index; argmax ties to the lowest index.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "../synth/bw_synth.h"

#define OR_KV_F16 1
#define OR_KV_BF16 2
#define OR_KV_FP8 3 /* OCP FP8 E4M3 */

/* ------------------------------------------------------------------------------------------ */
/* number formats                                                                              */
/* ------------------------------------------------------------------------------------------ */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits; exponent 0 = subnormal. */
double or_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1F;
  int f = h & 0x3FF;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25);
  return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of binary32 (1 sign, 8 exponent (bias 127), 7 fraction bits). */
double or_bf16_to_f64(uint16_t b) {
  int sign = (b >> 15) & 1;
  int e = (b >> 7) & 0xFF;
  int f = b & 0x7F;
  double v;
  if (e == 0)
    v = ldexp((double)f, -133);
  else if (e == 255)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(128 + f), e - 134);
  return sign ? -v : v;
}

/* Round v to a binary format with p significand bits, minimum normal exponent emin, maximum
 * exponent emax and exponent bias `bias`, to nearest with ties to even, and return its bit
 * pattern (1 sign bit, then the exponent field, then p-1 fraction bits). */
static uint16_t or_round_bits(double v, int p, int emin, int emax, int bias, int ebits) {
  uint16_t sign = 0;
  if (signbit(v)) {
    sign = (uint16_t)(1u << (p - 1 + ebits));
    v = -v;
  }
  uint16_t inf = (uint16_t)(((1u << ebits) - 1u) << (p - 1));
  if (isnan(v)) return (uint16_t)(sign | inf | (1u << (p - 2)));
  if (isinf(v)) return (uint16_t)(sign | inf);
  if (v == 0.0) return sign;
  int e2;
  frexp(v, &e2);
  int E = e2 - 1;                 /* v in [2^E, 2^(E+1)) */
  if (E < emin) E = emin;         /* subnormal range shares the quantum of the smallest binade */
  double units = ldexp(v, -(E - p + 1));
  double r = nearbyint(units);    /* default rounding mode: to nearest, ties to even */
  double rv = ldexp(r, E - p + 1);
  if (rv >= ldexp(1.0, emax + 1)) return (uint16_t)(sign | inf);
  if (rv == 0.0) return sign; /* underflow to a signed zero */
  int e3;
  frexp(rv, &e3);
  int Er = e3 - 1;
  if (Er < emin) {
    /* subnormal: exponent field 0, fraction = rv / 2^(emin - p + 1) */
    uint32_t frac = (uint32_t)ldexp(rv, -(emin - p + 1));
    return (uint16_t)(sign | frac);
  }
  uint32_t m = (uint32_t)ldexp(rv, -(Er - p + 1)); /* in [2^(p-1), 2^p) */
  uint32_t field = (uint32_t)(Er + bias);
  return (uint16_t)(sign | (field << (p - 1)) | (m - (1u << (p - 1))));
}

uint16_t or_f64_to_f16(double v) { return or_round_bits(v, 11, -14, 15, 15, 5); }
uint16_t or_f64_to_bf16(double v) { return or_round_bits(v, 8, -126, 127, 127, 8); }

/* OCP FP8 E4M3 (the "E4M3FN" of the OCP 8-bit floating point specification): 1 sign, 4 exponent
 * bits (bias 7), 3 fraction bits; exponent field 0 is subnormal (f * 2^-9); there is no
 * infinity, and only exponent field 15 with fraction 7 is NaN, so the largest finite value is
 * 1.75 * 2^8 = 448. */
double or_fp8_to_f64(uint8_t b) {
  int sign = (b >> 7) & 1;
  int e = (b >> 3) & 0xF;
  int f = b & 7;
  double v;
  if (e == 15 && f == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)f, -9);
  else
    v = ldexp((double)(8 + f), e - 10);
  return sign ? -v : v;
}

/* Round to E4M3, to nearest with ties to even, saturating: a magnitude whose rounding would
 * exceed 448 (that is, |v| >= 464, the midpoint to the next binade step) becomes 448, infinities
 * included. NaN becomes the NaN pattern. (The saturating reading of an FP8 cache: a stored key
 * or value is always finite.) */
uint8_t or_f64_to_fp8(double v) {
  if (isnan(v)) return 0x7F;
  uint8_t sign = signbit(v) ? 0x80 : 0;
  double a = fabs(v);
  if (a >= 464.0) return (uint8_t)(sign | 0x7E); /* 448 */
  /* below 464 the IEEE-style rounding of p = 4 significant bits, emin = -6, never reaches the
   * exponent field 15 with fraction 7 */
  return (uint8_t)(sign | or_round_bits(a, 4, -6, 8, 7, 4));
}

static double or_kv_round(double v, int dtype) {
  if (dtype == OR_KV_FP8) return or_fp8_to_f64(or_f64_to_fp8(v));
  return dtype == OR_KV_F16 ? or_f16_to_f64(or_f64_to_f16(v)) : or_bf16_to_f64(or_f64_to_bf16(v));
}

/* ------------------------------------------------------------------------------------------ */
/* int4 blocks: 32 weights, one fp16 scale, w = scale * (q - 8)                                */
/* ------------------------------------------------------------------------------------------ */

/* code q of element k of a row in the canonical layout: block b = k/32 occupies bytes
 * 16b..16b+15 of the row; byte i of a block holds element i (low nibble) and element i+16
 * (high nibble). */
int or_code(const uint8_t* row_codes, int64_t k) {
  int64_t b = k / 32;
  int i = (int)(k % 32);
  uint8_t byte = row_codes[16 * b + (i % 16)];
  return i < 16 ? (byte & 0xF) : (byte >> 4);
}

double or_weight(const uint8_t* codes, const uint16_t* scales, int64_t K, int64_t n, int64_t k) {
  double s = or_f16_to_f64(scales[n * (K / 32) + k / 32]);
  return s * (double)(or_code(codes + n * (K / 2), k) - 8);
}

void or_dequant(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K, double* W) {
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) W[n * K + k] = or_weight(codes, scales, K, n, k);
}

/* Quantise w[n][k] with given per-block scales: q = clamp(round_half_even(w / s) + 8, 0, 15),
 * packed into the canonical layout. A zero scale gives q = 8. */
void or_quantize(const double* W, const uint16_t* scales, int64_t N, int64_t K, uint8_t* codes) {
  memset(codes, 0, (size_t)(N * K / 2));
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      double s = or_f16_to_f64(scales[n * (K / 32) + k / 32]);
      double q = s != 0.0 ? nearbyint(W[n * K + k] / s) + 8.0 : 8.0;
      if (q < 0) q = 0;
      if (q > 15) q = 15;
      int64_t b = k / 32;
      int i = (int)(k % 32);
      uint8_t* byte = codes + n * (K / 2) + 16 * b + (i % 16);
      *byte |= (uint8_t)((int)q << (i < 16 ? 0 : 4));
    }
}

/* y[n] = sum_k W[n][k] x[k], k ascending, W[n][k] formed exactly in fp64. The block scales of
 * a row are decoded once per row (the same values the per-weight formula uses). */
void or_gemv(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K, const double* x,
             double* y) {
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(K / 32));
#pragma omp for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
      const uint8_t* rc = codes + n * (K / 2);
      const uint16_t* rs = scales + n * (K / 32);
      for (int64_t b = 0; b < K / 32; ++b) s[b] = or_f16_to_f64(rs[b]);
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double w = s[k / 32] * (double)(or_code(rc, k) - 8);
        acc += w * x[k];
      }
      y[n] = acc;
    }
    free(s);
  }
}

/* dense fp16 matrix [N][K] times x */
void or_gemv_f16(const uint16_t* W, int64_t N, int64_t K, const double* x, double* y) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) acc += or_f16_to_f64(W[n * K + k]) * x[k];
    y[n] = acc;
  }
}

/* ------------------------------------------------------------------------------------------ */
/* MXFP4 blocks: 32 E2M1 elements sharing one E8M0 scale                                       */
/* ------------------------------------------------------------------------------------------ */

/* The pages' engine keeps weights in a native 4-bit floating-point format beside FP16/BF16
 * ("Deep dive: bw24 ...", section 1, quantisation formats; the performance-strategy row of the
 * section 7 table). That format is NVIDIA's; the 4-bit float that CDNA4's matrix cores take is
 * the OCP Microscaling (MX) MXFP4 format, which is what this section defines: blocks of 32 E2M1
 * elements along K with one E8M0 scale each, w = scale * element.
 *
 * Canonical layout of an MXFP4 matrix [N][K] (K a multiple of 32):
 *   codes : N * K/2 bytes; row n occupies K/2 bytes; byte i of a row holds element 2i in bits
 *           0-3 and element 2i+1 in bits 4-7.
 *   scales: N * K/32 bytes, one E8M0 byte per block, row-major. */

/* E2M1: bit 3 sign, bits 2-1 exponent (bias 1), bit 0 fraction; exponent 0 is subnormal
 * (f * 0.5). No infinity or NaN: the eight magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double or_e2m1_to_f64(int c) {
  int sign = (c >> 3) & 1;
  int e = (c >> 1) & 3;
  int f = c & 1;
  double v = e == 0 ? 0.5 * (double)f : ldexp(1.0 + 0.5 * (double)f, e - 1);
  return sign ? -v : v;
}

/* E8M0: an unsigned exponent, 2^(e - 127); the byte 255 is NaN. */
double or_e8m0_to_f64(uint8_t e) { return e == 255 ? NAN : ldexp(1.0, (int)e - 127); }

/* element k of row n */
double or_mx_weight(const uint8_t* codes, const uint8_t* scales, int64_t K, int64_t n, int64_t k) {
  uint8_t byte = codes[n * (K / 2) + k / 2];
  int c = (k % 2) ? (byte >> 4) : (byte & 0xF);
  return or_e8m0_to_f64(scales[n * (K / 32) + k / 32]) * or_e2m1_to_f64(c);
}

void or_mx_dequant(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K, double* W) {
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) W[n * K + k] = or_mx_weight(codes, scales, K, n, k);
}

/* Y[m][n] = sum_k X[m][k] W[n][k] for M input rows (the GEMV is M = 1), k ascending, every
 * weight formed exactly in fp64. */
void or_mx_matmul(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K,
                  const double* X, int64_t M, double* Y) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t m = 0; m < M; ++m) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += or_mx_weight(codes, scales, K, n, k) * X[m * K + k];
      Y[m * N + n] = acc;
    }
}

/* ------------------------------------------------------------------------------------------ */
/* elementwise pieces                                                                          */
/* ------------------------------------------------------------------------------------------ */

void or_rmsnorm(const double* x, const uint16_t* gamma, int64_t n, double eps, double* out) {
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) ss += x[i] * x[i];
  double r = 1.0 / sqrt(ss / (double)n + eps);
  for (int64_t i = 0; i < n; ++i) out[i] = x[i] * r * or_f16_to_f64(gamma[i]);
}

/* rotate pairs (i, i + D/2) of one head by pos * base^(-2i/D) */
void or_rope(double* v, int D, int64_t pos, double base) {
  int half = D / 2;
  for (int i = 0; i < half; ++i) {
    double theta = (double)pos * pow(base, -2.0 * (double)i / (double)D);
    double c = cos(theta), s = sin(theta);
    double a = v[i], b = v[i + half];
    v[i] = a * c - b * s;
    v[i + half] = a * s + b * c;
  }
}

double or_silu(double z) { return z / (1.0 + exp(-z)); }

/* softmax of n logits (max subtracted first) */
void or_softmax(const double* s, int64_t n, double* p) {
  double m = -INFINITY;
  for (int64_t j = 0; j < n; ++j)
    if (s[j] > m) m = s[j];
  double z = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    p[j] = exp(s[j] - m);
    z += p[j];
  }
  for (int64_t j = 0; j < n; ++j) p[j] /= z;
}

/* index of the largest value, lowest index on ties */
int64_t or_argmax(const double* v, int64_t n) {
  int64_t best = 0;
  for (int64_t i = 1; i < n; ++i)
    if (v[i] > v[best]) best = i;
  return best;
}

/* top-k indices by value, descending; ties go to the lower index */
void or_topk(const double* v, int64_t n, int k, int32_t* idx) {
  unsigned char* taken = (unsigned char*)calloc((size_t)n, 1);
  for (int r = 0; r < k; ++r) {
    int64_t best = -1;
    for (int64_t i = 0; i < n; ++i) {
      if (taken[i]) continue;
      if (best < 0 || v[i] > v[best]) best = i;
    }
    idx[r] = (int32_t)best;
    taken[best] = 1;
  }
  free(taken);
}

/* Naive attention of one query over n keys: s_j = q.k_j / sqrt(D), p = softmax(s),
 * out = sum_j p_j v_j. K and V are [n][D]; probs (optional) receives p. */
void or_attention(const double* q, const double* K, const double* V, int64_t n, int D, double* out,
                  double* probs) {
  double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  double* p = probs ? probs : (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  double scale = 1.0 / sqrt((double)D);
  for (int64_t j = 0; j < n; ++j) {
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += q[d] * K[j * D + d];
    s[j] = dot * scale;
  }
  or_softmax(s, n, p);
  for (int d = 0; d < D; ++d) {
    double acc = 0.0;
    for (int64_t j = 0; j < n; ++j) acc += p[j] * V[j * D + d];
    out[d] = acc;
  }
  free(s);
  if (!probs) free(p);
}

/* The same attention with K/V read through a page table from a physical page pool.
 * pool holds pages of `page_tokens` slots; slot layout [page][slot][D] for K and for V
 * (two separate pools). Logical position j lives in page page_table[j / page_tokens],
 * slot j % page_tokens. Values are fp64. */
void or_attention_paged(const double* q, const double* Kpool, const double* Vpool,
                        const int32_t* page_table, int page_tokens, int64_t n, int D, double* out) {
  double* K = (double*)malloc(sizeof(double) * (size_t)(n * D > 0 ? n * D : 1));
  double* V = (double*)malloc(sizeof(double) * (size_t)(n * D > 0 ? n * D : 1));
  for (int64_t j = 0; j < n; ++j) {
    int64_t page = page_table[j / page_tokens];
    int64_t slot = j % page_tokens;
    for (int d = 0; d < D; ++d) {
      K[j * D + d] = Kpool[(page * page_tokens + slot) * D + d];
      V[j * D + d] = Vpool[(page * page_tokens + slot) * D + d];
    }
  }
  or_attention(q, K, V, n, D, out, NULL);
  free(K);
  free(V);
}

/* ------------------------------------------------------------------------------------------ */
/* model                                                                                       */
/* ------------------------------------------------------------------------------------------ */

typedef struct {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab;
  double rms_eps, rope_base;
  int32_t n_experts, top_k, expert_ffn, n_shared, shared_ffn;
  int32_t kv_dtype; /* OR_KV_F16, OR_KV_BF16 or OR_KV_FP8 */
} or_config;

typedef struct {
  uint8_t* codes;
  uint16_t* scales;
  int64_t N, K;
} or_mat;

typedef struct {
  or_config c;
  uint64_t seed;
  uint16_t** attn_norm;
  uint16_t** ffn_norm;
  or_mat* qkv;
  or_mat* o;
  or_mat* gate; /* dense: [L]; MoE: [L * n_experts] */
  or_mat* up;
  or_mat* down;
  or_mat* sgate; /* shared experts [L * n_shared] */
  or_mat* sup;
  or_mat* sdown;
  uint16_t** router; /* [L] -> [n_experts][d] */
  uint16_t* final_norm;
  or_mat lm_head;
} or_model;

static void or_mat_make(or_mat* m, uint64_t seed, uint32_t kind, uint32_t layer, uint32_t expert,
                        int64_t N, int64_t K) {
  m->N = N;
  m->K = K;
  m->codes = (uint8_t*)malloc((size_t)(N * K / 2));
  m->scales = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(N * K / 32));
  /* generate in row chunks in parallel (the generator is counter-based) */
  int64_t chunk = 256;
#pragma omp parallel for schedule(dynamic)
  for (int64_t r0 = 0; r0 < N; r0 += chunk) {
    int64_t nr = (r0 + chunk <= N) ? chunk : N - r0;
    bws_int4_matrix(seed, kind, layer, expert, N, K, r0, nr, m->codes + r0 * (K / 2),
                    m->scales + r0 * (K / 32));
  }
}

static void or_mat_free(or_mat* m) {
  free(m->codes);
  free(m->scales);
}

static int or_is_moe(const or_config* c) { return c->n_experts > 0; }

or_model* or_model_create(const or_config* cfg, uint64_t seed) {
  or_model* m = (or_model*)calloc(1, sizeof(or_model));
  m->c = *cfg;
  m->seed = seed;
  const or_config* c = &m->c;
  int L = c->n_layers, d = c->d_model;
  int64_t nqkv = (int64_t)(c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim;
  int64_t nattn = (int64_t)c->n_q_heads * c->head_dim;
  m->attn_norm = (uint16_t**)calloc((size_t)L, sizeof(uint16_t*));
  m->ffn_norm = (uint16_t**)calloc((size_t)L, sizeof(uint16_t*));
  m->qkv = (or_mat*)calloc((size_t)L, sizeof(or_mat));
  m->o = (or_mat*)calloc((size_t)L, sizeof(or_mat));
  for (int l = 0; l < L; ++l) {
    m->attn_norm[l] = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)d);
    m->ffn_norm[l] = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)d);
    bws_norm_gain(seed, BWS_ATTN_NORM, (uint32_t)l, d, m->attn_norm[l]);
    bws_norm_gain(seed, BWS_FFN_NORM, (uint32_t)l, d, m->ffn_norm[l]);
    or_mat_make(&m->qkv[l], seed, BWS_QKV, (uint32_t)l, 0, nqkv, d);
    or_mat_make(&m->o[l], seed, BWS_O, (uint32_t)l, 0, d, nattn);
  }
  if (!or_is_moe(c)) {
    m->gate = (or_mat*)calloc((size_t)L, sizeof(or_mat));
    m->up = (or_mat*)calloc((size_t)L, sizeof(or_mat));
    m->down = (or_mat*)calloc((size_t)L, sizeof(or_mat));
    for (int l = 0; l < L; ++l) {
      or_mat_make(&m->gate[l], seed, BWS_GATE, (uint32_t)l, 0, c->ffn_dim, d);
      or_mat_make(&m->up[l], seed, BWS_UP, (uint32_t)l, 0, c->ffn_dim, d);
      or_mat_make(&m->down[l], seed, BWS_DOWN, (uint32_t)l, 0, d, c->ffn_dim);
    }
  } else {
    int E = c->n_experts, S = c->n_shared;
    m->gate = (or_mat*)calloc((size_t)L * E, sizeof(or_mat));
    m->up = (or_mat*)calloc((size_t)L * E, sizeof(or_mat));
    m->down = (or_mat*)calloc((size_t)L * E, sizeof(or_mat));
    m->sgate = (or_mat*)calloc((size_t)(L * (S > 0 ? S : 1)), sizeof(or_mat));
    m->sup = (or_mat*)calloc((size_t)(L * (S > 0 ? S : 1)), sizeof(or_mat));
    m->sdown = (or_mat*)calloc((size_t)(L * (S > 0 ? S : 1)), sizeof(or_mat));
    m->router = (uint16_t**)calloc((size_t)L, sizeof(uint16_t*));
    for (int l = 0; l < L; ++l) {
      m->router[l] = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)E * d);
      bws_router(seed, (uint32_t)l, E, d, m->router[l]);
      for (int e = 0; e < E; ++e) {
        or_mat_make(&m->gate[l * E + e], seed, BWS_GATE, (uint32_t)l, 1u + (uint32_t)e,
                    c->expert_ffn, d);
        or_mat_make(&m->up[l * E + e], seed, BWS_UP, (uint32_t)l, 1u + (uint32_t)e, c->expert_ffn,
                    d);
        or_mat_make(&m->down[l * E + e], seed, BWS_DOWN, (uint32_t)l, 1u + (uint32_t)e, d,
                    c->expert_ffn);
      }
      for (int s = 0; s < S; ++s) {
        uint32_t ex = BWS_SHARED_EXPERT + (uint32_t)s;
        or_mat_make(&m->sgate[l * S + s], seed, BWS_GATE, (uint32_t)l, ex, c->shared_ffn, d);
        or_mat_make(&m->sup[l * S + s], seed, BWS_UP, (uint32_t)l, ex, c->shared_ffn, d);
        or_mat_make(&m->sdown[l * S + s], seed, BWS_DOWN, (uint32_t)l, ex, d, c->shared_ffn);
      }
    }
  }
  m->final_norm = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)d);
  bws_norm_gain(seed, BWS_FINAL_NORM, 0, d, m->final_norm);
  or_mat_make(&m->lm_head, seed, BWS_LM_HEAD, 0, 0, c->vocab, d);
  return m;
}

void or_model_free(or_model* m) {
  if (!m) return;
  const or_config* c = &m->c;
  int L = c->n_layers;
  for (int l = 0; l < L; ++l) {
    free(m->attn_norm[l]);
    free(m->ffn_norm[l]);
    or_mat_free(&m->qkv[l]);
    or_mat_free(&m->o[l]);
  }
  if (!or_is_moe(c)) {
    for (int l = 0; l < L; ++l) {
      or_mat_free(&m->gate[l]);
      or_mat_free(&m->up[l]);
      or_mat_free(&m->down[l]);
    }
  } else {
    int E = c->n_experts, S = c->n_shared;
    for (int l = 0; l < L; ++l) {
      free(m->router[l]);
      for (int e = 0; e < E; ++e) {
        or_mat_free(&m->gate[l * E + e]);
        or_mat_free(&m->up[l * E + e]);
        or_mat_free(&m->down[l * E + e]);
      }
      for (int s = 0; s < S; ++s) {
        or_mat_free(&m->sgate[l * S + s]);
        or_mat_free(&m->sup[l * S + s]);
        or_mat_free(&m->sdown[l * S + s]);
      }
    }
    free(m->router);
    free(m->sgate);
    free(m->sup);
    free(m->sdown);
  }
  free(m->gate);
  free(m->up);
  free(m->down);
  free(m->attn_norm);
  free(m->ffn_norm);
  free(m->qkv);
  free(m->o);
  free(m->final_norm);
  or_mat_free(&m->lm_head);
  free(m);
}

/* Access to the generated canonical tensors (for kernel-level checks). which: 0 qkv, 1 o,
 * 2 gate, 3 up, 4 down, 5 lm_head, 6 shared gate, 7 shared up, 8 shared down. For MoE, expert
 * selects the routed (or shared) expert. Returns 0 and fills the pointers, or -1. */
int or_model_matrix(const or_model* m, int which, int layer, int expert, const uint8_t** codes,
                    const uint16_t** scales, int64_t* N, int64_t* K) {
  const or_config* c = &m->c;
  const or_mat* mat = NULL;
  int E = c->n_experts, S = c->n_shared;
  int moe = or_is_moe(c);
  switch (which) {
    case 0: mat = &m->qkv[layer]; break;
    case 1: mat = &m->o[layer]; break;
    case 2: mat = moe ? &m->gate[layer * E + expert] : &m->gate[layer]; break;
    case 3: mat = moe ? &m->up[layer * E + expert] : &m->up[layer]; break;
    case 4: mat = moe ? &m->down[layer * E + expert] : &m->down[layer]; break;
    case 5: mat = &m->lm_head; break;
    case 6: mat = (moe && S) ? &m->sgate[layer * S + expert] : NULL; break;
    case 7: mat = (moe && S) ? &m->sup[layer * S + expert] : NULL; break;
    case 8: mat = (moe && S) ? &m->sdown[layer * S + expert] : NULL; break;
    default: break;
  }
  if (!mat) return -1;
  *codes = mat->codes;
  *scales = mat->scales;
  *N = mat->N;
  *K = mat->K;
  return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* KV state (logical view; no pages)                                                          */
/* ------------------------------------------------------------------------------------------ */

typedef struct {
  int64_t ctx0;         /* positions [0, ctx0) hold synthetic context */
  uint64_t synth_seed;  /* seed of that context */
  uint32_t synth_seq;   /* sequence index used in the generator key */
  int64_t cap;          /* positions [ctx0, ctx0 + cap) can be appended */
  double* app;          /* [L][cap][2][G][D] appended (already rounded) keys and values */
} or_seq;

typedef struct {
  int L, G, D;
  int dtype; /* cache dtype: selects the synthetic context's values */
  int n_seqs;
  or_seq* seqs;
} or_kv;

or_kv* or_kv_create(const or_model* m, int n_seqs, int64_t cap) {
  or_kv* kv = (or_kv*)calloc(1, sizeof(or_kv));
  kv->L = m->c.n_layers;
  kv->G = m->c.n_kv_heads;
  kv->D = m->c.head_dim;
  kv->dtype = m->c.kv_dtype;
  kv->n_seqs = n_seqs;
  kv->seqs = (or_seq*)calloc((size_t)n_seqs, sizeof(or_seq));
  for (int s = 0; s < n_seqs; ++s) {
    kv->seqs[s].cap = cap;
    kv->seqs[s].app = (double*)calloc((size_t)(kv->L * cap * 2 * kv->G * kv->D), sizeof(double));
  }
  return kv;
}

void or_kv_free(or_kv* kv) {
  if (!kv) return;
  for (int s = 0; s < kv->n_seqs; ++s) free(kv->seqs[s].app);
  free(kv->seqs);
  free(kv);
}

/* positions [0, ctx0) of sequence s hold the generator's synthetic K/V for
 * (synth_seed, layer, synth_seq) */
void or_kv_set_synth(or_kv* kv, int s, uint64_t synth_seed, uint32_t synth_seq, int64_t ctx0) {
  kv->seqs[s].ctx0 = ctx0;
  kv->seqs[s].synth_seed = synth_seed;
  kv->seqs[s].synth_seq = synth_seq;
}

static inline double or_kv_get(const or_kv* kv, const or_seq* sq, int l, int64_t pos, int which,
                               int g, int d) {
  if (pos < sq->ctx0)
    return bws_kv_value_dt(sq->synth_seed, (uint32_t)l, sq->synth_seq, pos, which, g, d, kv->G,
                           kv->D, kv->dtype);
  int64_t a = pos - sq->ctx0;
  return sq->app[((((int64_t)l * sq->cap + a) * 2 + which) * kv->G + g) * kv->D + d];
}

static inline double* or_kv_slot(or_kv* kv, or_seq* sq, int l, int64_t pos, int which, int g) {
  int64_t a = pos - sq->ctx0;
  return &sq->app[((((int64_t)l * sq->cap + a) * 2 + which) * kv->G + g) * kv->D];
}

/* store given (already rounded) keys and values of one position: vals [2][G][D] (for tests that
 * take a cached context from elsewhere; pos must lie in the appendable range) */
int or_kv_set(or_kv* kv, int s, int l, int64_t pos, const double* vals) {
  or_seq* sq = &kv->seqs[s];
  if (pos < sq->ctx0 || pos >= sq->ctx0 + sq->cap || l < 0 || l >= kv->L) return -1;
  for (int w = 0; w < 2; ++w)
    for (int g = 0; g < kv->G; ++g) {
      double* dst = or_kv_slot(kv, sq, l, pos, w, g);
      for (int d = 0; d < kv->D; ++d) dst[d] = vals[((int64_t)w * kv->G + g) * kv->D + d];
    }
  return 0;
}

/* read one cached element (for tests) */
double or_kv_read(const or_kv* kv, int s, int l, int64_t pos, int which, int g, int d) {
  return or_kv_get(kv, &kv->seqs[s], l, pos, which, g, d);
}

/* ------------------------------------------------------------------------------------------ */
/* forward                                                                                     */
/* ------------------------------------------------------------------------------------------ */

/* SwiGLU FFN: down * (silu(gate * h) (.) (up * h)) */
static void or_ffn(const or_mat* g, const or_mat* u, const or_mat* dn, const double* h,
                   double* out) {
  int64_t F = g->N;
  double* a = (double*)malloc(sizeof(double) * (size_t)F);
  double* b = (double*)malloc(sizeof(double) * (size_t)F);
  or_gemv(g->codes, g->scales, g->N, g->K, h, a);
  or_gemv(u->codes, u->scales, u->N, u->K, h, b);
  for (int64_t i = 0; i < F; ++i) a[i] = or_silu(a[i]) * b[i];
  or_gemv(dn->codes, dn->scales, dn->N, dn->K, a, out);
  free(a);
  free(b);
}

/* exported for tests: the dense FFN of one layer or one (shared) expert */
void or_model_ffn(const or_model* m, int layer, int expert, int shared, const double* h,
                  double* out) {
  const or_config* c = &m->c;
  if (!or_is_moe(c))
    or_ffn(&m->gate[layer], &m->up[layer], &m->down[layer], h, out);
  else if (shared)
    or_ffn(&m->sgate[layer * c->n_shared + expert], &m->sup[layer * c->n_shared + expert],
           &m->sdown[layer * c->n_shared + expert], h, out);
  else
    or_ffn(&m->gate[layer * c->n_experts + expert], &m->up[layer * c->n_experts + expert],
           &m->down[layer * c->n_experts + expert], h, out);
}

/* MoE FFN of one layer on input h. If sel_in is given, its set is adopted when it differs from
 * the oracle's top-k only by experts whose logits lie within tau of the k-th/(k+1)-th
 * boundary (a near tie: both selections are correct to the precision at hand); any other
 * difference returns -1. sel_out receives the set used. *adopted is incremented when sel_in
 * was adopted. */
static int or_moe_ffn(const or_model* m, int l, const double* h, double* out,
                      const int32_t* sel_in, int32_t* sel_out, double tau, int32_t* adopted) {
  const or_config* c = &m->c;
  int E = c->n_experts, k = c->top_k, d = c->d_model;
  double* r = (double*)malloc(sizeof(double) * (size_t)E);
  double* P = (double*)malloc(sizeof(double) * (size_t)E);
  int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  or_gemv_f16(m->router[l], E, d, h, r);
  or_softmax(r, E, P);
  or_topk(r, E, E, sel); /* full order: sel[0..k-1] is the top-k */
  int rc = 0;
  int32_t use[512];
  for (int i = 0; i < k; ++i) use[i] = sel[i];
  if (sel_in) {
    /* compare as sets */
    int same = 1;
    for (int i = 0; i < k && same; ++i) {
      int found = 0;
      for (int j = 0; j < k; ++j) found |= (sel_in[j] == use[i]);
      same &= found;
    }
    if (!same) {
      double kth = r[sel[k - 1]];
      double next = (k < E) ? r[sel[k]] : -INFINITY;
      int ok = 1;
      for (int i = 0; i < k && ok; ++i) {
        int e = sel_in[i];
        if (e < 0 || e >= E) {
          ok = 0;
          break;
        }
        int in_oracle = 0;
        for (int j = 0; j < k; ++j) in_oracle |= (use[j] == e);
        if (!in_oracle && !(r[e] >= next - tau && r[e] >= kth - tau)) ok = 0;
        for (int j = 0; j < i; ++j)
          if (sel_in[j] == e) ok = 0; /* duplicates are never valid */
      }
      for (int i = 0; i < k && ok; ++i) {
        int e = use[i];
        int in_gpu = 0;
        for (int j = 0; j < k; ++j) in_gpu |= (sel_in[j] == e);
        if (!in_gpu && !(r[e] <= kth + tau && r[e] <= next + tau)) ok = 0;
      }
      if (!ok) {
        rc = -1;
      } else {
        for (int i = 0; i < k; ++i) use[i] = sel_in[i];
        if (adopted) (*adopted)++;
      }
    }
  }
  if (sel_out)
    for (int i = 0; i < k; ++i) sel_out[i] = use[i];
  double z = 0.0;
  for (int i = 0; i < k; ++i) z += P[use[i]];
  for (int i = 0; i < d; ++i) out[i] = 0.0;
  double* y = (double*)malloc(sizeof(double) * (size_t)d);
  for (int i = 0; i < k; ++i) {
    int e = use[i];
    double gate = P[e] / z;
    or_ffn(&m->gate[l * E + e], &m->up[l * E + e], &m->down[l * E + e], h, y);
    for (int j = 0; j < d; ++j) out[j] += gate * y[j];
  }
  for (int s = 0; s < c->n_shared; ++s) {
    or_ffn(&m->sgate[l * c->n_shared + s], &m->sup[l * c->n_shared + s],
           &m->sdown[l * c->n_shared + s], h, y);
    for (int j = 0; j < d; ++j) out[j] += y[j];
  }
  free(y);
  free(r);
  free(P);
  free(sel);
  return rc;
}

/* exported for tests: router logits of one layer */
void or_model_router_logits(const or_model* m, int layer, const double* h, double* r) {
  or_gemv_f16(m->router[layer], m->c.n_experts, m->c.d_model, h, r);
}

/* exported for tests: the MoE FFN of one layer (sel_out may be NULL) */
int or_model_moe_ffn(const or_model* m, int layer, const double* h, double* out, int32_t* sel_out) {
  return or_moe_ffn(m, layer, h, out, NULL, sel_out, 0.0, NULL);
}

/* exported for tests: the MoE FFN of one layer with a proposed expert set sel_in (the near-tie
 * rule above); returns 0 (sel_in adopted, or equal to the oracle's set) or -1 (rejected) */
int or_model_moe_ffn_sel(const or_model* m, int layer, const double* h, double* out,
                         const int32_t* sel_in, int32_t* sel_out, double tau, int32_t* adopted) {
  return or_moe_ffn(m, layer, h, out, sel_in, sel_out, tau, adopted);
}

/* Decode T new tokens of sequence s at positions pos0 .. pos0+T-1. The keys and values of all
 * T tokens are cached before any of them attends; token t attends to positions 0..pos0+t.
 *   logits      [T][vocab] (optional)
 *   hidden      [T][d_model] residual stream after the last layer (optional)
 *   sel_out     [T][L][top_k] experts used (MoE, optional)
 *   sel_in      [T][L][top_k] candidate expert sets (MoE, optional; see or_moe_ffn)
 * Returns 0, or -1 if a candidate expert set was not a valid near-tie choice, or -2 if the
 * positions exceed the cache capacity. */
int or_forward(or_model* m, or_kv* kv, int s, const int32_t* tokens, int T, int64_t pos0,
               double* logits, double* hidden, int32_t* sel_out, const int32_t* sel_in,
               double tau, int32_t* adopted) {
  const or_config* c = &m->c;
  int L = c->n_layers, d = c->d_model, H = c->n_q_heads, G = c->n_kv_heads, D = c->head_dim;
  int rep = H / G;
  int64_t nqkv = (int64_t)(H + 2 * G) * D;
  or_seq* sq = &kv->seqs[s];
  if (pos0 < sq->ctx0 || pos0 + T > sq->ctx0 + sq->cap) return -2;
  int rc = 0;
  double* X = (double*)malloc(sizeof(double) * (size_t)T * d);
  double* h = (double*)malloc(sizeof(double) * (size_t)d);
  double* qkv = (double*)malloc(sizeof(double) * (size_t)T * nqkv);
  double* att = (double*)malloc(sizeof(double) * (size_t)T * H * D);
  double* y = (double*)malloc(sizeof(double) * (size_t)d);
  uint16_t* erow = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)d);
  for (int t = 0; t < T; ++t) {
    bws_embed_rows(m->seed, d, tokens[t], 1, erow);
    for (int i = 0; i < d; ++i) X[(int64_t)t * d + i] = or_f16_to_f64(erow[i]);
  }
  for (int l = 0; l < L; ++l) {
    /* attention block: q, k, v for every new token; cache k, v */
    for (int t = 0; t < T; ++t) {
      int64_t pos = pos0 + t;
      double* v3 = qkv + (int64_t)t * nqkv;
      or_rmsnorm(X + (int64_t)t * d, m->attn_norm[l], d, c->rms_eps, h);
      or_gemv(m->qkv[l].codes, m->qkv[l].scales, nqkv, d, h, v3);
      for (int hq = 0; hq < H; ++hq) or_rope(v3 + (int64_t)hq * D, D, pos, c->rope_base);
      for (int g = 0; g < G; ++g) or_rope(v3 + (int64_t)(H + g) * D, D, pos, c->rope_base);
      for (int g = 0; g < G; ++g) {
        double* kd = or_kv_slot(kv, sq, l, pos, 0, g);
        double* vd = or_kv_slot(kv, sq, l, pos, 1, g);
        for (int i = 0; i < D; ++i) {
          kd[i] = or_kv_round(v3[(int64_t)(H + g) * D + i], c->kv_dtype);
          vd[i] = or_kv_round(v3[(int64_t)(H + G + g) * D + i], c->kv_dtype);
        }
      }
    }
    for (int t = 0; t < T; ++t) {
      int64_t n = pos0 + t + 1;
      /* gather the logical K/V of every KV head for positions 0..pos0+t */
      double* Kc = (double*)malloc(sizeof(double) * (size_t)(G * n * D));
      double* Vc = (double*)malloc(sizeof(double) * (size_t)(G * n * D));
#pragma omp parallel for schedule(static)
      for (int64_t gj = 0; gj < (int64_t)G * n; ++gj) {
        int g = (int)(gj / n);
        int64_t j = gj % n;
        for (int i = 0; i < D; ++i) {
          Kc[(g * n + j) * D + i] = or_kv_get(kv, sq, l, j, 0, g, i);
          Vc[(g * n + j) * D + i] = or_kv_get(kv, sq, l, j, 1, g, i);
        }
      }
#pragma omp parallel for schedule(static)
      for (int hq = 0; hq < H; ++hq) {
        int g = hq / rep;
        or_attention(qkv + (int64_t)t * nqkv + (int64_t)hq * D, Kc + (int64_t)g * n * D,
                     Vc + (int64_t)g * n * D, n, D, att + ((int64_t)t * H + hq) * D, NULL);
      }
      free(Kc);
      free(Vc);
      or_gemv(m->o[l].codes, m->o[l].scales, d, (int64_t)H * D, att + (int64_t)t * H * D, y);
      for (int i = 0; i < d; ++i) X[(int64_t)t * d + i] += y[i];
    }
    /* FFN block */
    for (int t = 0; t < T; ++t) {
      or_rmsnorm(X + (int64_t)t * d, m->ffn_norm[l], d, c->rms_eps, h);
      if (!or_is_moe(c)) {
        or_ffn(&m->gate[l], &m->up[l], &m->down[l], h, y);
      } else {
        int32_t* so = sel_out ? sel_out + ((int64_t)t * L + l) * c->top_k : NULL;
        const int32_t* si = sel_in ? sel_in + ((int64_t)t * L + l) * c->top_k : NULL;
        if (or_moe_ffn(m, l, h, y, si, so, tau, adopted) != 0) rc = -1;
      }
      for (int i = 0; i < d; ++i) X[(int64_t)t * d + i] += y[i];
    }
  }
  if (hidden) memcpy(hidden, X, sizeof(double) * (size_t)T * d);
  if (logits) {
    for (int t = 0; t < T; ++t) {
      or_rmsnorm(X + (int64_t)t * d, m->final_norm, d, c->rms_eps, h);
      or_gemv(m->lm_head.codes, m->lm_head.scales, c->vocab, d, h, logits + (int64_t)t * c->vocab);
    }
  }
  free(X);
  free(h);
  free(qkv);
  free(att);
  free(y);
  free(erow);
  return rc;
}

int or_num_threads(void) { return omp_get_max_threads(); }
void or_set_num_threads(int n) { omp_set_num_threads(n); }
