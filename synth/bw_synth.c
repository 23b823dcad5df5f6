/*
 * bw_synth.c - seeded synthetic inputs (see bw_synth.h for the generator and distributions).
 * Built with gcc -O2 -ffp-contract=off so that the fp64 Box-Muller path is the same object code
 * wherever it is linked.
 */
#include "bw_synth.h"

#include <math.h>
#include <string.h>

uint64_t bws_key(uint64_t seed, uint32_t kind, uint32_t layer, uint32_t expert, uint32_t sub) {
  uint64_t k = bws_mix(seed ^ 0x5851F42D4C957F2DULL);
  k = bws_mix(k ^ ((uint64_t)kind << 40) ^ ((uint64_t)sub << 32) ^ (uint64_t)layer);
  k = bws_mix(k ^ ((uint64_t)expert * 0xD1B54A32D192ED03ULL));
  return k;
}

double bws_uniform(uint64_t h) {
  /* (m + 0.5) / 2^53 with m the top 53 bits: strictly inside (0,1) */
  return ((double)(h >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

double bws_gauss(uint64_t key, uint64_t i) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = bws_uniform(bws_hash(key, 2 * i));
  double u2 = bws_uniform(bws_hash(key, 2 * i + 1));
  double r = sqrt(-2.0 * log(u1));
  return r * cos(two_pi * u2);
}

uint16_t bws_f16_bits(double v) {
  uint16_t sign = 0;
  if (signbit(v)) {
    sign = 0x8000;
    v = -v;
  }
  if (isnan(v)) return (uint16_t)(sign | 0x7E00);
  if (v >= 65520.0) return (uint16_t)(sign | 0x7C00); /* rounds to inf */
  if (v < 6.103515625e-05) {
    /* subnormal range: units of 2^-24, round half to even */
    double units = v * 16777216.0; /* exact (power-of-two scale) */
    double fl = floor(units);
    double rem = units - fl;
    uint32_t m = (uint32_t)fl;
    if (rem > 0.5 || (rem == 0.5 && (m & 1u))) m += 1;
    return (uint16_t)(sign | m); /* m == 1024 becomes the smallest normal, as it should */
  }
  int e;
  double f = frexp(v, &e); /* v = f * 2^e, f in [0.5, 1) */
  /* v = (1 + m/1024) * 2^(e-1); mantissa units: f*2048 in [1024, 2048) */
  double units = f * 2048.0;
  double fl = floor(units);
  double rem = units - fl;
  uint32_t m = (uint32_t)fl;
  if (rem > 0.5 || (rem == 0.5 && (m & 1u))) m += 1;
  int exp_field = (e - 1) + 15;
  if (m == 2048) {
    m = 1024;
    exp_field += 1;
  }
  if (exp_field >= 31) return (uint16_t)(sign | 0x7C00);
  return (uint16_t)(sign | ((uint32_t)exp_field << 10) | (m - 1024));
}

void bws_fill_bytes(uint64_t key, uint64_t off, uint8_t* dst, size_t n) {
  size_t i = 0;
  while (i < n) {
    uint64_t b = off + i;
    uint64_t h = bws_hash(key, b >> 3);
    unsigned j = (unsigned)(b & 7u);
    for (; j < 8 && i < n; ++j, ++i) dst[i] = (uint8_t)(h >> (8 * j));
  }
}

void bws_fill_f16(uint64_t key, uint64_t off, uint16_t* dst, size_t n, double mean, double sd,
                  int absolute) {
  for (size_t i = 0; i < n; ++i) {
    double z = bws_gauss(key, off + i);
    double v = absolute ? fabs(sd * z) : mean + sd * z;
    dst[i] = bws_f16_bits(v);
  }
}

void bws_int4_matrix(uint64_t seed, uint32_t kind, uint32_t layer, uint32_t expert, int64_t N,
                     int64_t K, int64_t row0, int64_t nrows, uint8_t* codes, uint16_t* scales) {
  (void)N;
  int64_t row_bytes = K / 2;
  int64_t row_blocks = K / 32;
  if (codes)
    bws_fill_bytes(bws_key(seed, kind, layer, expert, BWS_SUB_CODES), (uint64_t)(row0 * row_bytes),
                   codes, (size_t)(nrows * row_bytes));
  if (scales)
    bws_fill_f16(bws_key(seed, kind, layer, expert, BWS_SUB_SCALES),
                 (uint64_t)(row0 * row_blocks), scales, (size_t)(nrows * row_blocks), 0.0, 0.02,
                 1);
}

void bws_mx_matrix(uint64_t seed, uint32_t kind, uint32_t layer, uint32_t expert, int64_t K,
                   int64_t row0, int64_t nrows, int e_lo, int e_hi, uint8_t* codes,
                   uint8_t* scales) {
  int64_t row_bytes = K / 2;
  int64_t row_blocks = K / 32;
  if (codes)
    bws_fill_bytes(bws_key(seed, kind, layer, expert, BWS_SUB_MX_CODES),
                   (uint64_t)(row0 * row_bytes), codes, (size_t)(nrows * row_bytes));
  if (scales) {
    uint64_t key = bws_key(seed, kind, layer, expert, BWS_SUB_MX_SCALES);
    uint64_t span = (uint64_t)(e_hi - e_lo + 1);
    for (int64_t i = 0; i < nrows * row_blocks; ++i)
      scales[i] = (uint8_t)(e_lo + (int)(bws_hash(key, (uint64_t)(row0 * row_blocks + i)) % span));
  }
}

void bws_norm_gain(uint64_t seed, uint32_t kind, uint32_t layer, int64_t n, uint16_t* dst) {
  bws_fill_f16(bws_key(seed, kind, layer, 0, 0), 0, dst, (size_t)n, 1.0, 0.1, 0);
}

void bws_embed_rows(uint64_t seed, int64_t d, int64_t row0, int64_t nrows, uint16_t* dst) {
  bws_fill_f16(bws_key(seed, BWS_EMBED, 0, 0, 0), (uint64_t)(row0 * d), dst, (size_t)(nrows * d),
               0.0, 1.0, 0);
}

void bws_router(uint64_t seed, uint32_t layer, int64_t n_experts, int64_t d, uint16_t* dst) {
  bws_fill_f16(bws_key(seed, BWS_ROUTER, layer, 0, 0), 0, dst, (size_t)(n_experts * d), 0.0, 0.02,
               0);
}

static inline int kv_code(uint64_t key, int64_t pos, int kv, int g, int d, int G, int D) {
  uint64_t idx = (((uint64_t)pos * 2u + (uint64_t)kv) * (uint64_t)G + (uint64_t)g) * (uint64_t)D +
                 (uint64_t)d;
  return (int)(bws_hash(key, idx) & 0xFFu) - 128;
}

static inline uint16_t kv_code_bits(int c, int dtype) {
  if (dtype == BWS_KV_FP8) {
    /* (c >> 3) / 8 = m / 8 with |m| <= 16: at most 4 significant bits, exact in E4M3
     * (1 sign, 4 exponent bits with bias 7, 3 fraction bits) */
    int m = c >> 3;
    uint16_t sign = m < 0 ? 0x80 : 0;
    if (m < 0) m = -m;
    if (m == 0) return sign;
    int k = 0;
    while ((m >> (k + 1)) != 0) ++k;         /* m in [2^k, 2^(k+1)) */
    int field = k - 3 + 7;                   /* m / 8 = 2^(k-3) (1 + frac) */
    int frac = (m - (1 << k)) << (3 - k);
    return (uint16_t)(sign | (field << 3) | frac);
  }
  /* c/64 with c in [-128, 127]: at most 8 significant bits, exact in bf16 and fp16 */
  double v = (double)c / 64.0;
  if (dtype == BWS_KV_F16) return bws_f16_bits(v);
  /* bf16: top half of the fp32 pattern (exact, so no rounding) */
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

double bws_kv_value(uint64_t seed, uint32_t layer, uint32_t seq, int64_t pos, int kv, int g,
                    int d, int G, int D) {
  uint64_t key = bws_key(seed, BWS_KV, layer, seq, 0);
  return (double)kv_code(key, pos, kv, g, d, G, D) / 64.0;
}

double bws_kv_value_dt(uint64_t seed, uint32_t layer, uint32_t seq, int64_t pos, int kv, int g,
                       int d, int G, int D, int dtype) {
  if (dtype != BWS_KV_FP8) return bws_kv_value(seed, layer, seq, pos, kv, g, d, G, D);
  uint64_t key = bws_key(seed, BWS_KV, layer, seq, 0);
  return (double)(kv_code(key, pos, kv, g, d, G, D) >> 3) / 8.0;
}

uint16_t bws_kv_bits(uint64_t seed, uint32_t layer, uint32_t seq, int64_t pos, int kv, int g,
                     int d, int G, int D, int dtype) {
  uint64_t key = bws_key(seed, BWS_KV, layer, seq, 0);
  return kv_code_bits(kv_code(key, pos, kv, g, d, G, D), dtype);
}

void bws_kv_fill(uint64_t seed, uint32_t layer, uint32_t seq, int64_t pos0, int64_t ntok, int G,
                 int D, int dtype, void* dst) {
  uint64_t key = bws_key(seed, BWS_KV, layer, seq, 0);
  uint16_t lut[256];
  for (int c = -128; c < 128; ++c) lut[c + 128] = kv_code_bits(c, dtype);
  uint16_t* d16 = (uint16_t*)dst;
  uint8_t* d8 = (uint8_t*)dst;
  size_t o = 0;
  for (int64_t t = 0; t < ntok; ++t)
    for (int kv = 0; kv < 2; ++kv)
      for (int g = 0; g < G; ++g)
        for (int d = 0; d < D; ++d, ++o) {
          uint16_t b = lut[kv_code(key, pos0 + t, kv, g, d, G, D) + 128];
          if (dtype == BWS_KV_FP8)
            d8[o] = (uint8_t)b;
          else
            d16[o] = b;
        }
}
