/*
 * bw_synth.h - seeded synthetic inputs for the int4 decode-step library and its CPU oracle.
 *
 * This module generates inputs only: weights, norm gains, embeddings, router matrices and
 * synthetic KV-cache context. It contains none of the decode step's arithmetic. Both the HIP
 * library and the oracle link the same compiled object of bw_synth.c, so the two sides see
 * identical bytes without either one reading the other's output.
 *
 * Generator: splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014; finaliser constants as in Vigna's public splitmix64.c), used as a
 * counter-based hash: value i of stream k is mix(k + (i+1) * golden_gamma). Every element is
 * therefore a pure function of (seed, tensor kind, layer, expert, index), independent of the
 * order or the thread it is generated in.
 *
 * Gaussians: Box-Muller in fp64 on two uniforms in (0,1) drawn from consecutive counters.
 * fp16 encoding is round-to-nearest-even with subnormals kept (no flush to zero).
 *
 * Distributions (one per tensor kind):
 *   int4 codes q      : uniform on 0..15 (packed bytes are uniform random bytes)
 *   int4 block scales : fp16(|0.02 z|)      z ~ N(0,1)
 *   embeddings        : fp16(z)
 *   RMSNorm gains     : fp16(1 + 0.1 z)
 *   MoE router matrix : fp16(0.02 z)
 *   MXFP4 codes       : uniform on 0..15 (uniform random bytes, two E2M1 codes each)
 *   MXFP4 scales      : E8M0 byte uniform on [e_lo, e_hi]
 *   synthetic KV      : c / 64 with c = (h & 0xFF) - 128, exact in bf16 and fp16; for an fp8
 *                       (OCP E4M3) cache (c >> 3) / 8, in [-2, 1.875], exact in E4M3
 */
#ifndef BW_SYNTH_H
#define BW_SYNTH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* tensor kinds (part of the stream key) */
enum {
  BWS_EMBED = 1,      /* [vocab][d_model] fp16                        */
  BWS_FINAL_NORM = 2, /* [d_model] fp16                               */
  BWS_LM_HEAD = 3,    /* int4 [vocab][d_model]                        */
  BWS_ATTN_NORM = 10, /* [d_model] fp16, per layer                    */
  BWS_QKV = 11,       /* int4 [(Hq+2Hkv)*D][d_model]: q rows, k rows, v rows */
  BWS_O = 12,         /* int4 [d_model][Hq*D]                         */
  BWS_FFN_NORM = 13,  /* [d_model] fp16                               */
  BWS_GATE = 14,      /* int4 [ffn][d_model]                          */
  BWS_UP = 15,        /* int4 [ffn][d_model]                          */
  BWS_DOWN = 16,      /* int4 [d_model][ffn]                          */
  BWS_ROUTER = 17,    /* fp16 [n_experts][d_model]                    */
  BWS_KV = 20         /* synthetic cached keys/values                 */
};

/* expert field of the key: 0 for a dense FFN, 1 + e for routed expert e (0-based), and
 * BWS_SHARED_EXPERT + s for shared expert s. */
#define BWS_SHARED_EXPERT 0x100000u

/* sub-streams of an int4 matrix, and of an MXFP4 matrix */
#define BWS_SUB_CODES 0u
#define BWS_SUB_SCALES 1u
#define BWS_SUB_MX_CODES 2u
#define BWS_SUB_MX_SCALES 3u

/* KV element dtype codes */
#define BWS_KV_F16 1
#define BWS_KV_BF16 2
#define BWS_KV_FP8 3 /* OCP FP8 E4M3 (one byte per element) */

static inline uint64_t bws_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* counter-based hash: element i of stream key */
static inline uint64_t bws_hash(uint64_t key, uint64_t i) {
  return bws_mix(key + (i + 1ULL) * 0x9E3779B97F4A7C15ULL);
}

/* stream key for (seed, kind, layer, expert, sub-stream) */
uint64_t bws_key(uint64_t seed, uint32_t kind, uint32_t layer, uint32_t expert, uint32_t sub);

/* uniform in (0,1) from a 64-bit hash (top 53 bits, centred) */
double bws_uniform(uint64_t h);

/* standard normal number i of a stream (Box-Muller on counters 2i, 2i+1) */
double bws_gauss(uint64_t key, uint64_t i);

/* fp64 -> fp16 bits, round to nearest even, subnormals kept, overflow -> inf */
uint16_t bws_f16_bits(double v);

/* Fill n bytes of a byte stream starting at byte offset off: byte b is byte (b % 8) of
 * bws_hash(key, b / 8), little-endian. */
void bws_fill_bytes(uint64_t key, uint64_t off, uint8_t* dst, size_t n);

/* Fill n fp16 values starting at element offset off: fp16(mean + sd * z) or fp16(|sd * z|)
 * when absolute != 0 (mean ignored). */
void bws_fill_f16(uint64_t key, uint64_t off, uint16_t* dst, size_t n, double mean, double sd,
                  int absolute);

/* One int4 matrix [N][K] in its canonical form, rows [row0, row0+nrows):
 *   codes : nrows * K/2 bytes. Row n occupies K/2 bytes; block b of the row is bytes
 *           16b..16b+15; byte i of a block holds element i in bits 0-3 and element i+16 in
 *           bits 4-7.
 *   scales: nrows * K/32 fp16 values, one per block, row-major.
 * Either output pointer may be NULL. K must be a multiple of 32. */
void bws_int4_matrix(uint64_t seed, uint32_t kind, uint32_t layer, uint32_t expert, int64_t N,
                     int64_t K, int64_t row0, int64_t nrows, uint8_t* codes, uint16_t* scales);

/* One MXFP4 matrix [N][K] (OCP MX: E2M1 elements, one E8M0 scale per 32), rows
 * [row0, row0+nrows):
 *   codes : nrows * K/2 bytes; byte i of a row holds element 2i in bits 0-3 and element 2i+1
 *           in bits 4-7 (uniform random bytes).
 *   scales: nrows * K/32 bytes, one per block, row-major, each uniform on [e_lo, e_hi].
 * Either output pointer may be NULL. K must be a multiple of 32; 0 <= e_lo <= e_hi <= 255. */
void bws_mx_matrix(uint64_t seed, uint32_t kind, uint32_t layer, uint32_t expert, int64_t K,
                   int64_t row0, int64_t nrows, int e_lo, int e_hi, uint8_t* codes,
                   uint8_t* scales);

/* Norm gains [n] for (kind in {BWS_ATTN_NORM, BWS_FFN_NORM, BWS_FINAL_NORM}, layer). */
void bws_norm_gain(uint64_t seed, uint32_t kind, uint32_t layer, int64_t n, uint16_t* dst);

/* Embedding rows [row0, row0+nrows) of a [vocab][d] table. */
void bws_embed_rows(uint64_t seed, int64_t d, int64_t row0, int64_t nrows, uint16_t* dst);

/* Router matrix [n_experts][d] of one layer. */
void bws_router(uint64_t seed, uint32_t layer, int64_t n_experts, int64_t d, uint16_t* dst);

/* Synthetic cached K or V element (kv = 0 for K, 1 for V) of sequence seq at position pos,
 * KV head g, dimension d, in a cache with G KV heads of size D. The value is
 * ((h & 0xFF) - 128) / 64 with h = bws_hash(bws_key(seed, BWS_KV, layer, seq, 0),
 * ((pos*2 + kv)*G + g)*D + d). */
double bws_kv_value(uint64_t seed, uint32_t layer, uint32_t seq, int64_t pos, int kv, int g,
                    int d, int G, int D);

/* The element of a cache of the given dtype: bws_kv_value for BWS_KV_F16 / BWS_KV_BF16, and
 * (c >> 3) / 8 (arithmetic shift of the same code c) for BWS_KV_FP8. */
double bws_kv_value_dt(uint64_t seed, uint32_t layer, uint32_t seq, int64_t pos, int kv, int g,
                       int d, int G, int D, int dtype);

/* The same element as bits of the dtype (bf16, fp16, or E4M3 in the low byte); exact. */
uint16_t bws_kv_bits(uint64_t seed, uint32_t layer, uint32_t seq, int64_t pos, int kv, int g,
                     int d, int G, int D, int dtype);

/* Fill the synthetic K and V of positions [pos0, pos0+ntok) of one (layer, seq) in the
 * order [tok][kv][g][d] (ntok*2*G*D values of the given dtype: 2 bytes each, 1 byte for fp8). */
void bws_kv_fill(uint64_t seed, uint32_t layer, uint32_t seq, int64_t pos0, int64_t ntok, int G,
                 int D, int dtype, void* dst);

#ifdef __cplusplus
}
#endif

#endif /* BW_SYNTH_H */
