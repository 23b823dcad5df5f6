/*
 * bw.h - C-ABI of the MI355X (gfx950) decode-step library libbw.so.
 *
 * The library runs one autoregressive decode step of a dense or MoE transformer whose linear
 * layers are int4 block-quantised (32 weights per block, one fp16 scale, w = scale * (q - 8)),
 * with grouped-query attention over a paged KV cache. Sources for the operation: the bw24
 * deep-dive page (10100.com) - section 2 (engine core: paged KV manager, dense/MoE model and
 * standard/MTP decoder strategies), section 4 (the Engine facade: callers only prefill and
 * decode; a session shares the weights and owns its KV cache), section 5 stage 4 (the verify
 * kernel unrolls K draft tokens along the sequence dimension over one shared KV cache) and
 * section 6 item 2 (logical sequence positions map to fixed physical pages through a page
 * table) - and the bw24 vs llama.cpp page (devpress.csdn.net) section 2.1 (each new token
 * reads the whole KV cache) and section 2.2 (linear layer and activation fused in one kernel).
 *
 * Conventions for every entry point:
 *  - Return value: BW_OK (0) or a negative BW_E* code. The text of the last error on the
 *    calling thread is returned by bw_last_error(). No C++ exception crosses this boundary.
 *  - Pointers named *_dev are device pointers (hipMalloc'd or from torch); pointers named
 *    *_host are host pointers. `stream` is a hipStream_t (NULL = the default stream).
 *  - Device work is enqueued asynchronously on `stream`; nothing here synchronises the stream
 *    except the calls documented as synchronous (model load, pool create/synthesise/read,
 *    bw_check_device_error, the debug readers).
 *  - Ownership: handles are owned by the caller until the matching *_free. The library owns
 *    all weight, KV-pool and workspace device memory behind a handle; it allocates at create
 *    time only and allocates nothing in bw_decode_step. Caller buffers are borrowed for the
 *    duration of the enqueued work.
 *  - Errors detected on the device (a page id or token id out of range) never fault: the
 *    offending read or write is skipped and a bit is set in the model's device error word,
 *    returned by bw_check_device_error.
 */
#ifndef BW_H
#define BW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define BW_OK 0
#define BW_EINVAL (-1)  /* bad argument (null pointer, size out of range, inconsistent shape) */
#define BW_ENOMEM (-2)  /* device or host allocation failed */
#define BW_EHIP (-3)    /* a HIP runtime call failed */
#define BW_ERANGE (-4)  /* a size exceeds what the handle was created for */
#define BW_ESTATE (-5)  /* handle used in the wrong state (e.g. pool of another model) */

/* KV cache element types */
#define BW_KV_F16 1
#define BW_KV_BF16 2
/* OCP FP8 E4M3 (one byte per element; no scale): a key or value is rounded to nearest, ties to
 * even, and saturates at +-448. The low-precision cache variant on CDNA4 of the pages' FP8 paths
 * ("Deep dive: bw24", section 1 and the comparison table of section 7). Halves the KV bytes. */
#define BW_KV_FP8 3

/* device error bits (bw_check_device_error) */
#define BW_DERR_PAGE 1   /* a page-table entry was outside [0, n_pages) */
#define BW_DERR_TOKEN 2  /* a token id was outside [0, vocab) */
#define BW_DERR_POS 4    /* a position seq_lens[b] + i was outside [0, max_positions) */
#define BW_DERR_PERSIST 8 /* the single-launch step gave up waiting (its deadline passed); later
                           * single-launch steps return at once until bw_check_device_error */

typedef struct bw_model bw_model;
typedef struct bw_kv_pool bw_kv_pool;
typedef struct bw_kv_tier bw_kv_tier;
typedef struct bw_expert_tier bw_expert_tier;

/* Model shape. Dense models set n_experts = 0; MoE models set ffn_dim = 0 and the expert
 * fields. All layers share one shape. */
typedef struct {
  int32_t n_layers;
  int32_t d_model;      /* multiple of 32 */
  int32_t n_q_heads;    /* multiple of n_kv_heads */
  int32_t n_kv_heads;
  int32_t head_dim;     /* 64 or 128 */
  int32_t ffn_dim;      /* dense SwiGLU width (multiple of 32) */
  int32_t vocab;
  float rms_eps;        /* RMSNorm epsilon (1e-6) */
  double rope_base;     /* RoPE base (1e6) */
  int32_t n_experts;    /* routed experts (MoE), 0 for dense */
  int32_t top_k;        /* experts per token (MoE) */
  int32_t expert_ffn;   /* SwiGLU width of a routed expert */
  int32_t n_shared;     /* ungated shared experts (MoE) */
  int32_t shared_ffn;   /* SwiGLU width of a shared expert */
  int32_t kv_dtype;     /* BW_KV_F16, BW_KV_BF16 or BW_KV_FP8 */
  int32_t page_tokens;  /* tokens per KV page; must be 16 */
  int32_t max_positions;/* largest position + 1 any step may use (RoPE table length) */
  int32_t max_tokens;   /* largest batch * t of one step (workspace size) */
} bw_model_config;

/* Create a model whose weights are generated from `seed` by the seeded input generator:
 * int4 codes uniform on 0..15, block scales fp16(|0.02 z|), embeddings fp16(z), norm gains
 * fp16(1 + 0.1 z), router fp16(0.02 z) (z standard normal). Generation runs on host threads;
 * the weights are then copied to the current HIP device. Synchronous.
 * Errors: BW_EINVAL for an unsupported shape, BW_ENOMEM, BW_EHIP. */
int bw_model_load_synthetic(const bw_model_config* cfg, uint64_t seed, bw_model** out);

/* Release a model and all device memory it owns. NULL is accepted. */
int bw_model_free(bw_model* model);

/* Copy one of the model's tensors to host memory in the canonical layout, so that a checker can
 * compare the library's weights with its own copy of the generated ones ("Deep dive: bw24",
 * section 4: one Engine owns the loaded weights that every session shares). Names:
 *   "embed" fp16 [vocab][d_model], "final_norm" fp16 [d_model],
 *   "lm_head.codes", "lm_head.scales",
 *   "layers.L.attn_norm", "layers.L.ffn_norm" fp16 [d_model],
 *   "layers.L.M.codes", "layers.L.M.scales" with M = qkv, o, gate, up, down (dense models),
 *   "layers.L.router" fp16 [n_experts][d_model] and "layers.L.experts.E.M.codes|scales",
 *   "layers.L.shared.S.M.codes|scales" with M = gate, up, down (MoE models).
 * An int4 matrix [N][K] exports as codes u8 [N][K/2] (canonical row order; block b of a row is
 * bytes 16b..16b+15, byte i holds element i in bits 0-3 and element i+16 in bits 4-7) and scales
 * fp16 [N][K/32] (one per block, canonical order), whatever its device tiling; QKV rows are q
 * heads, then k, then v. `bytes` must equal the tensor's size (bw_model_tensor_bytes).
 * Synchronous (waits for the device). Errors: BW_EINVAL (null argument, unknown name),
 * BW_ERANGE (wrong size), BW_EHIP. */
int bw_model_export_tensor(const bw_model* model, const char* name, void* host_dst, size_t bytes);

/* Size in bytes of a tensor bw_model_export_tensor writes. Errors: BW_EINVAL. */
int bw_model_tensor_bytes(const bw_model* model, const char* name, size_t* bytes);

/* Create a physical KV page pool of n_pages pages for `model`. One page holds page_tokens
 * positions of every layer; its device layout is
 *   pool[layer][page][kv_head][0 = K, 1 = V][slot 0..page_tokens-1][head_dim]
 * in the model's kv_dtype (one page-layer is 64 KiB at 8 KV heads x 128 dims x bf16, 32 KiB
 * with an FP8 cache).
 * The pool is zero-filled. Synchronous. Errors: BW_EINVAL, BW_ENOMEM, BW_EHIP. */
int bw_kv_pool_create(const bw_model* model, int32_t n_pages, bw_kv_pool** out);

/* Release a pool. NULL is accepted. */
int bw_kv_pool_free(bw_kv_pool* pool);

/* Fill every element of the pool with the 16-bit pattern `bits` (e.g. a NaN, to show that a
 * step never reads a slot it should not); an FP8 pool takes the low byte of `bits`.
 * Asynchronous on stream. */
int bw_kv_pool_fill(bw_kv_pool* pool, uint16_t bits, void* stream);

/* Write synthetic cached context: for sequence b (0 <= b < batch) and every layer, positions
 * [0, seq_lens_host[b]) receive the generator's synthetic K/V for (seed, layer, seq_ids_host[b])
 * (values c / 64 with c = (h & 0xFF) - 128, or (c >> 3) / 8 for an FP8 cache: exact in the
 * cache dtype), stored at page
 * page_table_host[b * max_pages + pos / page_tokens], slot pos % page_tokens.
 * Host pointers; synchronous. Errors: BW_EINVAL (a needed page id out of range). */
int bw_kv_pool_synthesize(bw_kv_pool* pool, uint64_t seed, const int32_t* seq_ids_host,
                          const int32_t* seq_lens_host, const int32_t* page_table_host,
                          int32_t batch, int32_t max_pages);

/* The same synthetic context from device arrays, queued on `stream` (no host round trip, nothing
 * allocated): seq_ids_dev [batch] (NULL: sequence b has id b), seq_lens_dev [batch] and
 * page_table_dev [batch * max_pages] are read by the kernel, which writes exactly the bits of
 * bw_kv_pool_synthesize (the generator is implemented on the device from the same definition).
 * The caller keeps the three arrays alive until the work on `stream` completes. The paged cache
 * that maps logical positions to fixed-size physical pages is the deep-dive page's (section 6
 * item 2). Errors: BW_EINVAL (null pool or array, batch outside [1, 65535], max_pages < 1),
 * BW_EHIP (launch). Range errors found on the device set bits in the device error word
 * (bw_check_device_error): BW_DERR_PAGE for a needed page id outside [0, n_pages) (that page is
 * skipped), BW_DERR_POS for a negative length or one needing more than max_pages pages (the
 * first max_pages pages are written). */
int bw_kv_pool_synthesize_async(bw_kv_pool* pool, uint64_t seed, const int32_t* seq_ids_dev,
                                const int32_t* seq_lens_dev, const int32_t* page_table_dev,
                                int32_t batch, int32_t max_pages, void* stream);

/* Copy one page-layer (n_kv_heads * 2 * page_tokens * head_dim elements, 2 bytes each or 1 for
 * FP8, in the pool layout above) to host memory. Synchronous. Errors: BW_EINVAL, BW_ERANGE. */
int bw_kv_pool_read(const bw_kv_pool* pool, int32_t layer, int32_t page, void* host_dst,
                    size_t bytes);

/* ---- host tier of the pool (L2 residency) ----
 * The deep-dive page ("Deep dive: bw24", section 6 item 3, Hy3 overflow) keeps hot KV pages in
 * VRAM and moves cold ones to locked host memory over PCIe, choosing them by their access time
 * stamps (least recently used first); a read of a page under migration waits for the copy. Here
 * a page is one physical page id across all layers (n_layers page-layers). The tier owns pinned
 * host memory (hipHostMalloc) for `host_pages` such pages and a copy stream of the default
 * priority. The caller owns the page tables: it decides where a restored page goes and maps it.
 *
 * Ordering: evict and restore queue their copies on the tier's stream after the work already
 * queued on the caller's `stream` (the steps that wrote or still read those pages). Before the
 * caller's stream reads a restored page, or writes a device page whose contents were just
 * evicted, it must call bw_kv_tier_wait (the dirty-page wait). Not thread-safe. */

/* Create the host tier. Synchronous. Errors: BW_EINVAL, BW_ENOMEM (pinned allocation), BW_EHIP. */
int bw_kv_tier_create(bw_kv_pool* pool, int32_t host_pages, bw_kv_tier** out);

/* Wait for the tier's copies and release it. NULL is accepted. */
int bw_kv_tier_free(bw_kv_tier* tier);

/* Record that a step reads the pages mapped for positions [0, seq_lens[b] + tokens) of each of
 * `batch` sequences (host arrays; page_table [batch][max_pages]): their access time becomes the
 * tier's clock, which then advances by one. Touched pages are resident (evictable). Errors:
 * BW_EINVAL (a needed page id out of range). */
int bw_kv_tier_touch(bw_kv_tier* tier, const int32_t* page_table_host, const int32_t* seq_lens_host,
                     int32_t batch, int32_t tokens, int32_t max_pages);

/* Evict up to n resident pages, least recently touched first (ties: lower page id), limited by
 * the free host slots: dev_pages_out[i] was copied to host slot host_slots_out[i], i < *n_out.
 * The pages are no longer resident; their device memory may be reused after bw_kv_tier_wait.
 * Asynchronous. Errors: BW_EINVAL, BW_EHIP. */
int bw_kv_tier_evict_lru(bw_kv_tier* tier, int32_t n, int32_t* dev_pages_out, int32_t* host_slots_out,
                         int32_t* n_out, void* stream);

/* Copy host slot host_slots[i] back to device page dev_pages[i] (any page id; the caller maps it
 * in its page table) for i < n, and free the slots. The pages become resident, touched now.
 * Asynchronous; bw_kv_tier_wait before a step reads them. Errors: BW_EINVAL (a slot holding no
 * page, a page out of range, a repeated slot or page), BW_EHIP. */
int bw_kv_tier_restore(bw_kv_tier* tier, const int32_t* host_slots, const int32_t* dev_pages, int32_t n,
                       void* stream);

/* Make `stream` wait for every copy the tier has queued so far. Errors: BW_EINVAL, BW_EHIP. */
int bw_kv_tier_wait(bw_kv_tier* tier, void* stream);

/* Resident device pages and occupied host slots. */
int bw_kv_tier_stats(const bw_kv_tier* tier, int32_t* resident_pages, int32_t* host_pages_used);

/* The eviction order alone (host arrays, no device): the up-to-n entries p with resident[p] != 0
 * of smallest stamps[p], ties to the lower p, in that order. Errors: BW_EINVAL. */
int bw_kv_lru_select(const uint64_t* stamps, const uint8_t* resident, int32_t n_pages, int32_t n,
                     int32_t* out, int32_t* n_out);

/* ---- host tier of the routed expert weights (MoE) ----
 * The deep-dive page ("Deep dive: bw24", section 6 item 3, the VRAM tier of Hy3; the comparison
 * table of section 7, memory and model management) keeps the weights of the currently active
 * experts in VRAM and moves cold ones to locked host memory by access time. Here a routed expert
 * (gate/up and down matrices, codes and scales) sits either in a device region or in a pinned
 * host slot, and the step's kernels read it wherever it is, through the model's per-layer expert
 * pointer tables: an expert on the host is read over PCIe by the kernels themselves, so every
 * step stays complete, only slower. Evicting an expert copies it to a host slot and repoints the
 * tables; its device region joins a free list. Restoring takes any free region (routed experts
 * all have one size) and copies the expert back. Copies and table updates are queued on the
 * caller's stream after the work already queued there. Shared experts always stay on the device.
 * Not thread-safe; free the tier before its model. */

/* Create the tier with `host_slots` pinned host slots (hipHostMalloc, one routed expert each).
 * Synchronous. Errors: BW_EINVAL, BW_ESTATE (a dense model), BW_ENOMEM, BW_EHIP. */
int bw_expert_tier_create(bw_model* model, int32_t host_slots, bw_expert_tier** out);

/* Restore every evicted expert (queued on `stream`), wait for the stream and release the tier.
 * NULL is accepted. Errors: BW_EHIP (the tier is then kept). */
int bw_expert_tier_free(bw_expert_tier* tier, void* stream);

/* Record the experts that the last bw_decode_step routed rows [0, n_rows) to: their access time
 * becomes the tier's clock, which then advances. Experts routed while on the host are marked for
 * bw_expert_tier_restore_routed. Synchronises `stream`. Errors: BW_EINVAL, BW_ERANGE, BW_EHIP. */
int bw_expert_tier_touch(bw_expert_tier* tier, int32_t n_rows, void* stream);

/* Evict up to n device-resident routed experts, least recently routed first (ties: lower layer,
 * then lower expert index), limited by the free host slots: (layers_out[i], experts_out[i]) for
 * i < *n_out. Asynchronous on `stream`. Errors: BW_EINVAL, BW_EHIP. */
int bw_expert_tier_evict_lru(bw_expert_tier* tier, int32_t n, int32_t* layers_out, int32_t* experts_out,
                             int32_t* n_out, void* stream);

/* Bring one evicted expert back into a free device region. Asynchronous on `stream`.
 * Errors: BW_EINVAL (out of range, or the expert is on the device), BW_EHIP. */
int bw_expert_tier_restore(bw_expert_tier* tier, int32_t layer, int32_t expert, void* stream);

/* Restore every expert that the last touched step routed to while it was on the host (hot
 * experts come back); *n_out receives their number. Asynchronous on `stream`. */
int bw_expert_tier_restore_routed(bw_expert_tier* tier, int32_t* n_out, void* stream);

/* Routed experts on the device and on the host. */
int bw_expert_tier_stats(const bw_expert_tier* tier, int32_t* resident, int32_t* on_host);

/* One decode step for `batch` sequences of `t` new tokens each (t = 1: plain decode; t > 1:
 * the verify step of speculative decoding, the t tokens laid out along the sequence).
 * Defined by the deep-dive page ("Deep dive: bw24", 10100.com): section 5 stage 4 (the verify
 * kernel takes the drafted tokens along the sequence dimension in one pass), section 6 item 2 (the
 * paged cache maps logical positions to fixed-size physical pages), and section 1 with the section 7
 * comparison table (the output equals token-by-token greedy argmax decoding); the bw24 vs
 * llama.cpp page (devpress.csdn.net) section 2.1 (each new token reads the whole cache).
 *   tokens_dev     int32 [batch * t]   token ids, row b*t + i is token i of sequence b
 *   seq_lens_dev   int32 [batch]       positions already cached BEFORE this call; token i of
 *                                      sequence b is at position seq_lens[b] + i
 *   page_table_dev int32 [batch * max_pages]  physical page of logical page j of sequence b;
 *                                      pages 0 .. (seq_lens[b] + t - 1) / page_tokens must be
 *                                      mapped (entries beyond may hold anything)
 *   logits_dev     float [batch * t * vocab] output logits, or NULL
 *   argmax_dev     int32 [batch * t]   greedy token per row (lowest index on ties), or NULL
 * The keys and values of all new tokens are written into the pool first; token i then attends
 * causally to positions 0 .. seq_lens[b] + i. The caller advances seq_lens afterwards.
 * The step's kernels are captured once per distinct argument set (pointers and sizes) into a
 * hipGraph on an internal stream and replayed on `stream`; the device buffers are read at
 * replay time, so a caller that keeps its buffers and updates their contents on the device
 * (e.g. feeding argmax_dev back as tokens_dev) replays one graph. The first call with a new
 * argument set pays the capture; no device memory is allocated by the library and the stream
 * is not synchronised.
 * Errors: BW_EINVAL (null handle or buffer, t < 1, batch < 1, pool of another model),
 * BW_ERANGE (batch * t > max_tokens). Page or token ids out of range are device errors. */
int bw_decode_step(bw_model* model, bw_kv_pool* pool, const int32_t* tokens_dev,
                   const int32_t* seq_lens_dev, const int32_t* page_table_dev, int32_t batch,
                   int32_t t, int32_t max_pages, float* logits_dev, int32_t* argmax_dev,
                   void* stream);

/* Turn step capture on (default) or off (every call then launches its kernels directly). */
int bw_set_graphs(bw_model* model, int32_t enable);

/* Batch-1 decode steps (batch = 1, t = 1) of a dense model run as ONE kernel launch when this is
 * on and the model's shape has a single-launch form: every layer's phases (QKV + RoPE + KV append,
 * attention, merge, O, gate/up, down) and the lm_head run in one resident workgroup per CU, and
 * the phases hand their small output vectors to each other through device memory, so the weight
 * stream is not broken by kernel boundaries (bw24 vs llama.cpp page, section 2.2: launches and
 * intermediate round trips are what fusion removes). Results match the kernel chain to fp32
 * rounding (exchanged activations keep 21 mantissa bits). Other steps, MoE models and traced steps
 * use the kernel chain.
 *   mode 0: off (kernel chain);
 *   mode 1 (default): on, ordinary launch of one workgroup per CU (the model load checked that
 *           one fits per CU, so on an otherwise idle GPU all are resident together);
 *   mode 2: on, cooperative launch (the runtime guarantees co-residency or refuses the launch).
 * Every wait inside the step is bounded either way (bw_debug_single_launch_deadline), so a
 * workgroup that cannot start never hangs the step: it ends with BW_DERR_PERSIST.
 * *available_out (may be NULL) receives 1 when the model has the single-launch form, else 0.
 * Errors: BW_EINVAL (null model, mode outside 0..2). */
int bw_set_single_launch(bw_model* model, int32_t mode, int32_t* available_out);

/* Row count from which a step (and bw_debug_matvec) runs its dense matrices -- QKV, O, gate/up,
 * down, lm_head -- as one int4 GEMM on the matrix cores over all batch * t rows, reading each
 * weight once (bw24 deep-dive page, section 5, stage 4: the drafted tokens of a verify step are
 * extra rows of one pass over the weights). Below it each row takes its own GEMV pass. 0 turns
 * the GEMM path off. Default 8. Routed experts always take the GEMV path.
 * Errors: BW_EINVAL (null model, min_rows < 0). */
int bw_set_gemm_min_rows(bw_model* model, int32_t min_rows);

/* Text of the last error on this thread ("" if none). */
const char* bw_last_error(void);

/* Greedy acceptance after a verify step: the bookkeeping of speculative decoding, on the device.
 * bw24 deep-dive page: section 1 (speculative output must equal plain token-by-token argmax
 * decoding), section 2 (the engine's verify-accept logic with a ring buffer of drafts and
 * logits), section 5 stage 4 (after the first mismatching draft the later positions' logits are
 * forced to -inf).
 * Row b*t + i of a bw_decode_step call with t tokens per sequence holds input x_i (x_0: the
 * last committed token, not yet cached; x_1..x_{t-1}: drafts) and its greedy token a_i. Draft
 * x_{j+1} is accepted while x_1..x_j were and x_{j+1} == a_j; with n accepted, a_0..a_n are
 * this step's committed tokens.
 *   tokens_dev   int32 [batch * t]  in: the step's inputs; out: tokens[b*t] = a_n, the next
 *                                   step's x_0 (the caller writes the next drafts into the rest)
 *   argmax_dev   int32 [batch * t]  the step's argmax output
 *   logits_dev   float [batch * t * vocab] the step's logits, or NULL; rows i > n become -inf
 *   seq_lens_dev int32 [batch]      in/out: advanced by n + 1 (keys and values of x_0..x_n stay;
 *                                   those of rejected drafts lie beyond and are overwritten by the
 *                                   next step before anything attends to them)
 *   ring_dev     int32 [batch * ring_cap] or NULL: committed tokens, token k of sequence b at
 *                                   ring[b * ring_cap + k % ring_cap]
 *   count_dev    int32 [batch] or NULL (with ring_dev): in/out, tokens committed so far
 *   accepted_dev int32 [batch] or NULL: n of this step
 * With t = 1 this is the bookkeeping of plain greedy decoding. Asynchronous on `stream`;
 * allocates nothing.
 * Errors: BW_EINVAL (null model, tokens, argmax or seq_lens; batch or t < 1; ring without
 * count or the reverse; ring_cap < t), BW_ERANGE (batch or t above 65535), BW_EHIP. */
int bw_spec_accept(bw_model* model, int32_t* tokens_dev, const int32_t* argmax_dev, float* logits_dev,
                   int32_t* seq_lens_dev, int32_t* ring_dev, int32_t* count_dev, int32_t ring_cap,
                   int32_t* accepted_dev, int32_t batch, int32_t t, void* stream);

/* Synchronise `stream`, copy the model's device error word to *flags_host (BW_DERR_* bits)
 * and clear it. */
int bw_check_device_error(bw_model* model, void* stream, int32_t* flags_host);

/* ---- MXFP4 weights on the matrix cores ----------------------------------------------------
 * A 4-bit floating-point weight format (bw24 deep-dive page, section 1, quantisation formats,
 * and the performance-strategy row of the section 7 table). The pages' engine uses NVIDIA's
 * NVFP4; the 4-bit float the CDNA4 matrix cores consume is OCP MX MXFP4, defined here: an
 * [N][K] matrix (K a multiple of 32) in blocks of 32 E2M1 elements along K, one E8M0 scale byte
 * per block, w = 2^(e - 127) * element (e = 255 is NaN).
 *   codes : [N][K/2] bytes, row-major; byte i of a row holds element 2i in bits 0-3 and element
 *           2i+1 in bits 4-7.
 *   scales: [N][K/32] E8M0 bytes, row-major.
 * These entry points take device pointers owned by the caller and run asynchronously on
 * `stream`. Products too large for fp32 come out as +-inf. */

/* y = W x for one input vector: x float32 [K], y float32 [N] (vector units; each weight is
 * decoded exactly to fp32 in registers, products and sums in fp32; a block with scale byte 255
 * makes its row NaN). K <= 16384; x 16-byte aligned.
 * Errors: BW_EINVAL (null pointer, N < 1, K not a multiple of 32 in [32, 16384]), BW_EHIP. */
int bw_mx_gemv(const uint8_t* codes_dev, const uint8_t* scales_dev, const float* x_dev, float* y_dev,
               int64_t N, int64_t K, void* stream);

/* Device workspace bytes bw_mx_gemm needs for these sizes on the current device.
 * Errors: BW_EINVAL (null bytes_out, M, N or K out of range). */
int bw_mx_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t* bytes_out);

/* Y = X W^T for M input rows on the scaled matrix cores (bw24 deep-dive page, section 5, stage
 * 4: the rows of a verify or batched step share one pass over the weights): X float32 [M][K]
 * (finite, 16-byte aligned), Y float32 [M][N]. The weights enter the products as stored (E2M1 with their E8M0
 * scales). X is first expanded into three MXFP8 terms (E4M3, one E8M0 scale per 32 along K), each
 * quantising the exact residual of the ones before it, which leaves at most 2^-12 of each
 * 32-element block's largest magnitude; each weight fragment feeds the three scaled products.
 * `workspace` (device, 256-byte aligned, at least bw_mx_gemm_workspace_bytes) holds the terms and
 * any split-K partials; calls sharing a workspace must not overlap. 1 <= M <= 2^22, K <= 2^20.
 * Errors: BW_EINVAL (null pointer, size out of range, misaligned workspace), BW_ERANGE
 * (workspace too small), BW_EHIP. */
int bw_mx_gemm(const uint8_t* codes_dev, const uint8_t* scales_dev, const float* X_dev, float* Y_dev, int64_t M,
               int64_t N, int64_t K, void* workspace, int64_t workspace_bytes, void* stream);

/* ---- parity-test entry points (same kernels as the step, exposed one at a time) ---------- */

/* Matrix selectors */
#define BW_MAT_QKV 0      /* [(Hq + 2 Hkv) * D][d_model]: q rows, then k rows, then v rows */
#define BW_MAT_O 1        /* [d_model][Hq * D]                                            */
#define BW_MAT_GATE 2     /* [ffn][d_model]  (MoE: routed expert `expert`)                 */
#define BW_MAT_UP 3       /* [ffn][d_model]                                                 */
#define BW_MAT_DOWN 4     /* [d_model][ffn]                                                 */
#define BW_MAT_LM_HEAD 5  /* [vocab][d_model]                                               */
#define BW_MAT_SGATE 6    /* shared expert `expert`                                         */
#define BW_MAT_SUP 7
#define BW_MAT_SDOWN 8

/* Dequantise one int4 matrix on the device with a plain kernel (w = s * (q - 8) per element)
 * and write it as fp32 [N][K] in canonical row and column order (dst_dev must hold N*K floats).
 * The step's own in-register unpacks (GEMV, batched GEMM) are checked bit for bit through
 * bw_debug_matvec with one-hot inputs, whose products are exact. Asynchronous. Errors: BW_EINVAL. */
int bw_debug_dequant(const bw_model* model, int32_t which, int32_t layer, int32_t expert,
                     float* dst_dev, void* stream);

/* y[m][n] = sum_k W[n][k] x[m][k] for m < n_vec with the step's GEMV (n_vec = 1) or the
 * batched MFMA path (n_vec > 1), canonical row order. x_dev float [n_vec][K], y_dev float
 * [n_vec][N]. Asynchronous. Errors: BW_EINVAL, BW_ERANGE (n_vec > max_tokens). */
int bw_debug_matvec(bw_model* model, int32_t which, int32_t layer, int32_t expert,
                    const float* x_dev, int32_t n_vec, float* y_dev, void* stream);

/* Attention alone over the pool for layer `layer`: q_dev float [batch * t][Hq][D] (already
 * rotated), causal as in bw_decode_step over positions 0 .. seq_lens[b] + i (the pool must
 * already hold them); out_dev float [batch * t][Hq][D]. Asynchronous. */
int bw_debug_attention(bw_model* model, bw_kv_pool* pool, int32_t layer, const float* q_dev,
                       const int32_t* seq_lens_dev, const int32_t* page_table_dev,
                       int32_t batch, int32_t t, int32_t max_pages, float* out_dev, void* stream);

/* bw_debug_attention for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels, with the
 * split-K partials [batch * t][n_q_heads][splits][head_dim + 2] (splits = ceil(max_pages / 4))
 * in a static device array of the library, 16 MiB per GPU, held until the process ends, instead
 * of the model's workspace. Calls no hipMalloc, hipFree or other allocating routine; the array's
 * device address is looked up once per device (hipGetSymbolAddress) on the first call there.
 * Every call on one GPU shares the array, so calls that overlap on one GPU (other streams or
 * threads) race; a call's partials are all written before they are read, so nothing needs
 * clearing between calls. Asynchronous on stream. Errors: BW_EINVAL (null or non-positive
 * argument), BW_ESTATE (pool of another model), BW_ERANGE (the partials would exceed 16 MiB, or
 * batch or t above 65535), BW_EHIP. */
int bw_attention_noalloc(bw_model* model, bw_kv_pool* pool, int32_t layer, const float* q_dev,
                         const int32_t* seq_lens_dev, const int32_t* page_table_dev, int32_t batch,
                         int32_t t, int32_t max_pages, float* out_dev, void* stream);

/* Round n fp32 values x_dev to the cache dtype kv_dtype with the conversion every kernel uses to
 * store a key or value: bits_dev[i] (uint16; an FP8 code in the low byte) and back_dev[i], the
 * stored value read back as fp32 the way the attention reads it. Asynchronous. Errors: BW_EINVAL. */
int bw_debug_kv_round(int32_t kv_dtype, const float* x_dev, int64_t n, uint16_t* bits_dev, float* back_dev,
                      void* stream);

/* Experts chosen by the last bw_decode_step (MoE): int32 [n_layers][batch * t][top_k],
 * copied to host. Synchronises `stream`. Errors: BW_ESTATE for a dense model. */
int bw_debug_read_experts(bw_model* model, int32_t n_rows, int32_t* host_dst, void* stream);

/* Residual stream after the last layer of the last bw_decode_step: float [batch * t][d_model],
 * copied to host. Synchronises `stream`. */
int bw_debug_read_hidden(bw_model* model, int32_t n_rows, float* host_dst, void* stream);

/* Copy row src of the lm_head (codes and scale) onto row dst, for tests that need two vocabulary
 * rows with bitwise equal logits (the greedy argmax must then take the lower index: "Deep dive:
 * bw24", section 1, output equal to token-by-token argmax decoding). Changes the model's weights.
 * Synchronous. Errors: BW_EINVAL (null model, row out of range), BW_EHIP. */
int bw_debug_copy_lm_head_row(bw_model* model, int32_t src, int32_t dst);

/* Timeout of each wait inside the single-launch step, in ticks of the GPU's 100 MHz real-time
 * counter (default 50,000,000 = 0.5 s). A wait that passes it raises BW_DERR_PERSIST and ends the
 * step on every workgroup; tests use a tiny value to exercise that path.
 * Errors: BW_EINVAL (null model), BW_ESTATE (no single-launch form). */
int bw_debug_single_launch_deadline(bw_model* model, uint64_t ticks);

/* Measurement hook of the single-launch step: while stamps_dev (device, n >= 16 * n_layers + 8
 * uint64) is set, workgroup 0 writes the GPU's 100 MHz real-time counter at each phase start and
 * when the phase's input has arrived: [16 l + 2 k] and [16 l + 2 k + 1] for phases k = 0..5 (QKV,
 * attention, merge, O, gate/up, down) of layer l (MoE models: k = 0..6, QKV, attention, merge, O,
 * router, top-k + expert gate/up, expert down, with [16 l + 14] / [16 l + 15] the start / end of
 * the expert gate/up matrix pass); [16 L + 0 / 1] lm_head start / input ready,
 * [16 L + 2] final argmax, [16 L + 3] step end, [16 L + 4] step start. NULL turns it off. With
 * n >= (16 n_layers + 8) x the step's workgroup count (one per CU), every workgroup w writes the
 * same record at w (16 n_layers + 8) (the final argmax and step end only in workgroup 0).
 * Errors: BW_EINVAL, BW_ESTATE (no single-launch form), BW_ERANGE (n too small). */
int bw_debug_single_launch_stamps(bw_model* model, uint64_t* stamps_dev, int32_t n);

/* ---- measurement hook ------------------------------------------------------------------- */

/* Kernel classes of one step, for bw_set_trace */
#define BW_K_QKV 0        /* RMSNorm + QKV GEMV + RoPE + KV append      */
#define BW_K_ATTN 1       /* split attention + merge                     */
#define BW_K_O 2          /* O GEMV + residual                           */
#define BW_K_GATE_UP 3    /* RMSNorm + gate/up GEMV + SwiGLU (dense)     */
#define BW_K_DOWN 4       /* down GEMV + residual (dense)                */
#define BW_K_LM_HEAD 5    /* final RMSNorm + lm_head GEMV (layer 0 slot) */
#define BW_K_ROUTER 6     /* RMSNorm + router GEMV + top-k (MoE)         */
#define BW_K_MOE_GATE_UP 7/* RMSNorm + selected experts' gate/up + SwiGLU */
#define BW_K_MOE_DOWN 8   /* gated experts' down + shared + residual     */

/* Record hipEvents around one kernel class in later bw_decode_step calls: before and after the
 * launch(es) of class `kernel_class` in layer l, events[2l] and events[2l+1] are recorded on the
 * step's stream (n_layers pairs; BW_K_LM_HEAD uses pair 0). `events` (an array of hipEvent_t
 * owned by the caller) is borrowed until the hook is cleared with events = NULL. For measuring
 * per-launch kernel time in a benchmark; the records add two stream markers per traced launch.
 * Errors: BW_EINVAL. */
int bw_set_trace(bw_model* model, int32_t kernel_class, void* const* events, int32_t n_layers);

#ifdef __cplusplus
}
#endif

#endif /* BW_H */
