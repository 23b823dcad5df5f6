// bw_internal.h - structures shared by the runtime and the kernel launchers of libbw.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bw {

// One int4 matrix on the device.
//  codes : [N][K/2] bytes. Row order is the device order (see the runtime: QKV rows are
//          interleaved in RoPE pairs, gate/up rows are interleaved as (gate_i, up_i)); within a
//          row the canonical block layout is kept: block b is bytes 16b..16b+15, byte i holds
//          element i (low nibble) and element i+16 (high nibble).
//  scales: fp16 [N][lpr][nb] with scales[n][j][c] = scale of block j + lpr*c of row n, so the
//          scales one lane needs for a row are contiguous. lpr = gcd(K/32, 64), nb = K/32/lpr.
struct Mat {
  const uint8_t* codes = nullptr;
  const uint16_t* scales = nullptr;
  int32_t N = 0, K = 0;
  int32_t lpr = 0, nb = 0;
};

// Per-layer expert tables (MoE): device arrays of pointers, routed experts first, then shared.
struct ExpertTab {
  const uint8_t* const* gu_codes = nullptr;   // [E + S] interleaved gate/up [2F][d]
  const uint16_t* const* gu_scales = nullptr;
  const uint8_t* const* dn_codes = nullptr;   // [E + S] down [d][F]
  const uint16_t* const* dn_scales = nullptr;
};

enum InMode { IN_PLAIN = 0, IN_RMSNORM = 1, IN_MOE_DOWN = 2 };
enum EpiMode {
  EPI_STORE = 0,      // y[m][row] = v (device row order)
  EPI_STORE_CANON = 1,// y[m][canonical row] = v (parity tests)
  EPI_RESID = 2,      // y[m][row] += v
  EPI_QKV = 3,        // RoPE pairs, q to qout, k/v rounded into the KV pool
  EPI_SWIGLU = 4,     // rows (2i, 2i+1) = (gate_i, up_i): y[m][i] = silu(g) * u
  EPI_LOGITS = 5,     // y[m][row] = v and per-workgroup argmax partial
  EPI_MOE_SWIGLU = 6  // virtual rows over the selected experts, SwiGLU into y[m][slot*F + i]
};

struct GemvParams {
  Mat w;
  int32_t n_rows;          // rows to compute (== w.N except for MoE virtual rows)
  // input rows: x[m * x_stride + k]
  const float* x = nullptr;
  int64_t x_stride = 0;
  const uint16_t* gamma = nullptr;  // RMSNorm gain (IN_RMSNORM)
  float eps = 1e-6f;
  // IN_RMSNORM of layer 0: the input row is the fp16 embedding of tokens[m] (rows >= vocab set
  // the error word and read row 0); workgroup 0 also stores it to x_out (the residual stream)
  const uint16_t* embed = nullptr;
  const int32_t* tokens = nullptr;
  int32_t vocab = 0;
  float* x_out = nullptr;
  // output
  float* y = nullptr;
  int64_t y_stride = 0;
  // EPI_STORE_CANON: canonical row of each device row; rows whose canonical index falls outside
  // [map_lo, map_lo + map_n) are skipped, the others stored at index - map_lo
  const int32_t* row_map = nullptr;
  int32_t map_lo = 0, map_n = 0x7fffffff;
  // EPI_QKV
  int32_t H = 0, G = 0, D = 0;
  const float2* rope = nullptr;     // [max_pos][D/2] (cos, sin)
  int32_t max_pos = 0;
  const int32_t* seq_lens = nullptr;
  int32_t t = 1;                    // tokens per sequence in this step (row m = b*t + i)
  const int32_t* page_table = nullptr;
  int32_t max_pages = 0;
  uint16_t* pool = nullptr;         // this layer's slice of the pool: [n_pages][G][2][16][D] elements
                                    // of the cache dtype (bytes for FP8, cast on use)
  int64_t pool_page_stride = 0;     // elements per page in the layer slice
  int32_t n_pages = 0;
  int32_t kv_dtype = 2;             // 1 = fp16, 2 = bf16, 3 = FP8 E4M3
  float* qout = nullptr;            // [M][H][D]
  int32_t* err = nullptr;
  // EPI_LOGITS: per-workgroup argmax partials [M][gridDim.x]
  float* amax_val = nullptr;
  int32_t* amax_idx = nullptr;
  // MoE
  const int32_t* sel = nullptr;     // [M][top_k] selected experts
  const float* gates = nullptr;     // [M][top_k] renormalised gates
  int32_t n_experts = 0, top_k = 0, n_shared = 0, Fe = 0, Fs = 0;
  ExpertTab ex;
  int32_t ex_lpr = 0, ex_nb = 0;    // lane split of the MoE virtual down K
};

struct AttnParams {
  const uint16_t* pool = nullptr;   // layer slice [n_pages][G][2][16][D] of the cache dtype (cast on use)
  int64_t pool_page_stride = 0;     // elements per page
  int32_t n_pages = 0;
  const float* q = nullptr;         // [M][H][D] rotated queries
  const int32_t* seq_lens = nullptr;
  const int32_t* page_table = nullptr;
  int32_t max_pages = 0;
  int32_t t = 1, H = 0, G = 0, D = 0;
  int32_t pages_per_split = 4;
  int32_t max_splits = 0;
  float scale = 0.f;                // 1/sqrt(D)
  float* part = nullptr;            // [M][H][max_splits][D + 2] (acc, m, l)
  float* out = nullptr;             // [M][H][D]
  int32_t* err = nullptr;
  int32_t* counters = nullptr;      // [batch][G] split arrival counters, zero between launches
  int32_t mfma = 1;                 // 8..16 query rows per KV head: the matrix-core kernel
};

// The single-launch batch-1 step of a dense model (bw_persist.hip).
struct PLayer {
  Mat qkv, o, gu, dn;               // gu, dn: dense FFN (unused for MoE)
  const uint16_t* attn_norm = nullptr;
  const uint16_t* ffn_norm = nullptr;
  const uint16_t* router = nullptr; // MoE: fp16 [E][d]
  ExpertTab ex;                     // MoE: expert matrices (routed, then shared)
  const uint8_t* dnc = nullptr;     // dense FFN by columns: W_down as per-workgroup column slices
};

constexpr int BW_DERR_PERSIST_BIT = 8;

struct PersistParams {
  const PLayer* layers = nullptr;   // device array [L]
  int32_t L = 0, H = 0, G = 0, V = 0;
  Mat lm;
  const uint16_t* final_norm = nullptr;
  const uint16_t* embed = nullptr;
  float eps = 1e-6f, attn_scale = 0.f;
  const float2* rope = nullptr;
  int32_t max_pos = 0;
  uint16_t* pool = nullptr;         // [L][n_pages][G][2][16][D] of the cache dtype (cast on use)
  int64_t layer_elems = 0, page_elems = 0;  // in elements of the cache dtype
  int32_t n_pages = 0;
  const int32_t* tokens = nullptr;  // [1]
  const int32_t* seq_lens = nullptr;// [1]
  const int32_t* page_table = nullptr;
  int32_t max_pages = 0;
  // exchange words (value with a 2-bit epoch tag in the low mantissa bits)
  uint32_t* xq = nullptr;           // [(H + 2G) D]: rotated q, rounded k and v (canonical dims)
  uint32_t* xp = nullptr;           // [H][splits][D + 2]: attention partials (acc, m, l)
  uint32_t* xa = nullptr;           // [H D]: attention output
  uint32_t* xm = nullptr;           // [d]: residual after attention
  uint32_t* xf = nullptr;           // [F]: SwiGLU output
  uint32_t* xx = nullptr;           // [d]: residual after the FFN (layer input)
  uint32_t* xdp = nullptr;          // FFN by columns: [owners][workgroups][2 x 16-byte-aligned halves] down partials
  int32_t n_xdp = 0;                // words of xdp
  uint64_t* xarg = nullptr;         // [workgroups]: argmax partial (value, index | tag << 30)
  float* logits = nullptr;          // [V] or null
  int32_t* argmax = nullptr;        // [1] or null
  uint32_t* epoch = nullptr;        // [1] steps run so far (tags derive from it)
  int32_t* err = nullptr;
  uint32_t* abort_flag = nullptr;
  uint64_t deadline_ticks = 50000000ull;  // one wait gives up after 0.5 s (100 MHz counter)
  // MoE (moe != 0): E experts, top_k routed + n_shared shared, each FFN width Fe
  int32_t moe = 0, E = 0, top_k = 0, n_shared = 0, Fe = 0;
  uint32_t* xr = nullptr;           // [E]: router logits (exchange)
  int32_t* sel_out = nullptr;       // optional: selected experts of layer l at sel_out[l * sel_stride + k]
  int64_t sel_stride = 0;
  uint64_t* stamps = nullptr;       // optional [L * 16 + 8]: real-time counter at phase starts (workgroup 0)
  int32_t stamp_stride = 0;         // > 0: every workgroup w writes its own record at w * stamp_stride
  bool plain_launch = false;        // ordinary launch instead of the cooperative one (see the runtime)
};

// launchers (bw_gemv.hip, bw_attn.hip, bw_misc.hip)
int launch_gemv(int in_mode, int epi, const GemvParams& p, int M, hipStream_t s, int* grid_out = nullptr);
int gemv_lane_split(int K, int* lpr, int* nb);
int launch_attention(const AttnParams& p, int kv_dtype, int batch, hipStream_t s);
int launch_embed(const uint16_t* embed, int32_t vocab, int32_t d, const int32_t* tokens, int M,
                 float* x, int32_t* err, hipStream_t s);
int launch_argmax_final(const float* val, const int32_t* idx, int parts, int M, int32_t* out,
                        hipStream_t s);
int launch_router(const uint16_t* wr, int E, int d, const float* x, const uint16_t* gamma,
                  float eps, int M, float* logits, hipStream_t s);
int launch_topk(const float* logits, int E, int k, int M, int32_t* sel, float* gates,
                hipStream_t s);
int launch_dequant(const Mat& w, const int32_t* row_map, int map_lo, int map_n, float* dst, hipStream_t s);
int launch_fill16(uint16_t* dst, size_t n, uint16_t bits, hipStream_t s);
int launch_kv_round(int kv_dtype, const float* x, int64_t n, uint16_t* bits, float* back, hipStream_t s);
// KV host tier: page ids of one packing launch, passed by value
struct PageList {
  static constexpr int kMax = 128;
  int32_t id[kMax];
};
// MXFP4 weights (bw_mx.hip)
constexpr int kMxGemvMaxK = 16384;
int launch_mx_gemv(const uint8_t* codes, const uint8_t* scales, const float* x, float* y, int64_t N, int K,
                   hipStream_t st);
int launch_mx_quant(const float* X, uint8_t* xq, uint32_t* xs, int64_t M, int K, int Kp, float* Y_zero,
                    int64_t y_elems, hipStream_t st);
int mx_gemm_splits(int64_t M, int64_t N, int K);
int64_t mx_gemm_workspace_bytes(int64_t M, int64_t N, int K, int splits);
int launch_mx_gemm(const uint8_t* codes, const uint8_t* scales, const float* X, float* Y, int64_t M, int64_t N,
                   int K, void* ws, int splits, hipStream_t st);
int launch_set_expert(const ExpertTab& tab, int e, const void* gc, const void* gs, const void* dc, const void* ds,
                      hipStream_t s);
int launch_page_pack(uint8_t* pool, int64_t layer_bytes, int64_t page_bytes, int L, const PageList& ids, int n,
                     uint8_t* stage, bool to_stage, hipStream_t s);

// batched path (bw_gemm.hip): matrix-core GEMM over all rows of a step. IN_PLAIN / IN_RMSNORM
// (rms = per-row RMSNorm factors from launch_rowrms); epilogues STORE_CANON, RESID, SWIGLU, LOGITS,
// QKV. part: gemm_part_elems(N, K, M) floats of k-split partials.
bool gemm_supported(int N, int K);
int gemm_ksplit(int N, int K, int M);
int64_t gemm_part_elems(int N, int K, int M);
int launch_gemm(int in_mode, int epi, const GemvParams& p, int M, const float* rms, float* part, uint16_t* xs,
                hipStream_t s);  // xs: [2][M][K] fp16 staging of X
int launch_rowrms(const float* x, int64_t stride, int K, float eps, int M, float* r, hipStream_t s);
// val / idx: at least M * max_parts partials (the lm_head's argmax workspace)
int launch_argmax_rows(const float* logits, int64_t ld, int N, int M, float* val, int32_t* idx, int max_parts,
                       int32_t* out, hipStream_t s);

// greedy acceptance after a verify step (bw_spec.hip)
int launch_spec_accept(int32_t* tokens, const int32_t* argmax, float* logits, int64_t V, int32_t* seq_lens,
                       int32_t* ring, int32_t* count, int cap, int32_t* accepted, int batch, int t, hipStream_t s);

// single-launch step (bw_persist.hip): -2 when (d, F, head dim, query heads per KV head) has no
// instantiation; query_only checks that one workgroup of it fits a CU
int launch_persist(const PersistParams& p, int d, int F, int kv_dtype, int D, int rep, int nwg, hipStream_t s,
                   bool query_only);
int launch_persist_reset(const PersistParams& p, int n_q, int n_p, int n_a, int n_d, int n_f, int n_arg, hipStream_t s);
// FFN by columns in the single launch: bytes of one layer's W_down column-slice copy for this
// shape and grid (0: the shape keeps the FFN by rows), and the kernel that writes that copy from
// the device matrix
int64_t persist_colffn_bytes(int d, int F, int nwg);
int64_t persist_colffn_xdp_words(int d, int F, int nwg);  // words of the partial-sum exchange
int launch_down_slices(const Mat& dn, int nwg, uint8_t* out, hipStream_t s);
// MoE form (router, top-k and expert phases): -2 when the shape has no instantiation
int launch_persist_moe(const PersistParams& p, int d, int kv_dtype, int D, int rep, int nwg, hipStream_t s,
                       bool query_only);

}  // namespace bw
