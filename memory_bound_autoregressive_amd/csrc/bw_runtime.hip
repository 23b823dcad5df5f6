// bw_runtime.hip - host side of libbw: model and pool objects, weight generation and layout, the
// decode-step launch sequence and the C-ABI entry points declared in include/bw.h.
//
// The step (bw24 deep-dive page, section 4: callers only prefill and decode; section 2: dense and
// MoE model strategies, standard and verify decoders) for M = batch * t token rows:
//   embed -> per layer [RMSNorm + QKV GEMV + RoPE + KV append] -> [split attention + merge]
//   -> [O GEMV + residual] -> dense: [RMSNorm + gate/up GEMV + SwiGLU] -> [down GEMV + residual]
//                             MoE:   [RMSNorm + router] -> [top-k] -> [RMSNorm + expert gate/up +
//                                    SwiGLU] -> [gated expert down + shared + residual]
//   -> [final RMSNorm + lm_head GEMV + argmax partials] -> [argmax].
// Every launch is enqueued on the caller's stream; nothing is allocated and nothing synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <functional>
#include <map>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "bw.h"
#include "bw_common.h"
#include "bw_internal.h"
#include "bw_synth.h"

using namespace bw;

// ---------------------------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------------------------

static thread_local std::string g_err;

static int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define HIP_OK(expr)                                                                        \
  do {                                                                                      \
    hipError_t e_ = (expr);                                                                 \
    if (e_ != hipSuccess) return fail(BW_EHIP, "%s: %s", #expr, hipGetErrorString(e_));    \
  } while (0)

// ---------------------------------------------------------------------------------------------
// host threads
// ---------------------------------------------------------------------------------------------

static int host_threads() {
  unsigned n = std::thread::hardware_concurrency();
  if (n == 0) n = 4;
  return (int)std::min(n, 16u);
}

template <class F>
static void parallel_for(int64_t n, F fn) {
  const int T = (int)std::min<int64_t>(host_threads(), std::max<int64_t>(n, 1));
  std::vector<std::thread> th;
  for (int t = 0; t < T; ++t)
    th.emplace_back([=] {
      for (int64_t i = t; i < n; i += T) fn(i);
    });
  for (auto& x : th) x.join();
}

// ---------------------------------------------------------------------------------------------
// device arena: weights live in a few large allocations
// ---------------------------------------------------------------------------------------------

struct Arena {
  std::vector<void*> blocks;
  char* cur = nullptr;
  size_t left = 0;
  int alloc(size_t bytes, void** out) {
    bytes = (bytes + 255) & ~(size_t)255;
    if (bytes > left) {
      size_t sz = std::max<size_t>(bytes, (size_t)1 << 30);
      void* p = nullptr;
      if (hipMalloc(&p, sz) != hipSuccess) return fail(BW_ENOMEM, "hipMalloc(%zu) failed", sz);
      blocks.push_back(p);
      cur = (char*)p;
      left = sz;
    }
    *out = cur;
    cur += bytes;
    left -= bytes;
    return 0;
  }
  void release() {
    for (void* p : blocks) (void)hipFree(p);
    blocks.clear();
    cur = nullptr;
    left = 0;
  }
};

// ---------------------------------------------------------------------------------------------
// objects
// ---------------------------------------------------------------------------------------------

struct LayerDev {
  uint16_t* attn_norm = nullptr;
  uint16_t* ffn_norm = nullptr;
  Mat qkv, o, gu, dn;            // dense gate/up interleaved, down
  uint16_t* router = nullptr;    // MoE [E][d]
  ExpertTab ex;                  // MoE device pointer tables
  std::vector<Mat> ex_gu, ex_dn; // MoE descriptors (routed then shared)
};

struct bw_model {
  bw_model_config c{};
  uint64_t seed = 0;
  Arena arena;
  std::vector<void*> ws;         // workspace allocations
  uint16_t* embed = nullptr;
  uint16_t* final_norm = nullptr;
  Mat lm;
  std::vector<LayerDev> L;
  float2* rope = nullptr;
  int32_t* qkv_map = nullptr;    // device row -> canonical row
  std::map<int, int32_t*> gu_map;// F -> [2F] device row -> (gate i -> i, up i -> F + i)
  // workspace
  float* x = nullptr;            // [T][d] residual stream
  float* q = nullptr;            // [T][H][D]
  float* attn_part = nullptr;    // [T][H][max_splits][D+2]
  float* attn_out = nullptr;     // [T][H*D]
  int32_t* attn_cnt = nullptr;   // [T][G] split counters (zero between launches)
  float* act = nullptr;          // [T][act_width]
  int64_t act_width = 0;
  float* logits = nullptr;       // [T][V]
  float* amax_val = nullptr;     // [T][lm_parts]
  int32_t* amax_idx = nullptr;
  int lm_parts = 0;
  float* router_logits = nullptr;// [T][E]
  int32_t* sel = nullptr;        // [L][T][k]
  float* gates = nullptr;        // [L][T][k]
  int32_t* err = nullptr;
  int pages_per_split = 4;
  int max_splits = 0;
  // batched path: steps with at least gemm_min_rows rows run the dense matrices as MFMA GEMMs
  float* gemm_part = nullptr;    // k-split partials of the largest dense GEMM
  uint16_t* gemm_x = nullptr;    // X of a GEMM as staged fp16 pairs [2][T][K max]
  float* rms = nullptr;          // [T] RMSNorm factors
  int gemm_min_rows = 8;
  // single-launch batch-1 step (dense models): exchange buffers and switches
  bool persist_ok = false;       // an instantiation exists and fits
  bool use_persist = true;
  int persist_nwg = 0;           // workgroups (one per CU)
  PersistParams pp{};            // step-independent parameters
  int n_xq = 0, n_xp = 0, n_xa = 0, n_xd = 0, n_xf = 0;
  // measurement hook
  int trace_class = -1;
  std::vector<hipEvent_t> trace_ev;
  // captured steps: one hipGraph per distinct argument set, replayed on the caller's stream
  hipStream_t cap_stream = nullptr;
  struct GraphEntry {
    std::vector<uintptr_t> key;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    uint64_t last_use = 0;
  };
  std::vector<GraphEntry> graphs;
  uint64_t use_clock = 0;
  bool use_graphs = true;
};

struct bw_kv_pool {
  const bw_model* m = nullptr;
  int32_t n_pages = 0;
  uint16_t* data = nullptr;      // elements of the cache dtype (bytes for FP8)
  int64_t page_elems = 0;        // elements of one page-layer
  int64_t layer_elems = 0;       // n_pages * page_elems
  int es = 2;                    // bytes per element
  // layer l's slice
  uint16_t* layer(int l) const { return (uint16_t*)((uint8_t*)data + (int64_t)l * layer_elems * es); }
};

static bool is_moe(const bw_model_config& c) { return c.n_experts > 0; }

// ---------------------------------------------------------------------------------------------
// weight layout
// ---------------------------------------------------------------------------------------------

// Retile fp16 scales [N][K/32] -> [N][lpr][nb] (scale of block j + lpr*c at [n][j][c]).
static void retile_scales(const uint16_t* src, int64_t N, int K, int lpr, int nb, uint16_t* dst) {
  const int nblk = K / 32;
  for (int64_t n = 0; n < N; ++n)
    for (int j = 0; j < lpr; ++j)
      for (int c = 0; c < nb; ++c) dst[n * nblk + j * nb + c] = src[n * nblk + j + lpr * c];
}

// Generate a matrix into host buffers, reorder its rows with dev_of_canon (nullptr = identity),
// retile the scales and upload it.
struct HostMat {
  std::vector<uint8_t> codes;
  std::vector<uint16_t> scales;
};

static void gen_canonical(uint64_t seed, uint32_t kind, uint32_t layer, uint32_t expert, int64_t N,
                          int K, HostMat& h) {
  h.codes.resize((size_t)N * K / 2);
  h.scales.resize((size_t)N * K / 32);
  const int64_t chunk = 512;
  const int64_t nchunks = (N + chunk - 1) / chunk;
  parallel_for(nchunks, [&](int64_t ci) {
    int64_t r0 = ci * chunk, nr = std::min(chunk, N - r0);
    bws_int4_matrix(seed, kind, layer, expert, N, K, r0, nr, h.codes.data() + r0 * (K / 2),
                    h.scales.data() + r0 * (K / 32));
  });
}

static int upload_mat(bw_model* m, const HostMat& h, int64_t N, int K,
                      const std::vector<int64_t>* canon_of_dev, Mat* out) {
  int lpr, nb;
  gemv_lane_split(K, &lpr, &nb);
  std::vector<uint8_t> codes((size_t)N * K / 2);
  std::vector<uint16_t> sc_perm((size_t)N * K / 32), sc((size_t)N * K / 32);
  const int64_t rb = K / 2, sb = K / 32;
  parallel_for(N, [&](int64_t d) {
    int64_t cr = canon_of_dev ? (*canon_of_dev)[d] : d;
    memcpy(&codes[d * rb], &h.codes[cr * rb], rb);
    memcpy(&sc_perm[d * sb], &h.scales[cr * sb], sb * 2);
  });
  retile_scales(sc_perm.data(), N, K, lpr, nb, sc.data());
  void *pc, *ps;
  if (int rc = m->arena.alloc(codes.size(), &pc)) return rc;
  if (int rc = m->arena.alloc(sc.size() * 2, &ps)) return rc;
  HIP_OK(hipMemcpy(pc, codes.data(), codes.size(), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(ps, sc.data(), sc.size() * 2, hipMemcpyHostToDevice));
  out->codes = (const uint8_t*)pc;
  out->scales = (const uint16_t*)ps;
  out->N = (int32_t)N;
  out->K = K;
  out->lpr = lpr;
  out->nb = nb;
  return 0;
}

// QKV device order: within the q block and the k block, the rows of each head are reordered to
// (0, D/2, 1, D/2 + 1, ...) so that the two rows of every RoPE pair are adjacent; v is unchanged.
static std::vector<int64_t> qkv_canon_of_dev(int H, int G, int D) {
  std::vector<int64_t> v((size_t)(H + 2 * G) * D);
  const int64_t nqk = (int64_t)(H + G) * D;
  for (int64_t dr = 0; dr < (int64_t)v.size(); ++dr) {
    if (dr < nqk) {
      int64_t head = dr / D, loc = dr % D;
      int64_t i = loc / 2, odd = loc % 2;
      v[dr] = head * D + i + odd * (D / 2);
    } else {
      v[dr] = dr;
    }
  }
  return v;
}

// gate/up interleave: device row 2i = gate row i, 2i + 1 = up row i
static int upload_gate_up(bw_model* m, uint64_t seed, uint32_t layer, uint32_t expert, int F, int d,
                          Mat* out) {
  HostMat g, u, gu;
  gen_canonical(seed, BWS_GATE, layer, expert, F, d, g);
  gen_canonical(seed, BWS_UP, layer, expert, F, d, u);
  gu.codes.resize((size_t)2 * F * d / 2);
  gu.scales.resize((size_t)2 * F * d / 32);
  const int64_t rb = d / 2, sb = d / 32;
  for (int64_t i = 0; i < F; ++i) {
    memcpy(&gu.codes[(2 * i) * rb], &g.codes[i * rb], rb);
    memcpy(&gu.codes[(2 * i + 1) * rb], &u.codes[i * rb], rb);
    memcpy(&gu.scales[(2 * i) * sb], &g.scales[i * sb], sb * 2);
    memcpy(&gu.scales[(2 * i + 1) * sb], &u.scales[i * sb], sb * 2);
  }
  return upload_mat(m, gu, 2 * (int64_t)F, d, nullptr, out);
}

static int upload_plain(bw_model* m, uint64_t seed, uint32_t kind, uint32_t layer, uint32_t expert,
                        int64_t N, int K, const std::vector<int64_t>* perm, Mat* out) {
  HostMat h;
  gen_canonical(seed, kind, layer, expert, N, K, h);
  return upload_mat(m, h, N, K, perm, out);
}

static int upload_f16(bw_model* m, const std::vector<uint16_t>& v, uint16_t** out) {
  void* p;
  if (int rc = m->arena.alloc(v.size() * 2, &p)) return rc;
  HIP_OK(hipMemcpy(p, v.data(), v.size() * 2, hipMemcpyHostToDevice));
  *out = (uint16_t*)p;
  return 0;
}

static int ws_alloc(bw_model* m, size_t bytes, void** out) {
  void* p = nullptr;
  if (bytes == 0) bytes = 256;
  if (hipMalloc(&p, bytes) != hipSuccess) return fail(BW_ENOMEM, "hipMalloc(%zu) failed", bytes);
  m->ws.push_back(p);
  *out = p;
  return 0;
}

static int make_gu_map(bw_model* m, int F) {
  if (m->gu_map.count(F)) return 0;
  std::vector<int32_t> v((size_t)2 * F);
  for (int i = 0; i < F; ++i) {
    v[2 * i] = i;
    v[2 * i + 1] = F + i;
  }
  void* p;
  if (int rc = ws_alloc(m, v.size() * 4, &p)) return rc;
  HIP_OK(hipMemcpy(p, v.data(), v.size() * 4, hipMemcpyHostToDevice));
  m->gu_map[F] = (int32_t*)p;
  return 0;
}

static int check_shape(const bw_model_config& c) {
  if (c.n_layers < 1 || c.d_model < 32 || c.d_model % 32) return fail(BW_EINVAL, "d_model must be a positive multiple of 32");
  if (c.n_q_heads < 1 || c.n_kv_heads < 1 || c.n_q_heads % c.n_kv_heads) return fail(BW_EINVAL, "n_q_heads must be a multiple of n_kv_heads");
  if (c.head_dim != 64 && c.head_dim != 128) return fail(BW_EINVAL, "head_dim must be 64 or 128");
  if (c.vocab < 1) return fail(BW_EINVAL, "vocab must be positive");
  if (c.page_tokens != kPageTokens) return fail(BW_EINVAL, "page_tokens must be 16");
  if (c.kv_dtype != BW_KV_F16 && c.kv_dtype != BW_KV_BF16 && c.kv_dtype != BW_KV_FP8)
    return fail(BW_EINVAL, "kv_dtype must be BW_KV_F16, BW_KV_BF16 or BW_KV_FP8");
  if (c.max_positions < 1 || c.max_tokens < 1) return fail(BW_EINVAL, "max_positions and max_tokens must be positive");
  if (c.max_positions > 65536) return fail(BW_EINVAL, "max_positions must be <= 65536");
  int qr = c.n_q_heads / c.n_kv_heads;
  (void)qr;
  if (is_moe(c)) {
    if (c.top_k < 1 || c.top_k > c.n_experts || c.top_k > 64) return fail(BW_EINVAL, "top_k must be in [1, min(64, n_experts)]");
    if (c.expert_ffn < 32 || c.expert_ffn % 32 || c.expert_ffn > 2048) return fail(BW_EINVAL, "expert_ffn must be a multiple of 32 up to 2048");
    if (c.n_shared < 0 || (c.n_shared > 0 && (c.shared_ffn < 32 || c.shared_ffn % 32 || c.shared_ffn > 2048))) return fail(BW_EINVAL, "shared_ffn must be a multiple of 32 up to 2048");
    if (c.n_experts > 1024) return fail(BW_EINVAL, "n_experts must be <= 1024");
  } else {
    if (c.ffn_dim < 32 || c.ffn_dim % 32) return fail(BW_EINVAL, "ffn_dim must be a positive multiple of 32");
  }
  return 0;
}

// The single-launch step (bw_persist.hip) for a model whose shape has an instantiation: one
// workgroup per CU, the geometry limits of the kernel checked here, exchange buffers allocated
// and tagged. Models without one keep the kernel chain only.
// MoE: every routed and shared expert has the same width Fe, and the F of the layout below is
// the concatenation of the slots (top_k routed, then the shared ones), slots x Fe.
static int launch_persist_any(const bw_model* m, const PersistParams& p, int nwg, hipStream_t s, bool query_only) {
  const auto& c = m->c;
  if (is_moe(c))
    return launch_persist_moe(p, c.d_model, c.kv_dtype, c.head_dim, c.n_q_heads / c.n_kv_heads, nwg, s, query_only);
  return launch_persist(p, c.d_model, c.ffn_dim, c.kv_dtype, c.head_dim, c.n_q_heads / c.n_kv_heads, nwg, s,
                        query_only);
}

static int persist_setup(bw_model* m) {
  const auto& c = m->c;
  const bool moe = is_moe(c);
  int dev = 0, ncu = 0;
  HIP_OK(hipGetDevice(&dev));
  HIP_OK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
  const int d = c.d_model, H = c.n_q_heads, G = c.n_kv_heads, D = c.head_dim;
  const int slots = moe ? c.top_k + c.n_shared : 0;
  const int F = moe ? slots * c.expert_ffn : c.ffn_dim;
  const int nwg = ncu;
  if (moe) {
    // the router phase gives each workgroup one expert's logit, and the top-k reads them with
    // one thread each; the expert slots' pointers and gates sit in a fixed LDS table
    const bool moe_fits = (c.n_shared == 0 || c.shared_ffn == c.expert_ffn) && c.n_experts <= nwg &&
                          c.n_experts <= 512 && c.n_experts + c.n_shared <= 480 && slots <= 32 && c.top_k <= 64;
    if (!moe_fits) return BW_OK;
  }
  const int S = nwg / G;
  const int Rd = (d + nwg - 1) / nwg;
  const int Rq = ((((H + 2 * G) * D + nwg - 1) / nwg) + 1) & ~1;
  const int Rg = (((2 * F + nwg - 1) / nwg) + 1) & ~1;
  int lpr, nb;
  gemv_lane_split(d, &lpr, &nb);
  // one merger workgroup per query head among the splits of its KV head (S >= H / G)
  const bool fits = H * D == d && S >= H / G && S <= 128 && Rd <= 64 && Rq <= 1024 && Rg <= 1024 &&
                    (H / G) * D <= 4096;
  if (!fits) return BW_OK;
  PersistParams& p = m->pp;
  if (moe) {
    p.moe = 1;
    p.E = c.n_experts;
    p.top_k = c.top_k;
    p.n_shared = c.n_shared;
    p.Fe = c.expert_ffn;
  }
  if (launch_persist_any(m, p, nwg, nullptr, true) != 0) {
    p = PersistParams{};
    return BW_OK;
  }
  std::vector<PLayer> layers(c.n_layers);
  // the FFN by columns (9B shape on 256 workgroups) reads W_down as per-workgroup column slices:
  // one copy per layer, written on the device from the uploaded matrix
  const int64_t dnc_bytes = moe ? 0 : persist_colffn_bytes(d, F, nwg);
  for (int l = 0; l < c.n_layers; ++l) {
    const LayerDev& Ld = m->L[l];
    layers[l] = PLayer{Ld.qkv, Ld.o, Ld.gu, Ld.dn, Ld.attn_norm, Ld.ffn_norm, Ld.router, Ld.ex};
    if (dnc_bytes > 0) {
      void* q;
      if (int rc = m->arena.alloc((size_t)dnc_bytes, &q)) return rc;
      if (launch_down_slices(Ld.dn, nwg, (uint8_t*)q, nullptr)) return fail(BW_EHIP, "W_down slice copy failed");
      layers[l].dnc = (const uint8_t*)q;
    }
  }
  void* ptr;
  if (dnc_bytes > 0) {
    p.n_xdp = (int32_t)persist_colffn_xdp_words(d, F, nwg);  // owners x producers x one record each
    if (int rc = ws_alloc(m, sizeof(uint32_t) * (size_t)p.n_xdp, &ptr)) return rc;
    p.xdp = (uint32_t*)ptr;
  }
  if (int rc = ws_alloc(m, sizeof(PLayer) * layers.size(), &ptr)) return rc;
  HIP_OK(hipMemcpy(ptr, layers.data(), sizeof(PLayer) * layers.size(), hipMemcpyHostToDevice));
  p.layers = (const PLayer*)ptr;
  p.L = c.n_layers;
  p.H = H;
  p.G = G;
  p.V = c.vocab;
  p.lm = m->lm;
  p.final_norm = m->final_norm;
  p.embed = m->embed;
  p.eps = c.rms_eps;
  p.attn_scale = (float)(1.0 / std::sqrt((double)D));
  p.rope = m->rope;
  p.max_pos = c.max_positions;
  p.err = m->err;
  m->n_xq = (H + 2 * G) * D;
  m->n_xp = H * S * (D + 2);
  m->n_xa = H * D;
  m->n_xd = d;
  m->n_xf = F;
  uint32_t** bufs[6] = {&p.xq, &p.xp, &p.xa, &p.xm, &p.xf, &p.xx};
  const int sizes[6] = {m->n_xq, m->n_xp, m->n_xa, m->n_xd, m->n_xf, m->n_xd};
  for (int i = 0; i < 6; ++i) {
    if (int rc = ws_alloc(m, sizeof(uint32_t) * sizes[i], &ptr)) return rc;
    *bufs[i] = (uint32_t*)ptr;
  }
  if (int rc = ws_alloc(m, sizeof(uint64_t) * nwg, &ptr)) return rc;
  p.xarg = (uint64_t*)ptr;
  if (moe) {
    if (int rc = ws_alloc(m, sizeof(uint32_t) * c.n_experts, &ptr)) return rc;
    p.xr = (uint32_t*)ptr;
    p.sel_out = m->sel;  // row 0 of each layer's selection table
    p.sel_stride = (int64_t)c.max_tokens * c.top_k;
  }

  if (int rc = ws_alloc(m, 256, &ptr)) return rc;
  HIP_OK(hipMemset(ptr, 0, 256));
  p.epoch = (uint32_t*)ptr;
  p.abort_flag = (uint32_t*)ptr + 16;
  if (launch_persist_reset(p, m->n_xq, m->n_xp, m->n_xa, m->n_xd, m->n_xf, nwg, nullptr)) return fail(BW_EHIP, "persistent-step reset failed");
  HIP_OK(hipDeviceSynchronize());
  p.plain_launch = true;  // mode 1 (see bw_set_single_launch)
  m->persist_nwg = nwg;
  m->persist_ok = true;
  return BW_OK;
}

extern "C" int bw_model_load_synthetic(const bw_model_config* cfg, uint64_t seed, bw_model** out) {
  if (!cfg || !out) return fail(BW_EINVAL, "null argument");
  *out = nullptr;
  if (int rc = check_shape(*cfg)) return rc;
  bw_model* m = new bw_model();
  m->c = *cfg;
  m->seed = seed;
  const bw_model_config& c = m->c;
  const int d = c.d_model, H = c.n_q_heads, G = c.n_kv_heads, D = c.head_dim, Lc = c.n_layers;
  auto bail = [&](int rc) {
    bw_model_free(m);
    return rc;
  };
  int rc = 0;
  // embeddings, norms
  {
    std::vector<uint16_t> e((size_t)c.vocab * d);
    const int64_t chunk = 256;
    parallel_for((c.vocab + chunk - 1) / chunk, [&](int64_t ci) {
      int64_t r0 = ci * chunk, nr = std::min<int64_t>(chunk, c.vocab - r0);
      bws_embed_rows(seed, d, r0, nr, e.data() + r0 * d);
    });
    if ((rc = upload_f16(m, e, &m->embed))) return bail(rc);
    std::vector<uint16_t> g(d);
    bws_norm_gain(seed, BWS_FINAL_NORM, 0, d, g.data());
    if ((rc = upload_f16(m, g, &m->final_norm))) return bail(rc);
  }
  const auto qkv_perm = qkv_canon_of_dev(H, G, D);
  m->L.resize(Lc);
  for (int l = 0; l < Lc; ++l) {
    LayerDev& Ld = m->L[l];
    std::vector<uint16_t> g(d);
    bws_norm_gain(seed, BWS_ATTN_NORM, l, d, g.data());
    if ((rc = upload_f16(m, g, &Ld.attn_norm))) return bail(rc);
    bws_norm_gain(seed, BWS_FFN_NORM, l, d, g.data());
    if ((rc = upload_f16(m, g, &Ld.ffn_norm))) return bail(rc);
    if ((rc = upload_plain(m, seed, BWS_QKV, l, 0, (int64_t)(H + 2 * G) * D, d, &qkv_perm, &Ld.qkv))) return bail(rc);
    if ((rc = upload_plain(m, seed, BWS_O, l, 0, d, H * D, nullptr, &Ld.o))) return bail(rc);
    if (!is_moe(c)) {
      if ((rc = upload_gate_up(m, seed, l, 0, c.ffn_dim, d, &Ld.gu))) return bail(rc);
      if ((rc = upload_plain(m, seed, BWS_DOWN, l, 0, d, c.ffn_dim, nullptr, &Ld.dn))) return bail(rc);
    } else {
      const int E = c.n_experts, S = c.n_shared;
      std::vector<uint16_t> r((size_t)E * d);
      bws_router(seed, l, E, d, r.data());
      if ((rc = upload_f16(m, r, &Ld.router))) return bail(rc);
      Ld.ex_gu.resize(E + S);
      Ld.ex_dn.resize(E + S);
      for (int e = 0; e < E + S; ++e) {
        const uint32_t ex = e < E ? 1u + (uint32_t)e : BWS_SHARED_EXPERT + (uint32_t)(e - E);
        const int F = e < E ? c.expert_ffn : c.shared_ffn;
        if ((rc = upload_gate_up(m, seed, l, ex, F, d, &Ld.ex_gu[e]))) return bail(rc);
        if ((rc = upload_plain(m, seed, BWS_DOWN, l, ex, d, F, nullptr, &Ld.ex_dn[e]))) return bail(rc);
      }
      std::vector<const void*> t0(E + S), t1(E + S), t2(E + S), t3(E + S);
      for (int e = 0; e < E + S; ++e) {
        t0[e] = Ld.ex_gu[e].codes;
        t1[e] = Ld.ex_gu[e].scales;
        t2[e] = Ld.ex_dn[e].codes;
        t3[e] = Ld.ex_dn[e].scales;
      }
      void* p;
      const size_t tb = sizeof(void*) * (E + S);
      if ((rc = m->arena.alloc(4 * tb, &p))) return bail(rc);
      if (hipMemcpy(p, t0.data(), tb, hipMemcpyHostToDevice) != hipSuccess ||
          hipMemcpy((char*)p + tb, t1.data(), tb, hipMemcpyHostToDevice) != hipSuccess ||
          hipMemcpy((char*)p + 2 * tb, t2.data(), tb, hipMemcpyHostToDevice) != hipSuccess ||
          hipMemcpy((char*)p + 3 * tb, t3.data(), tb, hipMemcpyHostToDevice) != hipSuccess)
        return bail(fail(BW_EHIP, "expert table upload failed"));
      Ld.ex.gu_codes = (const uint8_t* const*)p;
      Ld.ex.gu_scales = (const uint16_t* const*)((char*)p + tb);
      Ld.ex.dn_codes = (const uint8_t* const*)((char*)p + 2 * tb);
      Ld.ex.dn_scales = (const uint16_t* const*)((char*)p + 3 * tb);
    }
  }
  if ((rc = upload_plain(m, seed, BWS_LM_HEAD, 0, 0, c.vocab, d, nullptr, &m->lm))) return bail(rc);
  // RoPE table: angle pos * base^(-2i/D), evaluated in fp64, stored as fp32 (cos, sin)
  {
    std::vector<float2> t((size_t)c.max_positions * (D / 2));
    parallel_for(c.max_positions, [&](int64_t pos) {
      for (int i = 0; i < D / 2; ++i) {
        double th = (double)pos * std::pow(c.rope_base, -2.0 * i / D);
        t[pos * (D / 2) + i] = make_float2((float)std::cos(th), (float)std::sin(th));
      }
    });
    void* p;
    if ((rc = ws_alloc(m, t.size() * sizeof(float2), &p))) return bail(rc);
    if (hipMemcpy(p, t.data(), t.size() * sizeof(float2), hipMemcpyHostToDevice) != hipSuccess)
      return bail(fail(BW_EHIP, "rope upload failed"));
    m->rope = (float2*)p;
  }
  // row maps for the parity entry points
  {
    std::vector<int32_t> v(qkv_perm.begin(), qkv_perm.end());
    void* p;
    if ((rc = ws_alloc(m, v.size() * 4, &p))) return bail(rc);
    if (hipMemcpy(p, v.data(), v.size() * 4, hipMemcpyHostToDevice) != hipSuccess) return bail(fail(BW_EHIP, "map upload"));
    m->qkv_map = (int32_t*)p;
    if (!is_moe(c)) {
      if ((rc = make_gu_map(m, c.ffn_dim))) return bail(rc);
    } else {
      if ((rc = make_gu_map(m, c.expert_ffn))) return bail(rc);
      if (c.n_shared && (rc = make_gu_map(m, c.shared_ffn))) return bail(rc);
    }
  }
  // workspace
  {
    const int64_t T = c.max_tokens;
    m->max_splits = ((c.max_positions + kPageTokens - 1) / kPageTokens + m->pages_per_split - 1) / m->pages_per_split;
    int64_t aw = is_moe(c) ? (int64_t)c.top_k * c.expert_ffn + (int64_t)c.n_shared * c.shared_ffn : c.ffn_dim;
    aw = std::max<int64_t>(aw, 2 * (int64_t)std::max({c.ffn_dim, c.expert_ffn, c.shared_ffn}));
    aw = std::max<int64_t>(aw, (int64_t)(H + 2 * G) * D);
    aw = std::max<int64_t>(aw, d);
    m->act_width = aw;
    m->lm_parts = 4096;  // the GEMV launcher caps its grid at 4096 workgroups
    void* p;
    if ((rc = ws_alloc(m, sizeof(float) * T * d, &p))) return bail(rc);
    m->x = (float*)p;
    if ((rc = ws_alloc(m, sizeof(float) * T * H * D, &p))) return bail(rc);
    m->q = (float*)p;
    if ((rc = ws_alloc(m, sizeof(float) * T * H * m->max_splits * (D + 2), &p))) return bail(rc);
    m->attn_part = (float*)p;
    if ((rc = ws_alloc(m, sizeof(float) * T * H * D, &p))) return bail(rc);
    m->attn_out = (float*)p;
    if ((rc = ws_alloc(m, sizeof(int32_t) * T * G, &p))) return bail(rc);
    m->attn_cnt = (int32_t*)p;
    HIP_OK(hipMemset(m->attn_cnt, 0, sizeof(int32_t) * T * G));
    if ((rc = ws_alloc(m, sizeof(float) * T * aw, &p))) return bail(rc);
    m->act = (float*)p;
    if ((rc = ws_alloc(m, sizeof(float) * T * c.vocab, &p))) return bail(rc);
    m->logits = (float*)p;
    if ((rc = ws_alloc(m, sizeof(float) * T * m->lm_parts, &p))) return bail(rc);
    m->amax_val = (float*)p;
    if ((rc = ws_alloc(m, sizeof(int32_t) * T * m->lm_parts, &p))) return bail(rc);
    m->amax_idx = (int32_t*)p;
    {
      int64_t part = 0;
      const int64_t dims[9][2] = {{(int64_t)(H + 2 * G) * D, d}, {d, (int64_t)H * D}, {2 * (int64_t)c.ffn_dim, d},
                                  {d, c.ffn_dim}, {c.vocab, d}, {2 * (int64_t)c.expert_ffn, d}, {d, c.expert_ffn},
                                  {2 * (int64_t)c.shared_ffn, d}, {d, c.shared_ffn}};
      for (int64_t M = 1; M <= T; ++M)
        for (const auto& nk : dims)
          if (nk[0] > 0 && nk[1] > 0 && gemm_supported((int)nk[0], (int)nk[1]))
            part = std::max(part, gemm_part_elems((int)nk[0], (int)nk[1], (int)M));
      if ((rc = ws_alloc(m, sizeof(float) * std::max<int64_t>(part, 64), &p))) return bail(rc);
      m->gemm_part = (float*)p;
      if ((rc = ws_alloc(m, sizeof(float) * T, &p))) return bail(rc);
      m->rms = (float*)p;
      int64_t kmax = 0;
      for (const auto& nk : dims) kmax = std::max(kmax, nk[1]);
      if ((rc = ws_alloc(m, sizeof(uint16_t) * 2 * T * kmax, &p))) return bail(rc);
      m->gemm_x = (uint16_t*)p;
    }
    if ((rc = ws_alloc(m, 256, &p))) return bail(rc);
    m->err = (int32_t*)p;
    HIP_OK(hipMemset(m->err, 0, 256));
    if (is_moe(c)) {
      if ((rc = ws_alloc(m, sizeof(float) * T * c.n_experts, &p))) return bail(rc);
      m->router_logits = (float*)p;
      if ((rc = ws_alloc(m, sizeof(int32_t) * Lc * T * c.top_k, &p))) return bail(rc);
      m->sel = (int32_t*)p;
      if ((rc = ws_alloc(m, sizeof(float) * Lc * T * c.top_k, &p))) return bail(rc);
      m->gates = (float*)p;
    }
  }
  if ((rc = persist_setup(m))) return bail(rc);
  if (hipStreamCreateWithFlags(&m->cap_stream, hipStreamNonBlocking) != hipSuccess)
    return bail(fail(BW_EHIP, "stream creation failed"));
  if (hipDeviceSynchronize() != hipSuccess) return bail(fail(BW_EHIP, "device synchronisation failed"));
  *out = m;
  return BW_OK;
}

extern "C" int bw_model_free(bw_model* m) {
  if (!m) return BW_OK;
  (void)hipDeviceSynchronize();
  for (auto& g : m->graphs) {
    if (g.exec) (void)hipGraphExecDestroy(g.exec);
    if (g.graph) (void)hipGraphDestroy(g.graph);
  }
  if (m->cap_stream) (void)hipStreamDestroy(m->cap_stream);
  m->arena.release();
  for (void* p : m->ws) (void)hipFree(p);
  delete m;
  return BW_OK;
}

// ---------------------------------------------------------------------------------------------
// pool
// ---------------------------------------------------------------------------------------------

extern "C" int bw_kv_pool_create(const bw_model* m, int32_t n_pages, bw_kv_pool** out) {
  if (!m || !out) return fail(BW_EINVAL, "null argument");
  *out = nullptr;
  if (n_pages < 1) return fail(BW_EINVAL, "n_pages must be positive");
  const auto& c = m->c;
  bw_kv_pool* p = new bw_kv_pool();
  p->m = m;
  p->n_pages = n_pages;
  p->page_elems = (int64_t)c.n_kv_heads * 2 * kPageTokens * c.head_dim;
  p->layer_elems = p->page_elems * n_pages;
  p->es = c.kv_dtype == BW_KV_FP8 ? 1 : 2;
  const size_t bytes = (size_t)p->layer_elems * c.n_layers * p->es;
  void* d = nullptr;
  if (hipMalloc(&d, bytes) != hipSuccess) {
    delete p;
    return fail(BW_ENOMEM, "hipMalloc(%zu) for the KV pool failed", bytes);
  }
  if (hipMemset(d, 0, bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    (void)hipFree(d);
    delete p;
    return fail(BW_EHIP, "pool clear failed");
  }
  p->data = (uint16_t*)d;
  *out = p;
  return BW_OK;
}

extern "C" int bw_kv_pool_free(bw_kv_pool* p) {
  if (!p) return BW_OK;
  (void)hipDeviceSynchronize();
  (void)hipFree(p->data);
  delete p;
  return BW_OK;
}

extern "C" int bw_kv_pool_fill(bw_kv_pool* p, uint16_t bits, void* stream) {
  if (!p) return fail(BW_EINVAL, "null pool");
  // an FP8 pool is filled with the low byte of bits (its element count is even)
  const size_t n16 = (size_t)p->layer_elems * p->m->c.n_layers * p->es / 2;
  if (p->es == 1) bits = (uint16_t)((bits & 0xFFu) | ((bits & 0xFFu) << 8));
  if (launch_fill16(p->data, n16, bits, (hipStream_t)stream))
    return fail(BW_EHIP, "fill launch failed");
  return BW_OK;
}

// scatter staged page-layers to their physical pages, copying only the first nslot slots of
// each (kv, head) row so that unused slots keep their contents
__global__ void k_scatter_pages(const uint8_t* __restrict__ staged, const int32_t* __restrict__ dst_page,
                                const int32_t* __restrict__ nslot, uint8_t* __restrict__ layer_base,
                                int64_t page_bytes, int row_bytes) {
  const int i = blockIdx.x;
  const int64_t dst = (int64_t)dst_page[i] * page_bytes;
  const int ns = nslot[i];
  for (int64_t e = threadIdx.x; e < page_bytes; e += blockDim.x) {
    const int slot = (int)((e / row_bytes) % kPageTokens);
    if (slot < ns) layer_base[dst + e] = staged[(int64_t)i * page_bytes + e];
  }
}

// Device form of the synthetic context. The generator is implemented again here from its
// published definition (splitmix64 of Steele, Lea and Flood, OOPSLA 2014, used as a counter
// hash; finaliser constants as in Vigna's public splitmix64.c) with the stream-key derivation of
// the shared input generator, so both forms write the same bits.
__device__ __forceinline__ uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}
__device__ __forceinline__ uint64_t sm64_key(uint64_t seed, uint32_t kind, uint32_t layer, uint32_t expert) {
  uint64_t k = sm64_mix(seed ^ 0x5851F42D4C957F2DULL);
  k = sm64_mix(k ^ ((uint64_t)kind << 40) ^ (uint64_t)layer);
  return sm64_mix(k ^ ((uint64_t)expert * 0xD1B54A32D192ED03ULL));
}

// One workgroup per (logical page lp, sequence b, layer l): the page's first min(16, len - 16 lp)
// slots of every KV head, K and V, in the pool layout [g][kv][slot][d].
template <int DT>
__global__ void k_kv_synth(uint8_t* pool, int64_t layer_bytes, int64_t page_elems, int n_pages, uint64_t seed,
                           const int32_t* __restrict__ seq_ids, const int32_t* __restrict__ seq_lens,
                           const int32_t* __restrict__ page_table, int max_pages, int G, int D, int32_t* err) {
  const int lp = blockIdx.x, b = blockIdx.y, l = blockIdx.z;
  const int len = seq_lens[b];
  const int64_t np = len < 0 ? 0 : ((int64_t)len + kPageTokens - 1) / kPageTokens;  // no overflow near INT_MAX
  if (lp == 0 && l == 0 && threadIdx.x == 0 && (len < 0 || np > max_pages)) atomicOr(err, BW_DERR_POS);
  if (lp >= np || lp >= max_pages) return;
  const int page = page_table[(int64_t)b * max_pages + lp];
  if (page < 0 || page >= n_pages) {
    if (threadIdx.x == 0) atomicOr(err, BW_DERR_PAGE);
    return;
  }
  const int nslot = min(kPageTokens, len - lp * kPageTokens);
  const uint32_t seq = seq_ids ? (uint32_t)seq_ids[b] : (uint32_t)b;
  const uint64_t key = sm64_key(seed, BWS_KV, (uint32_t)l, seq);
  uint8_t* base = pool + (int64_t)l * layer_bytes + (int64_t)page * page_elems * (DT == 3 ? 1 : 2);
  for (int64_t e = threadIdx.x; e < page_elems; e += blockDim.x) {
    const int d = (int)(e % D), slot = (int)((e / D) % kPageTokens);
    const int kv = (int)((e / ((int64_t)D * kPageTokens)) & 1), g = (int)(e / ((int64_t)D * kPageTokens * 2));
    if (slot >= nslot) continue;
    const int64_t pos = (int64_t)lp * kPageTokens + slot;
    const uint64_t idx = (((uint64_t)pos * 2u + (uint64_t)kv) * (uint64_t)G + (uint64_t)g) * (uint64_t)D + (uint64_t)d;
    const int c = (int)(sm64_mix(key + (idx + 1ull) * 0x9E3779B97F4A7C15ULL) & 0xFFu) - 128;
    if constexpr (DT == 3) {
      base[e] = (uint8_t)f32_to_fp8((float)(c >> 3) * 0.125f);  // at most 4 significant bits: exact
    } else if constexpr (DT == 1) {
      ((uint16_t*)base)[e] = f32_to_f16((float)c * 0.015625f);  // at most 8 significant bits: exact
    } else {
      ((uint16_t*)base)[e] = (uint16_t)(__float_as_uint((float)c * 0.015625f) >> 16);
    }
  }
}

extern "C" int bw_kv_pool_synthesize_async(bw_kv_pool* p, uint64_t seed, const int32_t* seq_ids_dev,
                                           const int32_t* seq_lens_dev, const int32_t* page_table_dev,
                                           int32_t batch, int32_t max_pages, void* stream) {
  if (!p || !seq_lens_dev || !page_table_dev) return fail(BW_EINVAL, "null argument");
  if (batch < 1 || max_pages < 1) return fail(BW_EINVAL, "batch and max_pages must be positive");
  if (batch > 65535) return fail(BW_EINVAL, "batch must be <= 65535");
  const auto& c = p->m->c;
  const dim3 grid((unsigned)max_pages, (unsigned)batch, (unsigned)c.n_layers);
  const int64_t layer_bytes = p->layer_elems * p->es;
  hipStream_t s = (hipStream_t)stream;
#define BW_SYNTH_LAUNCH(DT)                                                                                \
  hipLaunchKernelGGL(k_kv_synth<DT>, grid, dim3(256), 0, s, (uint8_t*)p->data, layer_bytes, p->page_elems,   \
                     p->n_pages, seed, seq_ids_dev, seq_lens_dev, page_table_dev, max_pages, c.n_kv_heads, \
                     c.head_dim, p->m->err)
  if (c.kv_dtype == BW_KV_FP8) BW_SYNTH_LAUNCH(3);
  else if (c.kv_dtype == BW_KV_F16) BW_SYNTH_LAUNCH(1);
  else BW_SYNTH_LAUNCH(2);
#undef BW_SYNTH_LAUNCH
  if (hipGetLastError() != hipSuccess) return fail(BW_EHIP, "synthesis launch failed");
  return BW_OK;
}

extern "C" int bw_kv_pool_synthesize(bw_kv_pool* p, uint64_t seed, const int32_t* seq_ids,
                                     const int32_t* seq_lens, const int32_t* page_table,
                                     int32_t batch, int32_t max_pages) {
  if (!p || !seq_ids || !seq_lens || !page_table) return fail(BW_EINVAL, "null argument");
  if (batch < 1 || max_pages < 1) return fail(BW_EINVAL, "batch and max_pages must be positive");
  const auto& c = p->m->c;
  const int G = c.n_kv_heads, D = c.head_dim;
  const int dtype = c.kv_dtype == BW_KV_F16 ? BWS_KV_F16 : (c.kv_dtype == BW_KV_FP8 ? BWS_KV_FP8 : BWS_KV_BF16);
  const int es = p->es;
  // list of (sequence, logical page) to write
  struct Job { int b, lp, page, nslot; };
  std::vector<Job> jobs;
  for (int b = 0; b < batch; ++b) {
    if (seq_lens[b] < 0) return fail(BW_EINVAL, "negative seq_len");
    const int np = (seq_lens[b] + kPageTokens - 1) / kPageTokens;
    if (np > max_pages) return fail(BW_EINVAL, "seq_len %d needs more than max_pages pages", seq_lens[b]);
    for (int lp = 0; lp < np; ++lp) {
      const int page = page_table[(int64_t)b * max_pages + lp];
      if (page < 0 || page >= p->n_pages) return fail(BW_EINVAL, "page id %d out of range", page);
      jobs.push_back({b, lp, page, std::min(kPageTokens, seq_lens[b] - lp * kPageTokens)});
    }
  }
  if (jobs.empty()) return BW_OK;
  const int64_t pb = p->page_elems * es;  // bytes of one page-layer
  const int64_t chunk = std::min<int64_t>((int64_t)jobs.size(), std::max<int64_t>(1, (256ll << 20) / pb));
  std::vector<uint8_t> host((size_t)(chunk * pb));
  std::vector<int32_t> pid(chunk), ns(chunk);
  void *dstage = nullptr, *dpid = nullptr, *dns = nullptr;
  if (hipMalloc(&dstage, (size_t)(chunk * pb)) != hipSuccess || hipMalloc(&dpid, chunk * 4) != hipSuccess ||
      hipMalloc(&dns, chunk * 4) != hipSuccess) {
    if (dstage) (void)hipFree(dstage);
    if (dpid) (void)hipFree(dpid);
    return fail(BW_ENOMEM, "staging allocation failed");
  }
  int rc = BW_OK;
  for (int l = 0; l < c.n_layers && rc == BW_OK; ++l) {
    for (int64_t j0 = 0; j0 < (int64_t)jobs.size() && rc == BW_OK; j0 += chunk) {
      const int64_t nj = std::min<int64_t>(chunk, (int64_t)jobs.size() - j0);
      parallel_for(nj, [&](int64_t i) {
        const Job& jb = jobs[j0 + i];
        std::vector<uint8_t> tmp((size_t)kPageTokens * 2 * G * D * es);
        bws_kv_fill(seed, l, (uint32_t)seq_ids[jb.b], (int64_t)jb.lp * kPageTokens, jb.nslot, G, D, dtype, tmp.data());
        uint8_t* dst = host.data() + i * pb;
        // [tok][kv][g][d] -> [g][kv][slot][d]
        for (int t = 0; t < jb.nslot; ++t)
          for (int kv = 0; kv < 2; ++kv)
            for (int g = 0; g < G; ++g)
              memcpy(dst + ((((int64_t)g * 2 + kv) * kPageTokens + t) * D) * es,
                     tmp.data() + ((((int64_t)t * 2 + kv) * G + g) * D) * es, (size_t)D * es);
        pid[i] = jb.page;
        ns[i] = jb.nslot;
      });
      if (hipMemcpy(dstage, host.data(), (size_t)(nj * pb), hipMemcpyHostToDevice) != hipSuccess ||
          hipMemcpy(dpid, pid.data(), nj * 4, hipMemcpyHostToDevice) != hipSuccess ||
          hipMemcpy(dns, ns.data(), nj * 4, hipMemcpyHostToDevice) != hipSuccess) {
        rc = fail(BW_EHIP, "staging copy failed");
        break;
      }
      hipLaunchKernelGGL(k_scatter_pages, dim3((unsigned)nj), dim3(256), 0, 0, (const uint8_t*)dstage,
                         (const int32_t*)dpid, (const int32_t*)dns, (uint8_t*)p->layer(l), pb, D * es);
      if (hipDeviceSynchronize() != hipSuccess) rc = fail(BW_EHIP, "scatter failed");
    }
  }
  (void)hipFree(dstage);
  (void)hipFree(dpid);
  (void)hipFree(dns);
  return rc;
}

extern "C" int bw_kv_pool_read(const bw_kv_pool* p, int32_t layer, int32_t page, void* host_dst,
                               size_t bytes) {
  if (!p || !host_dst) return fail(BW_EINVAL, "null argument");
  if (layer < 0 || layer >= p->m->c.n_layers || page < 0 || page >= p->n_pages)
    return fail(BW_EINVAL, "layer or page out of range");
  const size_t pb = (size_t)p->page_elems * p->es;
  if (bytes < pb) return fail(BW_ERANGE, "destination too small");
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(host_dst, (const uint8_t*)p->layer(layer) + (int64_t)page * pb, pb, hipMemcpyDeviceToHost));
  return BW_OK;
}

// ---------------------------------------------------------------------------------------------
// host tier of the pool: pinned host page slots, least recently used pages evicted first
// ---------------------------------------------------------------------------------------------
// The deep-dive page's Hy3 overflow (section 6 item 3) keeps hot KV pages in VRAM and moves cold
// ones to locked host memory over PCIe, evicting by the pages' access time stamps; a read of a
// page under migration waits until the copy is done. Here a page is one physical page id across
// all layers. A kernel packs up to 128 pages into a contiguous device staging buffer (or unpacks
// them), and each run of consecutive host slots is one DMA copy, all on the tier's own stream: a
// strided copy per page (L rows of one page-layer) reached 45 GB/s for 64 KiB rows and 37 GB/s
// for 32 KiB rows, against 57 GB/s for one contiguous copy.

struct bw_kv_tier {
  bw_kv_pool* pool = nullptr;
  int32_t host_pages = 0;
  uint8_t* host = nullptr;          // [host_pages][n_layers][page_bytes], pinned
  std::vector<uint64_t> stamp;      // per device page: tier clock at its last touch
  std::vector<uint8_t> resident;    // per device page: holds cached positions the tier may evict
  std::vector<uint8_t> slot_used;   // per host slot
  std::vector<int32_t> free_slots;  // host slots not holding a page (the last one is used first)
  uint64_t clock = 1;
  hipStream_t copy = nullptr;       // copy stream (default priority)
  hipEvent_t after = nullptr;       // caller's stream position before a batch of copies
  hipEvent_t done = nullptr;        // copy stream position after the latest batch of copies
  uint8_t* stage = nullptr;         // device staging buffer [stage_pages][n_layers][page_bytes]
  int32_t stage_pages = 0;
};

extern "C" int bw_kv_lru_select(const uint64_t* stamps, const uint8_t* resident, int32_t n_pages, int32_t n,
                                int32_t* out, int32_t* n_out) {
  if (!stamps || !resident || !out || !n_out) return fail(BW_EINVAL, "null argument");
  if (n_pages < 0 || n < 0) return fail(BW_EINVAL, "negative size");
  std::vector<int32_t> cand;
  for (int32_t p = 0; p < n_pages; ++p)
    if (resident[p]) cand.push_back(p);
  const size_t k = std::min<size_t>((size_t)n, cand.size());
  std::partial_sort(cand.begin(), cand.begin() + k, cand.end(), [&](int32_t a, int32_t b) {
    return stamps[a] != stamps[b] ? stamps[a] < stamps[b] : a < b;
  });
  for (size_t i = 0; i < k; ++i) out[i] = cand[i];
  *n_out = (int32_t)k;
  return BW_OK;
}

extern "C" int bw_kv_tier_free(bw_kv_tier* t) {
  if (!t) return BW_OK;
  if (t->copy) (void)hipStreamSynchronize(t->copy);
  if (t->after) (void)hipEventDestroy(t->after);
  if (t->done) (void)hipEventDestroy(t->done);
  if (t->copy) (void)hipStreamDestroy(t->copy);
  if (t->host) (void)hipHostFree(t->host);
  if (t->stage) (void)hipFree(t->stage);
  delete t;
  return BW_OK;
}

extern "C" int bw_kv_tier_create(bw_kv_pool* pool, int32_t host_pages, bw_kv_tier** out) {
  if (!pool || !out) return fail(BW_EINVAL, "null argument");
  *out = nullptr;
  if (host_pages < 1) return fail(BW_EINVAL, "host_pages must be positive");
  const size_t page_bytes = (size_t)pool->page_elems * pool->es;
  const size_t bytes = (size_t)host_pages * pool->m->c.n_layers * page_bytes;
  bw_kv_tier* t = new bw_kv_tier();
  t->pool = pool;
  t->host_pages = host_pages;
  if (hipHostMalloc((void**)&t->host, bytes, hipHostMallocDefault) != hipSuccess) {
    t->host = nullptr;
    bw_kv_tier_free(t);
    return fail(BW_ENOMEM, "hipHostMalloc(%zu) for the host tier failed", bytes);
  }
  if (hipStreamCreateWithFlags(&t->copy, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&t->after, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&t->done, hipEventDisableTiming) != hipSuccess) {
    bw_kv_tier_free(t);
    return fail(BW_EHIP, "tier stream or event creation failed");
  }
  const size_t per_page = (size_t)pool->m->c.n_layers * page_bytes;
  t->stage_pages = (int32_t)std::max<size_t>(1, std::min<size_t>({(size_t)host_pages, (size_t)PageList::kMax,
                                                                   ((size_t)256 << 20) / per_page}));
  if (hipMalloc((void**)&t->stage, t->stage_pages * per_page) != hipSuccess) {
    t->stage = nullptr;
    bw_kv_tier_free(t);
    return fail(BW_ENOMEM, "hipMalloc for the tier's staging buffer failed");
  }
  t->stamp.assign(pool->n_pages, 0);
  t->resident.assign(pool->n_pages, 0);
  t->slot_used.assign(host_pages, 0);
  for (int32_t s = host_pages - 1; s >= 0; --s) t->free_slots.push_back(s);
  *out = t;
  return BW_OK;
}

extern "C" int bw_kv_tier_touch(bw_kv_tier* t, const int32_t* page_table, const int32_t* seq_lens, int32_t batch,
                                int32_t tokens, int32_t max_pages) {
  if (!t || !page_table || !seq_lens) return fail(BW_EINVAL, "null argument");
  if (batch < 1 || tokens < 0 || max_pages < 1) return fail(BW_EINVAL, "bad batch, tokens or max_pages");
  for (int32_t b = 0; b < batch; ++b) {
    if (seq_lens[b] < 0) return fail(BW_EINVAL, "negative seq_len");
    const int64_t np = ((int64_t)seq_lens[b] + tokens + kPageTokens - 1) / kPageTokens;
    if (np > max_pages) return fail(BW_EINVAL, "sequence %d needs more than max_pages pages", b);
    for (int64_t j = 0; j < np; ++j) {
      const int32_t pg = page_table[(int64_t)b * max_pages + j];
      if (pg < 0 || pg >= t->pool->n_pages) return fail(BW_EINVAL, "page id %d out of range", pg);
      t->stamp[pg] = t->clock;
      t->resident[pg] = 1;
    }
  }
  ++t->clock;
  return BW_OK;
}

// pages[i] <-> host slots[i], i < n, in chunks through the staging buffer; one DMA copy per run of
// consecutive host slots within a chunk
static int tier_move(bw_kv_tier* t, const int32_t* pages, const int32_t* slots, int32_t n, bool to_host) {
  const bw_kv_pool* p = t->pool;
  const int L = p->m->c.n_layers;
  const int64_t pb = p->page_elems * p->es, lb = p->layer_elems * p->es, per = (int64_t)L * pb;
  for (int32_t c0 = 0; c0 < n; c0 += t->stage_pages) {
    const int32_t m = std::min(t->stage_pages, n - c0);
    PageList ids;
    for (int32_t i = 0; i < m; ++i) ids.id[i] = pages[c0 + i];
    if (to_host && launch_page_pack((uint8_t*)p->data, lb, pb, L, ids, m, t->stage, true, t->copy))
      return fail(BW_EHIP, "page packing launch failed");
    for (int32_t i = 0; i < m;) {
      int32_t j = i + 1;
      while (j < m && slots[c0 + j] == slots[c0 + j - 1] + 1) ++j;
      uint8_t* h = t->host + (int64_t)slots[c0 + i] * per;
      uint8_t* d = t->stage + (int64_t)i * per;
      HIP_OK(hipMemcpyAsync(to_host ? (void*)h : (void*)d, to_host ? (const void*)d : (const void*)h, (size_t)((j - i) * per),
                            to_host ? hipMemcpyDeviceToHost : hipMemcpyHostToDevice, t->copy));
      i = j;
    }
    if (!to_host && launch_page_pack((uint8_t*)p->data, lb, pb, L, ids, m, t->stage, false, t->copy))
      return fail(BW_EHIP, "page unpacking launch failed");
  }
  return BW_OK;
}

extern "C" int bw_kv_tier_evict_lru(bw_kv_tier* t, int32_t n, int32_t* dev_pages, int32_t* host_slots,
                                    int32_t* n_out, void* stream) {
  if (!t || !dev_pages || !host_slots || !n_out) return fail(BW_EINVAL, "null argument");
  if (n < 0) return fail(BW_EINVAL, "negative n");
  const int32_t k = std::min<int32_t>(n, (int32_t)t->free_slots.size());
  int32_t got = 0;
  int rc = bw_kv_lru_select(t->stamp.data(), t->resident.data(), t->pool->n_pages, k, dev_pages, &got);
  if (rc != BW_OK) return rc;
  *n_out = got;
  if (got == 0) return BW_OK;
  // the copies start after the work already queued on the caller's stream (the steps that wrote
  // these pages)
  HIP_OK(hipEventRecord(t->after, (hipStream_t)stream));
  HIP_OK(hipStreamWaitEvent(t->copy, t->after, 0));
  for (int32_t i = 0; i < got; ++i) {  // the free list is kept descending: lowest slots first
    const int32_t slot = t->free_slots.back();
    t->free_slots.pop_back();
    t->slot_used[slot] = 1;
    host_slots[i] = slot;
    t->resident[dev_pages[i]] = 0;
    t->stamp[dev_pages[i]] = 0;
  }
  const int rc2 = tier_move(t, dev_pages, host_slots, got, true);
  if (rc2 != BW_OK) return rc2;
  HIP_OK(hipEventRecord(t->done, t->copy));
  return BW_OK;
}

extern "C" int bw_kv_tier_restore(bw_kv_tier* t, const int32_t* host_slots, const int32_t* dev_pages, int32_t n,
                                  void* stream) {
  if (!t || (n > 0 && (!host_slots || !dev_pages))) return fail(BW_EINVAL, "null argument");
  if (n < 0) return fail(BW_EINVAL, "negative n");
  for (int32_t i = 0; i < n; ++i) {
    if (host_slots[i] < 0 || host_slots[i] >= t->host_pages || !t->slot_used[host_slots[i]])
      return fail(BW_EINVAL, "host slot %d holds no page", host_slots[i]);
    if (dev_pages[i] < 0 || dev_pages[i] >= t->pool->n_pages) return fail(BW_EINVAL, "page id %d out of range", dev_pages[i]);
    for (int32_t j = 0; j < i; ++j)
      if (host_slots[j] == host_slots[i] || dev_pages[j] == dev_pages[i])
        return fail(BW_EINVAL, "slot or page repeated");
  }
  if (n == 0) return BW_OK;
  // after the work queued on the caller's stream (a step that still reads a target page)
  HIP_OK(hipEventRecord(t->after, (hipStream_t)stream));
  HIP_OK(hipStreamWaitEvent(t->copy, t->after, 0));
  const int rc2 = tier_move(t, dev_pages, host_slots, n, false);
  if (rc2 != BW_OK) return rc2;
  for (int32_t i = 0; i < n; ++i) {
    t->resident[dev_pages[i]] = 1;
    t->stamp[dev_pages[i]] = t->clock;
    // the slot is free again; a later eviction into it runs after this copy on the same stream
    t->slot_used[host_slots[i]] = 0;
    t->free_slots.push_back(host_slots[i]);
  }
  std::sort(t->free_slots.begin(), t->free_slots.end(), std::greater<int32_t>());
  HIP_OK(hipEventRecord(t->done, t->copy));
  return BW_OK;
}

extern "C" int bw_kv_tier_wait(bw_kv_tier* t, void* stream) {
  if (!t) return fail(BW_EINVAL, "null tier");
  HIP_OK(hipStreamWaitEvent((hipStream_t)stream, t->done, 0));
  return BW_OK;
}

extern "C" int bw_kv_tier_stats(const bw_kv_tier* t, int32_t* resident_pages, int32_t* host_pages_used) {
  if (!t || !resident_pages || !host_pages_used) return fail(BW_EINVAL, "null argument");
  int32_t r = 0;
  for (uint8_t v : t->resident) r += v;
  *resident_pages = r;
  *host_pages_used = t->host_pages - (int32_t)t->free_slots.size();
  return BW_OK;
}

// ---------------------------------------------------------------------------------------------
// host tier of the routed expert weights (MoE)
// ---------------------------------------------------------------------------------------------

// The device addresses of one routed expert's four parts.
struct ExpertRegion {
  const uint8_t* gc = nullptr;   // gate/up codes [2 Fe][d / 2]
  const uint16_t* gs = nullptr;  // gate/up scales
  const uint8_t* dc = nullptr;   // down codes [d][Fe / 2]
  const uint16_t* ds = nullptr;  // down scales
};

struct bw_expert_tier {
  bw_model* m = nullptr;
  int32_t host_slots = 0;
  size_t part[4] = {0, 0, 0, 0};  // bytes of each part (gate/up codes, scales, down codes, scales)
  size_t off[4] = {0, 0, 0, 0};   // offset of each part inside a host slot (256-byte aligned)
  size_t slot_bytes = 0;
  uint8_t* host = nullptr;        // pinned [host_slots][slot_bytes] (hipHostMalloc)
  uint8_t* host_dev = nullptr;    // the same memory as kernels address it
  std::vector<uint64_t> stamp;    // [L * E]: tier clock when a touched step last routed the expert
  std::vector<int32_t> slot_of;   // [L * E]: host slot of an evicted expert, -1 on the device
  std::vector<ExpertRegion> dev_of;   // [L * E]: device region of a resident expert
  std::vector<ExpertRegion> free_dev; // device regions holding no expert (one per evicted expert)
  std::vector<int32_t> free_slots;    // host slots holding no expert (kept descending)
  std::vector<uint8_t> routed_on_host;// [L * E]: routed by the last touched step while on the host
  uint64_t clock = 1;
};

static ExpertRegion region_of(const LayerDev& Ld, int e) {
  return {Ld.ex_gu[e].codes, Ld.ex_gu[e].scales, Ld.ex_dn[e].codes, Ld.ex_dn[e].scales};
}

// point expert e of layer l (tables on the device, descriptors on the host) at region r
static int expert_point(bw_expert_tier* t, int l, int e, const ExpertRegion& r, hipStream_t s) {
  LayerDev& Ld = t->m->L[l];
  if (launch_set_expert(Ld.ex, e, r.gc, r.gs, r.dc, r.ds, s)) return fail(BW_EHIP, "expert table update failed");
  Ld.ex_gu[e].codes = r.gc;
  Ld.ex_gu[e].scales = r.gs;
  Ld.ex_dn[e].codes = r.dc;
  Ld.ex_dn[e].scales = r.ds;
  return BW_OK;
}

static ExpertRegion slot_region(const bw_expert_tier* t, int32_t slot) {
  uint8_t* b = t->host_dev + (size_t)slot * t->slot_bytes;
  return {b + t->off[0], (const uint16_t*)(b + t->off[1]), b + t->off[2], (const uint16_t*)(b + t->off[3])};
}

// copy the four parts of an expert between two regions, in stream order
static int expert_copy(const bw_expert_tier* t, const ExpertRegion& dst, const ExpertRegion& src, hipStream_t s) {
  const void* sp[4] = {src.gc, src.gs, src.dc, src.ds};
  void* dp[4] = {(void*)dst.gc, (void*)dst.gs, (void*)dst.dc, (void*)dst.ds};
  for (int i = 0; i < 4; ++i) HIP_OK(hipMemcpyAsync(dp[i], sp[i], t->part[i], hipMemcpyDefault, s));
  return BW_OK;
}

static int expert_evict(bw_expert_tier* t, int l, int e, hipStream_t s) {
  const int E = t->m->c.n_experts;
  const int32_t slot = t->free_slots.back();
  t->free_slots.pop_back();
  const ExpertRegion host = slot_region(t, slot), dev = t->dev_of[l * E + e];
  if (int rc = expert_copy(t, host, dev, s)) return rc;
  if (int rc = expert_point(t, l, e, host, s)) return rc;
  t->free_dev.push_back(dev);
  t->slot_of[l * E + e] = slot;
  t->dev_of[l * E + e] = ExpertRegion{};
  return BW_OK;
}

static int expert_restore(bw_expert_tier* t, int l, int e, hipStream_t s) {
  const int E = t->m->c.n_experts;
  const int32_t slot = t->slot_of[l * E + e];
  const ExpertRegion dev = t->free_dev.back();
  t->free_dev.pop_back();
  if (int rc = expert_copy(t, dev, slot_region(t, slot), s)) return rc;
  if (int rc = expert_point(t, l, e, dev, s)) return rc;
  t->dev_of[l * E + e] = dev;
  t->slot_of[l * E + e] = -1;
  t->routed_on_host[l * E + e] = 0;
  t->stamp[l * E + e] = t->clock;
  // the slot is free again; a later eviction into it is queued after this copy on the same stream
  t->free_slots.push_back(slot);
  std::sort(t->free_slots.begin(), t->free_slots.end(), std::greater<int32_t>());
  return BW_OK;
}

extern "C" int bw_expert_tier_create(bw_model* m, int32_t host_slots, bw_expert_tier** out) {
  if (!m || !out) return fail(BW_EINVAL, "null argument");
  *out = nullptr;
  if (!is_moe(m->c)) return fail(BW_ESTATE, "the model has no routed experts");
  if (host_slots < 1) return fail(BW_EINVAL, "host_slots must be positive");
  const auto& c = m->c;
  const int L = c.n_layers, E = c.n_experts, d = c.d_model, F = c.expert_ffn;
  bw_expert_tier* t = new bw_expert_tier();
  t->m = m;
  t->host_slots = host_slots;
  t->part[0] = (size_t)2 * F * d / 2;
  t->part[1] = (size_t)2 * F * d / 32 * 2;
  t->part[2] = (size_t)d * F / 2;
  t->part[3] = (size_t)d * F / 32 * 2;
  size_t o = 0;
  for (int i = 0; i < 4; ++i) {
    t->off[i] = o;
    o += (t->part[i] + 255) & ~(size_t)255;
  }
  t->slot_bytes = o;
  if (hipHostMalloc((void**)&t->host, (size_t)host_slots * o, hipHostMallocDefault) != hipSuccess) {
    delete t;
    return fail(BW_ENOMEM, "hipHostMalloc(%zu) for the expert tier failed", (size_t)host_slots * o);
  }
  if (hipHostGetDevicePointer((void**)&t->host_dev, t->host, 0) != hipSuccess || !t->host_dev) {
    (void)hipHostFree(t->host);
    delete t;
    return fail(BW_EHIP, "no device address for the expert tier's host memory");
  }
  t->stamp.assign((size_t)L * E, 0);
  t->slot_of.assign((size_t)L * E, -1);
  t->routed_on_host.assign((size_t)L * E, 0);
  t->dev_of.resize((size_t)L * E);
  for (int l = 0; l < L; ++l)
    for (int e = 0; e < E; ++e) t->dev_of[(size_t)l * E + e] = region_of(m->L[l], e);
  for (int32_t sl = host_slots - 1; sl >= 0; --sl) t->free_slots.push_back(sl);
  *out = t;
  return BW_OK;
}

extern "C" int bw_expert_tier_free(bw_expert_tier* t, void* stream) {
  if (!t) return BW_OK;
  const int E = t->m->c.n_experts, L = t->m->c.n_layers;
  int rc = BW_OK;
  for (int l = 0; l < L && rc == BW_OK; ++l)
    for (int e = 0; e < E && rc == BW_OK; ++e)
      if (t->slot_of[l * E + e] >= 0) rc = expert_restore(t, l, e, (hipStream_t)stream);
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess && rc == BW_OK) rc = fail(BW_EHIP, "stream synchronisation failed");
  if (rc != BW_OK) return rc;  // an expert may still point at the host memory: keep it
  (void)hipHostFree(t->host);
  delete t;
  return BW_OK;
}

extern "C" int bw_expert_tier_touch(bw_expert_tier* t, int32_t n_rows, void* stream) {
  if (!t) return fail(BW_EINVAL, "null tier");
  const auto& c = t->m->c;
  if (n_rows < 1 || n_rows > c.max_tokens) return fail(BW_ERANGE, "n_rows out of range");
  const int L = c.n_layers, E = c.n_experts, k = c.top_k;
  std::vector<int32_t> sel((size_t)L * c.max_tokens * k);
  HIP_OK(hipStreamSynchronize((hipStream_t)stream));
  HIP_OK(hipMemcpy(sel.data(), t->m->sel, sel.size() * sizeof(int32_t), hipMemcpyDeviceToHost));
  std::fill(t->routed_on_host.begin(), t->routed_on_host.end(), 0);
  for (int l = 0; l < L; ++l)
    for (int r = 0; r < n_rows; ++r)
      for (int j = 0; j < k; ++j) {
        const int e = sel[((size_t)l * c.max_tokens + r) * k + j];
        if (e < 0 || e >= E) continue;
        t->stamp[(size_t)l * E + e] = t->clock;
        if (t->slot_of[(size_t)l * E + e] >= 0) t->routed_on_host[(size_t)l * E + e] = 1;
      }
  ++t->clock;
  return BW_OK;
}

extern "C" int bw_expert_tier_evict_lru(bw_expert_tier* t, int32_t n, int32_t* layers_out, int32_t* experts_out,
                                        int32_t* n_out, void* stream) {
  if (!t || !layers_out || !experts_out || !n_out) return fail(BW_EINVAL, "null argument");
  if (n < 0) return fail(BW_EINVAL, "negative n");
  const int E = t->m->c.n_experts, LE = t->m->c.n_layers * E;
  std::vector<uint8_t> resident(LE);
  for (int i = 0; i < LE; ++i) resident[i] = t->slot_of[i] < 0 ? 1 : 0;
  const int32_t k = std::min<int32_t>(n, (int32_t)t->free_slots.size());
  std::vector<int32_t> pick(std::max(k, 1));
  int32_t got = 0;
  if (int rc = bw_kv_lru_select(t->stamp.data(), resident.data(), LE, k, pick.data(), &got)) return rc;
  for (int32_t i = 0; i < got; ++i) {
    if (int rc = expert_evict(t, pick[i] / E, pick[i] % E, (hipStream_t)stream)) return rc;
    layers_out[i] = pick[i] / E;
    experts_out[i] = pick[i] % E;
  }
  *n_out = got;
  return BW_OK;
}

extern "C" int bw_expert_tier_restore(bw_expert_tier* t, int32_t layer, int32_t expert, void* stream) {
  if (!t) return fail(BW_EINVAL, "null tier");
  const int E = t->m->c.n_experts;
  if (layer < 0 || layer >= t->m->c.n_layers || expert < 0 || expert >= E) return fail(BW_EINVAL, "expert out of range");
  if (t->slot_of[layer * E + expert] < 0) return fail(BW_EINVAL, "expert %d of layer %d is on the device", expert, layer);
  return expert_restore(t, layer, expert, (hipStream_t)stream);
}

extern "C" int bw_expert_tier_restore_routed(bw_expert_tier* t, int32_t* n_out, void* stream) {
  if (!t || !n_out) return fail(BW_EINVAL, "null argument");
  const int E = t->m->c.n_experts, LE = t->m->c.n_layers * E;
  int32_t n = 0;
  for (int i = 0; i < LE; ++i)
    if (t->routed_on_host[i] && t->slot_of[i] >= 0) {
      if (int rc = expert_restore(t, i / E, i % E, (hipStream_t)stream)) return rc;
      ++n;
    }
  *n_out = n;
  return BW_OK;
}

extern "C" int bw_expert_tier_stats(const bw_expert_tier* t, int32_t* resident, int32_t* on_host) {
  if (!t || !resident || !on_host) return fail(BW_EINVAL, "null argument");
  int32_t h = 0;
  for (int32_t v : t->slot_of) h += v >= 0 ? 1 : 0;
  *on_host = h;
  *resident = (int32_t)t->slot_of.size() - h;
  return BW_OK;
}

// ---------------------------------------------------------------------------------------------
// the step
// ---------------------------------------------------------------------------------------------

static AttnParams attn_params(bw_model* m, const bw_kv_pool* pool, int l, const float* q,
                              const int32_t* seq_lens, const int32_t* page_table, int t,
                              int max_pages, float* out) {
  const auto& c = m->c;
  AttnParams a;
  a.pool = pool->layer(l);
  a.pool_page_stride = pool->page_elems;
  a.n_pages = pool->n_pages;
  a.q = q;
  a.seq_lens = seq_lens;
  a.page_table = page_table;
  a.max_pages = max_pages;
  a.t = t;
  a.H = c.n_q_heads;
  a.G = c.n_kv_heads;
  a.D = c.head_dim;
  a.pages_per_split = m->pages_per_split;
  a.max_splits = m->max_splits;
  a.scale = (float)(1.0 / std::sqrt((double)c.head_dim));
  a.part = m->attn_part;
  a.out = out;
  a.err = m->err;
  a.counters = m->attn_cnt;
  return a;
}

static inline void trace_mark(bw_model* m, int cls, int layer, int which, hipStream_t s) {
  if (m->trace_class == cls && (size_t)(2 * layer + which) < m->trace_ev.size())
    (void)hipEventRecord(m->trace_ev[2 * layer + which], s);
}

extern "C" int bw_set_trace(bw_model* m, int32_t kernel_class, void* const* events, int32_t n_layers) {
  if (!m) return fail(BW_EINVAL, "null model");
  if (!events) {
    m->trace_class = -1;
    m->trace_ev.clear();
    return BW_OK;
  }
  if (kernel_class < 0 || kernel_class > BW_K_MOE_DOWN || n_layers < 1) return fail(BW_EINVAL, "bad trace request");
  m->trace_ev.assign((hipEvent_t*)events, (hipEvent_t*)events + 2 * n_layers);
  m->trace_class = kernel_class;
  return BW_OK;
}

// One dense matrix product of a step: the MFMA GEMM when the step has gemm_min_rows rows or more
// (weights read once for all rows), else the GEMV (one pass over the weights per row, each pass at
// the HBM rate). The batched path computes the RMSNorm factors and the layer-0 embedding in their
// own small kernels; its logits skip the per-workgroup argmax partials (argmax_rows follows).
static bool batched(const bw_model* m, const Mat& w, int M) {
  return m->gemm_min_rows > 0 && M >= m->gemm_min_rows && gemm_supported(w.N, w.K);
}

static int run_dense(bw_model* m, int in_mode, int epi, GemvParams p, int M, hipStream_t s, int* grid_out = nullptr) {
  if (!batched(m, p.w, M)) return launch_gemv(in_mode, epi, p, M, s, grid_out);
  if (in_mode == IN_RMSNORM) {
    if (p.embed) {
      if (launch_embed(p.embed, p.vocab, p.w.K, p.tokens, M, p.x_out, p.err, s)) return -1;
      p.embed = nullptr;
    }
    if (launch_rowrms(p.x, p.x_stride, p.w.K, p.eps, M, m->rms, s)) return -1;
  }
  return launch_gemm(in_mode, epi, p, M, m->rms, m->gemm_part, m->gemm_x, s);
}

// enqueue every kernel of one step on stream s (arguments already validated)
static int enqueue_step(bw_model* m, bw_kv_pool* pool, const int32_t* tokens, const int32_t* seq_lens,
                        const int32_t* page_table, int32_t batch, int32_t t, int32_t max_pages,
                        float* logits_out, int32_t* argmax_out, hipStream_t s) {
  const int M = batch * t;
  const auto& c = m->c;
  const int d = c.d_model, H = c.n_q_heads, G = c.n_kv_heads, D = c.head_dim;
  for (int l = 0; l < c.n_layers; ++l) {
    const LayerDev& Ld = m->L[l];
    // RMSNorm + QKV + RoPE + KV append
    GemvParams g;
    g.w = Ld.qkv;
    g.n_rows = Ld.qkv.N;
    g.x = m->x;
    g.x_stride = d;
    g.gamma = Ld.attn_norm;
    g.eps = c.rms_eps;
    g.H = H;
    g.G = G;
    g.D = D;
    g.rope = m->rope;
    g.max_pos = c.max_positions;
    g.seq_lens = seq_lens;
    g.t = t;
    g.page_table = page_table;
    g.max_pages = max_pages;
    g.pool = pool->layer(l);
    g.pool_page_stride = pool->page_elems;
    g.n_pages = pool->n_pages;
    g.kv_dtype = c.kv_dtype;
    g.qout = m->q;
    g.err = m->err;
    if (l == 0) {  // the embedding gather runs in layer 0's input stage
      g.embed = m->embed;
      g.tokens = tokens;
      g.vocab = c.vocab;
      g.x_out = m->x;
    }
    trace_mark(m, BW_K_QKV, l, 0, s);
    if (run_dense(m, IN_RMSNORM, EPI_QKV, g, M, s)) return fail(BW_EHIP, "qkv launch failed (layer %d)", l);
    trace_mark(m, BW_K_QKV, l, 1, s);
    // attention
    AttnParams a = attn_params(m, pool, l, m->q, seq_lens, page_table, t, max_pages, m->attn_out);
    trace_mark(m, BW_K_ATTN, l, 0, s);
    if (launch_attention(a, c.kv_dtype, batch, s)) return fail(BW_EHIP, "attention launch failed (layer %d)", l);
    trace_mark(m, BW_K_ATTN, l, 1, s);
    // O + residual
    GemvParams o;
    o.w = Ld.o;
    o.n_rows = Ld.o.N;
    o.x = m->attn_out;
    o.x_stride = (int64_t)H * D;
    o.y = m->x;
    o.y_stride = d;
    trace_mark(m, BW_K_O, l, 0, s);
    if (run_dense(m, IN_PLAIN, EPI_RESID, o, M, s)) return fail(BW_EHIP, "o launch failed (layer %d)", l);
    trace_mark(m, BW_K_O, l, 1, s);
    if (!is_moe(c)) {
      GemvParams gu;
      gu.w = Ld.gu;
      gu.n_rows = Ld.gu.N;
      gu.x = m->x;
      gu.x_stride = d;
      gu.gamma = Ld.ffn_norm;
      gu.eps = c.rms_eps;
      gu.y = m->act;
      gu.y_stride = m->act_width;
      trace_mark(m, BW_K_GATE_UP, l, 0, s);
      if (run_dense(m, IN_RMSNORM, EPI_SWIGLU, gu, M, s)) return fail(BW_EHIP, "gate/up launch failed (layer %d)", l);
      trace_mark(m, BW_K_GATE_UP, l, 1, s);
      GemvParams dn;
      dn.w = Ld.dn;
      dn.n_rows = Ld.dn.N;
      dn.x = m->act;
      dn.x_stride = m->act_width;
      dn.y = m->x;
      dn.y_stride = d;
      trace_mark(m, BW_K_DOWN, l, 0, s);
      if (run_dense(m, IN_PLAIN, EPI_RESID, dn, M, s)) return fail(BW_EHIP, "down launch failed (layer %d)", l);
      trace_mark(m, BW_K_DOWN, l, 1, s);
    } else {
      int32_t* sel = m->sel + (int64_t)l * c.max_tokens * c.top_k;
      float* gates = m->gates + (int64_t)l * c.max_tokens * c.top_k;
      trace_mark(m, BW_K_ROUTER, l, 0, s);
      if (launch_router(Ld.router, c.n_experts, d, m->x, Ld.ffn_norm, c.rms_eps, M, m->router_logits, s))
        return fail(BW_EHIP, "router launch failed (layer %d)", l);
      if (launch_topk(m->router_logits, c.n_experts, c.top_k, M, sel, gates, s))
        return fail(BW_EHIP, "top-k launch failed (layer %d)", l);
      trace_mark(m, BW_K_ROUTER, l, 1, s);
      GemvParams gu;
      gu.w.K = d;
      gu.n_rows = c.top_k * 2 * c.expert_ffn + c.n_shared * 2 * c.shared_ffn;
      gu.x = m->x;
      gu.x_stride = d;
      gu.gamma = Ld.ffn_norm;
      gu.eps = c.rms_eps;
      gu.y = m->act;
      gu.y_stride = m->act_width;
      gu.sel = sel;
      gu.gates = gates;
      gu.n_experts = c.n_experts;
      gu.top_k = c.top_k;
      gu.n_shared = c.n_shared;
      gu.Fe = c.expert_ffn;
      gu.Fs = c.shared_ffn;
      gu.ex = Ld.ex;
      trace_mark(m, BW_K_MOE_GATE_UP, l, 0, s);
      if (launch_gemv(IN_RMSNORM, EPI_MOE_SWIGLU, gu, M, s)) return fail(BW_EHIP, "expert gate/up launch failed (layer %d)", l);
      trace_mark(m, BW_K_MOE_GATE_UP, l, 1, s);
      GemvParams dn = gu;
      dn.n_rows = d;
      dn.x = m->act;
      dn.x_stride = m->act_width;
      dn.gamma = nullptr;
      dn.y = m->x;
      dn.y_stride = d;
      trace_mark(m, BW_K_MOE_DOWN, l, 0, s);
      if (int e = launch_gemv(IN_MOE_DOWN, EPI_RESID, dn, M, s))
        return fail(BW_EHIP, "expert down launch failed (layer %d, code %d: -2 = unsupported K %d)", l, e,
                    c.top_k * c.expert_ffn + c.n_shared * c.shared_ffn);
      trace_mark(m, BW_K_MOE_DOWN, l, 1, s);
    }
  }
  // final RMSNorm + lm_head + argmax; a step that asks for neither (a prefill chunk before the
  // last) ends with the layers
  if (!logits_out && !argmax_out) return BW_OK;
  GemvParams lm;
  lm.w = m->lm;
  lm.n_rows = m->lm.N;
  lm.x = m->x;
  lm.x_stride = d;
  lm.gamma = m->final_norm;
  lm.eps = c.rms_eps;
  lm.y = logits_out ? logits_out : m->logits;
  lm.y_stride = c.vocab;
  lm.amax_val = m->amax_val;
  lm.amax_idx = m->amax_idx;
  int lm_grid = 0;
  trace_mark(m, BW_K_LM_HEAD, 0, 0, s);
  if (run_dense(m, IN_RMSNORM, EPI_LOGITS, lm, M, s, &lm_grid)) return fail(BW_EHIP, "lm_head launch failed");
  trace_mark(m, BW_K_LM_HEAD, 0, 1, s);
  if (batched(m, lm.w, M)) {
    if (argmax_out && launch_argmax_rows(lm.y, lm.y_stride, c.vocab, M, m->amax_val, m->amax_idx, m->lm_parts,
                                         argmax_out, s))
      return fail(BW_EHIP, "argmax launch failed");
    return BW_OK;
  }
  if (lm_grid > m->lm_parts) return fail(BW_EHIP, "lm_head grid exceeds the argmax workspace");
  if (argmax_out && launch_argmax_final(m->amax_val, m->amax_idx, lm_grid, M, argmax_out, s))
    return fail(BW_EHIP, "argmax launch failed");
  return BW_OK;
}

extern "C" int bw_decode_step(bw_model* m, bw_kv_pool* pool, const int32_t* tokens,
                              const int32_t* seq_lens, const int32_t* page_table, int32_t batch,
                              int32_t t, int32_t max_pages, float* logits_out, int32_t* argmax_out,
                              void* stream) {
  if (!m || !pool || !tokens || !seq_lens || !page_table) return fail(BW_EINVAL, "null argument");
  if (pool->m != m) return fail(BW_ESTATE, "pool belongs to another model");
  if (batch < 1 || t < 1 || max_pages < 1) return fail(BW_EINVAL, "batch, t and max_pages must be positive");
  if (batch * t > m->c.max_tokens) return fail(BW_ERANGE, "batch * t = %d exceeds max_tokens %d", batch * t, m->c.max_tokens);
  hipStream_t s = (hipStream_t)stream;
  // the single launch holds one attention split's page ids in LDS (at most 256 per split);
  // a longer page table takes the kernel chain
  const bool persist_pages =
      m->persist_ok && (max_pages + m->persist_nwg / m->c.n_kv_heads - 1) / (m->persist_nwg / m->c.n_kv_heads) <= 256;
  if (m->persist_ok && m->use_persist && persist_pages && batch == 1 && t == 1 && m->trace_class < 0) {
    // the whole step as one launch (no capture needed: one launch per step)
    PersistParams p = m->pp;
    p.pool = pool->data;
    p.layer_elems = pool->layer_elems;
    p.page_elems = pool->page_elems;
    p.n_pages = pool->n_pages;
    p.tokens = tokens;
    p.seq_lens = seq_lens;
    p.page_table = page_table;
    p.max_pages = max_pages;
    p.logits = logits_out;
    p.argmax = argmax_out;
    if (launch_persist_any(m, p, m->persist_nwg, s, false))
      return fail(BW_EHIP, "single-launch step failed to launch");
    return BW_OK;
  }
  if (!m->use_graphs || m->trace_class >= 0)
    return enqueue_step(m, pool, tokens, seq_lens, page_table, batch, t, max_pages, logits_out, argmax_out, s);
  // replay a captured step when the arguments match one, else capture one (a one-time cost)
  const std::vector<uintptr_t> key = {(uintptr_t)pool, (uintptr_t)tokens, (uintptr_t)seq_lens, (uintptr_t)page_table,
                                      (uintptr_t)batch, (uintptr_t)t, (uintptr_t)max_pages, (uintptr_t)logits_out,
                                      (uintptr_t)argmax_out};
  ++m->use_clock;
  for (auto& g : m->graphs)
    if (g.key == key) {
      g.last_use = m->use_clock;
      HIP_OK(hipGraphLaunch(g.exec, s));
      return BW_OK;
    }
  bw_model::GraphEntry e;
  e.key = key;
  e.last_use = m->use_clock;
  HIP_OK(hipStreamBeginCapture(m->cap_stream, hipStreamCaptureModeRelaxed));
  int rc = enqueue_step(m, pool, tokens, seq_lens, page_table, batch, t, max_pages, logits_out, argmax_out, m->cap_stream);
  hipError_t ce = hipStreamEndCapture(m->cap_stream, &e.graph);
  if (rc) {
    if (e.graph) (void)hipGraphDestroy(e.graph);
    return rc;
  }
  if (ce != hipSuccess) return fail(BW_EHIP, "step capture failed: %s", hipGetErrorString(ce));
  if (hipGraphInstantiate(&e.exec, e.graph, nullptr, nullptr, 0) != hipSuccess) {
    (void)hipGraphDestroy(e.graph);
    return fail(BW_EHIP, "graph instantiation failed");
  }
  if (m->graphs.size() >= 8) {  // evict the least recently used
    size_t v = 0;
    for (size_t i = 1; i < m->graphs.size(); ++i)
      if (m->graphs[i].last_use < m->graphs[v].last_use) v = i;
    (void)hipGraphExecDestroy(m->graphs[v].exec);
    (void)hipGraphDestroy(m->graphs[v].graph);
    m->graphs.erase(m->graphs.begin() + v);
  }
  m->graphs.push_back(e);
  HIP_OK(hipGraphLaunch(e.exec, s));
  return BW_OK;
}

extern "C" int bw_set_graphs(bw_model* m, int32_t enable) {
  if (!m) return fail(BW_EINVAL, "null model");
  m->use_graphs = enable != 0;
  return BW_OK;
}

extern "C" int bw_set_single_launch(bw_model* m, int32_t mode, int32_t* available) {
  if (!m) return fail(BW_EINVAL, "null model");
  if (mode < 0 || mode > 2) return fail(BW_EINVAL, "mode must be 0, 1 or 2");
  m->use_persist = mode != 0;
  m->pp.plain_launch = mode != 2;
  if (available) *available = m->persist_ok ? 1 : 0;
  return BW_OK;
}

extern "C" int bw_set_gemm_min_rows(bw_model* m, int32_t min_rows) {
  if (!m) return fail(BW_EINVAL, "null model");
  if (min_rows < 0) return fail(BW_EINVAL, "min_rows must be >= 0");
  m->gemm_min_rows = min_rows;
  return BW_OK;
}

extern "C" const char* bw_last_error(void) { return g_err.c_str(); }

extern "C" int bw_spec_accept(bw_model* m, int32_t* tokens, const int32_t* argmax, float* logits, int32_t* seq_lens,
                              int32_t* ring, int32_t* count, int32_t ring_cap, int32_t* accepted, int32_t batch,
                              int32_t t, void* stream) {
  if (!m || !tokens || !argmax || !seq_lens) return fail(BW_EINVAL, "null argument");
  if (batch < 1 || t < 1) return fail(BW_EINVAL, "batch and t must be positive");
  if (t > 65535 || batch > 65535) return fail(BW_ERANGE, "batch and t are at most 65535");
  if ((ring == nullptr) != (count == nullptr)) return fail(BW_EINVAL, "ring and count go together");
  if (ring != nullptr && ring_cap < t) return fail(BW_EINVAL, "ring_cap %d is below t = %d", ring_cap, t);
  if (launch_spec_accept(tokens, argmax, logits, m->c.vocab, seq_lens, ring, count, ring_cap, accepted, batch, t,
                         (hipStream_t)stream))
    return fail(BW_EHIP, "acceptance kernel failed to launch");
  return BW_OK;
}

extern "C" int bw_check_device_error(bw_model* m, void* stream, int32_t* flags) {
  if (!m || !flags) return fail(BW_EINVAL, "null argument");
  HIP_OK(hipStreamSynchronize((hipStream_t)stream));
  HIP_OK(hipMemcpy(flags, m->err, 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemset(m->err, 0, 4));
  if (m->persist_ok && (*flags & BW_DERR_PERSIST) &&
      launch_persist_reset(m->pp, m->n_xq, m->n_xp, m->n_xa, m->n_xd, m->n_xf, m->persist_nwg, (hipStream_t)stream))
    return fail(BW_EHIP, "persistent-step reset failed");
  HIP_OK(hipDeviceSynchronize());
  return BW_OK;
}

// ---------------------------------------------------------------------------------------------
// parity-test entry points
// ---------------------------------------------------------------------------------------------

// matrix descriptor, its device->canonical row map and the canonical row count
static int find_mat(const bw_model* m, int which, int layer, int expert, Mat* w, const int32_t** map,
                    int* n_canon, int* half) {
  const auto& c = m->c;
  *map = nullptr;
  *half = -1;  // for interleaved gate/up: 0 = gate half, 1 = up half
  if (which == BW_MAT_LM_HEAD) {
    *w = m->lm;
    *n_canon = m->lm.N;
    return 0;
  }
  if (layer < 0 || layer >= c.n_layers) return fail(BW_EINVAL, "layer out of range");
  const LayerDev& Ld = m->L[layer];
  switch (which) {
    case BW_MAT_QKV: *w = Ld.qkv; *map = m->qkv_map; *n_canon = Ld.qkv.N; return 0;
    case BW_MAT_O: *w = Ld.o; *n_canon = Ld.o.N; return 0;
    case BW_MAT_DOWN:
      if (!is_moe(c)) { *w = Ld.dn; *n_canon = Ld.dn.N; return 0; }
      if (expert < 0 || expert >= c.n_experts) return fail(BW_EINVAL, "expert out of range");
      *w = Ld.ex_dn[expert]; *n_canon = w->N; return 0;
    case BW_MAT_SDOWN:
      if (!is_moe(c) || expert < 0 || expert >= c.n_shared) return fail(BW_EINVAL, "shared expert out of range");
      *w = Ld.ex_dn[c.n_experts + expert]; *n_canon = w->N; return 0;
    case BW_MAT_GATE:
    case BW_MAT_UP:
    case BW_MAT_SGATE:
    case BW_MAT_SUP: {
      const bool shared = which == BW_MAT_SGATE || which == BW_MAT_SUP;
      if (!is_moe(c)) {
        if (shared) return fail(BW_EINVAL, "dense model has no shared expert");
        *w = Ld.gu;
      } else if (shared) {
        if (expert < 0 || expert >= c.n_shared) return fail(BW_EINVAL, "shared expert out of range");
        *w = Ld.ex_gu[c.n_experts + expert];
      } else {
        if (expert < 0 || expert >= c.n_experts) return fail(BW_EINVAL, "expert out of range");
        *w = Ld.ex_gu[expert];
      }
      const int F = w->N / 2;
      *map = m->gu_map.at(F);
      *n_canon = F;
      *half = (which == BW_MAT_GATE || which == BW_MAT_SGATE) ? 0 : 1;
      return 0;
    }
    default: return fail(BW_EINVAL, "unknown matrix selector %d", which);
  }
}

// ---------------------------------------------------------------------------------------------
// tensor export in the canonical layout
// ---------------------------------------------------------------------------------------------

// A named tensor of the model: an fp16 vector or matrix (plain), or one part of an int4 matrix.
struct TensorRef {
  const void* fp16 = nullptr;  // plain fp16 tensor
  int64_t elems = 0;
  Mat w;                       // int4 matrix (codes or scales part)
  bool is_mat = false, scales = false;
  const int32_t* map = nullptr;// device -> canonical row (device memory), or null
  int half = -1;               // interleaved gate/up: 0 = gate rows, 1 = up rows
  int n_canon = 0;             // canonical rows
};

static int parse_tensor(const bw_model* m, const char* name, TensorRef* t) {
  const auto& c = m->c;
  const std::string s(name);
  auto part = [&](const std::string& rest, int which, int layer, int expert) -> int {
    // rest: ".codes" or ".scales"
    if (rest != ".codes" && rest != ".scales") return fail(BW_EINVAL, "tensor %s: expected .codes or .scales", name);
    if (int rc = find_mat(m, which, layer, expert, &t->w, &t->map, &t->n_canon, &t->half)) return rc;
    t->is_mat = true;
    t->scales = rest == ".scales";
    return BW_OK;
  };
  if (s == "embed") { t->fp16 = m->embed; t->elems = (int64_t)c.vocab * c.d_model; return BW_OK; }
  if (s == "final_norm") { t->fp16 = m->final_norm; t->elems = c.d_model; return BW_OK; }
  if (s.rfind("lm_head", 0) == 0) return part(s.substr(7), BW_MAT_LM_HEAD, 0, 0);
  int l = -1, e = -1, n = 0;
  char kind[32] = {0}, mat[16] = {0}, tail[16] = {0};
  if (sscanf(name, "layers.%d.%31[a-z_]%n", &l, kind, &n) < 2 || l < 0 || l >= c.n_layers)
    return fail(BW_EINVAL, "unknown tensor %s", name);
  const std::string k(kind), rest = s.substr(n);
  if (k == "attn_norm" && rest.empty()) { t->fp16 = m->L[l].attn_norm; t->elems = c.d_model; return BW_OK; }
  if (k == "ffn_norm" && rest.empty()) { t->fp16 = m->L[l].ffn_norm; t->elems = c.d_model; return BW_OK; }
  if (k == "router" && rest.empty() && is_moe(c)) {
    t->fp16 = m->L[l].router;
    t->elems = (int64_t)c.n_experts * c.d_model;
    return BW_OK;
  }
  if (k == "experts" || k == "shared") {
    if (!is_moe(c) || sscanf(rest.c_str(), ".%d.%15[a-z]%15s", &e, mat, tail) != 3)
      return fail(BW_EINVAL, "unknown tensor %s", name);
    const std::string mm(mat);
    const bool sh = k == "shared";
    const int which = mm == "gate" ? (sh ? BW_MAT_SGATE : BW_MAT_GATE)
                    : mm == "up"   ? (sh ? BW_MAT_SUP : BW_MAT_UP)
                    : mm == "down" ? (sh ? BW_MAT_SDOWN : BW_MAT_DOWN) : -1;
    if (which < 0) return fail(BW_EINVAL, "unknown tensor %s", name);
    return part(tail, which, l, e);
  }
  const int which = k == "qkv" ? BW_MAT_QKV : k == "o" ? BW_MAT_O : k == "gate" ? BW_MAT_GATE
                  : k == "up" ? BW_MAT_UP : k == "down" ? BW_MAT_DOWN : -1;
  if (which < 0 || (is_moe(c) && (which == BW_MAT_GATE || which == BW_MAT_UP || which == BW_MAT_DOWN)))
    return fail(BW_EINVAL, "unknown tensor %s", name);
  return part(rest, which, l, 0);
}

static size_t tensor_bytes(const TensorRef& t) {
  if (!t.is_mat) return (size_t)t.elems * 2;
  return t.scales ? (size_t)t.n_canon * (t.w.K / 32) * 2 : (size_t)t.n_canon * (t.w.K / 2);
}

extern "C" int bw_model_tensor_bytes(const bw_model* m, const char* name, size_t* bytes) {
  if (!m || !name || !bytes) return fail(BW_EINVAL, "null argument");
  TensorRef t;
  if (int rc = parse_tensor(m, name, &t)) return rc;
  *bytes = tensor_bytes(t);
  return BW_OK;
}

extern "C" int bw_model_export_tensor(const bw_model* m, const char* name, void* host_dst, size_t bytes) {
  if (!m || !name || !host_dst) return fail(BW_EINVAL, "null argument");
  TensorRef t;
  if (int rc = parse_tensor(m, name, &t)) return rc;
  const size_t want = tensor_bytes(t);
  if (bytes != want) return fail(BW_ERANGE, "tensor %s holds %zu bytes, not %zu", name, want, bytes);
  HIP_OK(hipDeviceSynchronize());
  if (!t.is_mat) {
    HIP_OK(hipMemcpy(host_dst, t.fp16, want, hipMemcpyDeviceToHost));
    return BW_OK;
  }
  const Mat& w = t.w;
  const int64_t rb = w.K / 2, nblk = w.K / 32;
  // device rows and their canonical rows (gate/up: the requested half of the interleave)
  std::vector<int32_t> map;
  if (t.map) {
    map.resize(w.N);
    HIP_OK(hipMemcpy(map.data(), t.map, sizeof(int32_t) * w.N, hipMemcpyDeviceToHost));
  }
  const int64_t lo = t.half < 0 ? 0 : (int64_t)t.half * t.n_canon;
  auto canon_of = [&](int64_t r) -> int64_t {
    const int64_t cr = t.map ? (int64_t)map[r] - lo : r;
    return cr >= 0 && cr < t.n_canon ? cr : -1;
  };
  if (!t.scales) {
    std::vector<uint8_t> dev((size_t)w.N * rb);
    HIP_OK(hipMemcpy(dev.data(), w.codes, dev.size(), hipMemcpyDeviceToHost));
    uint8_t* dst = (uint8_t*)host_dst;
    for (int64_t r = 0; r < w.N; ++r)
      if (const int64_t cr = canon_of(r); cr >= 0) memcpy(dst + cr * rb, dev.data() + r * rb, rb);
  } else {
    std::vector<uint16_t> dev((size_t)w.N * nblk);
    HIP_OK(hipMemcpy(dev.data(), w.scales, dev.size() * 2, hipMemcpyDeviceToHost));
    uint16_t* dst = (uint16_t*)host_dst;
    // device scales are tiled per row as [lpr][nb]: block b sits at (b % lpr) * nb + b / lpr
    for (int64_t r = 0; r < w.N; ++r)
      if (const int64_t cr = canon_of(r); cr >= 0)
        for (int64_t b = 0; b < nblk; ++b) dst[cr * nblk + b] = dev[r * nblk + (b % w.lpr) * w.nb + b / w.lpr];
  }
  return BW_OK;
}

extern "C" int bw_debug_copy_lm_head_row(bw_model* m, int32_t src, int32_t dst) {
  if (!m) return fail(BW_EINVAL, "null model");
  const Mat& w = m->lm;
  if (src < 0 || src >= w.N || dst < 0 || dst >= w.N) return fail(BW_EINVAL, "row out of range");
  const int64_t rb = w.K / 2, sb = (w.K / 32) * 2;
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy((uint8_t*)w.codes + dst * rb, w.codes + src * rb, rb, hipMemcpyDeviceToDevice));
  HIP_OK(hipMemcpy((uint8_t*)w.scales + dst * sb, (const uint8_t*)w.scales + src * sb, sb, hipMemcpyDeviceToDevice));
  HIP_OK(hipDeviceSynchronize());
  return BW_OK;
}

extern "C" int bw_debug_dequant(const bw_model* m, int32_t which, int32_t layer, int32_t expert,
                                float* dst, void* stream) {
  if (!m || !dst) return fail(BW_EINVAL, "null argument");
  Mat w;
  const int32_t* map;
  int n, half;
  if (int rc = find_mat(m, which, layer, expert, &w, &map, &n, &half)) return rc;
  // interleaved gate/up: keep only the requested half (canonical rows [half*F, half*F + F))
  const int lo = half < 0 ? 0 : half * n;
  if (launch_dequant(w, map, lo, n, dst, (hipStream_t)stream)) return fail(BW_EHIP, "dequant launch failed");
  return BW_OK;
}

extern "C" int bw_debug_matvec(bw_model* m, int32_t which, int32_t layer, int32_t expert,
                               const float* x, int32_t n_vec, float* y, void* stream) {
  if (!m || !x || !y) return fail(BW_EINVAL, "null argument");
  if (n_vec < 1) return fail(BW_EINVAL, "n_vec must be positive");
  if (n_vec > m->c.max_tokens) return fail(BW_ERANGE, "n_vec exceeds max_tokens");
  Mat w;
  const int32_t* map;
  int n, half;
  if (int rc = find_mat(m, which, layer, expert, &w, &map, &n, &half)) return rc;
  GemvParams g;
  g.w = w;
  g.n_rows = w.N;
  g.x = x;
  g.x_stride = w.K;
  g.row_map = map;
  g.map_lo = half < 0 ? 0 : half * n;
  g.map_n = n;
  g.y = y;
  g.y_stride = n;
  if (run_dense(m, IN_PLAIN, EPI_STORE_CANON, g, n_vec, (hipStream_t)stream)) return fail(BW_EHIP, "matrix product launch failed");
  return BW_OK;
}

extern "C" int bw_debug_attention(bw_model* m, bw_kv_pool* pool, int32_t layer, const float* q,
                                  const int32_t* seq_lens, const int32_t* page_table, int32_t batch,
                                  int32_t t, int32_t max_pages, float* out, void* stream) {
  if (!m || !pool || !q || !seq_lens || !page_table || !out) return fail(BW_EINVAL, "null argument");
  if (pool->m != m) return fail(BW_ESTATE, "pool belongs to another model");
  if (layer < 0 || layer >= m->c.n_layers) return fail(BW_EINVAL, "layer out of range");
  if (batch < 1 || t < 1 || batch * t > m->c.max_tokens) return fail(BW_ERANGE, "batch * t out of range");
  AttnParams a = attn_params(m, pool, layer, q, seq_lens, page_table, t, max_pages, out);
  if (launch_attention(a, m->c.kv_dtype, batch, (hipStream_t)stream)) return fail(BW_EHIP, "attention launch failed");
  return BW_OK;
}

// ---------------------------------------------------------------------------------------------
// attention that allocates nothing: split partials in a static device array
// ---------------------------------------------------------------------------------------------

// The split-K partials [rows][heads][splits][head_dim + 2] of bw_attention_noalloc live here, one
// copy per GPU for the life of the process. In host code the name is only a stand-in: the device
// address comes from hipGetSymbolAddress, once per device (noalloc_scratch below).
constexpr size_t kNoallocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64] = {};  // per device id

static int noalloc_scratch(void** out) {
  int dev = 0;
  HIP_OK(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return fail(BW_EINVAL, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return fail(BW_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return BW_OK;
}

extern "C" int bw_attention_noalloc(bw_model* m, bw_kv_pool* pool, int32_t layer, const float* q,
                                    const int32_t* seq_lens, const int32_t* page_table, int32_t batch,
                                    int32_t t, int32_t max_pages, float* out, void* stream) {
  if (!m || !pool || !q || !seq_lens || !page_table || !out) return fail(BW_EINVAL, "null argument");
  if (pool->m != m) return fail(BW_ESTATE, "pool belongs to another model");
  if (layer < 0 || layer >= m->c.n_layers) return fail(BW_EINVAL, "layer out of range");
  if (batch < 1 || t < 1 || max_pages < 1) return fail(BW_EINVAL, "batch, t and max_pages must be positive");
  if (batch > 65535 || t > 65535) return fail(BW_ERANGE, "batch and t are at most 65535");
  AttnParams a = attn_params(m, pool, layer, q, seq_lens, page_table, t, max_pages, out);
  // splits of this call: enough for max_pages at the vector-unit kernel's split length (the
  // matrix-core kernel takes longer splits, so fewer)
  a.max_splits = (max_pages + a.pages_per_split - 1) / a.pages_per_split;
  const double need = (double)batch * t * a.H * a.max_splits * (a.D + 2) * sizeof(float);
  if (need > (double)kNoallocScratchBytes)
    return fail(BW_ERANGE, "attention partials need %.0f bytes, more than the %zu-byte static scratch", need,
                kNoallocScratchBytes);
  void* ptr = nullptr;
  if (int rc = noalloc_scratch(&ptr)) return rc;
  a.part = (float*)ptr;
  a.counters = nullptr;  // the attention kernels keep no arrival counters
  if (launch_attention(a, m->c.kv_dtype, batch, (hipStream_t)stream)) return fail(BW_EHIP, "attention launch failed");
  return BW_OK;
}

// ---------------------------------------------------------------------------------------------
// MXFP4 weights
// ---------------------------------------------------------------------------------------------

extern "C" int bw_mx_gemv(const uint8_t* codes, const uint8_t* scales, const float* x, float* y, int64_t N,
                          int64_t K, void* stream) {
  if (!codes || !scales || !x || !y) return fail(BW_EINVAL, "null argument");
  if (N < 1 || N > ((int64_t)1 << 40)) return fail(BW_EINVAL, "N out of range");
  if (K < 32 || K % 32 || K > kMxGemvMaxK) return fail(BW_EINVAL, "K must be a multiple of 32 in [32, %d]", kMxGemvMaxK);
  if ((uintptr_t)x % 16) return fail(BW_EINVAL, "x must be 16-byte aligned");
  if (launch_mx_gemv(codes, scales, x, y, N, (int)K, (hipStream_t)stream)) return fail(BW_EHIP, "MXFP4 GEMV launch failed");
  return BW_OK;
}

static int mx_gemm_check(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || M > ((int64_t)1 << 22)) return fail(BW_EINVAL, "M out of range");
  if (N < 1 || N > ((int64_t)1 << 36)) return fail(BW_EINVAL, "N out of range");
  if (K < 32 || K % 32 || K > ((int64_t)1 << 20)) return fail(BW_EINVAL, "K must be a multiple of 32 in [32, 2^20]");
  return BW_OK;
}

extern "C" int bw_mx_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t* bytes_out) {
  if (!bytes_out) return fail(BW_EINVAL, "null argument");
  if (int rc = mx_gemm_check(M, N, K)) return rc;
  *bytes_out = mx_gemm_workspace_bytes(M, N, (int)K, mx_gemm_splits(M, N, (int)K));
  return BW_OK;
}

extern "C" int bw_mx_gemm(const uint8_t* codes, const uint8_t* scales, const float* X, float* Y, int64_t M, int64_t N,
                          int64_t K, void* workspace, int64_t workspace_bytes, void* stream) {
  if (!codes || !scales || !X || !Y || !workspace) return fail(BW_EINVAL, "null argument");
  if (int rc = mx_gemm_check(M, N, K)) return rc;
  const int splits = mx_gemm_splits(M, N, (int)K);
  const int64_t need = mx_gemm_workspace_bytes(M, N, (int)K, splits);
  if (workspace_bytes < need) return fail(BW_ERANGE, "workspace of %lld bytes, %lld needed", (long long)workspace_bytes,
                                          (long long)need);
  if ((uintptr_t)workspace % 256) return fail(BW_EINVAL, "workspace must be 256-byte aligned");
  if ((uintptr_t)X % 16) return fail(BW_EINVAL, "X must be 16-byte aligned");
  if (launch_mx_gemm(codes, scales, X, Y, M, N, (int)K, workspace, splits, (hipStream_t)stream))
    return fail(BW_EHIP, "MXFP4 GEMM launch failed");
  return BW_OK;
}

extern "C" int bw_debug_kv_round(int32_t kv_dtype, const float* x, int64_t n, uint16_t* bits, float* back,
                                 void* stream) {
  if (!x || !bits || !back) return fail(BW_EINVAL, "null argument");
  if (n < 1 || n > (int64_t)1 << 31) return fail(BW_EINVAL, "n out of range");
  if (kv_dtype != BW_KV_F16 && kv_dtype != BW_KV_BF16 && kv_dtype != BW_KV_FP8) return fail(BW_EINVAL, "bad kv_dtype");
  if (launch_kv_round(kv_dtype, x, n, bits, back, (hipStream_t)stream)) return fail(BW_EHIP, "launch failed");
  return BW_OK;
}

extern "C" int bw_debug_read_experts(bw_model* m, int32_t n_rows, int32_t* host_dst, void* stream) {
  if (!m || !host_dst) return fail(BW_EINVAL, "null argument");
  if (!is_moe(m->c)) return fail(BW_ESTATE, "dense model");
  if (n_rows < 1 || n_rows > m->c.max_tokens) return fail(BW_ERANGE, "n_rows out of range");
  HIP_OK(hipStreamSynchronize((hipStream_t)stream));
  const auto& c = m->c;
  for (int l = 0; l < c.n_layers; ++l)
    HIP_OK(hipMemcpy(host_dst + (size_t)l * n_rows * c.top_k, m->sel + (size_t)l * c.max_tokens * c.top_k,
                     sizeof(int32_t) * n_rows * c.top_k, hipMemcpyDeviceToHost));
  return BW_OK;
}

extern "C" int bw_debug_single_launch_stamps(bw_model* m, uint64_t* stamps_dev, int32_t n) {
  if (!m) return fail(BW_EINVAL, "null model");
  if (!m->persist_ok) return fail(BW_ESTATE, "the model has no single-launch step");
  const int rec = m->c.n_layers * 16 + 8;
  if (stamps_dev && n < rec) return fail(BW_ERANGE, "need %d stamps", rec);
  m->pp.stamps = stamps_dev;
  m->pp.stamp_stride = stamps_dev && (int64_t)n >= (int64_t)rec * m->persist_nwg ? rec : 0;
  return BW_OK;
}

extern "C" int bw_debug_single_launch_deadline(bw_model* m, uint64_t ticks) {
  if (!m) return fail(BW_EINVAL, "null model");
  if (!m->persist_ok) return fail(BW_ESTATE, "the model has no single-launch step");
  m->pp.deadline_ticks = ticks;
  return BW_OK;
}

extern "C" int bw_debug_read_hidden(bw_model* m, int32_t n_rows, float* host_dst, void* stream) {
  if (!m || !host_dst) return fail(BW_EINVAL, "null argument");
  if (n_rows < 1 || n_rows > m->c.max_tokens) return fail(BW_ERANGE, "n_rows out of range");
  HIP_OK(hipStreamSynchronize((hipStream_t)stream));
  HIP_OK(hipMemcpy(host_dst, m->x, sizeof(float) * n_rows * m->c.d_model, hipMemcpyDeviceToHost));
  return BW_OK;
}
