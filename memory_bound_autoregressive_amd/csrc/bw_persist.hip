// bw_persist.hip - the whole batch-1 decode step of a dense model as one persistent kernel.
//
// Why: a batch-1 step is a chain of ~6 matrix passes per layer, each moving 10-60 MB. As separate
// kernels every pass pays a launch gap, a ramp of its first loads and a tail, ~5 us, against
// 1.3-8 us of streaming. The pages attribute the same loss to kernel launches and intermediate
// round trips and answer it by fusion (bw24 vs llama.cpp page, section 2.2). Here one workgroup
// per CU stays resident for the whole step; the phases of a layer hand their (small) output
// vectors to each other through device memory, and each workgroup issues its next weight loads
// before it waits for the next input, so weight streaming continues across phase boundaries.
//
// Exchange. Each phase output element is one 32-bit word: the fp32 value with its two lowest
// mantissa bits replaced by an epoch tag (a relative change below 2^-21). Producers store words
// with agent-scope relaxed atomic stores (written through the XCD-local L2); consumers read them
// with 16-byte loads that are coherent across the XCD L2s (sc1) and re-read every word whose tag
// is not the one they wait for. A word is written once per layer, and consecutive writes of a
// word carry different tags (mod 4), so a consumer can neither take a stale word nor wait on a
// word that was already overwritten (every phase needs all of its predecessor's output, so no
// workgroup is more than one phase ahead of any other). No fences are used. The exact fp32
// residual rows stay in the LDS of the workgroup that owns them; only their exchanged copies are
// tagged. Keys and values are rounded to the cache dtype before exchange, which leaves their low
// bits zero.
//
// Every wait is bounded: a deadline on the real-time counter, and a device abort flag that any
// waiter raises and every waiter polls. An aborted step sets BW_DERR_PERSIST in the error word and
// all workgroups return; the abort flag stays raised (later steps return at once) until the host
// clears it (bw_check_device_error), which also re-tags the exchange buffers.
//
// Phases of layer l (tags T(l) = epoch * (L + 2) + l + 1; the embedding writes T(-1)):
//   QKV   in x (RMSNorm)      rows (Hq + 2Hkv) D, RoPE + KV append      out xq
//   ATTN  in xq (q, new k/v)  (KV head, split) over the paged cache     out xp (acc, m, l)
//   MERGE in xp               H*D outputs                               out xa
//   O     in xa               d rows, residual (row owner)              out xm
//   GU    in xm (RMSNorm)     2F rows, SwiGLU pairs                     out xf
//   DOWN  in xf               d rows, residual (row owner)              out xx
// then LM (in xx, RMSNorm; logits + per-workgroup argmax) and ARGMAX (workgroup 0). Each buffer
// above is written once per layer, so two consecutive writes of a word differ in tag by 1, 2
// (xx across a step boundary) or 3 (the others across a step boundary). The argmax partials are
// written once per step and carry the epoch itself (difference 1).
#include <algorithm>
#include <type_traits>

#include "bw_common.h"
#include "bw_dot.h"
#include "bw_lanes.h"
#include "bw_mfma.h"
#include "bw_internal.h"

namespace bw {

constexpr int kPT = 512;           // threads per workgroup
constexpr int kPW = kPT / kWave;   // waves per workgroup
constexpr uint32_t kRsrc3 = 0x00020000u;
constexpr int kCohSC1 = 16;        // cache policy: coherent across the XCD L2s
constexpr float kNoScore = -1.0e30f;               // running max of a split without positions
constexpr int kOOB = 0x7FFFFFF0;  // buffer offset past every buffer: the load returns zero, touches nothing
// argmax index of a workgroup with no candidate (every logit NaN): the largest index the 30-bit
// field of an argmax partial holds, so it survives the packing and loses every tie to a real row
constexpr int kNoIdx = 0x3FFFFFFF;

// ---- exchange words ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t xenc(float v, uint32_t tag) { return (__float_as_uint(v) & ~3u) | (tag & 3u); }
__device__ __forceinline__ float xdec(uint32_t w) { return __uint_as_float(w & ~3u); }
__device__ __forceinline__ bool xok(uint32_t w, uint32_t tag) { return ((w ^ tag) & 3u) == 0u; }
__device__ __forceinline__ __amdgpu_buffer_rsrc_t xrsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, kRsrc3);
}
__device__ __forceinline__ u32x4 xload4(__amdgpu_buffer_rsrc_t r, int idx4) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, idx4 * 16, 0, kCohSC1);
}
// A buffer descriptor whose words are provably uniform: a pointer kept across phases may sit in
// vector registers, and a descriptor built from those would make every load through it a loop
// over lanes; readfirstlane puts the words back in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* p, int bytes) {
  const uint64_t a = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a), hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), 0, __builtin_amdgcn_readfirstlane(bytes),
                                           kRsrc3);
}
__device__ __forceinline__ uint32_t xload1(__amdgpu_buffer_rsrc_t r, int idx) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, idx * 4, 0, kCohSC1);
}
__device__ __forceinline__ void xstore(uint32_t* base, int idx, float v, uint32_t tag) {
  __hip_atomic_store(base + idx, xenc(v, tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Ctl {
  uint32_t* abort_flag;
  int32_t* err;
  int* bail;         // LDS flag of this workgroup
  uint64_t t0;       // real-time counter at the start of the current wait
  uint64_t deadline; // ticks of the 100 MHz real-time counter one wait may take
};

// The abort flag as a coherent buffer load, issued in the same batch as a wait's reloads so that
// one memory round trip serves both.
__device__ __forceinline__ uint32_t load_abort(const Ctl& c) {
  return __builtin_amdgcn_raw_buffer_load_b32(__builtin_amdgcn_make_buffer_rsrc(c.abort_flag, 0, 4, kRsrc3), 0, 0,
                                              kCohSC1);
}

// true when this wait must give up: the step was aborted elsewhere (flag: the abort flag as last
// loaded) or the deadline passed
__device__ __forceinline__ bool give_up(Ctl& c, uint32_t flag) {
  if (*c.bail) return true;
  if (flag != 0u || __builtin_amdgcn_s_memrealtime() - c.t0 > c.deadline) {
    atomicOr(c.err, BW_DERR_PERSIST_BIT);
    __hip_atomic_store(c.abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *c.bail = 1;
    return true;
  }
  return false;
}

// Waits on up to N words (idx[i] < 0: unused) in two parts: poll_words_issue loads every word
// once (unconditionally; an unused slot reads zero past the buffer), the caller may then issue its
// weight loads, and poll_words_wait checks the first results outside the retry loop, so that
// check waits for the word loads only, not for weight loads issued after them.
template <int N>
__device__ __forceinline__ void poll_words_issue(__amdgpu_buffer_rsrc_t r, const int (&idx)[N], uint32_t (&w)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) w[i] = __builtin_amdgcn_raw_buffer_load_b32(r, idx[i] >= 0 ? idx[i] * 4 : kOOB, 0, kCohSC1);
}
template <int N>
__device__ __forceinline__ void poll_words_wait(__amdgpu_buffer_rsrc_t r, const int (&idx)[N], uint32_t tag, uint32_t (&w)[N],
                                                Ctl& c) {
  c.t0 = __builtin_amdgcn_s_memrealtime();
  bool all = true;
#pragma unroll
  for (int i = 0; i < N; ++i) all &= idx[i] < 0 || xok(w[i], tag);
  uint32_t flag = 0u;
  while (!all && !give_up(c, flag)) {
    __builtin_amdgcn_s_sleep(1);
    flag = load_abort(c);
    // branch-free reloads (a word already seen reads past the buffer), so they all go out
    // before the one wait below
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const bool need = idx[i] >= 0 && !xok(w[i], tag);
      const uint32_t nw = __builtin_amdgcn_raw_buffer_load_b32(r, need ? idx[i] * 4 : kOOB, 0, kCohSC1);
      w[i] = need ? nw : w[i];
    }
    all = true;
#pragma unroll
    for (int i = 0; i < N; ++i) all &= idx[i] < 0 || xok(w[i], tag);
  }
}

// This thread's index, opaque to the compiler: every phase starts from a fresh copy, so the
// per-thread address terms of a phase are formed inside it instead of being hoisted out of the
// layer loop and held in registers for the whole step.
__device__ __forceinline__ int phase_tid() {
  int t;
  asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"((int)threadIdx.x));
  return t;
}
__device__ __forceinline__ int wave_of(int tid) { return __builtin_amdgcn_readfirstlane(tid >> 6); }

// A small read-only struct as wave-uniform values: each 32-bit word goes through readfirstlane,
// so pointers built from it (buffer descriptors) are known uniform and loads through them need no
// per-lane loop.
template <typename T>
__device__ __forceinline__ T load_uniform(const T* src) {
  static_assert(sizeof(T) % 4 == 0, "word-sized struct");
  T r;
  const uint32_t* a = reinterpret_cast<const uint32_t*>(src);
  uint32_t* b = reinterpret_cast<uint32_t*>(&r);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) b[i] = __builtin_amdgcn_readfirstlane(a[i]);
  return r;
}

// measurement hook: workgroup 0 (or every workgroup, at its own record) stores the real-time
// counter at a phase start
__device__ __forceinline__ void stamp(const PersistParams& p, int idx) {
  if (p.stamps != nullptr && threadIdx.x == 0 && (p.stamp_stride > 0 || blockIdx.x == 0))
    p.stamps[(int64_t)blockIdx.x * p.stamp_stride + idx] = __builtin_amdgcn_s_memrealtime();
}

// ---- LDS layout ---------------------------------------------------------------------------------

struct Lds {
  float* xs;     // staged input vector [Kmax] (bank-swizzled blocks)
  float* bs;     // block sums [Kmax / 32]
  float* ydot;   // row dot products of the current phase [kMaxRows]
  float* resid;  // exact residual rows owned by this workgroup [kMaxOwn]
  float* red;    // reduction scratch [32]
  float* mrg;    // merge scratch [kMrg]
  int* pgid;     // page ids of this workgroup's attention split [kMaxSplitPages]
  float* att;    // attention scratch
  uint32_t* ltab;  // two slots of the layer table (this layer's and the next one's PLayer)
};
constexpr int kMaxRows = 1024;  // rows per workgroup per phase held in ydot
#ifndef BW_LM_RW
#define BW_LM_RW 4
#endif
constexpr int kLmRW = BW_LM_RW;  // row steps per group of the lm_head pass
constexpr int kMaxOwn = 64;     // residual rows per workgroup
constexpr int kMaxSplitPages = 256;  // pages of one attention split (workgroup)
constexpr int kMaxSplit = kPT / 4;  // attention splits per KV head (workgroups / KV heads)
constexpr int kMergeNA = 8;         // split partial words per thread in one poll round of a merger
constexpr int kLW = (int)(sizeof(PLayer) / 4);  // words of one layer's table entry
static_assert(sizeof(PLayer) % 16 == 0 && kLW <= kWave, "layer table entry in whole 16-byte words");
// merge scratch: (m, l) of [splits], factors [splits], partial sums [kPT], the denominator
// MoE scratch inside mrg (free outside the merge phase), in floats: top-k candidates [kMoeMaxE]
// (uint64 keys), maxima of 16-key rows [32] (uint64), the threshold (uint64) and candidate count,
// chosen experts [64] and their keys [64] (uint64), slot gates, slot matrix pointers [slots][4],
// and the gate/up matrix pointers of every expert [E + shared][2]
constexpr int kMoeMaxE = 512, kMoeCand = 0, kMoeGmax = kMoeCand + 2 * kMoeMaxE, kMoeThr = kMoeGmax + 64;
constexpr int kMoeCnt = kMoeThr + 2, kMoeChosen = kMoeThr + 8, kMoeChosenKey = kMoeChosen + 64;
constexpr int kMoeGate = kMoeChosenKey + 128, kMoePtr = kMoeGate + 64;
constexpr int kMoeMaxSlots = 32;
constexpr int kMoeAll = kMoePtr + 2 * 4 * kMoeMaxSlots;
constexpr int kMoeMaxEx = 480;  // routed + shared experts
constexpr int kMrgMerge = 3 * kMaxSplit + kPT + 8;
constexpr int kMrgMoe = kMoeAll + 2 * 2 * kMoeMaxEx;
constexpr int kMrg = kMrgMerge > kMrgMoe ? kMrgMerge : kMrgMoe;
static_assert(kMoeGmax % 4 == 0 && kMoeThr % 2 == 0 && kMoeChosenKey % 2 == 0 && kMoePtr % 4 == 0 && kMoeAll % 4 == 0,
              "MoE tables aligned");

// Router logit as a 64-bit key whose unsigned order is the top-k order: the float's bits mapped
// to an order-preserving integer (NaN as -inf, -0 as +0) above the complemented expert index, so
// that of equal logits the lower index ranks first and no two keys are equal. Zero is below every
// key (padding).
__device__ __forceinline__ uint64_t moe_key(float v, int e) {
  if (v != v) v = -INFINITY;
  if (v == 0.f) v = 0.f;
  const uint32_t b = __float_as_uint(v);
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}
__device__ __forceinline__ float moe_key_value(uint64_t k) {
  const uint32_t o = (uint32_t)(k >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// ---- staging of a GEMV input from the exchange ------------------------------------------------
// xs gets the K values (times the RMSNorm factor and gain when NORM), bs the per-block sums.
// stage_issue loads every chunk once (and the gain), the caller then issues the phase's first
// weight loads, and stage_finish waits (its first check needs only the chunk loads: waits count
// loads in issue order), normalises and stores. The caller synchronises before stage_issue's
// data is used by other threads' previous phase; stage_finish ends with a barrier.
template <int K>
struct XStage {
  static constexpr int N4 = K / 4, PER = (N4 + kPT - 1) / kPT;
  u32x4 v[PER];
  uint32_t g[PER][2];
};

template <int K, bool NORM>
__device__ __forceinline__ void stage_issue(int tid, const uint32_t* xin, const uint16_t* gamma, XStage<K>& x) {
  using X = XStage<K>;
  const __amdgpu_buffer_rsrc_t r = xrsrc(xin, (int64_t)K * 4);
  const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc((void*)gamma, 0, K * 2, kRsrc3);
#pragma unroll
  for (int i = 0; i < X::PER; ++i) {
    const int q = tid + i * kPT;
    if constexpr (NORM) {
      const auto gv = __builtin_amdgcn_raw_buffer_load_b64(rg, q < X::N4 ? q * 8 : kOOB, 0, 0);
      x.g[i][0] = gv[0];
      x.g[i][1] = gv[1];
    }
    x.v[i] = __builtin_amdgcn_raw_buffer_load_b128(r, q < X::N4 ? q * 16 : kOOB, 0, kCohSC1);
  }
}

template <int K, bool NORM>
__device__ __forceinline__ void stage_finish(int tid, const uint32_t* xin, uint32_t tag, float eps, XStage<K>& x, Lds& s,
                                             Ctl& c) {
  using X = XStage<K>;
  constexpr int N4 = X::N4, PER = X::PER;
  auto& v = x.v;
  {
    const __amdgpu_buffer_rsrc_t r = xrsrc(xin, (int64_t)K * 4);
    c.t0 = __builtin_amdgcn_s_memrealtime();
    bool all = true;
#pragma unroll
    for (int i = 0; i < PER; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) all &= tid + i * kPT >= N4 || xok(v[i][k], tag);
    uint32_t flag = 0u;
    while (!all && !give_up(c, flag)) {
      __builtin_amdgcn_s_sleep(1);
      flag = load_abort(c);
      all = true;
#pragma unroll
      for (int i = 0; i < PER; ++i) {  // branch-free, as in poll_words_wait
        const int q = tid + i * kPT;
        bool ok = true;
#pragma unroll
        for (int k = 0; k < 4; ++k) ok &= xok(v[i][k], tag);
        ok = ok || q >= N4;
        const u32x4 nv = __builtin_amdgcn_raw_buffer_load_b128(r, ok ? kOOB : q * 16, 0, kCohSC1);
        v[i] = ok ? v[i] : nv;
      }
#pragma unroll
      for (int i = 0; i < PER; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) all &= tid + i * kPT >= N4 || xok(v[i][k], tag);
    }
  }
  float scale = 1.f;
  if constexpr (NORM) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (tid + i * kPT < N4)
#pragma unroll
        for (int k = 0; k < 4; ++k) ss = fmaf(xdec(v[i][k]), xdec(v[i][k]), ss);
    ss = wsum(ss);
    if ((tid & 63) == 0) s.red[wave_of(tid)] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kPW; ++w) tot += s.red[w];
    scale = 1.0f / sqrtf(tot / (float)K + eps);
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int q = tid + i * kPT;  // chunk q = elements 4q..4q+3; block q / 8 sits in 8 adjacent lanes
    const bool in = q < N4;
    const int k = 4 * q;
    float4 f = make_float4(xdec(v[i][0]), xdec(v[i][1]), xdec(v[i][2]), xdec(v[i][3]));
    if constexpr (NORM) {
      f.x *= scale * f16_to_f32((uint16_t)(x.g[i][0] & 0xFFFFu));
      f.y *= scale * f16_to_f32((uint16_t)(x.g[i][0] >> 16));
      f.z *= scale * f16_to_f32((uint16_t)(x.g[i][1] & 0xFFFFu));
      f.w *= scale * f16_to_f32((uint16_t)(x.g[i][1] >> 16));
    }
    float cs = in ? (f.x + f.y) + (f.z + f.w) : 0.f;
    // elements 16..31 of a block pair with the high nibbles, which block_dot_hs reads 16x too large
    if ((k & 31) >= 16) f = make_float4(f.x * 0.0625f, f.y * 0.0625f, f.z * 0.0625f, f.w * 0.0625f);
    if (in) *(float4*)xs_chunk(s.xs, k >> 5, (k & 31) >> 2) = f;
    cs = sum8(cs);
    if (in && (q & 7) == 0) s.bs[q >> 3] = cs;
  }
  __syncthreads();
}

// ---- block dot product on high-nibble-scaled x ------------------------------------------------
// As block_dot (bw_dot.h), with one AND fewer per code pair: the high nibbles are masked in place
// ((w >> s) & 0x00F000F0 reads as two fp16 subnormals 16 q 2^-24, exact), and the x values they
// pair with (elements 16..31 of the block) were staged divided by 16 (exact), so every product is
// still q x 2^-24. Per code dword: one shift and four ANDs for eight codes.
__device__ __forceinline__ float block_dot_hs(u32x4 q, const float4* xv, float bsum) {
  float d = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w = q[k], w8 = q[k] >> 8;
    const float4 lo = xv[k], hi = xv[4 + k];
    d = mix2(w & 0x000F000Fu, lo.x, lo.z, d);    // elements 4k, 4k+2
    d = mix2(w & 0x00F000F0u, hi.x, hi.z, d);    // elements 16+4k, 16+4k+2 (x / 16)
    d = mix2(w8 & 0x000F000Fu, lo.y, lo.w, d);   // elements 4k+1, 4k+3
    d = mix2(w8 & 0x00F000F0u, hi.y, hi.w, d);   // elements 16+4k+1, 16+4k+3 (x / 16)
  }
  return fmaf(16777216.0f, d, -8.0f * bsum);
}

// ---- GEMV over a row range --------------------------------------------------------------------
// Rows [r0, r1) of w; wave v takes groups v, v + kPW, ... of RW row steps (64 / LPR rows each).
template <int LPR, int NB, int RW>
struct PGroup {
  u32x4 q[RW][NB];
  uint16_t sc[RW][NB];
  int row[RW];
};

// Loads of one group, as buffer loads on the matrix: every load is issued unconditionally and rows
// past r1 get an offset beyond the buffer, which returns zero without touching memory. With no load
// under a branch (and none through a flat pointer, which would also count against the LDS wait
// counter) the compiler's wait counts stay exact: computing a group waits for that group's loads
// only, while the next group's are in flight.
constexpr int kNT = 2;            // cache policy: non-temporal (each weight is read once per step)

template <int LPR, int NB, int RW>
__device__ __forceinline__ void pload(int tid, const Mat w, int r0, int r1, int gi, PGroup<LPR, NB, RW>& g) {
  constexpr int RPW = kWave / LPR;
  const int lane = tid & 63, j = lane % LPR, rsub = lane / LPR;
  constexpr int nblk = LPR * NB;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc((void*)w.codes, 0, w.N * (nblk * 16), kRsrc3);
  const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc((void*)w.scales, 0, w.N * (nblk * 2), kRsrc3);
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int row = r0 + (gi * RW + r) * RPW + rsub;
    g.row[r] = row;
    const bool ok = row < r1;
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      g.q[r][c] = __builtin_amdgcn_raw_buffer_load_b128(rc, ok ? row * (nblk * 16) + (j + LPR * c) * 16 : kOOB, 0, kNT);
      g.sc[r][c] = __builtin_amdgcn_raw_buffer_load_b16(rsc, ok ? (row * nblk + j * NB + c) * 2 : kOOB, 0, 0);
    }
  }
}

template <int LPR, int NB, int RW>
__device__ __forceinline__ void pcompute(int tid, const PGroup<LPR, NB, RW>& g, int r0, int r1, const Lds& s) {
  const int lane = tid & 63, j = lane % LPR;
  float acc[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) acc[r] = 0.f;
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    __builtin_amdgcn_sched_barrier(0);
    // with many blocks per lane, the block index goes through an opaque move, so the chunk
    // addresses are formed per block instead of all NB x 8 of them being hoisted into registers
    int b = j + LPR * c;
    if constexpr (NB > 12) asm volatile("v_mov_b32 %0, %1" : "=v"(b) : "v"(j + LPR * c));
    float4 xb[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) xb[k] = *(const float4*)xs_chunk(s.xs, b, k);
    const float sb = s.bs[b];
#pragma unroll
    for (int r = 0; r < RW; ++r) acc[r] = fmaf(f16_to_f32(g.sc[r][c]), block_dot_hs(g.q[r][c], xb, sb), acc[r]);
  }
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    acc[r] = sum_lanes(acc[r], LPR);
    if (j == 0 && g.row[r] < r1) s.ydot[g.row[r] - r0] = acc[r];
  }
}

// first group of this wave (issued before the input is waited for)
template <int LPR, int NB, int RW>
__device__ __forceinline__ void gemv_first(int tid, const Mat w, int r0, int r1, PGroup<LPR, NB, RW>& g) {
  pload<LPR, NB, RW>(tid, w, r0, r1, wave_of(tid), g);
}

// The rest of the rows; ydot is complete after the caller's __syncthreads. DB: the A/B groups
// alternate so that the next group's loads are in flight while the current one is computed;
// otherwise one group is kept (for phases whose group covers a wave's whole share of the rows,
// so the loop runs once and no second register set is needed).
template <int LPR, int NB, int RW, bool DB>
__device__ __forceinline__ void gemv_rest(int tid, const Mat w, int r0, int r1, PGroup<LPR, NB, RW>& cur, const Lds& s) {
  constexpr int GROUP = (kWave / LPR) * RW;
  const int n_groups = (r1 - r0 + GROUP - 1) / GROUP;
  int gi = wave_of(tid);
  if (gi >= n_groups) return;
  if constexpr (DB) {
    PGroup<LPR, NB, RW> alt;
    while (true) {
      pload<LPR, NB, RW>(tid, w, r0, r1, gi + kPW, alt);
      pcompute<LPR, NB, RW>(tid, cur, r0, r1, s);
      gi += kPW;
      if (gi >= n_groups) break;
      pload<LPR, NB, RW>(tid, w, r0, r1, gi + kPW, cur);
      pcompute<LPR, NB, RW>(tid, alt, r0, r1, s);
      gi += kPW;
      if (gi >= n_groups) break;
    }
  } else {
    while (true) {
      pcompute<LPR, NB, RW>(tid, cur, r0, r1, s);
      gi += kPW;
      if (gi >= n_groups) break;
      pload<LPR, NB, RW>(tid, w, r0, r1, gi, cur);
    }
  }
}

// As gemv_rest, with each group's loads done by load(gi, group): the MoE phases pick the matrix
// of a row step or of a block column.
template <int LPR, int NB, int RW, bool DB, typename LoadF>
__device__ __forceinline__ void gemv_rest_f(int tid, int r0, int r1, PGroup<LPR, NB, RW>& cur, const Lds& s,
                                            LoadF&& load) {
  constexpr int GROUP = (kWave / LPR) * RW;
  const int n_groups = (r1 - r0 + GROUP - 1) / GROUP;
  int gi = wave_of(tid);
  if (gi >= n_groups) return;
  if constexpr (DB) {
    PGroup<LPR, NB, RW> alt;
    while (true) {
      load(gi + kPW, alt);
      pcompute<LPR, NB, RW>(tid, cur, r0, r1, s);
      gi += kPW;
      if (gi >= n_groups) break;
      load(gi + kPW, cur);
      pcompute<LPR, NB, RW>(tid, alt, r0, r1, s);
      gi += kPW;
      if (gi >= n_groups) break;
    }
  } else {
    while (true) {
      pcompute<LPR, NB, RW>(tid, cur, r0, r1, s);
      gi += kPW;
      if (gi >= n_groups) break;
      load(gi, cur);
    }
  }
}

// ---- dense FFN by columns ---------------------------------------------------------------------
// Workgroup w computes its gate/up rows (the SwiGLU outputs of ffn columns [C w, C w + C), C =
// F / 256), keeps those C values in LDS and multiplies them at once by the same C columns of
// W_down, for every one of the d rows. The d partial sums go to the owners of the rows, which add
// the 256 partials of each row to their residual rows. So the FFN streams its gate/up and down
// weights in one pass with no exchange between them; the F-long SwiGLU vector is never gathered.
// The slice's columns form units of U columns (16 when C is a multiple of 16, else 4); a unit
// lies inside one 32-column block and takes that block's scale.
//   9B  (d 4096, F 12288): C 48 = 3 units of 16, 8 rows per thread, 2 blocks per slice at most;
//   27B (d 5120, F 17408) would take C 68 = 17 units of 4, 10 rows per thread, 3 blocks per slice
//   at most (laid out and tested, not used: see with_colffn).
//
// W_down column-slice copy (written once at load from the device matrix): for slice w and thread
// t, CH chunks of 16 bytes at ((w CH + c) 512 + t) 16, so chunk c of all threads is contiguous.
// The thread's RT rows go in pairs (rows RT t + 2j, RT t + 2j + 1), PW words per pair, so a pair
// can be computed as soon as its words have arrived (loads complete in issue order):
//   code words: the pair's 2 C codes, flat code f = r C + c (row 2j + r, slice column c) in word
//               f / 8 of the pair; nibble n (bits 4n..4n+3) of a word holds flat code 8 (f / 8) + 2n
//               for n < 4 and 8 (f / 8) + 2 (n - 4) + 1 otherwise, so (word >> 4m) & 0x000F000F
//               is the fp16-subnormal pair of flat codes (2m, 2m + 1), which C even keeps in one row;
//   scale words: fp16 e = r S + b (row 2j + r, b-th block the slice touches, S blocks at most per
//               slice) in word 2 C / 8 + e / 2 of the pair, half e % 2 (zero past the slice's last block);
// and zero words up to the chunk boundary after the last pair.
constexpr int kCfWG = 256;  // workgroups of the layout (one slice each)

template <int KD_, int KF_>
struct CfGeo {
  static constexpr int COLS = KF_ / kCfWG;               // ffn columns per workgroup
  static constexpr int UW = COLS % 16 == 0 ? 16 : 4;     // columns per unit
  static constexpr int NU = COLS / UW;
  static constexpr int RT = KD_ / kPT;                   // W_down rows per thread
  static constexpr int OWN = KD_ / kCfWG;                // residual rows per owner (= 2 RT)
  static constexpr int RTP = (RT + 3) & ~3;              // words of half a partial record (16-byte aligned)
  static constexpr int span() {                          // blocks one slice touches, at most
    int m = 0;
    for (int w = 0; w < kCfWG; ++w) {
      const int b = ((w * COLS + COLS - 1) >> 5) - ((w * COLS) >> 5) + 1;
      m = b > m ? b : m;
    }
    return m;
  }
  static constexpr int NSB = span();
  static constexpr int PCW = 2 * COLS / 8;               // code words of a row pair
  static constexpr int PW = PCW + NSB;                   // words of a row pair (2 NSB scales)
  static constexpr int CH = (RT / 2 * PW + 3) / 4;       // 16-byte chunks per thread
  static constexpr int XS = 96;                          // LDS offset of the unit sums after the C values
  static_assert(KF_ % kCfWG == 0 && COLS % 4 == 0 && (2 * COLS) % 8 == 0 && OWN == 2 * RT && RT % 2 == 0 &&
                    COLS <= XS && XS + NU <= 128 && NSB <= 4,
                "FFN-by-columns geometry");
};

// this thread's chunks of slice w (every load unconditional, non-temporal)
template <class G>
__device__ __forceinline__ void cf_issue(int tid, const uint8_t* dnc, int w, u32x4 (&q)[G::CH]) {
  const __amdgpu_buffer_rsrc_t r = uniform_rsrc(dnc + (int64_t)w * G::CH * kPT * 16, G::CH * kPT * 16);
#pragma unroll
  for (int c = 0; c < G::CH; ++c) q[c] = __builtin_amdgcn_raw_buffer_load_b128(r, (c * kPT + tid) * 16, 0, kNT);
}

// the RT partial sums sum_u s_b(u) sum_{c in unit u} (q_c - 8) x_c of this thread's rows, units in
// order, row pairs in load order; xc: the slice's C SwiGLU values, then (at XS) the sums of its
// units (LDS); col0 = C w
template <class G>
__device__ __forceinline__ void cf_partials(const u32x4 (&q)[G::CH], const float* xc, int col0, float (&out)[G::RT]) {
  float xv[G::COLS], su[G::NU];
#pragma unroll
  for (int c = 0; c < G::COLS; c += 4) {
    const float4 v = *(const float4*)(xc + c);
    xv[c] = v.x;
    xv[c + 1] = v.y;
    xv[c + 2] = v.z;
    xv[c + 3] = v.w;
  }
#pragma unroll
  for (int u = 0; u < G::NU; ++u) su[u] = xc[G::XS + u];
#pragma unroll
  for (int i = 0; i < G::RT; ++i) {
    const int base = (i >> 1) * G::PW, r = i & 1;  // the row's pair and its place in the pair
    float o = 0.f;
#pragma unroll
    for (int u = 0; u < G::NU; ++u) {
      const int rb = ((col0 + G::UW * u) >> 5) - (col0 >> 5);  // the unit's block among the slice's (uniform)
      float acc = 0.f;
#pragma unroll
      for (int pr = 0; pr < G::UW / 2; ++pr) {
        const int f = r * G::COLS + G::UW * u + 2 * pr, k = base + (f >> 3), m = (f & 7) >> 1;
        acc = mix2((q[k >> 2][k & 3] >> (4 * m)) & 0x000F000Fu, xv[G::UW * u + 2 * pr], xv[G::UW * u + 2 * pr + 1], acc);
      }
      const float d = fmaf(16777216.0f, acc, -8.0f * su[u]);
      float sv = 0.f;
#pragma unroll
      for (int b = 0; b < G::NSB; ++b) {
        const int e = r * G::NSB + b, k = base + G::PCW + (e >> 1);
        const uint32_t sw = q[k >> 2][k & 3];
        const float sb = f16_to_f32((uint16_t)((e & 1) ? (sw >> 16) : (sw & 0xFFFFu)));
        sv = b == 0 ? sb : (rb == b ? sb : sv);
      }
      o = fmaf(sv, d, o);
    }
    out[i] = o;
  }
}

// ---- MoE expert matrices ----------------------------------------------------------------------
// mp: per slot (top_k routed experts in rank order, then the shared ones) the device pointers of
// its gate/up codes and scales and its down codes and scales, staged in LDS after the top-k.
__device__ __forceinline__ const void* lds_ptr(const uint64_t* mp, int i) {
  const uint64_t v = mp[i];
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}

// Rows [r0, r1) of the concatenated gate/up matrices (slot k holds rows [2 Fe k, 2 Fe (k + 1)), its
// expert's own rows 0 .. 2 Fe - 1, gate and up interleaved). One row per wave per row step
// (LPR = 64), so the matrix of each row step is uniform.
template <int LPR, int NB, int RW>
__device__ __forceinline__ void pload_moe_gu(int tid, const uint64_t* mp, int Fe, int r0, int r1, int gi,
                                             PGroup<LPR, NB, RW>& g) {
  static_assert(LPR == kWave, "one row per wave per row step");
  const int j = tid & 63;
  constexpr int nblk = LPR * NB;
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int row = r0 + gi * RW + r;
    g.row[r] = row;
    const bool ok = row < r1;
    const int slot = ok ? row / (2 * Fe) : 0, lr = row - slot * 2 * Fe;
    const __amdgpu_buffer_rsrc_t rc =
        __builtin_amdgcn_make_buffer_rsrc((void*)lds_ptr(mp, slot * 4 + 0), 0, 2 * Fe * (nblk * 16), kRsrc3);
    const __amdgpu_buffer_rsrc_t rsc =
        __builtin_amdgcn_make_buffer_rsrc((void*)lds_ptr(mp, slot * 4 + 1), 0, 2 * Fe * (nblk * 2), kRsrc3);
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      g.q[r][c] = __builtin_amdgcn_raw_buffer_load_b128(rc, ok ? lr * (nblk * 16) + (j + LPR * c) * 16 : kOOB, 0, kNT);
      g.sc[r][c] = __builtin_amdgcn_raw_buffer_load_b16(rsc, ok ? (lr * nblk + j * NB + c) * 2 : kOOB, 0, 0);
    }
  }
}

// Rows [r0, r1) of the down projection over the concatenated expert outputs: a lane's block
// column c is block j of slot c's matrix [d][Fe] (Fe = 32 LPR), so every load of column c reads
// slot c's matrix.
template <int LPR, int NB, int RW>
__device__ __forceinline__ void pload_moe_dn(int tid, const uint64_t* mp, int d, int r0, int r1, int gi,
                                             PGroup<LPR, NB, RW>& g) {
  constexpr int RPW = kWave / LPR;
  const int lane = tid & 63, j = lane % LPR, rsub = lane / LPR;
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int row = r0 + (gi * RW + r) * RPW + rsub;
    g.row[r] = row;
    const bool ok = row < r1;
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      const __amdgpu_buffer_rsrc_t rc =
          __builtin_amdgcn_make_buffer_rsrc((void*)lds_ptr(mp, c * 4 + 2), 0, d * (LPR * 16), kRsrc3);
      const __amdgpu_buffer_rsrc_t rsc =
          __builtin_amdgcn_make_buffer_rsrc((void*)lds_ptr(mp, c * 4 + 3), 0, d * (LPR * 2), kRsrc3);
      g.q[r][c] = __builtin_amdgcn_raw_buffer_load_b128(rc, ok ? row * (LPR * 16) + j * 16 : kOOB, 0, kNT);
      g.sc[r][c] = __builtin_amdgcn_raw_buffer_load_b16(rsc, ok ? (row * LPR + j) * 2 : kOOB, 0, 0);
    }
  }
}

// ---- attention over the paged cache -----------------------------------------------------------

// K and V of one page for KV head g, as buffer loads on the layer's pool slice (an invalid page id
// reads zeros without touching memory). K is loaded as the A operand of the score products: lane
// l holds token l % 16 and, per 32-dim chunk c, the 8 dims kdim(c, l / 16) ..+7 (16-bit caches:
// one 16-byte load per chunk; FP8: one 16-byte load per two chunks, dims 64 u + 16 (l / 16) ..+15).
// V is loaded as 16-byte pieces for staging in LDS: piece k = l + 64 u holds token k / (D / 8),
// dims 8 (k % (D / 8)) ..+7 (FP8: token k / (D / 16), dims 16 (k % (D / 16)) ..+15).
template <int D, int KVDT>
struct PageRegs {
  static constexpr int NC = D / 32;                          // 32-dim chunks of the scores
  static constexpr int NK = KVDT == 3 ? NC / 2 : NC;         // K loads per lane
  static constexpr int NVL = KVDT == 3 ? D / 64 : D / 32;    // V loads per lane
  u32x4 k[NK];
  u32x4 v[NVL];
};

// head dims of the 8 K elements a lane holds in chunk c (lane group grp = lane / 16); a score sums
// over all dims, so any order that K and the query parts share gives the same sum
template <int KVDT>
__device__ __forceinline__ int kdim(int c, int grp) {
  return KVDT == 3 ? 64 * (c >> 1) + 16 * grp + 8 * (c & 1) : 32 * c + 8 * grp;
}

template <int D, int KVDT>
__device__ __forceinline__ void load_page(int lane, const typename KvT<KVDT>::E* pool, int64_t page_elems,
                                          int n_pages, int page, int g, PageRegs<D, KVDT>& pr) {
  using PR = PageRegs<D, KVDT>;
  constexpr int ES = KvT<KVDT>::ES;
  const int c16 = lane & 15, grp = lane >> 4;
  // the descriptor covers this KV head's K and V of the page, or no bytes for an invalid page id
  // (every load then reads zeros): the offsets need no selection, which the compiler would turn
  // into a branch around each load and a wait for every load in flight at the join
  const bool ok = page >= 0 && page < n_pages;
  const __amdgpu_buffer_rsrc_t r =
      uniform_rsrc(pool + (ok ? (int64_t)page * page_elems + (int64_t)(g * 2) * kPageTokens * D : 0),
                   ok ? 2 * kPageTokens * D * ES : 0);
  if constexpr (KVDT == 3) {
#pragma unroll
    for (int u = 0; u < PR::NK; ++u) pr.k[u] = __builtin_amdgcn_raw_buffer_load_b128(r, c16 * D + 64 * u + 16 * grp, 0, 0);
#pragma unroll
    for (int u = 0; u < PR::NVL; ++u) {
      const int k = lane + 64 * u;
      pr.v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, kPageTokens * D + (k / (D / 16)) * D + 16 * (k % (D / 16)), 0, 0);
    }
  } else {
#pragma unroll
    for (int c = 0; c < PR::NK; ++c)
      pr.k[c] = __builtin_amdgcn_raw_buffer_load_b128(r, (c16 * D + 32 * c + 8 * grp) * 2, 0, 0);
#pragma unroll
    for (int u = 0; u < PR::NVL; ++u) {
      const int k = lane + 64 * u;
      pr.v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, (kPageTokens * D + (k / (D / 8)) * D + 8 * (k % (D / 8))) * 2, 0, 0);
    }
  }
}

// 8 elements of the new token's key or value (cache dtype bits staged in LDS)
template <int KVDT>
__device__ __forceinline__ typename KvT<KVDT>::C8 lds_chunk8(const uint16_t* bits, int d0) {
  return *(const typename KvT<KVDT>::C8*)((const typename KvT<KVDT>::E*)bits + d0);
}

// ---- parameters -------------------------------------------------------------------------------

constexpr int kVPitch = 8;  // LDS row of a staged V page: D + 8 16-bit elements (conflict-free transpose reads)

template <int D, int QR>
struct alignas(16) AttnLds {
  alignas(16) uint16_t qpart[2][QR * D];  // the scaled query rows as hi and lo parts (16-bit operand type)
  float m[kPW][QR], l[kPW][QR];
  float acc[kPW][QR * D];
  alignas(16) uint16_t knew[D];  // cache dtype bits (the first D bytes for FP8)
  alignas(16) uint16_t vnew[D];
  alignas(16) uint16_t vst[kPW][kPageTokens * (D + kVPitch)];  // each wave's staged V page (16-bit)
};

// The next layer's table entry, issued by the first kLW threads ahead of the last phase's input
// polls (the polls' first check waits for it anyway) and stored to its LDS slot after them.
__device__ __forceinline__ uint32_t ltab_issue(const PersistParams& p, int l1, int tid) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)p.layers, 0, p.L * kLW * 4, kRsrc3);
  return __builtin_amdgcn_raw_buffer_load_b32(r, tid < kLW && l1 < p.L ? (l1 * kLW + tid) * 4 : kOOB, 0, 0);
}

// ---- the kernel -------------------------------------------------------------------------------

// RWQ, RWO, RWG, RWF: row steps per register group of the QKV, O, gate/up and down passes; a
// group that covers a wave's whole share of a phase is loaded in full before the phase's wait.
// COLF: the dense FFN by columns (see cf_issue), for the shape and grid it is laid out for.
template <int LPR_D, int NB_D, int LPR_F, int NB_F, int KVDT, int D, int QR, int RWQ, int RWO, int RWG, int RWF,
          bool MOE, bool COLF>
__global__ __launch_bounds__(kPT) void k_persist(PersistParams p) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  constexpr int KD = LPR_D * NB_D * 32;  // d_model (= Hq * D)
  constexpr int KF = LPR_F * NB_F * 32;  // ffn dim
  constexpr int KMAX = KD > KF ? KD : KF;
  // A phase alternates two register groups (the next one's loads in flight while one is computed)
  // only where a group is small: at most 12 blocks per lane (60 registers of codes and scales).
  constexpr bool DBQ = RWQ < 3 && RWQ * NB_D <= 12, DBO = RWO < 2 && RWO * NB_D <= 12;
  constexpr bool DBG = RWG < 6 && RWG * NB_D <= 12, DBF = RWF < 2 && RWF * NB_F <= 12;
  // lm_head row steps per group: about eight blocks per lane
  constexpr int LMRW = NB_D <= 2 ? kLmRW : (kLmRW * 2 >= NB_D ? kLmRW * 2 / NB_D : 1);
  __shared__ int bail;
  Lds s;
  s.xs = lds;
  s.bs = s.xs + KMAX;
  s.ydot = s.bs + KMAX / 32;
  s.resid = s.ydot + kMaxRows;
  s.red = s.resid + kMaxOwn;
  s.mrg = s.red + 32;
  s.pgid = reinterpret_cast<int*>(s.mrg + kMrg);
  s.att = s.mrg + kMrg + kMaxSplitPages;
  s.ltab = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(s.att) + sizeof(AttnLds<D, QR>));
  AttnLds<D, QR>& al = *reinterpret_cast<AttnLds<D, QR>*>(s.att);

  const int nwg = gridDim.x, w = blockIdx.x;
  if (threadIdx.x == 0) bail = 0;
  Ctl ctl{p.abort_flag, p.err, &bail, 0, p.deadline_ticks};
  __syncthreads();
  // a previous step that aborted leaves the flag raised: nothing runs until the host clears it
  if (__hip_atomic_load(p.abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
    if (threadIdx.x == 0 && w == 0) atomicOr(p.err, BW_DERR_PERSIST_BIT);
    return;
  }

  const int L = p.L, H = p.H, G = p.G;
  stamp(p, L * 16 + 4);
  // layer 0's table entry into slot 0; later entries are loaded one layer ahead (ltab_issue)
  if (threadIdx.x < kLW) s.ltab[threadIdx.x] = reinterpret_cast<const uint32_t*>(p.layers)[threadIdx.x];
  const uint32_t epoch = p.epoch[0];
  const uint32_t base_tag = epoch * (uint32_t)(L + 2);
  const int pos = p.seq_lens[0];
  const int kv_len = pos + 1;
  const bool pos_ok = pos >= 0 && pos < p.max_pos && pos / kPageTokens < p.max_pages;
  const int HD = H * D, GD = G * D;
  const int Nq = HD + 2 * GD;

  // row ownership: residual rows [w*Rd, ...), QKV / GU rows in even-aligned ranges
  const int Rd = (KD + nwg - 1) / nwg;
  const int d0 = min(w * Rd, KD), d1 = min(d0 + Rd, KD);
  const int Rq = (((Nq + nwg - 1) / nwg) + 1) & ~1;
  const int q0 = min(w * Rq, Nq), q1 = min(q0 + Rq, Nq);
  const int Rg = (((2 * KF + nwg - 1) / nwg) + 1) & ~1;
  const int g0 = min(w * Rg, 2 * KF), g1 = min(g0 + Rg, 2 * KF);
  const int Rv = (p.V + nwg - 1) / nwg;
  const int v0 = min(w * Rv, p.V), v1 = min(v0 + Rv, p.V);
  // attention splits per KV head: all workgroups, but no more than one merge round of the
  // mergers covers (kPT / D split groups x 8 words per thread), so that a merger polls once;
  // workgroups past S G take no split
  const int S = min(nwg / G, (kPT / D) * kMergeNA);
  const int ag = w / S, as = w - ag * S;  // this workgroup's (KV head, split); ag >= G: idle

  // ---- embedding: owned residual rows
  {
    const int tid = phase_tid();
    const int lane = tid & 63, wave = wave_of(tid);
    (void)lane;
    (void)wave;
    int tok = p.tokens[0];
    if (tok < 0 || tok >= p.V) {
      if (tid == 0 && w == 0) atomicOr(p.err, 2);
      tok = 0;
    }
    const uint32_t tag = base_tag;  // T(-1)
    for (int r = d0 + tid; r < d1; r += kPT) {
      const float v = f16_to_f32(p.embed[(int64_t)tok * KD + r]);
      s.resid[r - d0] = v;
      xstore(p.xx, r, v, tag);
    }
  }
  if (!pos_ok && threadIdx.x == 0 && w == 0) atomicOr(p.err, 4);

  // This workgroup's attention split: pages [apg0, apg1) of KV head ag (the same for every layer).
  // Each wave's first page id is read once per step; its K/V are loaded during each layer's QKV pass.
  int apg0, apg1, first_page;
  {
    int n_pg = (kv_len + kPageTokens - 1) / kPageTokens;
    n_pg = max(0, min(n_pg, p.max_pages));
    const int pps = (n_pg + S - 1) / S;
    apg0 = ag < G ? as * pps : 0;
    apg1 = ag < G ? min(n_pg, apg0 + pps) : 0;
    const int tid = phase_tid();
    for (int i = tid; i < apg1 - apg0 && i < kMaxSplitPages; i += kPT) s.pgid[i] = p.page_table[apg0 + i];
    __syncthreads();
    const int pg = apg0 + wave_of(tid);
    first_page = pg < apg1 ? s.pgid[pg - apg0] : -1;
  }

  // Per-step constants of the QKV epilogue, read before any weight is in flight: the new token's
  // page and the RoPE factors of this thread's row pair (at most one pair per thread).
  const int page_new = pos_ok ? __builtin_amdgcn_readfirstlane(p.page_table[pos / kPageTokens]) : -1;
  float2 rope_cs = make_float2(1.f, 0.f);
  {
    const int tid = phase_tid();
    const int dr = q0 + 2 * tid;
    if (pos_ok && dr < q1 && dr < HD + GD) {
      const int local = dr < HD ? dr : dr - HD;
      const int i = (local % D) >> 1;
      rope_cs = p.rope[(int64_t)pos * (D >> 1) + i];
    }
  }

  // Each phase issues its input loads first, then its first weight group, then waits for the
  // input (O's weights go out during the merge, whose input loads precede them the same way).

  for (int l = 0; l < L; ++l) {
    // this layer's descriptors, read once with scalar loads (the table is constant for the step),
    // so the matrix pointers are uniform registers and the loops below never re-read them
    const PLayer Ly = load_uniform(reinterpret_cast<const PLayer*>(s.ltab + (l & 1) * kLW));
    const uint32_t tin = base_tag + (uint32_t)l;       // T(l - 1)
    const uint32_t tout = base_tag + (uint32_t)l + 1;  // T(l)
    typedef typename KvT<KVDT>::E KE;
    KE* pool = (KE*)p.pool + (int64_t)l * p.layer_elems;
    PageRegs<D, KVDT> kv_first;

    // ================= QKV =================
    stamp(p, l * 16 + 0);
    {
      const int tid = phase_tid();
      const int lane = tid & 63, wave = wave_of(tid);
      (void)lane;
      (void)wave;
      XStage<KD> xin;
      stage_issue<KD, true>(tid, p.xx, Ly.attn_norm, xin);
      PGroup<LPR_D, NB_D, RWQ> cur;
      gemv_first<LPR_D, NB_D, RWQ>(tid, Ly.qkv, q0, q1, cur);
      __syncthreads();
      stage_finish<KD, true>(tid, p.xx, tin, p.eps, xin, s, ctl);
      if (bail) return;
      stamp(p, l * 16 + 1);
      // this layer's first attention page, after the input wait (waits count loads in issue
      // order): its id is known, only the new token's slot changes in this step, and that slot
      // is taken from the exchange
      load_page<D, KVDT>(lane, pool, p.page_elems, p.n_pages, first_page, ag, kv_first);
      gemv_rest<LPR_D, NB_D, RWQ, DBQ>(tid, Ly.qkv, q0, q1, cur, s);
      __syncthreads();
      if (2 * tid < q1 - q0) {
        // one RoPE pair (q, k) or two adjacent value dims per thread; k and v are rounded to the
        // cache dtype, stored in the pool and exchanged as the rounded values
        const int pi = tid, dr = q0 + 2 * pi;
        const float a = s.ydot[2 * pi], b = s.ydot[2 * pi + 1];
        const bool is_v = dr >= HD + GD;
        const int local = dr < HD ? dr : (is_v ? dr - HD - GD : dr - HD);
        const int head = local / D;
        int dd0, dd1;
        float o0 = a, o1 = b;
        if (!is_v) {
          const int i = (local - head * D) >> 1;
          o0 = a * rope_cs.x - b * rope_cs.y;
          o1 = a * rope_cs.y + b * rope_cs.x;
          dd0 = i;
          dd1 = i + (D >> 1);
        } else {
          dd0 = local - head * D;
          dd1 = dd0 + 1;
        }
        if (dr < HD) {
          xstore(p.xq, head * D + dd0, o0, tout);
          xstore(p.xq, head * D + dd1, o1, tout);
        } else {
          const int which = is_v ? 1 : 0;
          const uint16_t k0 = f32_to_kv<KVDT>(o0), k1 = f32_to_kv<KVDT>(o1);
          const int xb = HD + which * GD + head * D;
          xstore(p.xq, xb + dd0, kv_to_f32<KVDT>(k0), tout);
          xstore(p.xq, xb + dd1, kv_to_f32<KVDT>(k1), tout);
          if (page_new >= 0 && page_new < p.n_pages) {
            KE* dst = pool + (int64_t)page_new * p.page_elems +
                      ((int64_t)(head * 2 + which) * kPageTokens + (pos % kPageTokens)) * D;
            dst[dd0] = (KE)k0;
            dst[dd1] = (KE)k1;
          } else if (pos_ok) {
            atomicOr(p.err, 1);
          }
        }
      }
    }

    // ================= ATTENTION (KV head ag, split as) =================
    // Both products of a page on the matrix cores (16 x 16 tiles):
    // - scores^T = K Q^T: K (16 tokens x 32 dims per product) as the A operand; the B operand's
    //   columns 2h and 2h + 1 hold the hi and lo parts of query head h (16 significant bits), so
    //   head h's scores are the sum of result columns 2h and 2h + 1 (adjacent lanes);
    // - O += P V: P (rows 2h and 2h + 1: the hi and lo parts of head h's probabilities) as the A
    //   operand, V (16 tokens x 16 dims) as the B operand, read from the wave's staged page with
    //   transposing LDS reads; rows 2h and 2h + 1 of the result sit in one lane and add up there.
    // Lane l of a 16 x 16 result holds column l % 16, rows 4 (l / 16) ..+3.
    stamp(p, l * 16 + 2);
    {
      const int tid = phase_tid();
      const int lane = tid & 63, wave = wave_of(tid);
      constexpr int MT = KVDT == 3 ? 2 : KVDT;  // an FP8 cache is widened to bf16 (exact)
      using MM = MfmaT<MT>;
      typedef typename MM::e8 e8;
      typedef typename MM::e4 e4;
      typedef typename std::remove_reference<decltype(e8{}[0])>::type el8;
      typedef typename std::remove_reference<decltype(e4{}[0])>::type el4;
      using PR = PageRegs<D, KVDT>;
      constexpr int NC = D / 32, NV16 = D / 16, VP = D + kVPitch;
      static_assert(2 * QR <= 16, "two parts per query head fit one 16-wide tile");
      const int c16 = lane & 15, grp = lane >> 4;
      const bool active = ag < G;
      const int pg0 = apg0, pg1 = apg1;
      const int pg_new = pos / kPageTokens, slot_new = pos % kPageTokens;
      int pg = pg0 + wave;
      int page = first_page;
      // q rows of this KV head and the new key / value
      if (active) {
        const __amdgpu_buffer_rsrc_t r = xrsrc(p.xq, (int64_t)Nq * 4);
        constexpr int NQW = (QR * D + 2 * D + kPT - 1) / kPT;
        int idx[NQW];
        uint32_t word[NQW];
#pragma unroll
        for (int i = 0; i < NQW; ++i) {
          const int e = tid + i * kPT;
          if (e < QR * D) {
            const int qr = e / D, dd = e - qr * D;
            idx[i] = (ag * QR + qr) * D + dd;
          } else if (e < QR * D + 2 * D) {
            const int e2 = e - QR * D, which = e2 / D, dd = e2 - which * D;
            idx[i] = HD + which * GD + ag * D + dd;
          } else {
            idx[i] = -1;
          }
        }
        poll_words_issue<NQW>(r, idx, word);
        poll_words_wait<NQW>(r, idx, tout, word, ctl);
#pragma unroll
        for (int i = 0; i < NQW; ++i) {
          const int e = tid + i * kPT;
          if (e < QR * D) {
            const float x = xdec(word[i]) * p.attn_scale;
            const uint16_t hb = part_bits<MT>(x);
            al.qpart[0][e] = hb;
            al.qpart[1][e] = part_bits<MT>(x - kv_to_f32<MT>(hb));
          } else if (e < QR * D + 2 * D) {
            const int e2 = e - QR * D, which = e2 / D, dd = e2 - which * D;
            const uint16_t bits = f32_to_kv<KVDT>(xdec(word[i]));
            if (which == 0) ((KE*)al.knew)[dd] = (KE)bits;
            else ((KE*)al.vnew)[dd] = (KE)bits;
          }
        }
      }
      __syncthreads();
      stamp(p, l * 16 + 3);
      if (bail) return;
      // the query parts as the B operand: column c16 = 2h + part, dims kdim(c, grp) ..+7
      e8 qp[NC];
      {
        const int qh = c16 >> 1;
        const bool qcol = qh < QR;
        const uint16_t* qs = al.qpart[c16 & 1] + (qcol ? qh : 0) * D;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const u32x4 v = *(const u32x4*)(qs + kdim<KVDT>(c, grp));
          qp[c] = __builtin_bit_cast(e8, qcol ? v : u32x4{0u, 0u, 0u, 0u});
        }
      }
      float mrun = -INFINITY, lrun = 0.f;  // of head c16 / 2 (even lanes with c16 < 2 QR)
      bool first = true;                   // no page computed yet: the accumulators are zero
      f32x4 o[NV16];
#pragma unroll
      for (int c = 0; c < NV16; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
      uint16_t* vl = al.vst[wave];
      const uint16_t* vrow = vl + (4 * grp + (c16 >> 2)) * VP + 4 * (c16 & 3);
      // the rows of the probability operand: row c16 = part c16 & 1 of head c16 / 2; zero beyond 2 QR
      const int prow_part = c16 < 2 * QR ? (c16 & 1) : 2;
      for (; active && pg < pg1; pg += kPW) {
        const bool valid = page >= 0 && page < p.n_pages;
        if (!valid && lane == 0) atomicOr(p.err, 1);
        const int pgn = pg + kPW;
        const int page_n = pgn < pg1 ? s.pgid[pgn - pg0] : -1;
        if (pg == pg_new) {  // the new token's slot comes from the exchange
          if (c16 == slot_new) {
#pragma unroll
            for (int u = 0; u < PR::NK; ++u)
              kv_first.k[u] = *(const u32x4*)((const KE*)al.knew + (KVDT == 3 ? 64 * u + 16 * grp : 32 * u + 8 * grp));
          }
#pragma unroll
          for (int u = 0; u < PR::NVL; ++u) {
            const int k = lane + 64 * u;
            const int tk = KVDT == 3 ? k / (D / 16) : k / (D / 8);
            const int d0 = KVDT == 3 ? 16 * (k % (D / 16)) : 8 * (k % (D / 8));
            if (tk == slot_new) kv_first.v[u] = *(const u32x4*)((const KE*)al.vnew + d0);
          }
        }
        if (valid) {
          // stage V (this wave's buffer; a wave's LDS operations run in order); slots past the
          // sequence end are zeros, so stale contents never meet a zero probability
          const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int u = 0; u < PR::NVL; ++u) {
            const int k = lane + 64 * u;
            if constexpr (KVDT == 3) {
              const int tk = k / (D / 16);
              const bool live = pg * kPageTokens + tk < kv_len;
              uint16_t* dst = vl + tk * VP + 16 * (k % (D / 16));
              *(u32x4*)dst = live ? fp8x8_to_bf16x8(u32x2{kv_first.v[u][0], kv_first.v[u][1]}) : z;
              *(u32x4*)(dst + 8) = live ? fp8x8_to_bf16x8(u32x2{kv_first.v[u][2], kv_first.v[u][3]}) : z;
            } else {
              const int tk = k / (D / 8);
              *(u32x4*)(vl + tk * VP + 8 * (k % (D / 8))) = pg * kPageTokens + tk < kv_len ? kv_first.v[u] : z;
            }
          }
          // scores^T
          f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            u32x4 kr;
            if constexpr (KVDT == 3)
              kr = fp8x8_to_bf16x8((c & 1) ? u32x2{kv_first.k[c >> 1][2], kv_first.k[c >> 1][3]}
                                           : u32x2{kv_first.k[c >> 1][0], kv_first.k[c >> 1][1]});
            else
              kr = kv_first.k[c];
            sc = MM::mm32(__builtin_bit_cast(e8, kr), qp[c], sc);
          }
          // even lane c16 = 2h: head h's scores are its column plus the next lane's
          float sv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float t = sc[i] + row_from<1>(sc[i]);
            const int j = pg * kPageTokens + 4 * grp + i;
            sv[i] = j < kv_len ? t : -INFINITY;
          }
          float pm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
          pm = max_xor32(max_xor16(pm));
          const float mnew = fmaxf(mrun, pm);
          float pv[4], psum = 0.f, alpha = 1.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pv[i] = mnew == -INFINITY ? 0.f : __expf(sv[i] - mnew);
            psum += pv[i];
          }
          if (mnew != -INFINITY) alpha = __expf(mrun - mnew);
          psum = sum_xor32(sum_xor16(psum));
          lrun = lrun * alpha + psum;
          mrun = mnew;
          // the probability operand: odd lane 2h + 1 takes head h's values from lane 2h
          e4 pa;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float ph = pv[i], pl = row_to<1>(pv[i]);  // pl: the even neighbour's value
            const float x = prow_part == 0 ? ph : pl;
            const uint16_t hb = part_bits<MT>(x);
            const uint16_t lb = part_bits<MT>(x - kv_to_f32<MT>(hb));
            pa[i] = __builtin_bit_cast(el4, prow_part == 0 ? hb : (prow_part == 1 ? lb : (uint16_t)0));
          }
          // rescale the accumulators when a running max moved (never on the first page, whose
          // accumulators are zero): rows 2h and 2h + 1 take head h's factor from lane 2h
          if (!first && __ballot(c16 < 2 * QR && alpha != 1.f) != 0) {
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
              const float a = __shfl(alpha, (lane & ~15) | (4 * grp + i));
#pragma unroll
              for (int c = 0; c < NV16; ++c) {
                o[c][i] *= a;
                o[c][i + 1] *= a;
              }
            }
          }
          first = false;
          typedef short s4 __attribute__((ext_vector_type(4)));
#pragma unroll
          for (int c = 0; c < NV16; ++c) {
            const s4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(vrow + 16 * c));
            o[c] = MM::mm16(pa, __builtin_bit_cast(e4, t), o[c]);
          }
        }
        page = page_n;
        load_page<D, KVDT>(lane, pool, p.page_elems, p.n_pages, pgn < pg1 ? page : -1, ag, kv_first);
      }
      if constexpr (!MOE) stamp(p, l * 16 + 12);  // MoE: the down phase's slot
      // rows 2h (hi) and 2h + 1 (lo) of head h add up in the lane; then the waves merge in LDS
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const int h = 2 * grp + (i >> 1);
        if (h < QR) {
#pragma unroll
          for (int c = 0; c < NV16; ++c) al.acc[wave][h * D + 16 * c + c16] = o[c][i] + o[c][i + 1];
        }
      }
      if (grp == 0 && c16 < 2 * QR && (c16 & 1) == 0) {
        al.m[wave][c16 >> 1] = mrun;
        al.l[wave][c16 >> 1] = lrun;
      }
      __syncthreads();
      if constexpr (!MOE) stamp(p, l * 16 + 13);
      if (active) {
        for (int e = tid; e < QR * D; e += kPT) {
          const int qr = e / D, dd = e - qr * D;
          float M = -INFINITY;
#pragma unroll
          for (int v = 0; v < kPW; ++v) M = fmaxf(M, al.m[v][qr]);
          float a = 0.f, lsum = 0.f;
          if (M != -INFINITY) {
#pragma unroll
            for (int v = 0; v < kPW; ++v) {
              const float f = __expf(al.m[v][qr] - M);
              a = fmaf(al.acc[v][e], f, a);
              lsum = fmaf(al.l[v][qr], f, lsum);
            }
          }
          const int h = ag * QR + qr;
          uint32_t* dst = p.xp + ((int64_t)h * S + as) * (D + 2);
          xstore(dst, dd, a, tout);
          if (dd == 0) {
            xstore(dst, D, M == -INFINITY ? kNoScore : M, tout);
            xstore(dst, D + 1, lsum, tout);
          }
        }
      }
    }

    // ================= MERGE (one workgroup per query head) =================
    // Split q < QR of KV head g combines the S split partials of query head g * QR + q and stores
    // that head's D outputs; every other workgroup goes on to the O phase at once (its O weights
    // go out here), so the attention output takes one exchange from the splits to the mergers
    // (S producers each) and one all-gather into O.
    stamp(p, l * 16 + 4);
    PGroup<LPR_D, NB_D, RWO> o_pre;
    {
      const int tid = phase_tid();
      const int lane = tid & 63, wave = wave_of(tid);
      (void)lane;
      (void)wave;
      if (ag < G && as < QR) {
        const int h = ag * QR + as;
        const __amdgpu_buffer_rsrc_t r = xrsrc(p.xp, (int64_t)H * S * (D + 2) * 4);
        constexpr int SG = kPT / D;  // split groups: thread t takes output t % D of splits t / D + SG i
        constexpr int NA = kMergeNA;  // partial words per thread per round
        static_assert(kPT % D == 0 && 3 * kMaxSplit + kPT + 1 <= kMrg, "merge scratch");
        const int dd = tid % D, sg = tid / D;
        float* ml = s.mrg;                  // [S][2]: running max, denominator
        float* fm = s.mrg + 2 * kMaxSplit;  // [S]: exp(m - M)
        float* part = fm + kMaxSplit;       // [SG][D]
        float* den = part + kPT;            // [1]
        int idx[1 + NA];
        uint32_t word[1 + NA];
        idx[0] = tid < 2 * S ? (h * S + (tid >> 1)) * (D + 2) + D + (tid & 1) : -1;
#pragma unroll
        for (int i = 0; i < NA; ++i) {
          const int sp = sg + SG * i;
          idx[1 + i] = sp < S ? (h * S + sp) * (D + 2) + dd : -1;
        }
        poll_words_issue<1 + NA>(r, idx, word);
        gemv_first<LPR_D, NB_D, RWO>(tid, Ly.o, d0, d1, o_pre);
        poll_words_wait<1 + NA>(r, idx, tout, word, ctl);
        if (idx[0] >= 0) ml[tid] = xdec(word[0]);
        __syncthreads();
        stamp(p, l * 16 + 5);
        if (bail) return;
        // max over the splits, factors, denominator (fixed-order reductions: deterministic)
        if (wave == 0) {
          float M = kNoScore;
          for (int sp = lane; sp < S; sp += kWave) M = fmaxf(M, ml[2 * sp]);
          M = wmax(M);
          float dpart = 0.f;
          for (int sp = lane; sp < S; sp += kWave) {
            const float f = __expf(ml[2 * sp] - M);
            fm[sp] = f;
            dpart = fmaf(ml[2 * sp + 1], f, dpart);
          }
          dpart = wsum(dpart);
          if (lane == 0) den[0] = dpart;
        }
        __syncthreads();
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < NA; ++i)
          if (idx[1 + i] >= 0) a = fmaf(xdec(word[1 + i]), fm[sg + SG * i], a);
        // more splits than SG * NA (small models with many splits per KV head)
        for (int base = SG * NA; base < S; base += SG * NA) {
          int idx2[NA];
          uint32_t w2[NA];
#pragma unroll
          for (int i = 0; i < NA; ++i) {
            const int sp = base + sg + SG * i;
            idx2[i] = sp < S ? (h * S + sp) * (D + 2) + dd : -1;
          }
          poll_words_issue<NA>(r, idx2, w2);
          poll_words_wait<NA>(r, idx2, tout, w2, ctl);
#pragma unroll
          for (int i = 0; i < NA; ++i)
            if (idx2[i] >= 0) a = fmaf(xdec(w2[i]), fm[base + sg + SG * i], a);
        }
        part[sg * D + dd] = a;
        __syncthreads();
        if (bail) return;
        if (tid < D) {
          float o = 0.f;
#pragma unroll
          for (int g2 = 0; g2 < SG; ++g2) o += part[g2 * D + tid];
          const float dn = den[0];
          xstore(p.xa, h * D + tid, dn > 0.f ? o / dn : 0.f, tout);
        }
      } else {
        gemv_first<LPR_D, NB_D, RWO>(tid, Ly.o, d0, d1, o_pre);
        stamp(p, l * 16 + 5);
      }
    }

    // ================= O + residual =================
    stamp(p, l * 16 + 6);
    {
      const int tid = phase_tid();
      const int lane = tid & 63, wave = wave_of(tid);
      (void)lane;
      (void)wave;
      PGroup<LPR_D, NB_D, RWO>& cur = o_pre;
      XStage<KD> xin;
      stage_issue<KD, false>(tid, p.xa, nullptr, xin);
      stage_finish<KD, false>(tid, p.xa, tout, 0.f, xin, s, ctl);
      if (bail) return;
      stamp(p, l * 16 + 7);
      gemv_rest<LPR_D, NB_D, RWO, DBO>(tid, Ly.o, d0, d1, cur, s);
      __syncthreads();
      for (int r = d0 + tid; r < d1; r += kPT) {
        const float v = s.resid[r - d0] + s.ydot[r - d0];
        s.resid[r - d0] = v;
        xstore(p.xm, r, v, tout);
      }
    }

    if constexpr (COLF) {
    using CG = CfGeo<KD, KF>;
    static_assert(!MOE, "FFN by columns: dense models");
    // ================= gate/up + SwiGLU + down by columns =================
    // The W_down slice goes out in place of the gate/up pass's last next-group load, so the two
    // matrices stream back to back; the SwiGLU values stay in LDS.
    stamp(p, l * 16 + 8);
    {
      const int tid = phase_tid();
      constexpr int GROUP = (kWave / LPR_D) * RWG;
      constexpr int NG = (2 * CG::COLS + GROUP * kPW - 1) / (GROUP * kPW);  // groups per wave (the last may be empty)
      const int wave = wave_of(tid);
      XStage<KD> xin;
      stage_issue<KD, true>(tid, p.xm, Ly.ffn_norm, xin);
      PGroup<LPR_D, NB_D, RWG> ga[2];
      pload<LPR_D, NB_D, RWG>(tid, Ly.gu, g0, g1, wave, ga[0]);
      __syncthreads();
      stage_finish<KD, true>(tid, p.xm, tout, p.eps, xin, s, ctl);
      if (bail) return;
      stamp(p, l * 16 + 9);
      u32x4 dq[CG::CH];
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        if (i + 1 < NG) pload<LPR_D, NB_D, RWG>(tid, Ly.gu, g0, g1, wave + (i + 1) * kPW, ga[(i + 1) & 1]);
        else cf_issue<CG>(tid, Ly.dnc, w, dq);
        pcompute<LPR_D, NB_D, RWG>(tid, ga[i & 1], g0, g1, s);
      }
      __syncthreads();
      // the slice's SwiGLU values and the sums of its units (waves 0 and 1)
      if (tid < 2 * kWave) {
        float v = 0.f;
        if (tid < CG::COLS) {
          v = silu(s.ydot[2 * tid]) * s.ydot[2 * tid + 1];
          s.xs[tid] = v;
        }
        v = sum_lanes(v, CG::UW);
        if (tid < CG::COLS && tid % CG::UW == 0) s.xs[CG::XS + tid / CG::UW] = v;
      }
      __syncthreads();
      float part[CG::RT];
      cf_partials<CG>(dq, s.xs, w * CG::COLS, part);
      // rows RT t .. RT t + RT - 1 belong to owner t / 2, at RTP (t % 2) of this producer's record
      const __amdgpu_buffer_rsrc_t rp = xrsrc(p.xdp, (int64_t)p.n_xdp * 4);
      const int off = (((tid >> 1) * kCfWG + w) * (2 * CG::RTP) + (tid & 1) * CG::RTP) * 4;
#pragma unroll
      for (int c = 0; c < CG::RT / 4; ++c) {
        u32x4 a;
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = xenc(part[4 * c + i], tout);
        __builtin_amdgcn_raw_buffer_store_b128(a, rp, off + 16 * c, 0, kCohSC1);
      }
      if constexpr (CG::RT % 4 != 0) {
        u32x2 a;
        a[0] = xenc(part[CG::RT - 2], tout);
        a[1] = xenc(part[CG::RT - 1], tout);
        __builtin_amdgcn_raw_buffer_store_b64(a, rp, off + 16 * (CG::RT / 4), 0, kCohSC1);
      }
    }

    // ================= down partials -> owned residual rows =================
    // Thread t reads producer t / 2's partials of its RT rows; the 256 producers of each of the OWN
    // rows are summed through LDS in a fixed order.
    stamp(p, l * 16 + 10);
    {
      const int tid = phase_tid();
      constexpr int N4 = CG::RT / 4, N2 = (CG::RT % 4) / 2;
      const __amdgpu_buffer_rsrc_t rp = xrsrc(p.xdp, (int64_t)p.n_xdp * 4);
      const int off = ((w * kCfWG + (tid >> 1)) * (2 * CG::RTP) + (tid & 1) * CG::RTP) * 4;
      const uint32_t nxt = ltab_issue(p, l + 1, tid);
      u32x4 v[N4 > 0 ? N4 : 1];
      u32x2 v2 = {0u, 0u};
#pragma unroll
      for (int c = 0; c < N4; ++c) v[c] = __builtin_amdgcn_raw_buffer_load_b128(rp, off + 16 * c, 0, kCohSC1);
      if constexpr (N2) v2 = __builtin_amdgcn_raw_buffer_load_b64(rp, off + 16 * N4, 0, kCohSC1);
      {
        auto ok4 = [&](const u32x4& a) { return xok(a[0], tout) && xok(a[1], tout) && xok(a[2], tout) && xok(a[3], tout); };
        auto ok2 = [&](const u32x2& a) { return !N2 || (xok(a[0], tout) && xok(a[1], tout)); };
        auto all_ok = [&]() {
          bool all = ok2(v2);
#pragma unroll
          for (int c = 0; c < N4; ++c) all &= ok4(v[c]);
          return all;
        };
        ctl.t0 = __builtin_amdgcn_s_memrealtime();
        bool all = all_ok();
        uint32_t flag = 0u;
        while (!all && !give_up(ctl, flag)) {
          __builtin_amdgcn_s_sleep(1);
          flag = load_abort(ctl);
#pragma unroll
          for (int c = 0; c < N4; ++c) {  // branch-free reloads, as in stage_finish
            const bool ok = ok4(v[c]);
            const u32x4 nv = __builtin_amdgcn_raw_buffer_load_b128(rp, ok ? kOOB : off + 16 * c, 0, kCohSC1);
            v[c] = ok ? v[c] : nv;
          }
          if constexpr (N2) {
            const bool ok = ok2(v2);
            const u32x2 nv = __builtin_amdgcn_raw_buffer_load_b64(rp, ok ? kOOB : off + 16 * N4, 0, kCohSC1);
            v2 = ok ? v2 : nv;
          }
          all = all_ok();
        }
      }
      stamp(p, l * 16 + 11);
      if (tid < kLW) s.ltab[((l + 1) & 1) * kLW + tid] = nxt;
      // transpose through LDS: [producer][OWN rows] (past the unit sums the FFN phase may still read)
      float* tp = s.xs + 128;
#pragma unroll
      for (int c = 0; c < N4; ++c) {
        *(float2*)(tp + CG::RT * tid + 4 * c) = make_float2(xdec(v[c][0]), xdec(v[c][1]));
        *(float2*)(tp + CG::RT * tid + 4 * c + 2) = make_float2(xdec(v[c][2]), xdec(v[c][3]));
      }
      if constexpr (N2) *(float2*)(tp + CG::RT * tid + 4 * N4) = make_float2(xdec(v2[0]), xdec(v2[1]));
      __syncthreads();
      if (bail) return;
      // thread t < 16 OWN: row t % OWN over producers t / OWN + 16 j; then the 16 groups (fixed order)
      float* red = s.mrg;  // [16][OWN]
      if (tid < 16 * CG::OWN) {
        float x = 0.f;
#pragma unroll
        for (int j = 0; j < kCfWG / 16; ++j) x += tp[tid + 16 * j * CG::OWN];
        red[tid] = x;
      }
      __syncthreads();
      if (tid < CG::OWN) {
        float dsum = 0.f;
#pragma unroll
        for (int g = 0; g < 16; ++g) dsum += red[g * CG::OWN + tid];
        const float r = s.resid[tid] + dsum;
        s.resid[tid] = r;
        xstore(p.xx, d0 + tid, r, tout);
      }
    }
    } else if constexpr (!MOE) {
    // ================= gate/up + SwiGLU =================
    stamp(p, l * 16 + 8);
    {
      const int tid = phase_tid();
      const int lane = tid & 63, wave = wave_of(tid);
      (void)lane;
      (void)wave;
      XStage<KD> xin;
      stage_issue<KD, true>(tid, p.xm, Ly.ffn_norm, xin);
      PGroup<LPR_D, NB_D, RWG> cur;
      gemv_first<LPR_D, NB_D, RWG>(tid, Ly.gu, g0, g1, cur);
      __syncthreads();
      stage_finish<KD, true>(tid, p.xm, tout, p.eps, xin, s, ctl);
      if (bail) return;
      stamp(p, l * 16 + 9);
      gemv_rest<LPR_D, NB_D, RWG, DBG>(tid, Ly.gu, g0, g1, cur, s);
      __syncthreads();
      for (int pi = tid; 2 * pi < g1 - g0; pi += kPT) {
        const float gv = s.ydot[2 * pi], uv = s.ydot[2 * pi + 1];
        xstore(p.xf, (g0 >> 1) + pi, silu(gv) * uv, tout);
      }
    }

    // ================= down + residual =================
    stamp(p, l * 16 + 10);
    {
      const int tid = phase_tid();
      const int lane = tid & 63, wave = wave_of(tid);
      (void)lane;
      (void)wave;
      XStage<KF> xin;
      const uint32_t nxt = ltab_issue(p, l + 1, tid);
      stage_issue<KF, false>(tid, p.xf, nullptr, xin);
      PGroup<LPR_F, NB_F, RWF> cur;
      gemv_first<LPR_F, NB_F, RWF>(tid, Ly.dn, d0, d1, cur);
      __syncthreads();
      stage_finish<KF, false>(tid, p.xf, tout, 0.f, xin, s, ctl);
      if (bail) return;
      stamp(p, l * 16 + 11);
      if (tid < kLW) s.ltab[((l + 1) & 1) * kLW + tid] = nxt;
      gemv_rest<LPR_F, NB_F, RWF, DBF>(tid, Ly.dn, d0, d1, cur, s);
      __syncthreads();
      for (int r = d0 + tid; r < d1; r += kPT) {
        const float v = s.resid[r - d0] + s.ydot[r - d0];
        s.resid[r - d0] = v;
        xstore(p.xx, r, v, tout);
      }
    }
    } else {
    static_assert((KMAX + KMAX / 32 + kMaxRows + kMaxOwn + 32) % 4 == 0, "MoE scratch 16-byte aligned");
    // ================= MoE router (one row of the router per workgroup) =================
    stamp(p, l * 16 + 8);
    {
      const int tid = phase_tid();
      const int wave = wave_of(tid);
      XStage<KD> xin;
      stage_issue<KD, true>(tid, p.xm, Ly.ffn_norm, xin);
      // this workgroup's router row, 4 fp16 per thread, issued before the input wait
      const bool has_row = w < p.E;
      const bool mine = 4 * tid < KD;
      const __amdgpu_buffer_rsrc_t rr =
          __builtin_amdgcn_make_buffer_rsrc((void*)(Ly.router + (int64_t)(has_row ? w : 0) * KD), 0, KD * 2, kRsrc3);
      const auto wv = __builtin_amdgcn_raw_buffer_load_b64(rr, mine ? tid * 8 : kOOB, 0, kNT);
      // the gate/up matrices' addresses of every expert, for the slots the top-k fills next
      const int n_ex = p.E + p.n_shared;
      const auto pgc = __builtin_amdgcn_raw_buffer_load_b64(xrsrc(Ly.ex.gu_codes, (int64_t)n_ex * 8),
                                                            tid < n_ex ? tid * 8 : kOOB, 0, 0);
      const auto pgs = __builtin_amdgcn_raw_buffer_load_b64(xrsrc(Ly.ex.gu_scales, (int64_t)n_ex * 8),
                                                            tid < n_ex ? tid * 8 : kOOB, 0, 0);
      __syncthreads();
      stage_finish<KD, true>(tid, p.xm, tout, p.eps, xin, s, ctl);
      if (bail) return;
      stamp(p, l * 16 + 9);
      // elements 4 tid .. +3 from the staged layout (the second half of a block is staged / 16);
      // the staged input stays in LDS for the expert gate/up phase
      float dot = 0.f;
      if (mine) {
        const float4 xv = *(const float4*)xs_chunk(s.xs, tid >> 3, tid & 7);
        dot = fmaf(f16_to_f32((uint16_t)(wv[0] & 0xFFFFu)), xv.x, dot);
        dot = fmaf(f16_to_f32((uint16_t)(wv[0] >> 16)), xv.y, dot);
        dot = fmaf(f16_to_f32((uint16_t)(wv[1] & 0xFFFFu)), xv.z, dot);
        dot = fmaf(f16_to_f32((uint16_t)(wv[1] >> 16)), xv.w, dot);
        if ((tid & 7) >= 4) dot *= 16.f;
      }
      dot = wsum(dot);
      if ((tid & 63) == 0) s.red[wave] = dot;
      if (tid < n_ex) {
        uint32_t* all = reinterpret_cast<uint32_t*>(s.mrg + kMoeAll) + 4 * tid;
        all[0] = pgc[0];
        all[1] = pgc[1];
        all[2] = pgs[0];
        all[3] = pgs[1];
      }
      __syncthreads();
      if (tid == 0 && has_row) {
        float tot = 0.f;
#pragma unroll
        for (int v = 0; v < kPW; ++v) tot += s.red[v];
        xstore(p.xr, w, tot, tout);
      }
    }

    // ================= MoE top-k + expert gate/up + SwiGLU =================
    stamp(p, l * 16 + 10);
    {
      const int tid = phase_tid();
      uint64_t* cand = reinterpret_cast<uint64_t*>(s.mrg + kMoeCand);  // [Ep] top-k candidates
      uint64_t* gmax = reinterpret_cast<uint64_t*>(s.mrg + kMoeGmax);  // [Ep / 16] row maxima
      uint64_t* thr = reinterpret_cast<uint64_t*>(s.mrg + kMoeThr);
      int* cnt = reinterpret_cast<int*>(s.mrg + kMoeCnt);
      int* chosen = reinterpret_cast<int*>(s.mrg + kMoeChosen);              // [top_k]
      uint64_t* ckey = reinterpret_cast<uint64_t*>(s.mrg + kMoeChosenKey);   // [top_k]
      float* gate = s.mrg + kMoeGate;                                        // [slots]
      uint64_t* mp = reinterpret_cast<uint64_t*>(s.mrg + kMoePtr);           // [slots][4]
      const uint64_t* all = reinterpret_cast<const uint64_t*>(s.mrg + kMoeAll);  // [E + shared][2]
      const int Ep = (p.E + 31) & ~31;
      const int nrows = Ep / 16;
      // Top-k, descending, ties to the lower index, over keys whose unsigned order is that order.
      // The maxima of the 16-key rows are distinct keys, so the k-th largest of them bounds the
      // k-th largest key from below: only keys at or above it can be chosen, and a candidate's rank
      // among all keys is its rank among the candidates.
      uint64_t my = 0;
      {
        const __amdgpu_buffer_rsrc_t r = xrsrc(p.xr, (int64_t)p.E * 4);
        int idx[1] = {tid < p.E ? tid : -1};
        uint32_t word[1];
        poll_words_issue<1>(r, idx, word);
        poll_words_wait<1>(r, idx, tout, word, ctl);
        if (tid < p.E) my = moe_key(xdec(word[0]), tid);
        const uint64_t rmax = max16_u64(my);  // every lane, so no DPP source lane is inactive
        if (tid < Ep) {
          cand[tid] = 0ull;
          if ((tid & 15) == 0) gmax[tid >> 4] = rmax;
        }
      }
      __syncthreads();
      if (bail) return;
      stamp(p, l * 16 + 11);
      if (tid < nrows && nrows >= p.top_k) {
        const uint64_t g = gmax[tid];
        int rank = 0;
        for (int j = 0; j < nrows; ++j) {
          const uint64_t o = gmax[j];
          rank += (o > g || (o == g && j < tid)) ? 1 : 0;
        }
        if (rank == p.top_k - 1) thr[0] = g;
      }
      if (tid == 0) {
        cnt[0] = 0;
        if (nrows < p.top_k) thr[0] = 0ull;
      }
      __syncthreads();
      const bool is_cand = tid < p.E && my >= thr[0];
      if (is_cand) cand[atomicAdd(cnt, 1)] = my;
      __syncthreads();
      if (is_cand) {
        const int nc = (cnt[0] + 15) & ~15;  // entries past the count hold zero keys
        int rank = 0;
        for (int j = 0; j < nc; j += 16) {
          ulong2 u[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) u[q] = *(const ulong2*)(cand + j + 2 * q);
#pragma unroll
          for (int q = 0; q < 8; ++q) rank += (u[q].x > my ? 1 : 0) + (u[q].y > my ? 1 : 0);
        }
        if (rank < p.top_k) {
          chosen[rank] = tid;
          ckey[rank] = my;
        }
      }
      __syncthreads();
      // slot k: the k-th routed expert (gate: its softmax weight renormalised over the top-k) or a
      // shared expert (gate 1); its matrices' pointers go to LDS
      // (the down matrices' addresses are loaded here and land in LDS after the gate/up pass)
      const int e_slot = tid < NB_F ? (tid < p.top_k ? chosen[tid] : p.E + (tid - p.top_k)) : 0;
      const int n_ex = p.E + p.n_shared;
      const auto pdc = __builtin_amdgcn_raw_buffer_load_b64(xrsrc(Ly.ex.dn_codes, (int64_t)n_ex * 8),
                                                            tid < NB_F ? e_slot * 8 : kOOB, 0, 0);
      const auto pds = __builtin_amdgcn_raw_buffer_load_b64(xrsrc(Ly.ex.dn_scales, (int64_t)n_ex * 8),
                                                            tid < NB_F ? e_slot * 8 : kOOB, 0, 0);
      if (tid < NB_F) {
        const int k = tid;
        const int e = e_slot;
        float g = 1.f;
        if (k < p.top_k) {
          const float mx = moe_key_value(ckey[0]);
          float z = 0.f;
          for (int q = 0; q < p.top_k; ++q) z += __expf(moe_key_value(ckey[q]) - mx);
          g = __expf(moe_key_value(ckey[k]) - mx) / z;
        }
        gate[k] = g;
        mp[k * 4 + 0] = all[e * 2 + 0];
        mp[k * 4 + 1] = all[e * 2 + 1];
        if (w == 0 && k < p.top_k && p.sel_out != nullptr) p.sel_out[(int64_t)l * p.sel_stride + k] = e;
      }
      __syncthreads();
      stamp(p, l * 16 + 14);
      PGroup<LPR_D, NB_D, RWG> cur;
      pload_moe_gu<LPR_D, NB_D, RWG>(tid, mp, p.Fe, g0, g1, wave_of(tid), cur);
      gemv_rest_f<LPR_D, NB_D, RWG, (RWG < 5)>(tid, g0, g1, cur, s, [&](int gi, PGroup<LPR_D, NB_D, RWG>& gg) {
        pload_moe_gu<LPR_D, NB_D, RWG>(tid, mp, p.Fe, g0, g1, gi, gg);
      });
      if (tid < NB_F) {
        uint32_t* dn = reinterpret_cast<uint32_t*>(mp + tid * 4 + 2);
        dn[0] = pdc[0];
        dn[1] = pdc[1];
        dn[2] = pds[0];
        dn[3] = pds[1];
      }
      __syncthreads();
      stamp(p, l * 16 + 15);
      for (int pi = tid; 2 * pi < g1 - g0; pi += kPT) {
        const int r = g0 + 2 * pi;
        const int slot = r / (2 * p.Fe), i = (r - slot * 2 * p.Fe) >> 1;
        const float gv = s.ydot[2 * pi], uv = s.ydot[2 * pi + 1];
        xstore(p.xf, slot * p.Fe + i, gate[slot] * (silu(gv) * uv), tout);
      }
    }

    // ================= MoE down (over the concatenated gated expert outputs) + residual ========
    stamp(p, l * 16 + 12);
    {
      const int tid = phase_tid();
      const uint64_t* mp = reinterpret_cast<const uint64_t*>(s.mrg + kMoePtr);
      XStage<KF> xin;
      const uint32_t nxt = ltab_issue(p, l + 1, tid);
      stage_issue<KF, false>(tid, p.xf, nullptr, xin);
      PGroup<LPR_F, NB_F, RWF> cur;
      pload_moe_dn<LPR_F, NB_F, RWF>(tid, mp, KD, d0, d1, wave_of(tid), cur);
      __syncthreads();
      stage_finish<KF, false>(tid, p.xf, tout, 0.f, xin, s, ctl);
      if (bail) return;
      stamp(p, l * 16 + 13);
      if (tid < kLW) s.ltab[((l + 1) & 1) * kLW + tid] = nxt;
      gemv_rest_f<LPR_F, NB_F, RWF, DBF>(tid, d0, d1, cur, s, [&](int gi, PGroup<LPR_F, NB_F, RWF>& gg) {
        pload_moe_dn<LPR_F, NB_F, RWF>(tid, mp, KD, d0, d1, gi, gg);
      });
      __syncthreads();
      for (int r = d0 + tid; r < d1; r += kPT) {
        const float v = s.resid[r - d0] + s.ydot[r - d0];
        s.resid[r - d0] = v;
        xstore(p.xx, r, v, tout);
      }
    }
    }
  }

  // ================= final RMSNorm + lm_head + argmax partial =================
  stamp(p, L * 16 + 0);
  const uint32_t tfin = base_tag + (uint32_t)L;  // T(L - 1)
  // ================= final RMSNorm + lm_head + argmax partial =================
  {
    const int tid = phase_tid();
    const int lane = tid & 63, wave = wave_of(tid);
    (void)lane;
    (void)wave;
    XStage<KD> xin;
    stage_issue<KD, true>(tid, p.xx, p.final_norm, xin);
    __syncthreads();
    stage_finish<KD, true>(tid, p.xx, tfin, p.eps, xin, s, ctl);
    if (bail) return;
    stamp(p, L * 16 + 1);
    float best_v = -INFINITY;
    int best_i = kNoIdx;
    const Mat lm = p.lm;
    for (int c0 = v0; c0 < v1; c0 += kMaxRows) {
      const int c1 = min(v1, c0 + kMaxRows);
      PGroup<LPR_D, NB_D, LMRW> cur;
      gemv_first<LPR_D, NB_D, LMRW>(tid, lm, c0, c1, cur);
      gemv_rest<LPR_D, NB_D, LMRW, true>(tid, lm, c0, c1, cur, s);
      __syncthreads();
      for (int r = c0 + tid; r < c1; r += kPT) {
        const float v = s.ydot[r - c0];
        if (p.logits) p.logits[r] = v;
        if (v > best_v || (v == best_v && r < best_i)) { best_v = v; best_i = r; }
      }
      __syncthreads();
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(best_v, o);
      const int oi = __shfl_xor(best_i, o);
      if (ov > best_v || (ov == best_v && oi < best_i)) { best_v = ov; best_i = oi; }
    }
    if (lane == 0) {
      s.red[wave] = best_v;
      reinterpret_cast<int*>(s.red)[16 + wave] = best_i;
    }
    __syncthreads();
    if (tid == 0) {
      float bv = s.red[0];
      int bi = reinterpret_cast<int*>(s.red)[16];
      for (int v = 1; v < kPW; ++v) {
        const float ov = s.red[v];
        const int oi = reinterpret_cast<int*>(s.red)[16 + v];
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      // (value, index | tag << 30) as one 64-bit word: the value is exchanged exactly
      const uint64_t word = ((uint64_t)(((uint32_t)bi & 0x3FFFFFFFu) | ((epoch & 3u) << 30)) << 32) | __float_as_uint(bv);
      __hip_atomic_store(p.xarg + w, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (w != 0) return;
  // ================= argmax over the workgroup partials (workgroup 0) =================
  stamp(p, L * 16 + 2);
  {
    const int tid = phase_tid();
    const int lane = tid & 63, wave = wave_of(tid);
    (void)lane;
    (void)wave;
    float bv = -INFINITY;
    int bi = kNoIdx;
    for (int k = tid; k < nwg; k += kPT) {
      uint64_t word = __hip_atomic_load(p.xarg + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ctl.t0 = __builtin_amdgcn_s_memrealtime();
      while ((uint32_t)(word >> 62) != (epoch & 3u)) {
        if (give_up(ctl, __hip_atomic_load(ctl.abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) break;
        __builtin_amdgcn_s_sleep(1);
        word = __hip_atomic_load(p.xarg + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      const float v = __uint_as_float((uint32_t)word);
      const int i = (int)((word >> 32) & 0x3FFFFFFFu);
      if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    __syncthreads();
    if (lane == 0) {
      s.red[wave] = bv;
      reinterpret_cast<int*>(s.red)[16 + wave] = bi;
    }
    __syncthreads();
    if (tid == 0) {
      float b2 = s.red[0];
      int i2 = reinterpret_cast<int*>(s.red)[16];
      for (int v = 1; v < kPW; ++v) {
        const float ov = s.red[v];
        const int oi = reinterpret_cast<int*>(s.red)[16 + v];
        if (ov > b2 || (ov == b2 && oi < i2)) { b2 = ov; i2 = oi; }
      }
      if (!bail) {
        if (p.argmax) p.argmax[0] = i2 == kNoIdx ? 0 : i2;  // every logit NaN: token 0, as the chain
        p.epoch[0] = epoch + 1;  // every workgroup has read it: all have reached the final phase
      }
      if (p.stamps != nullptr) p.stamps[L * 16 + 3] = __builtin_amdgcn_s_memrealtime();
    }
  }
}

// Re-tag every exchange word so that no word matches the first tag the next step waits for
// (T(-1) + 2 for the layer-input vector, T(0) + 2 for the others, epoch + 2 for the argmax).
__global__ void k_persist_reset(PersistParams p, int n_q, int n_p, int n_a, int n_d, int n_f, int n_arg) {
  const uint32_t epoch = p.epoch[0];
  const uint32_t base_tag = epoch * (uint32_t)(p.L + 2);
  const uint32_t bad_in = base_tag + 2, bad = base_tag + 3;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_q) p.xq[i] = xenc(0.f, bad);
  if (i < n_p) p.xp[i] = xenc(0.f, bad);
  if (i < n_a) p.xa[i] = xenc(0.f, bad);
  if (i < n_d) {
    p.xm[i] = xenc(0.f, bad);
    p.xx[i] = xenc(0.f, bad_in);
  }
  if (i < n_f) p.xf[i] = xenc(0.f, bad);
  if (p.xr != nullptr && i < p.E) p.xr[i] = xenc(0.f, bad);
  if (p.xdp != nullptr && i < p.n_xdp) p.xdp[i] = xenc(0.f, bad);
  if (i < n_arg) p.xarg[i] = (uint64_t)((epoch + 2) & 3u) << 62;
  if (i == 0) p.abort_flag[0] = 0u;
}

// ---- host side ----------------------------------------------------------------------------------

template <int LPR_D, int NB_D, int LPR_F, int NB_F, int KVDT, int D, int QR>
static size_t persist_lds_bytes() {
  constexpr int KD = LPR_D * NB_D * 32, KF = LPR_F * NB_F * 32;
  constexpr int KMAX = KD > KF ? KD : KF;
  return sizeof(float) * ((size_t)KMAX + KMAX / 32 + kMaxRows + kMaxOwn + 32 + kMrg + kMaxSplitPages) +
         sizeof(AttnLds<D, QR>) + 2 * sizeof(PLayer);
}

template <int LPR_D, int NB_D, int LPR_F, int NB_F, int KVDT, int D, int QR, int RWQ, int RWO, int RWG, int RWF,
          bool MOE = false, bool COLF = false>
static int launch_persist_t(const PersistParams& p, int nwg, hipStream_t s, bool query_only) {
  auto kern = k_persist<LPR_D, NB_D, LPR_F, NB_F, KVDT, D, QR, RWQ, RWO, RWG, RWF, MOE, COLF>;
  const size_t lds = persist_lds_bytes<LPR_D, NB_D, LPR_F, NB_F, KVDT, D, QR>();
  if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) return -1;
  if (query_only) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kPT, lds) != hipSuccess) return -1;
    return per_cu >= 1 ? 0 : -2;
  }
  PersistParams a = p;
  if (p.plain_launch) {
    hipLaunchKernelGGL(kern, dim3(nwg), dim3(kPT), lds, s, a);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  void* args[] = {&a};
  if (hipLaunchCooperativeKernel((const void*)kern, dim3(nwg), dim3(kPT), args, lds, s) != hipSuccess) return -1;
  return 0;
}

// Shapes with an instantiation: (d, ffn, head dim, query heads per KV head) with the row steps
// per wave group sized for 256 workgroups
// shapes laid out for the FFN by columns (on 256 workgroups). The 27B shape (68 columns, units of
// 4) passes the same tests but timed no faster than its FFN by rows (4109 against 4089 us per
// step): its longer slice arithmetic is exposed at the end of the fused pass, so it keeps the rows.
template <class F>
static int64_t with_colffn(int d, int ffn, int nwg, F&& f) {
  if (nwg != kCfWG) return 0;
  if (d == 4096 && ffn == 12288) return f(CfGeo<4096, 12288>{});
  return 0;
}

int64_t persist_colffn_bytes(int d, int F, int nwg) {
  return with_colffn(d, F, nwg, [](auto g) { return (int64_t)kCfWG * decltype(g)::CH * kPT * 16; });
}

int64_t persist_colffn_xdp_words(int d, int F, int nwg) {
  return with_colffn(d, F, nwg, [](auto g) { return (int64_t)kCfWG * kCfWG * 2 * decltype(g)::RTP; });
}

// One 16-byte chunk (slice w, chunk c, thread t) of the W_down column-slice copy (see the layout
// above cf_issue), from the device matrix (codes [d][F/2], scales tiled [d][lpr][nb]).
template <class G>
__global__ void k_down_slices(Mat dn, uint8_t* out) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= (int64_t)kCfWG * G::CH * kPT) return;
  const int t = (int)(g % kPT), c = (int)((g / kPT) % G::CH), w = (int)(g / ((int64_t)kPT * G::CH));
  const int nblk = dn.K / 32, col0 = w * G::COLS, b0 = col0 >> 5, b_last = (col0 + G::COLS - 1) >> 5;
  auto scale = [&](int row, int b) {
    return b > b_last ? (uint16_t)0 : dn.scales[(int64_t)row * nblk + (b % dn.lpr) * dn.nb + b / dn.lpr];
  };
  u32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int kw = 4 * c + e, j = kw / G::PW, k = kw % G::PW;  // row pair j, word k of the pair
    uint32_t word = 0u;
    if (j < G::RT / 2 && k < G::PCW) {
      for (int n = 0; n < 8; ++n) {
        const int f = 8 * k + (n < 4 ? 2 * n : 2 * (n - 4) + 1);
        const int row = G::RT * t + 2 * j + f / G::COLS, col = col0 + f % G::COLS, in = col % 32;
        const uint8_t byte = dn.codes[(int64_t)row * (dn.K / 2) + (col / 32) * 16 + (in % 16)];
        const uint32_t q = in < 16 ? (byte & 15u) : (byte >> 4);
        word |= q << (4 * n);
      }
    } else if (j < G::RT / 2) {
      for (int h = 0; h < 2; ++h) {
        const int sidx = 2 * (k - G::PCW) + h, r = sidx / G::NSB, b = sidx % G::NSB;
        if (r < 2) word |= (uint32_t)scale(G::RT * t + 2 * j + r, b0 + b) << (16 * h);
      }
    }
    v[e] = word;
  }
  *(u32x4*)(out + g * 16) = v;
}

int launch_down_slices(const Mat& dn, int nwg, uint8_t* out, hipStream_t s) {
  int rc = -2;  // no layout for this shape
  with_colffn(dn.N, dn.K, nwg, [&](auto g) -> int64_t {
    using G = decltype(g);
    const int64_t n = (int64_t)kCfWG * G::CH * kPT;
    hipLaunchKernelGGL(k_down_slices<G>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dn, out);
    rc = hipGetLastError() == hipSuccess ? 0 : -1;
    return 1;
  });
  return rc;
}

int launch_persist(const PersistParams& p, int d, int F, int kv_dtype, int D, int rep, int nwg, hipStream_t s,
                   bool query_only) {
  // the 9B shape on 256 workgroups: the FFN by columns
  if (persist_colffn_bytes(d, F, nwg) > 0 && D == 128 && d == 4096 && rep == 4) {
    if (kv_dtype == 1) return launch_persist_t<64, 2, 64, 6, 1, 128, 4, 3, 2, 2, 1, false, true>(p, nwg, s, query_only);
    if (kv_dtype == 2) return launch_persist_t<64, 2, 64, 6, 2, 128, 4, 3, 2, 2, 1, false, true>(p, nwg, s, query_only);
    if (kv_dtype == 3) return launch_persist_t<64, 2, 64, 6, 3, 128, 4, 3, 2, 2, 1, false, true>(p, nwg, s, query_only);
  }
  // FP8 E4M3 caches
#define BW_P8(DM, FF, LD, ND, LF, NF, DD, QR, RQ, RO, RG, RF)                        \
  if (kv_dtype == 3 && d == DM && F == FF && D == DD && rep == QR)                  \
    return launch_persist_t<LD, ND, LF, NF, 3, DD, QR, RQ, RO, RG, RF>(p, nwg, s, query_only);
  BW_P8(4096, 12288, 64, 2, 64, 6, 128, 4, 3, 2, 2, 1)
  BW_P8(5120, 17408, 32, 5, 32, 17, 128, 5, 1, 1, 1, 1)
  BW_P8(256, 1024, 8, 1, 32, 1, 64, 2, 1, 1, 1, 1)
#undef BW_P8
  if (kv_dtype == 3) return -2;
#define BW_P(DM, FF, LD, ND, LF, NF, DD, QR, RQ, RO, RG, RF)                                                  \
  if (d == DM && F == FF && D == DD && rep == QR) {                                                           \
    return kv_dtype == 1 ? launch_persist_t<LD, ND, LF, NF, 1, DD, QR, RQ, RO, RG, RF>(p, nwg, s, query_only) \
                         : launch_persist_t<LD, ND, LF, NF, 2, DD, QR, RQ, RO, RG, RF>(p, nwg, s, query_only); \
  }
  BW_P(4096, 12288, 64, 2, 64, 6, 128, 4, 3, 2, 2, 1)  // dense-9b: 24 / 16 / 96 / 16 rows per workgroup
  BW_P(5120, 17408, 32, 5, 32, 17, 128, 5, 1, 1, 1, 1)  // dense-27b: 28 / 20 / 136 / 20 rows per workgroup
  BW_P(256, 1024, 8, 1, 32, 1, 64, 2, 1, 1, 1, 1)       // tiny
#undef BW_P
  return -2;
}

// MoE shapes: (d, slots x expert width, head dim, query heads per KV head). The gate/up pass reads
// one row per wave per row step (LPR_D = 64), the down pass one slot's Fe / 32 blocks per lane
// column (Fe = 32 LPR_F, NB_F = slots).
int launch_persist_moe(const PersistParams& p, int d, int kv_dtype, int D, int rep, int nwg, hipStream_t s,
                       bool query_only) {
  const int slots = p.top_k + p.n_shared;
#define BW_PM(DM, FE, SL, LD, ND, LF, DD, QR, RQ, RO, RG, RF)                                                    \
  if (d == DM && p.Fe == FE && slots == SL && D == DD && rep == QR) {                                           \
    static_assert(DM == LD * ND * 32 && FE == LF * 32, "d and Fe match the lane split");                        \
    if (kv_dtype == 3) return launch_persist_t<LD, ND, LF, SL, 3, DD, QR, RQ, RO, RG, RF, true>(p, nwg, s, query_only); \
    return kv_dtype == 1 ? launch_persist_t<LD, ND, LF, SL, 1, DD, QR, RQ, RO, RG, RF, true>(p, nwg, s, query_only) \
                         : launch_persist_t<LD, ND, LF, SL, 2, DD, QR, RQ, RO, RG, RF, true>(p, nwg, s, query_only); \
  }
  BW_PM(2048, 512, 9, 64, 1, 16, 128, 4, 2, 1, 5, 1)  // moe-35b-a3b: 12 / 8 / 36 / 8 rows per workgroup
#undef BW_PM
  return -2;
}

int launch_persist_reset(const PersistParams& p, int n_q, int n_p, int n_a, int n_d, int n_f, int n_arg, hipStream_t s) {
  const int n = std::max({n_q, n_p, n_a, n_d, n_f, n_arg, p.xr != nullptr ? p.E : 0, p.xdp != nullptr ? p.n_xdp : 0});
  hipLaunchKernelGGL(k_persist_reset, dim3((n + 255) / 256), dim3(256), 0, s, p, n_q, n_p, n_a, n_d, n_f, n_arg);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace bw
