// bw_spec.hip - greedy acceptance after a speculative verify step.
//
// bw24 deep-dive page (10100.com): section 1 requires speculative output identical to plain
// token-by-token argmax decoding; section 2 puts the verify-accept logic in the engine, with a
// ring buffer for draft tokens and logits; section 5 stage 4 has the verify kernel mask the
// positions after the first mismatching draft so that their logits read -inf.
//
// Row i of sequence b holds the input x_i (x_0 = the last committed token, x_1..x_{t-1} the
// drafts) and the step's greedy token a_i, the prediction for the position after x_i. Draft
// x_{j+1} stands while x_1..x_j stood and x_{j+1} == a_j. With n drafts standing, a_0..a_n are
// the committed tokens of this step (a_0..a_{n-1} equal the standing drafts, a_n is the token
// after them), the cache holds valid keys and values for x_0..x_n, so seq_lens advances by
// n + 1, and a_n is the next step's x_0. Rows n+1..t-1 were computed from rejected drafts.
#include "bw_common.h"
#include "bw_internal.h"

namespace bw {

// Grid (t, batch), 256 threads. Every block finds its sequence's n from the t inputs and
// argmaxes (t is small), a block with row i > n fills that logits row with -inf, and block
// (0, b) does the bookkeeping. Only block (0, b) writes x_0 of sequence b, which no block reads.
__global__ __launch_bounds__(256) void k_spec_accept(int32_t* __restrict__ tokens, const int32_t* __restrict__ argmax,
                                                     float* __restrict__ logits, int64_t V,
                                                     int32_t* __restrict__ seq_lens, int32_t* __restrict__ ring,
                                                     int32_t* __restrict__ count, int cap,
                                                     int32_t* __restrict__ accepted, int t) {
  const int i = blockIdx.x, b = blockIdx.y;
  const int32_t* x = tokens + (int64_t)b * t;
  const int32_t* a = argmax + (int64_t)b * t;
  int n = 0;
  while (n + 1 < t && x[n + 1] == a[n]) ++n;
  if (logits != nullptr && i > n) {
    float* row = logits + ((int64_t)b * t + i) * V;
    for (int64_t k = threadIdx.x; k < V; k += blockDim.x) row[k] = -INFINITY;
  }
  if (i == 0 && threadIdx.x == 0) {
    if (ring != nullptr) {
      const int c = count[b];
      for (int j = 0; j <= n; ++j) ring[(int64_t)b * cap + (c + j) % cap] = a[j];
      count[b] = c + n + 1;
    }
    if (accepted != nullptr) accepted[b] = n;
    seq_lens[b] += n + 1;
    tokens[(int64_t)b * t] = a[n];
  }
}

int launch_spec_accept(int32_t* tokens, const int32_t* argmax, float* logits, int64_t V, int32_t* seq_lens,
                       int32_t* ring, int32_t* count, int cap, int32_t* accepted, int batch, int t, hipStream_t s) {
  hipLaunchKernelGGL(k_spec_accept, dim3(t, batch), dim3(256), 0, s, tokens, argmax, logits, V, seq_lens, ring, count,
                     cap, accepted, t);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace bw
