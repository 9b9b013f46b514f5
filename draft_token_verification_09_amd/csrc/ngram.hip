// Prompt n-gram lookup drafting, batched over sequences.
//
// "Accelerating Autoregressive LLM Inference 3x with Lossless Speculative Decoding
// and EAGLE Heads" (x078.com): prompt n-gram lookup as a zero-VRAM draft
// mechanism proposing K candidates, with the lookup's maximum n set to 4 in its
// deployment snippet (section 1).  Reading: for n = n_max down to n_min, the
// earliest j with c[j:j+n] == c[L-n:L] and j + n <= L - 1 wins; the draft is
// c[j+n : min(j+n+K, L)].
//
// One workgroup per sequence.  Instead of testing every (n, j) pair, each lane
// takes candidate end positions e = j + n - 1 in [0, L-2] and measures how many
// tokens ending at e match the suffix ending at L-1 (at most n_max); a match of
// length >= n at end e is an occurrence for n starting at j = e - n + 1, so the
// earliest occurrence for n is the smallest such e.  Each lane keeps its earliest e
// per n in registers, a wave minimum and one shared-memory atomic min per wave and n
// combine them, and the largest n with an occurrence wins.  The context goes
// through shared memory in tiles of kTile tokens (plus the n_max - 1 before each
// tile), loaded with independent reads, so the comparisons never wait on memory.
// The first tile is read before the context length arrives (it does not depend on it);
// when the whole context fits in it, the suffix and the proposed tokens come from shared
// memory too, so the kernel waits on global memory once before its stores.
#include "device_common.h"
#include "host_runtime.h"
#include "spec_verify.h"

namespace specv {

constexpr int kTile = 4096;
constexpr int kNgramThreads = 1024;  // one workgroup per sequence, 16 waves

__global__ __launch_bounds__(kNgramThreads) void ngram_propose_kernel(const int32_t* context, const int32_t* context_len,
                                                                 int L_max, int n_min, int n_max, int K,
                                                                 int32_t* out_draft, int32_t* out_len,
                                                                 int32_t* out_match_n) {
  __shared__ int s_suffix[SPEC_MAX_NGRAM_N];
  __shared__ int s_first[SPEC_MAX_NGRAM_N + 1];
  __shared__ int s_ctx[kTile + SPEC_MAX_NGRAM_N];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t* c = context + static_cast<size_t>(b) * L_max;
  int32_t* od = out_draft + static_cast<size_t>(b) * K;
  const int L = context_len[b];
  const int pre = min(kTile, L_max);  // the first tile: tokens [0, pre), in bounds whatever L is
  for (int i = tid; i < pre; i += kNgramThreads) s_ctx[i] = c[i];
  if (L < 1 || L > L_max) {
    for (int k = tid; k < K; k += kNgramThreads) od[k] = -1;
    if (tid == 0) {
      out_len[b] = 0;
      if (out_match_n) out_match_n[b] = -1;
    }
    return;
  }
  const bool one_tile = L <= pre;  // the whole context is in the first tile, and stays there
  if (tid <= n_max) s_first[tid] = INT_MAX;
  __syncthreads();  // the first tile is in shared memory
  if (tid < n_max) s_suffix[tid] = tid < L ? (one_tile ? s_ctx[L - 1 - tid] : c[L - 1 - tid]) : 0;
  // This lane's earliest end position per n.  A lane visits end positions in increasing
  // order, so first[n] is set once, when the lane's longest match so far first reaches n.
  int first[SPEC_MAX_NGRAM_N + 1];
#pragma unroll
  for (int n = 0; n <= SPEC_MAX_NGRAM_N; ++n) first[n] = INT_MAX;
  int reached = 0;
  for (int t0 = 0; t0 <= L - 2; t0 += kTile) {
    // end positions e in [t0, t1) need tokens [lo, t1)
    const int t1 = min(t0 + kTile, L - 1);
    const int lo = max(0, t0 - (n_max - 1));
    __syncthreads();  // the previous tile's comparisons (and the suffix) are done
    if (t0 > 0)       // the first tile, [0, t1) within [0, pre), is already loaded
      for (int i = tid; i < t1 - lo; i += kNgramThreads) s_ctx[i] = c[lo + i];
    __syncthreads();
    for (int e = t0 + tid; e < t1; e += kNgramThreads) {
      int ml = 0;
      while (ml < n_max && ml <= e && s_ctx[e - ml - lo] == s_suffix[ml]) ++ml;
      if (ml > reached) {
#pragma unroll
        for (int n = 1; n <= SPEC_MAX_NGRAM_N; ++n)
          if (n > reached && n <= ml) first[n] = e;
        reached = ml;
      }
    }
  }
#pragma unroll
  for (int n = 1; n <= SPEC_MAX_NGRAM_N; ++n) {
    if (n > n_max) break;
    const int m = wave_min_int(first[n]);
    if ((tid & 63) == 0 && m != INT_MAX) atomicMin(&s_first[n], m);
  }
  __syncthreads();
  int best_n = 0, best_e = -1;
  for (int n = n_max; n >= n_min; --n) {
    if (s_first[n] != INT_MAX) {
      best_n = n;
      best_e = s_first[n];
      break;
    }
  }
  const int start = best_e + 1;  // first continuation token
  const int len = best_n ? min(K, L - start) : 0;
  for (int k = tid; k < K; k += kNgramThreads) od[k] = k < len ? (one_tile ? s_ctx[start + k] : c[start + k]) : -1;
  if (tid == 0) {
    out_len[b] = len;
    if (out_match_n) out_match_n[b] = best_n;
  }
}

}  // namespace specv

using namespace specv;

extern "C" {

spec_status_t ngram_propose(const int32_t* context, const int32_t* context_len,
                            int B, int L_max, int n_min, int n_max, int K,
                            int32_t* out_draft_tokens, int32_t* out_draft_len, int32_t* out_match_n,
                            spec_stream_t stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (B < 0 || L_max < 1 || K < 1 || n_min < 1 || n_max < n_min)
    return fail(SPEC_ERR_INVALID_ARG, "need B >= 0, L_max >= 1, K >= 1, 1 <= n_min <= n_max");
  if (n_max > SPEC_MAX_NGRAM_N) return fail(SPEC_ERR_UNSUPPORTED, "n_max = %d exceeds SPEC_MAX_NGRAM_N", n_max);
  if (K > SPEC_MAX_K) return fail(SPEC_ERR_UNSUPPORTED, "K = %d exceeds SPEC_MAX_K", K);
  if (B == 0) return SPEC_OK;
  if (!context || !context_len || !out_draft_tokens || !out_draft_len)
    return fail(SPEC_ERR_INVALID_ARG, "a required pointer is NULL");
  LaunchScope scope("ngram_propose", s);
  scope.launch(ngram_propose_kernel, dim3(static_cast<unsigned>(B)), dim3(kNgramThreads), s, context, context_len, L_max, n_min, n_max, K, out_draft_tokens, out_draft_len, out_match_n);
  return scope.finish();
}

}  // extern "C"
