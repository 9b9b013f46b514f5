// Prompt n-gram lookup drafting, batched over sequences: one workgroup of 1024 lanes per
// sequence runs the lookup of ngram_body.h ("Accelerating Autoregressive LLM Inference 3x
// with Lossless Speculative Decoding and EAGLE Heads" (x078.com), section 1's deployment
// snippet: lookup maximum n = 4, K candidates).
#include "device_common.h"
#include "host_runtime.h"
#include "ngram_body.h"
#include "spec_verify.h"

namespace specv {

constexpr int kNgramThreads = 1024;  // one workgroup per sequence, 16 waves

__global__ __launch_bounds__(kNgramThreads) void ngram_propose_kernel(const int32_t* context, const int32_t* context_len,
                                                                 int L_max, int n_min, int n_max, int K,
                                                                 int32_t* out_draft, int32_t* out_len,
                                                                 int32_t* out_match_n) {
  ngram_propose_body<kNgramThreads>(static_cast<int>(blockIdx.x), context, context_len, L_max, n_min, n_max, K,
                                    out_draft, out_len, out_match_n);
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
