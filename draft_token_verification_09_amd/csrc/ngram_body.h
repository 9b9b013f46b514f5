// Prompt n-gram lookup, one workgroup per sequence: the body shared by ngram_propose's own
// kernel and the fused propose-and-verify kernel of chain.hip.
//
// "Accelerating Autoregressive LLM Inference 3x with Lossless Speculative Decoding
// and EAGLE Heads" (x078.com): prompt n-gram lookup as a zero-VRAM draft
// mechanism proposing K candidates, with the lookup's maximum n set to 4 in its
// deployment snippet (section 1).  Reading: for n = n_max down to n_min, the
// earliest j with c[j:j+n] == c[L-n:L] and j + n <= L - 1 wins; the draft is
// c[j+n : min(j+n+K, L)].
//
// Instead of testing every (n, j) pair, each lane takes candidate end positions
// e = j + n - 1 in [0, L-2] and measures how many tokens ending at e match the suffix
// ending at L-1 (at most n_max); a match of length >= n at end e is an occurrence for n
// starting at j = e - n + 1, so the earliest occurrence for n is the smallest such e.
// A lane visits its end positions in increasing order, so the first time its longest match
// reaches n is its earliest occurrence for n: it then takes a shared-memory atomic min per
// newly reached n (a few per lane), and the largest n with an occurrence wins.  The
// context goes through shared memory in tiles of kTile tokens (plus the n_max - 1 before
// each tile), loaded with independent reads, so the comparisons never wait on memory.  The
// first tile is read before the context length arrives (it does not depend on it); when
// the whole context fits in it, the suffix and the proposed tokens come from shared memory
// too, so the body waits on global memory once before its stores.
#pragma once

#include "device_common.h"
#include "spec_verify.h"

namespace specv {

constexpr int kTile = 4096;

// Copy tokens [lo, lo + n) of the context row c into s[0, n) with every lane's loads of a batch
// in flight together (kBatch per lane) before any is stored: a copy whose loads each wait for the
// previous store would pay one memory round trip per token a lane copies, which next to a
// streaming pass on the same device costs microseconds each.
template <int NT>
__device__ __forceinline__ void stage_tokens(int* s, const int32_t* c, int lo, int n) {
  constexpr int kBatch = 8;
  for (int base = 0; base < n; base += NT * kBatch) {
    int v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = base + j * NT + static_cast<int>(threadIdx.x);
      v[j] = i < n ? c[lo + i] : 0;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = base + j * NT + static_cast<int>(threadIdx.x);
      if (i < n) s[i] = v[j];
    }
  }
}

// Shared-memory ints a context tile of TILE tokens takes (with the n-gram overlap).
template <int TILE>
constexpr int kTileInts = TILE + SPEC_MAX_NGRAM_N;

// Proposal of sequence b by a workgroup of NT lanes, through context tiles of TILE tokens held
// in s_ctx (shared memory of kTileInts<TILE> ints).  Returns the draft length (0 with no match
// or an invalid context length) in every lane, and leaves the draft in out_draft[b].
template <int NT, int TILE>
__device__ __forceinline__ int ngram_propose_in(int* s_ctx, int b, const int32_t* context, const int32_t* context_len,
                                                int L_max, int n_min, int n_max, int K, int32_t* out_draft,
                                                int32_t* out_len, int32_t* out_match_n) {
  __shared__ int s_suffix[SPEC_MAX_NGRAM_N];
  __shared__ int s_first[SPEC_MAX_NGRAM_N + 1];
  const int tid = threadIdx.x;
  const int32_t* c = context + static_cast<size_t>(b) * L_max;
  int32_t* od = out_draft + static_cast<size_t>(b) * K;
  const int L = context_len[b];
  const int pre = min(TILE, L_max);  // the first tile: tokens [0, pre), in bounds whatever L is
  stage_tokens<NT>(s_ctx, c, 0, pre);
  if (L < 1 || L > L_max) {
    for (int k = tid; k < K; k += NT) od[k] = -1;
    if (tid == 0) {
      out_len[b] = 0;
      if (out_match_n) out_match_n[b] = -1;
    }
    return 0;
  }
  const bool one_tile = L <= pre;  // the whole context is in the first tile, and stays there
  if (tid <= n_max) s_first[tid] = INT_MAX;
  __syncthreads();  // the first tile is in shared memory
  if (tid < n_max) s_suffix[tid] = tid < L ? (one_tile ? s_ctx[L - 1 - tid] : c[L - 1 - tid]) : 0;
  int reached = 0;  // this lane's longest match so far
  for (int t0 = 0; t0 <= L - 2; t0 += TILE) {
    // end positions e in [t0, t1) need tokens [lo, t1)
    const int t1 = min(t0 + TILE, L - 1);
    const int lo = max(0, t0 - (n_max - 1));
    __syncthreads();  // the previous tile's comparisons (and the suffix) are done
    if (t0 > 0)  // the first tile, [0, t1) within [0, pre), is already loaded
      stage_tokens<NT>(s_ctx, c, lo, t1 - lo);
    __syncthreads();
    for (int e = t0 + tid; e < t1; e += NT) {
      int ml = 0;
      while (ml < n_max && ml <= e && s_ctx[e - ml - lo] == s_suffix[ml]) ++ml;
      for (int n = reached + 1; n <= ml; ++n) atomicMin(&s_first[n], e);
      reached = max(reached, ml);
    }
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
  for (int k = tid; k < K; k += NT) od[k] = k < len ? (one_tile ? s_ctx[start + k] : c[start + k]) : -1;
  if (tid == 0) {
    out_len[b] = len;
    if (out_match_n) out_match_n[b] = best_n;
  }
  return len;
}

// The same with the tile in a shared array of its own.
template <int NT, int TILE = kTile>
__device__ __forceinline__ int ngram_propose_body(int b, const int32_t* context, const int32_t* context_len,
                                                  int L_max, int n_min, int n_max, int K, int32_t* out_draft,
                                                  int32_t* out_len, int32_t* out_match_n) {
  __shared__ int s_ctx[kTileInts<TILE>];
  return ngram_propose_in<NT, TILE>(s_ctx, b, context, context_len, L_max, n_min, n_max, K, out_draft, out_len,
                                    out_match_n);
}

}  // namespace specv
