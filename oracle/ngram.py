"""Prompt n-gram lookup drafting -- the oracle (test infrastructure only).

Method: "Accelerating Autoregressive LLM Inference 3x with Lossless Speculative
Decoding and EAGLE Heads" (x078.com): the draft mechanism may be a zero-VRAM
prompt n-gram lookup proposing K = 5 candidates; its deployment snippet (section 1)
sets the lookup's maximum n to 4.

Readings taken where the page is silent:
  * For n = n_max down to n_min, look for the current suffix c[L-n:L] earlier in
    the context: the smallest j with c[j:j+n] == c[L-n:L] and j + n <= L - 1
    (so that at least one token follows the match; overlap with the suffix is allowed).
  * The first (largest) n with a match wins; the draft is the continuation
    c[j+n : min(j+n+K, L)], so 1 <= draft_len <= K.  With no match draft_len = 0.
  * The drafted tokens are verified with a one-hot draft distribution
    (alpha = p(x)), which the chain oracle implements for draft logits = None.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class NgramResult:
    draft: np.ndarray      # [B, K] int32, -1 padded
    draft_len: np.ndarray  # [B] int32
    match_n: np.ndarray    # [B] int32 (0 = no match)
    match_pos: np.ndarray  # [B] int32 start j of the match (-1 = none)


def ngram_propose_sequence(context: np.ndarray, n_min: int, n_max: int, K: int):
    """Returns (draft tokens list, matched n, match start j) for one context."""
    c = np.asarray(context, dtype=np.int64)
    L = c.shape[0]
    for n in range(n_max, n_min - 1, -1):
        if n > L - 1:
            continue
        suffix = c[L - n:]
        windows = np.lib.stride_tricks.sliding_window_view(c, n)[: L - n]  # starts j = 0 .. L-1-n
        hits = np.flatnonzero(np.all(windows == suffix, axis=1))
        if hits.size:
            j = int(hits[0])
            cont = c[j + n: min(j + n + K, L)]
            return [int(v) for v in cont], n, j
    return [], 0, -1


def ngram_propose(context, context_len, n_min: int, n_max: int, K: int) -> NgramResult:
    context = np.asarray(context)
    B = context.shape[0]
    if not 1 <= n_min <= n_max:
        raise ValueError("need 1 <= n_min <= n_max")
    draft = np.full((B, K), -1, dtype=np.int32)
    dlen = np.zeros((B,), dtype=np.int32)
    mn = np.zeros((B,), dtype=np.int32)
    mpos = np.full((B,), -1, dtype=np.int32)
    for b in range(B):
        L = int(context_len[b])
        if not 1 <= L <= context.shape[1]:
            raise ValueError("context length out of range")
        toks, n, j = ngram_propose_sequence(context[b, :L], n_min, n_max, K)
        draft[b, : len(toks)] = toks
        dlen[b] = len(toks)
        mn[b] = n
        mpos[b] = j
    return NgramResult(draft=draft, draft_len=dlen, match_n=mn, match_pos=mpos)
