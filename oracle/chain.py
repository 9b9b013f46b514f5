"""Chain verification by modified rejection sampling -- the oracle (test infrastructure only).

Method: "Speculative Decoding in Production: From Draft Models to EAGLE-3 Dynamic
Trees ..." (blog.llmgo.top), section I.1 "Verification via Modified Rejection
Sampling": for each draft token x_k compute alpha = min(1, p(x_k)/q(x_k)) (step 1),
draw r ~ U(0,1) and accept while r <= alpha, stopping at the first rejection
(step 2); on rejection draw the replacement from max(0, p - q) normalised
(step 3).  The same page states the invariance theorem that this reproduces p.

Readings taken where that page is silent (each also named at its use):
  * p = softmax(target_logits / T), q = softmax(draft_logits / T), one T per sequence.
  * The target supplies K + 1 rows: row k scores draft token k, row K is the
    "next position" used for a bonus token when all drafted tokens are accepted.
  * With a per-sequence draft length k_b <= K only rows 0..k_b (target) and
    0..k_b - 1 (draft) are used; the bonus comes from target row k_b.
  * No draft logits means a one-hot draft distribution at the drafted token
    (prompt-lookup drafting): q(x) = 1 so alpha = p(x), and the residual is p
    with the drafted token removed.
  * Sampling from a weight vector w: inclusive prefix sums C in vocabulary
    order, t = u * C[V-1]; the result is the smallest i with C[i] >= t.
  * q(x) = 0 gives alpha = 1 if p(x) > 0 else 0; an all-zero residual falls back
    to sampling p itself (both unreachable in exact arithmetic when x ~ q).
  * Temperature 0 means greedy verification (the invariance theorem of section I.1
    covers greedy decoding; the "Speculative decoding: Medusa, EAGLE, vLLM" usage
    example runs at temperature 0): draft k is accepted iff it equals the argmax of
    target row k (raw logits, smallest index on ties), and the token emitted after
    the last accepted draft is the argmax of the next target row.  No uniform and
    no draft logit is used.

Everything is float64; each sequence is verified by a plain sequential loop.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .common import widen_logits
from .tree import argmax_first


def softmax_at_temperature(logits: np.ndarray, temperature: float) -> np.ndarray:
    """p_i = exp(l_i / T) / sum_j exp(l_j / T), evaluated as exp(z - max z) / sum(...) in float64.

    Temperature divides the logits (a reading: the pages name temperature without a formula).
    -inf logits get probability 0; the row needs at least one finite logit."""
    if not temperature > 0.0:
        raise ValueError("temperature must be > 0")
    z = np.asarray(logits, dtype=np.float64) / float(temperature)
    m = np.max(z)
    if not np.isfinite(m):
        raise ValueError("a row needs at least one finite logit and no +inf/NaN")
    e = np.exp(z - m)
    return e / np.sum(e)


def acceptance_probability(p_x: float, q_x: float) -> float:
    """alpha = min(1, p(x) / q(x))  ("Speculative Decoding in Production", section I.1, step 1).

    q(x) = 0 (unreachable when x was drawn from q) is read as alpha = 1 if p(x) > 0 else 0."""
    if q_x > 0.0:
        return min(1.0, p_x / q_x)
    return 1.0 if p_x > 0.0 else 0.0


def accept_test(r: float, alpha: float) -> bool:
    """Accept the drafted token iff r <= alpha  ("Speculative Decoding in Production", section I.1, step 2)."""
    return r <= alpha


def residual_weights(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Unnormalised residual max(0, p(x) - q(x))  ("Speculative Decoding in Production", section I.1, step 3)."""
    return np.maximum(0.0, p - q)


def inverse_cdf_sample(w: np.ndarray, u: float):
    """Draw an index from weights w >= 0 with one uniform u in (0, 1].

    Reading: C = inclusive prefix sums of w in vocabulary order, W = C[-1], t = u * W,
    result = smallest i with C[i] >= t (the last i with w_i > 0 if rounding left none).
    Returns (index, gap, W) where gap = min(t - C[i-1], C[i] - t) / W is the distance
    from t to the nearer boundary of the chosen interval, relative to W."""
    if not (0.0 < u <= 1.0):
        raise ValueError("u must lie in (0, 1]")
    C = np.cumsum(np.asarray(w, dtype=np.float64))
    W = float(C[-1])
    if not W > 0.0:
        raise ValueError("weights sum to zero")
    t = u * W
    hits = np.flatnonzero(C >= t)
    if hits.size:
        i = int(hits[0])
    else:
        i = int(np.flatnonzero(np.asarray(w) > 0.0)[-1])
    lo = float(C[i - 1]) if i > 0 else 0.0
    gap = min(t - lo, float(C[i]) - t) / W
    return i, gap, W


@dataclass
class ChainSequenceResult:
    num_accepted: int            # n: drafted tokens accepted before the first rejection
    tokens: List[int]            # x_0..x_{n-1}, then the resampled / bonus token
    p_x: List[float]             # p_k(x_k) for k < k_b
    q_x: List[float]             # q_k(x_k) for k < k_b
    alpha: List[float]           # alpha_k for k < k_b
    accept_margins: List[float]  # |u_k - alpha_k| for every accept test that was decided (k <= n, k < k_b)
    cdf_gap: float               # boundary distance of the final draw (relative to its total mass)
    mode: str                    # "residual", "bonus" or "residual_zero_fallback"
    final_mass: float            # W of the final draw
    row_max: List[float] = field(default_factory=list)


def verify_chain_sequence(
    target_rows: np.ndarray,
    draft_rows: Optional[np.ndarray],
    tokens: np.ndarray,
    draft_len: int,
    temperature: float,
    u_accept: np.ndarray,
    u_final: float,
) -> ChainSequenceResult:
    """Verify one sequence's chain of drafted tokens.

    target_rows: [K+1, V] float64 logits; draft_rows: [K, V] float64 logits or None (one-hot q);
    tokens: [K] drafted ids (only the first draft_len are used); u_accept: [K]; u_final: scalar."""
    K1, V = target_rows.shape
    K = K1 - 1
    kb = int(draft_len)
    if not 0 <= kb <= K:
        raise ValueError("draft_len out of range")
    if not temperature > 0.0:
        raise ValueError("temperature must be > 0")
    for k in range(kb):
        if not 0 <= int(tokens[k]) < V:
            raise ValueError("draft token out of range")
        if not 0.0 < float(u_accept[k]) <= 1.0:
            raise ValueError("accept uniform outside (0, 1]")
    if not 0.0 < float(u_final) <= 1.0:
        raise ValueError("final uniform outside (0, 1]")

    p_rows = [softmax_at_temperature(target_rows[k], temperature) for k in range(kb + 1)]
    if draft_rows is None:
        q_rows = []
        for k in range(kb):
            q = np.zeros(V)
            q[int(tokens[k])] = 1.0
            q_rows.append(q)
    else:
        q_rows = [softmax_at_temperature(draft_rows[k], temperature) for k in range(kb)]

    # Step 1 for every drafted position (computed for all k < k_b, as the GPU does).
    p_x, q_x, alpha = [], [], []
    for k in range(kb):
        x = int(tokens[k])
        p_x.append(float(p_rows[k][x]))
        q_x.append(float(q_rows[k][x]))
        alpha.append(acceptance_probability(p_x[-1], q_x[-1]))

    # Step 2: accept while r <= alpha; the first rejection ends verification.
    n = kb
    margins = []
    for k in range(kb):
        margins.append(abs(float(u_accept[k]) - alpha[k]))
        if not accept_test(float(u_accept[k]), alpha[k]):
            n = k
            break

    # Step 3 (rejection) or the bonus draw from the next target row (all accepted).
    if n < kb:
        w = residual_weights(p_rows[n], q_rows[n])
        mode = "residual"
        if not np.sum(w) > 0.0:
            w = p_rows[n]
            mode = "residual_zero_fallback"
    else:
        w = p_rows[kb]
        mode = "bonus"
    y, gap, W = inverse_cdf_sample(w, float(u_final))

    out = [int(tokens[k]) for k in range(n)] + [int(y)]
    return ChainSequenceResult(
        num_accepted=n, tokens=out, p_x=p_x, q_x=q_x, alpha=alpha, accept_margins=margins,
        cdf_gap=gap, mode=mode, final_mass=W,
    )


def verify_chain_greedy_sequence(target_rows: np.ndarray, tokens: np.ndarray, draft_len: int) -> ChainSequenceResult:
    """Greedy (temperature 0) verification of one sequence's chain: accept draft k while it
    equals argmax_first(target row k); emit the argmax of the row after the last accepted
    draft.  p_x, q_x and alpha are not defined at temperature 0 and are reported as 0."""
    K1, V = target_rows.shape
    K = K1 - 1
    kb = int(draft_len)
    if not 0 <= kb <= K:
        raise ValueError("draft_len out of range")
    for k in range(kb):
        if not 0 <= int(tokens[k]) < V:
            raise ValueError("draft token out of range")
    n = kb
    for k in range(kb):
        if int(tokens[k]) != argmax_first(target_rows[k]):
            n = k
            break
    out = [int(tokens[k]) for k in range(n)] + [argmax_first(target_rows[n])]
    return ChainSequenceResult(
        num_accepted=n, tokens=out, p_x=[0.0] * kb, q_x=[0.0] * kb, alpha=[0.0] * kb, accept_margins=[],
        cdf_gap=float("inf"), mode="greedy", final_mass=0.0,
    )


@dataclass
class ChainBatchResult:
    tokens: np.ndarray        # [B, K+1] int32, -1 padded
    num_accepted: np.ndarray  # [B] int32
    probs: np.ndarray         # [B, K, 3] float64: p(x), q(x), alpha for k < k_b, 0 elsewhere
    sequences: List[ChainSequenceResult]


def verify_chain(target, draft, dtype: str, tokens, temperature, u_accept, u_final,
                 draft_len=None, seqs=None) -> ChainBatchResult:
    """Batched chain verification: a loop over sequences of verify_chain_sequence, or of
    verify_chain_greedy_sequence for a sequence whose temperature is 0.

    target: [B, K+1, V] and draft: [B, K, V] (or None) as float32 or bf16 uint16 bits;
    tokens [B, K] int; temperature [B]; u_accept [B, K]; u_final [B]; draft_len [B] or None.
    `seqs` restricts the work to a subset of sequence indices (others are left zero / -1)."""
    target = np.asarray(target)
    B, K1, V = target.shape
    K = K1 - 1
    out_tok = np.full((B, K + 1), -1, dtype=np.int32)
    out_n = np.zeros((B,), dtype=np.int32)
    probs = np.zeros((B, K, 3), dtype=np.float64)
    results: List[Optional[ChainSequenceResult]] = [None] * B
    for b in (range(B) if seqs is None else seqs):
        kb = K if draft_len is None else int(draft_len[b])
        t_rows = widen_logits(target[b], dtype)
        if float(temperature[b]) == 0.0:
            r = verify_chain_greedy_sequence(t_rows, np.asarray(tokens)[b], kb)
        else:
            d_rows = None if draft is None else widen_logits(np.asarray(draft)[b], dtype)
            r = verify_chain_sequence(t_rows, d_rows, np.asarray(tokens)[b], kb, float(temperature[b]),
                                      np.asarray(u_accept)[b], float(u_final[b]))
        results[b] = r
        out_tok[b, : len(r.tokens)] = r.tokens
        out_n[b] = r.num_accepted
        for k in range(kb):
            probs[b, k] = (r.p_x[k], r.q_x[k], r.alpha[k])
    return ChainBatchResult(tokens=out_tok, num_accepted=out_n, probs=probs, sequences=results)
