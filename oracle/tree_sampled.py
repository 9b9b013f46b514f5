"""Stochastic (temperature > 0) tree verification -- oracle (TEST INFRASTRUCTURE ONLY).

The pages verify drafted trees ("Speculative Decoding in Production ..." (blog.llmgo.top),
section III.2: a rejected branch B1 and an accepted sibling B2) and sample at temperature
above zero, but state the acceptance rule only for a chain (section I.1: accept x with
probability min(1, p(x)/q(x)), else draw from max(0, p - q) normalised).  Reading, taken
from the published multi-candidate form of that rule (SpecInfer's multi-step speculative
sampling): the children of a node were drawn independently from the draft distribution
q at that node, and are tried in node-index order against a residual target r:

    r_1 = p (the target distribution at the node)
    child j with token x: accept with probability min(1, r_j(x) / q(x));
        accepted -> move to the child and repeat there with its own p and q;
        rejected -> r_{j+1} = max(0, r_j - q) normalised
    every child rejected -> emit a token drawn from r_{m+1}; stop
    a node without children (reached by acceptance) -> emit a bonus token from its p; stop

so a chain-shaped tree is exactly chain verification, and marginalising over the
children's draws and the accept tests recovers p (checked by exact enumeration).

Further readings, shared with chain verification: p = softmax(target / T) and
q = softmax(draft / T) of the node's rows; u_accept[i] is the uniform of the test of
node i; the final draw uses u_final with the inclusive inverse-CDF convention;
q(x) = 0 gives alpha = 1 if r(x) > 0 else 0; a residual with no mass left keeps the
previous r (unreachable in exact arithmetic when the children were drawn from q).
Temperature must be > 0 (temperature 0 is greedy tree verification).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .chain import acceptance_probability, accept_test, inverse_cdf_sample, residual_weights, softmax_at_temperature
from .common import widen_logits


@dataclass
class SampledTreeResult:
    accept_len: int
    path_nodes: List[int]            # accepted nodes from the root side, root excluded
    tokens: List[int]                # their tokens, then the emitted token
    tests: List[tuple] = field(default_factory=list)  # (node, alpha, accepted) in the order decided
    accept_margins: List[float] = field(default_factory=list)
    final_weights: Optional[np.ndarray] = None
    cdf_gap: float = float("inf")
    mode: str = ""                   # "residual", "bonus", "residual_zero_fallback" or "invalid"


def _children(parent):
    kids = [[] for _ in range(len(parent))]
    for i in range(1, len(parent)):
        kids[int(parent[i])].append(i)
    return kids


def verify_tree_sampled_sequence(target_rows, draft_rows, parent, node_token, temperature, u_accept, u_final,
                                 max_depth) -> SampledTreeResult:
    """One tree.  target_rows, draft_rows: [N1, V] float64 logits (draft row i is the draft
    distribution that node i's children were drawn from; leaves' draft rows are unused)."""
    N1, V = target_rows.shape
    invalid = SampledTreeResult(accept_len=-1, path_nodes=[], tokens=[], mode="invalid")
    if int(parent[0]) != -1 or any(not 0 <= int(parent[i]) < i for i in range(1, N1)):
        return invalid
    if any(not 0 <= int(node_token[i]) < V for i in range(1, N1)):
        return invalid
    if not (temperature > 0.0 and np.isfinite(temperature)):
        return invalid
    if any(not 0.0 < float(u_accept[i]) <= 1.0 for i in range(1, N1)) or not 0.0 < float(u_final) <= 1.0:
        return invalid
    kids = _children(parent)
    res = SampledTreeResult(accept_len=0, path_nodes=[], tokens=[])
    cur = 0
    while True:
        p = softmax_at_temperature(target_rows[cur], temperature)
        if not kids[cur]:
            w, res.mode = p, "bonus"
            break
        q = softmax_at_temperature(draft_rows[cur], temperature)
        r = p
        moved = fell_back = False
        for c in kids[cur]:
            x = int(node_token[c])
            alpha = acceptance_probability(float(r[x]), float(q[x]))
            ok = accept_test(float(u_accept[c]), alpha)
            res.tests.append((c, alpha, ok))
            res.accept_margins.append(abs(float(u_accept[c]) - alpha))
            if ok:
                res.path_nodes.append(c)
                res.tokens.append(x)
                cur = c
                moved = True
                break
            nxt = residual_weights(r, q)
            mass = float(np.sum(nxt))
            if mass > 0.0:
                r = nxt / mass
            else:
                fell_back = True
        if not moved:
            w = r
            res.mode = "residual_zero_fallback" if fell_back else "residual"
            break
    if len(res.path_nodes) > max_depth:
        return invalid
    y, gap, _ = inverse_cdf_sample(w, float(u_final))
    res.accept_len = len(res.path_nodes)
    res.tokens.append(int(y))
    res.final_weights = np.asarray(w, dtype=np.float64)
    res.cdf_gap = gap
    return res


@dataclass
class SampledTreeBatchResult:
    accept_len: np.ndarray   # [B] int32 (-1 = invalid input)
    tokens: np.ndarray       # [B, max_depth + 1] int32, -1 padded
    path_nodes: np.ndarray   # [B, max_depth + 1] int32, -1 padded
    sequences: list


def verify_tree_sampled(target, draft, dtype: str, parent, node_token, temperature, u_accept, u_final,
                        max_depth: int, seqs=None) -> SampledTreeBatchResult:
    """Batched: target, draft [B, N1, V] (float32 or bf16 bits), parent and node_token [B, N1],
    temperature [B], u_accept [B, N1], u_final [B]."""
    target = np.asarray(target)
    B, N1, V = target.shape
    D1 = max_depth + 1
    acc = np.zeros(B, dtype=np.int32)
    tok = np.full((B, D1), -1, dtype=np.int32)
    nodes = np.full((B, D1), -1, dtype=np.int32)
    out = [None] * B
    for b in (range(B) if seqs is None else seqs):
        r = verify_tree_sampled_sequence(widen_logits(target[b], dtype), widen_logits(np.asarray(draft)[b], dtype),
                                         np.asarray(parent)[b], np.asarray(node_token)[b], float(temperature[b]),
                                         np.asarray(u_accept)[b], float(u_final[b]), max_depth)
        out[b] = r
        acc[b] = r.accept_len
        if r.accept_len >= 0:
            tok[b, : len(r.tokens)] = r.tokens
            nodes[b, : len(r.path_nodes)] = r.path_nodes
    return SampledTreeBatchResult(accept_len=acc, tokens=tok, path_nodes=nodes, sequences=out)
