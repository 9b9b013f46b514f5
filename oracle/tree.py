"""Greedy tree verification -- the oracle (test infrastructure only).

Method: "Speculative Decoding in Production: From Draft Models to EAGLE-3 Dynamic
Trees ..." (blog.llmgo.top), section III.2 "The Tree Attention Verification
Mechanism": all branches of the flattened draft tree are scored in one target
pass, and a branch whose tokens match is accepted even when a sibling branch is
rejected.  "Speculative decoding: Medusa, EAGLE, vLLM" (vikram-blog.pages.dev),
"System Topology & Data Flow" figure: branch [t1, t2, t3] accepted (3 tokens),
sibling [t1, t2', t4] rejected; its usage example runs at temperature 0 (greedy).

Readings taken where the pages are silent:
  * Row i of the target logits is the next-token distribution after the path
    root -> node i; row 0 belongs to the root (the last committed token).
  * Greedy matching: node i is accepted iff its parent is accepted and its token
    equals the argmax of the parent's row; argmax ties go to the smallest
    vocabulary index; raw logits are compared (temperature cannot change an argmax).
  * The accepted path ends at the deepest accepted node (smallest node index on
    ties); its tokens are emitted root-first, then the argmax of that node's row
    as the bonus token.
  * Nodes are listed parents-first: parent[0] = -1 and 0 <= parent[i] < i.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List

import numpy as np

from .common import widen_logits


def argmax_first(row: np.ndarray) -> int:
    """Index of the largest value; the smallest such index when several are equal."""
    return int(np.argmax(row))


@dataclass
class TreeSequenceResult:
    accept_len: int
    tokens: List[int]      # path tokens root-first (root excluded), then the bonus token
    path_nodes: List[int]  # node indices root-first (root excluded)
    argmax: List[int]      # per-node row argmax
    accepted: List[bool]


def verify_tree_greedy_sequence(rows: np.ndarray, parent: np.ndarray, node_token: np.ndarray,
                                max_depth: int) -> TreeSequenceResult:
    N1, V = rows.shape
    if int(parent[0]) != -1:
        raise ValueError("parent[0] must be -1 (the root)")
    for i in range(1, N1):
        if not 0 <= int(parent[i]) < i:
            raise ValueError("nodes must be listed parents-first")
        if not 0 <= int(node_token[i]) < V:
            raise ValueError("node token out of range")
    amax = [argmax_first(rows[i]) for i in range(N1)]
    accepted = [False] * N1
    depth = [0] * N1
    accepted[0] = True
    for i in range(1, N1):
        par = int(parent[i])
        depth[i] = depth[par] + 1
        accepted[i] = accepted[par] and int(node_token[i]) == amax[par]
    best = 0
    for i in range(1, N1):
        if accepted[i] and depth[i] > depth[best]:
            best = i
    if depth[best] > max_depth:
        raise ValueError("accepted path deeper than max_depth")
    path = []
    v = best
    while v != 0:
        path.append(v)
        v = int(parent[v])
    path.reverse()
    toks = [int(node_token[v]) for v in path] + [amax[best]]
    return TreeSequenceResult(accept_len=depth[best], tokens=toks, path_nodes=path, argmax=amax,
                              accepted=accepted)


@dataclass
class TreeBatchResult:
    accept_len: np.ndarray  # [B]
    tokens: np.ndarray      # [B, max_depth + 1], -1 padded
    path_nodes: np.ndarray  # [B, max_depth + 1], -1 padded
    argmax: np.ndarray      # [B, N1]
    sequences: list


def verify_tree_greedy(target, dtype: str, parent, node_token, max_depth: int, seqs=None) -> TreeBatchResult:
    target = np.asarray(target)
    B, N1, V = target.shape
    acc = np.zeros((B,), dtype=np.int32)
    tok = np.full((B, max_depth + 1), -1, dtype=np.int32)
    nodes = np.full((B, max_depth + 1), -1, dtype=np.int32)
    amax = np.zeros((B, N1), dtype=np.int32)
    res = [None] * B
    for b in (range(B) if seqs is None else seqs):
        r = verify_tree_greedy_sequence(widen_logits(target[b], dtype), np.asarray(parent)[b],
                                        np.asarray(node_token)[b], max_depth)
        res[b] = r
        acc[b] = r.accept_len
        tok[b, : len(r.tokens)] = r.tokens
        nodes[b, : len(r.path_nodes)] = r.path_nodes
        amax[b] = r.argmax
    return TreeBatchResult(accept_len=acc, tokens=tok, path_nodes=nodes, argmax=amax, sequences=res)
