"""Seeded workload recipes for batched draft-token verification.

Every random draw comes from ``numpy.random.Philox`` keyed by
``SeedSequence([seed, role, index])``: one independent stream per role
(target logits, draft noise, peak positions, draft sampling, accept uniforms,
final uniforms, tree shape, tree tokens, tree boosts, prompts) and per sequence
index, so any subset of sequences can be regenerated alone and generation can
run on several threads.

Logits are generated in float32.  bf16 inputs are the round-to-nearest-even
bf16 bit patterns of those float32 values, stored as ``uint16``; every consumer
(oracle and GPU) reads the identical bits.

Uniforms live on the grid ``(k + 1) * 2**-24`` for a 24-bit draw ``k``: the
interval (0, 1], exactly representable in float32 and float64 alike.

Draft tokens are drawn from the draft distribution with the Gumbel-max trick
(argmax of logits / T plus independent Gumbel noise), which samples the
temperature-scaled softmax exactly without evaluating it.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

_ROLES = {
    "target": 1,
    "draft_noise": 2,
    "peaks": 3,
    "draft_sample": 4,
    "u_accept": 5,
    "u_final": 6,
    "tree_shape": 7,
    "tree_tokens": 8,
    "tree_boost": 9,
    "prompt": 10,
    "ngram_target": 11,
    "draft_len": 12,
    "kv": 13,
    "commit": 14,
    "parents": 15,
}


def philox(seed: int, role: str, index: int = 0) -> np.random.Generator:
    """Independent Philox stream for (seed, role, index)."""
    return np.random.Generator(
        np.random.Philox(np.random.SeedSequence([int(seed), _ROLES[role], int(index)]))
    )


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (used here only to draw drafts)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def uniforms_open_closed(rng: np.random.Generator, shape) -> np.ndarray:
    """float32 uniforms on the grid (k + 1) * 2**-24, k uniform in [0, 2**24): the interval (0, 1]."""
    k = rng.integers(0, 1 << 24, size=shape, dtype=np.int64)
    return ((k + 1).astype(np.float64) * 2.0**-24).astype(np.float32)


def _gumbel_argmax(rng: np.random.Generator, logits_row: np.ndarray, temperature: float) -> int:
    """Sample an index with probability proportional to exp(logit / T) (Gumbel-max trick)."""
    u = rng.random(logits_row.shape[0])
    with np.errstate(divide="ignore"):
        g = -np.log(-np.log(u))
    return int(np.argmax(logits_row.astype(np.float64) / temperature + g))


def _threads(n_items: int, threads: Optional[int]) -> int:
    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    return max(1, min(threads, n_items))


def _parallel(fn, n_items: int, threads: Optional[int]):
    nt = _threads(n_items, threads)
    if nt == 1:
        return [fn(i) for i in range(n_items)]
    with ThreadPoolExecutor(nt) as ex:
        return list(ex.map(fn, range(n_items)))


# --------------------------------------------------------------------------------------
# Chain verification inputs
# --------------------------------------------------------------------------------------


@dataclass
class ChainInputs:
    """Inputs of one batched chain verification.

    target:  [B, K+1, V] float32, or uint16 bf16 bits when dtype == "bf16"
    draft:   [B, K, V] same dtype, or None (one-hot draft distribution)
    tokens:  [B, K] int32 draft tokens
    draft_len: [B] int32 in [0, K], or None (every sequence drafts K tokens)
    temperature: [B] float32 > 0
    u_accept: [B, K] float32 in (0, 1]
    u_final:  [B] float32 in (0, 1]
    """

    target: np.ndarray
    draft: Optional[np.ndarray]
    dtype: str
    tokens: np.ndarray
    draft_len: Optional[np.ndarray]
    temperature: np.ndarray
    u_accept: np.ndarray
    u_final: np.ndarray
    name: str = ""

    @property
    def B(self) -> int:
        return int(self.target.shape[0])

    @property
    def K(self) -> int:
        return int(self.tokens.shape[1])

    @property
    def V(self) -> int:
        return int(self.target.shape[2])

    def subset(self, idx) -> "ChainInputs":
        idx = np.asarray(idx)
        return ChainInputs(
            target=self.target[idx],
            draft=None if self.draft is None else self.draft[idx],
            dtype=self.dtype,
            tokens=self.tokens[idx],
            draft_len=None if self.draft_len is None else self.draft_len[idx],
            temperature=self.temperature[idx],
            u_accept=self.u_accept[idx],
            u_final=self.u_final[idx],
            name=self.name,
        )


def chain_inputs(
    seed: int,
    *,
    B: int,
    K: int,
    V: int,
    dtype: str,
    target_sigma: float,
    draft_sigma: float,
    temperature: float,
    peaks: int = 0,
    peak_shift: float = 0.0,
    name: str = "",
    threads: Optional[int] = None,
) -> ChainInputs:
    """Target rows N(0, target_sigma^2) (plus `peaks` distinct tokens per row shifted by
    `peak_shift`); draft rows = target + N(0, draft_sigma^2); draft token k ~ softmax(draft_k / T)."""
    if dtype not in ("f32", "bf16"):
        raise ValueError(dtype)
    store = np.uint16 if dtype == "bf16" else np.float32
    target = np.empty((B, K + 1, V), dtype=store)
    draft = np.empty((B, K, V), dtype=store)
    tokens = np.empty((B, K), dtype=np.int32)
    u_acc = np.empty((B, K), dtype=np.float32)
    u_fin = np.empty((B,), dtype=np.float32)

    def one(b: int) -> None:
        t = philox(seed, "target", b).standard_normal((K + 1, V), dtype=np.float32)
        t *= np.float32(target_sigma)
        if peaks:
            rp = philox(seed, "peaks", b)
            for r in range(K + 1):
                idx = rp.choice(V, size=min(peaks, V), replace=False)
                t[r, idx] += np.float32(peak_shift)
        d = philox(seed, "draft_noise", b).standard_normal((K, V), dtype=np.float32)
        d *= np.float32(draft_sigma)
        d += t[:K]
        if dtype == "bf16":
            target[b] = bf16_bits_from_f32(t)
            draft[b] = bf16_bits_from_f32(d)
            d_seen = f32_from_bf16_bits(draft[b])
        else:
            target[b] = t
            draft[b] = d
            d_seen = d
        rs = philox(seed, "draft_sample", b)
        for k in range(K):
            tokens[b, k] = _gumbel_argmax(rs, d_seen[k], temperature)
        u_acc[b] = uniforms_open_closed(philox(seed, "u_accept", b), (K,))
        u_fin[b] = uniforms_open_closed(philox(seed, "u_final", b), (1,))[0]

    _parallel(one, B, threads)
    return ChainInputs(
        target=target,
        draft=draft,
        dtype=dtype,
        tokens=tokens,
        draft_len=None,
        temperature=np.full((B,), temperature, dtype=np.float32),
        u_accept=u_acc,
        u_final=u_fin,
        name=name,
    )


def chain_shared_rows(seed: int, index: int, *, target: np.ndarray, draft: Optional[np.ndarray], dtype: str, B: int,
                      temperature: float, tokens: Optional[np.ndarray] = None, name: str = "") -> ChainInputs:
    """B sequences that all score the same rows (target [K+1, V] and draft [K, V], stored as
    `dtype`: float32 values or uint16 bf16 bits), each with its own fresh draws: draft
    tokens x_k ~ softmax(draft_k / T) by Gumbel-max over [B, K, V] at once (or, with
    draft None, the given one-hot tokens [K]) and fresh uniforms.  `index` selects an
    independent batch of draws, for statistics over many calls."""
    store = np.uint16 if dtype == "bf16" else np.float32
    target = np.asarray(target, dtype=store)
    K1, V = target.shape
    K = K1 - 1
    if draft is None:
        toks = np.broadcast_to(np.asarray(tokens, dtype=np.int32), (B, K)).copy()
    else:
        draft = np.asarray(draft, dtype=store)
        seen = f32_from_bf16_bits(draft) if dtype == "bf16" else draft
        u = philox(seed, "draft_sample", index).random((B, K, V))
        with np.errstate(divide="ignore"):
            g = -np.log(-np.log(u))
        toks = np.argmax(seen.astype(np.float64)[None] / temperature + g, axis=-1).astype(np.int32)
    return ChainInputs(
        target=np.broadcast_to(target, (B, K1, V)).copy(),
        draft=None if draft is None else np.broadcast_to(draft, (B, K, V)).copy(),
        dtype=dtype,
        tokens=toks,
        draft_len=None,
        temperature=np.full((B,), temperature, dtype=np.float32),
        u_accept=uniforms_open_closed(philox(seed, "u_accept", index), (B, K)),
        u_final=uniforms_open_closed(philox(seed, "u_final", index), (B,)),
        name=name,
    )


def chain_config_small_f32(seed: int = 0, B: int = 1, K: int = 5, V: int = 32000, **kw) -> ChainInputs:
    """Chain verify, fp32: target N(0, 2^2) per position, draft = target + N(0, 1), T = 1.0."""
    return chain_inputs(seed, B=B, K=K, V=V, dtype="f32", target_sigma=2.0, draft_sigma=1.0,
                        temperature=1.0, name=f"chain_f32_B{B}_K{K}_V{V}", **kw)


def chain_config_high_accept_bf16(seed: int = 0, B: int = 64, K: int = 5, V: int = 128256, **kw) -> ChainInputs:
    """Chain verify, bf16, high acceptance: target N(0, 3^2) with 20 peak tokens per row at +8,
    draft = target + N(0, 0.7^2), T = 0.8."""
    return chain_inputs(seed, B=B, K=K, V=V, dtype="bf16", target_sigma=3.0, draft_sigma=0.7,
                        temperature=0.8, peaks=20, peak_shift=8.0,
                        name=f"chain_bf16_hi_B{B}_K{K}_V{V}", **kw)


def chain_config_low_accept_bf16(seed: int = 0, B: int = 256, K: int = 8, V: int = 152064, **kw) -> ChainInputs:
    """Chain verify, bf16, low acceptance: target N(0, 2^2), draft = target + N(0, 3^2), T = 1.0."""
    return chain_inputs(seed, B=B, K=K, V=V, dtype="bf16", target_sigma=2.0, draft_sigma=3.0,
                        temperature=1.0, name=f"chain_bf16_lo_B{B}_K{K}_V{V}", **kw)


# --------------------------------------------------------------------------------------
# Greedy tree verification inputs
# --------------------------------------------------------------------------------------


@dataclass
class TreeInputs:
    """target: [B, N1, V] (row i = next-token logits after node i; row 0 = root);
    parent: [B, N1] int32 (parent[:, 0] = -1, parent[i] < i); node_token: [B, N1] int32."""

    target: np.ndarray
    dtype: str
    parent: np.ndarray
    node_token: np.ndarray
    max_depth: int
    name: str = ""

    @property
    def B(self) -> int:
        return int(self.target.shape[0])

    @property
    def N1(self) -> int:
        return int(self.target.shape[1])

    @property
    def V(self) -> int:
        return int(self.target.shape[2])


def _tree_shape(rng: np.random.Generator, n_nodes: int, depth: int, max_branch: int) -> np.ndarray:
    """Level-by-level budgeted construction: each node of the current frontier draws a
    branching factor in {1..max_branch}; a level's size is capped so that every later level
    can still hold one node, and the last level must absorb exactly the remaining budget.
    Shapes that cannot meet the budget are redrawn.  Returns parent[0..n_nodes] (BFS order)."""
    while True:
        parent = [-1]
        frontier = [0]
        remaining = n_nodes
        ok = True
        for level in range(1, depth + 1):
            levels_after = depth - level
            cap = remaining - levels_after
            new = []
            for node in frontier:
                if len(new) >= cap:
                    break
                br = int(rng.integers(1, max_branch + 1))
                br = min(br, cap - len(new))
                for _ in range(br):
                    parent.append(node)
                    new.append(len(parent) - 1)
            if level == depth and len(new) != remaining:
                ok = False
                break
            if not new:
                ok = False
                break
            remaining -= len(new)
            frontier = new
        if ok and remaining == 0:
            return np.asarray(parent, dtype=np.int32)


def tree_inputs(
    seed: int,
    *,
    B: int,
    n_nodes: int,
    depth: int,
    V: int,
    dtype: str = "bf16",
    sigma: float = 2.0,
    boost: float = 10.0,
    p_boost: float = 0.7,
    max_branch: int = 4,
    name: str = "",
    threads: Optional[int] = None,
) -> TreeInputs:
    """Random draft trees (n_nodes draft nodes + root, exactly `depth` levels); node tokens
    uniform over V; target rows N(0, sigma^2); for each node with children, with probability
    p_boost one child (chosen uniformly) has its token boosted by `boost` in that node's row."""
    N1 = n_nodes + 1
    store = np.uint16 if dtype == "bf16" else np.float32
    target = np.empty((B, N1, V), dtype=store)
    parent = np.empty((B, N1), dtype=np.int32)
    node_token = np.empty((B, N1), dtype=np.int32)

    def one(b: int) -> None:
        par = _tree_shape(philox(seed, "tree_shape", b), n_nodes, depth, max_branch)
        tok = philox(seed, "tree_tokens", b).integers(0, V, size=N1, dtype=np.int64).astype(np.int32)
        tok[0] = 0
        rows = philox(seed, "target", b).standard_normal((N1, V), dtype=np.float32)
        rows *= np.float32(sigma)
        rb = philox(seed, "tree_boost", b)
        children = [[] for _ in range(N1)]
        for i in range(1, N1):
            children[par[i]].append(i)
        for i in range(N1):
            hit = rb.random() < p_boost
            pick = int(rb.integers(0, max(1, len(children[i]))))
            if hit and children[i]:
                rows[i, tok[children[i][pick]]] += np.float32(boost)
        target[b] = bf16_bits_from_f32(rows) if dtype == "bf16" else rows
        parent[b] = par
        node_token[b] = tok

    _parallel(one, B, threads)
    return TreeInputs(target=target, dtype=dtype, parent=parent, node_token=node_token,
                      max_depth=depth, name=name or f"tree_{dtype}_B{B}_N{n_nodes}_V{V}")


def tree_config_eagle_bf16(seed: int = 0, B: int = 32, n_nodes: int = 60, depth: int = 6,
                           V: int = 128256, **kw) -> TreeInputs:
    """Greedy tree verify, bf16: 60-node trees of depth 6, branching {1..4}, rows N(0, 2^2),
    matching child token +10 with probability 0.7 per node."""
    return tree_inputs(seed, B=B, n_nodes=n_nodes, depth=depth, V=V, dtype="bf16", sigma=2.0,
                       boost=10.0, p_boost=0.7, **kw)


@dataclass
class SampledTreeInputs:
    """target, draft: [B, N1, V] (row i = logits after node i; draft row i is the
    distribution node i's children were drawn from); parent, node_token [B, N1] int32;
    temperature [B]; u_accept [B, N1]; u_final [B]."""

    target: np.ndarray
    draft: np.ndarray
    dtype: str
    parent: np.ndarray
    node_token: np.ndarray
    temperature: np.ndarray
    u_accept: np.ndarray
    u_final: np.ndarray
    max_depth: int
    name: str = ""

    @property
    def B(self) -> int:
        return int(self.target.shape[0])

    @property
    def N1(self) -> int:
        return int(self.target.shape[1])

    @property
    def V(self) -> int:
        return int(self.target.shape[2])


def tree_sampled_inputs(seed: int, *, B: int, n_nodes: int, depth: int, V: int, dtype: str = "bf16",
                        target_sigma: float = 3.0, draft_sigma: float = 0.7, temperature: float = 0.8,
                        peaks: int = 20, peak_shift: float = 8.0, max_branch: int = 4, parent=None,
                        name: str = "", threads: Optional[int] = None) -> SampledTreeInputs:
    """Random draft trees (the shapes of tree_inputs unless `parent` is given); target rows
    N(0, target_sigma^2) with `peaks` tokens per row shifted by `peak_shift`; draft rows =
    target + N(0, draft_sigma^2); the children of every node drawn independently from
    softmax(draft row / T) of that node (Gumbel-max on the stored values)."""
    store = np.uint16 if dtype == "bf16" else np.float32
    if parent is None:
        parent = np.stack([_tree_shape(philox(seed, "tree_shape", b), n_nodes, depth, max_branch) for b in range(B)])
    parent = np.asarray(parent, dtype=np.int32)
    N1 = parent.shape[1]
    target = np.empty((B, N1, V), dtype=store)
    draft = np.empty((B, N1, V), dtype=store)
    node_token = np.zeros((B, N1), dtype=np.int32)
    u_acc = np.empty((B, N1), dtype=np.float32)
    u_fin = np.empty((B,), dtype=np.float32)

    def one(b: int) -> None:
        t = philox(seed, "target", b).standard_normal((N1, V), dtype=np.float32)
        t *= np.float32(target_sigma)
        if peaks:
            rp = philox(seed, "peaks", b)
            for r in range(N1):
                idx = rp.choice(V, size=min(peaks, V), replace=False)
                t[r, idx] += np.float32(peak_shift)
        d = philox(seed, "draft_noise", b).standard_normal((N1, V), dtype=np.float32)
        d *= np.float32(draft_sigma)
        d += t
        if dtype == "bf16":
            target[b] = bf16_bits_from_f32(t)
            draft[b] = bf16_bits_from_f32(d)
            d_seen = f32_from_bf16_bits(draft[b])
        else:
            target[b] = t
            draft[b] = d
            d_seen = d
        rs = philox(seed, "draft_sample", b)
        for i in range(1, N1):
            node_token[b, i] = _gumbel_argmax(rs, d_seen[parent[b, i]], temperature)
        u_acc[b] = uniforms_open_closed(philox(seed, "u_accept", b), (N1,))
        u_fin[b] = uniforms_open_closed(philox(seed, "u_final", b), (1,))[0]

    _parallel(one, B, threads)
    return SampledTreeInputs(target=target, draft=draft, dtype=dtype, parent=parent, node_token=node_token,
                             temperature=np.full((B,), temperature, dtype=np.float32), u_accept=u_acc,
                             u_final=u_fin, max_depth=depth,
                             name=name or f"tree_sampled_{dtype}_B{B}_N{N1 - 1}_V{V}")


def tree_sampled_config_bf16(seed: int = 0, B: int = 32, n_nodes: int = 60, depth: int = 6, V: int = 128256,
                             **kw) -> SampledTreeInputs:
    """Stochastic tree verify, bf16: the greedy workload's tree shapes (60 nodes, depth 6,
    branching {1..4}) with the high-acceptance chain recipe per node (target N(0, 3^2) +
    20 peaks at +8, draft = target + N(0, 0.7^2), T = 0.8); children drawn from q."""
    return tree_sampled_inputs(seed, B=B, n_nodes=n_nodes, depth=depth, V=V, dtype="bf16", **kw)


def tree_parents(seed: int = 0, *, B: int = 32, n_nodes: int = 60, depth: int = 6, max_branch: int = 4) -> np.ndarray:
    """The topologies of tree_inputs(seed, ...) alone: parent [B, n_nodes + 1] int32."""
    return np.stack([_tree_shape(philox(seed, "tree_shape", b), n_nodes, depth, max_branch) for b in range(B)])


def random_parents(seed: int, *, B: int, N1: int, kind: str = "mixed", window: int = 8) -> np.ndarray:
    """Parents-first trees of N1 nodes: "random" (parent of i uniform over the `window`
    nodes before it), "chain" (parent i - 1), "star" (every parent the root), or "mixed"
    (one of the three per sequence).  Returns parent [B, N1] int32."""
    out = np.empty((B, N1), dtype=np.int32)
    for b in range(B):
        rng = philox(seed, "parents", b)
        k = kind if kind != "mixed" else ("random", "chain", "star")[int(rng.integers(0, 3))]
        par = np.empty(N1, dtype=np.int64)
        par[0] = -1
        idx = np.arange(1, N1)
        if k == "chain":
            par[1:] = idx - 1
        elif k == "star":
            par[1:] = 0
        else:
            lo = np.maximum(0, idx - window)
            par[1:] = lo + (rng.random(N1 - 1) * (idx - lo)).astype(np.int64)
        out[b] = par
    return out


def kv_entries(seed: int, *, planes: int, B: int, rows: int, W: int) -> np.ndarray:
    """Random 16-bit cache entries [planes, B, rows, W] (uint16 bit patterns)."""
    out = np.empty((planes, B, rows, W), dtype=np.uint16)

    def one(b: int) -> None:
        out[:, b] = philox(seed, "kv", b).integers(0, 1 << 16, size=(planes, rows, W), dtype=np.uint16)

    _parallel(one, B, None)
    return out


def commit_requests(seed: int, *, B: int, N1: int, P: int, L_cap: int):
    """Random commit inputs: accept_len [B] in [0, min(P, N1 - 1)], path [B, P] of that
    many distinct nodes in [1, N1) in increasing order (-1 padded), cache_len [B] with
    room for the commit.  Returns (accept_len, path, cache_len) as int32 arrays."""
    acc = np.zeros(B, dtype=np.int32)
    path = np.full((B, P), -1, dtype=np.int32)
    clen = np.zeros(B, dtype=np.int32)
    top = min(P, N1 - 1)
    for b in range(B):
        rng = philox(seed, "commit", b)
        n = int(rng.integers(0, top + 1))
        acc[b] = n
        path[b, :n] = np.sort(rng.choice(np.arange(1, N1), size=n, replace=False))
        clen[b] = int(rng.integers(0, L_cap - n))
    return acc, path, clen


# --------------------------------------------------------------------------------------
# n-gram prompt lookup inputs
# --------------------------------------------------------------------------------------


@dataclass
class NgramPrompts:
    context: np.ndarray      # [B, L_max] int32
    context_len: np.ndarray  # [B] int32


def _zipf_cdf(V: int, s: float) -> np.ndarray:
    ranks = np.arange(1, V + 1, dtype=np.float64)
    w = ranks ** (-s)
    c = np.cumsum(w)
    return c / c[-1]


def ngram_prompts(seed: int, *, B: int, L: int, V: int, zipf_s: float = 1.1, p_copy: float = 0.1,
                  span_lo: int = 16, span_hi: int = 64, lengths: Optional[np.ndarray] = None,
                  threads: Optional[int] = None) -> NgramPrompts:
    """Prompts built from spans of U{span_lo..span_hi} tokens: each span is, with probability
    p_copy, a copy of an earlier segment of the same length, otherwise i.i.d. tokens whose
    rank follows a Zipf(zipf_s) law bounded to V (token id = rank - 1)."""
    cdf = _zipf_cdf(V, zipf_s)
    ctx = np.zeros((B, L), dtype=np.int32)
    lens = np.full((B,), L, dtype=np.int32) if lengths is None else np.asarray(lengths, dtype=np.int32)

    def one(b: int) -> None:
        rng = philox(seed, "prompt", b)
        n = int(lens[b])
        pos = 0
        while pos < n:
            span = min(int(rng.integers(span_lo, span_hi + 1)), n - pos)
            copy = rng.random() < p_copy
            if copy and pos >= span:
                src = int(rng.integers(0, pos - span + 1))
                ctx[b, pos:pos + span] = ctx[b, src:src + span]
            else:
                ctx[b, pos:pos + span] = np.searchsorted(cdf, rng.random(span), side="right").astype(np.int32)
            pos += span
        np.clip(ctx[b], 0, V - 1, out=ctx[b])

    _parallel(one, B, threads)
    return NgramPrompts(context=ctx, context_len=lens)


def ngram_config_prompts(seed: int = 0, B: int = 128, L: int = 4096, V: int = 32000, **kw) -> NgramPrompts:
    """n-gram prompt lookup workload: 4096-token Zipf(1.1) prompts over V = 32000 with 10 % copied spans."""
    return ngram_prompts(seed, B=B, L=L, V=V, **kw)


def ngram_target_inputs(seed: int, proposals: np.ndarray, draft_len: np.ndarray, *, V: int,
                        sigma: float = 2.0, boost: float = 6.0, temperature: float = 1.0,
                        dtype: str = "bf16", threads: Optional[int] = None) -> ChainInputs:
    """Target logits for verifying n-gram proposals: rows N(0, sigma^2), with proposal k boosted
    by `boost` in row k.  The proposals are an input here (whoever computed them)."""
    proposals = np.asarray(proposals, dtype=np.int32)
    draft_len = np.asarray(draft_len, dtype=np.int32)
    B, K = proposals.shape
    store = np.uint16 if dtype == "bf16" else np.float32
    target = np.empty((B, K + 1, V), dtype=store)
    u_acc = np.empty((B, K), dtype=np.float32)
    u_fin = np.empty((B,), dtype=np.float32)

    def one(b: int) -> None:
        t = philox(seed, "ngram_target", b).standard_normal((K + 1, V), dtype=np.float32)
        t *= np.float32(sigma)
        for k in range(int(draft_len[b])):
            t[k, proposals[b, k]] += np.float32(boost)
        target[b] = bf16_bits_from_f32(t) if dtype == "bf16" else t
        u_acc[b] = uniforms_open_closed(philox(seed, "u_accept", b), (K,))
        u_fin[b] = uniforms_open_closed(philox(seed, "u_final", b), (1,))[0]

    _parallel(one, B, threads)
    return ChainInputs(target=target, draft=None, dtype=dtype, tokens=proposals.copy(), draft_len=draft_len.copy(),
                       temperature=np.full((B,), temperature, dtype=np.float32), u_accept=u_acc,
                       u_final=u_fin, name=f"ngram_verify_{dtype}_B{B}_K{K}_V{V}")
