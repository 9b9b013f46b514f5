"""The steps on either side of tree verification -- oracle (TEST INFRASTRUCTURE ONLY).

Before verification the draft tree is flattened into one sequence and scored in a
single target pass under a two-dimensional mask; after it, the cache entries of the
accepted path are committed.

Pages:
  * "Speculative Decoding in Production: From Draft Models to EAGLE-3 Dynamic Trees
    for 3x-5x Lossless Acceleration" (blog.llmgo.top), section III.2 "The Tree
    Attention Verification Mechanism": the candidate tree becomes one concatenated
    sequence and a 2-D mask lets the target verify every branch in one pass.
  * "Speculative decoding: Medusa, EAGLE, vLLM" (vikram-blog.pages.dev), "System
    Topology & Data Flow": the tokens of the accepted branch go into the KV cache.

Readings taken where the pages are silent:
  * Node order is parents first (parent[0] = -1, 0 <= parent[i] < i), as in the
    verification step.  mask[i, j] = 1 iff node j is on the path from the root to
    node i, node i itself included; depth[i] = number of edges from the root.  A tree
    that breaks the order gets an all-zero mask and depth -1 for every node.
  * The one pass covers the root (the token emitted by the previous step) and every
    node, so it yields one cache entry per node.  Committing writes the root's entry
    to cache position cache_len and, for k = 1..n with n = accept_len, the entry of
    the k-th accepted node (path_nodes[k - 1]: the accepted nodes from the root
    side, root excluded, as verification reports them) to cache_len + k; the new
    length is cache_len + n + 1.  The token emitted after the path has no entry yet:
    it is the next step's root.
  * Without path_nodes the accepted nodes are 1, ..., n (chain verification).
  * A sequence with accept_len < 0 (flagged invalid by verification), a path node
    outside [0, N1), n beyond the path row, or a commit that would pass the cache
    capacity writes nothing and reports new length -1.
"""

from __future__ import annotations

import numpy as np


def _ordered(parent):
    """True iff parent lists a rooted tree parents first."""
    if len(parent) == 0 or int(parent[0]) != -1:
        return False
    return all(0 <= int(parent[i]) < i for i in range(1, len(parent)))


def tree_attention_mask_sequence(parent):
    """(mask [N1, N1] uint8, depth [N1] int32) of one tree: walk each node up to the root."""
    parent = np.asarray(parent)
    N1 = parent.shape[0]
    mask = np.zeros((N1, N1), dtype=np.uint8)
    depth = np.full(N1, -1, dtype=np.int32)
    if not _ordered(parent):
        return mask, depth
    for i in range(N1):
        v, d = i, 0
        mask[i, v] = 1
        while v != 0:
            v = int(parent[v])
            mask[i, v] = 1
            d += 1
        depth[i] = d
    return mask, depth


def tree_attention_mask(parent):
    """Batched: parent [B, N1] -> (mask [B, N1, N1] uint8, depth [B, N1] int32)."""
    parent = np.asarray(parent)
    B, N1 = parent.shape
    mask = np.zeros((B, N1, N1), dtype=np.uint8)
    depth = np.zeros((B, N1), dtype=np.int32)
    for b in range(B):
        mask[b], depth[b] = tree_attention_mask_sequence(parent[b])
    return mask, depth


def commit_path(kv_nodes, path_nodes, accept_len, cache_len, kv_cache):
    """Commit the accepted path's entries; returns the new cache lengths [B] int32.

    kv_nodes [planes, B, N1, W] and kv_cache [planes, B, L_cap, W] (any dtype, the
    entry is W elements of it); kv_cache is updated in place.  path_nodes [B, P]
    holds the accepted nodes from the root side, root excluded (-1 padded), or is
    None for the chain reading.
    """
    planes, B, N1, _ = kv_nodes.shape
    L_cap = kv_cache.shape[2]
    new_len = np.full(B, -1, dtype=np.int32)
    for b in range(B):
        n = int(accept_len[b])
        start = int(cache_len[b])
        if n < 0 or start < 0 or start + n + 1 > L_cap:
            continue
        if path_nodes is None:
            nodes = list(range(n + 1))
        else:
            row = path_nodes[b]
            if n > len(row):
                continue
            nodes = [0] + [int(row[k]) for k in range(n)]
        if any(not 0 <= v < N1 for v in nodes):
            continue
        for k, v in enumerate(nodes):
            kv_cache[:, b, start + k, :] = kv_nodes[:, b, v, :]
        new_len[b] = start + n + 1
    return new_len
