"""Pins of the tree-attention mask and path-commit oracle (CPU only).

Mask: the pages' draft-tree figure (golden), the causal mask of a chain and the
star tree (closed forms), the reflexive-transitive closure of the parent relation
computed by boolean matrix products (a different computation from the oracle's
walk), and the row recursion row(i) = row(parent(i)) + e_i.
Commit: the pages' accepted-branch figure run through greedy verification then
the commit (golden), entries that carry their node index, untouched cache rows,
and each invalid case.  Planted mistakes at the end must each fail a pin.
"""

import json
import os

import numpy as np
import pytest

import oracle
import oracle.tree_io as tio

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _fixture(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def random_tree(rng, N1, kind="random"):
    if N1 == 1:
        return np.array([-1])
    if kind == "chain":
        return np.arange(-1, N1 - 1)
    if kind == "star":
        return np.concatenate([[-1], np.zeros(N1 - 1, dtype=np.int64)])
    par = [-1] + [int(rng.integers(max(0, i - 4), i)) for i in range(1, N1)]
    return np.asarray(par)


def closure_mask(parent):
    """Reflexive-transitive closure of child -> parent by repeated boolean products."""
    N1 = len(parent)
    A = np.zeros((N1, N1), dtype=np.int64)
    for i in range(1, N1):
        A[i, parent[i]] = 1
    M = np.eye(N1, dtype=np.int64)
    for _ in range(N1):
        M = ((M + M @ A) > 0).astype(np.int64)
    return M.astype(np.uint8)


# ------------------------------------------------------------------ mask pins
def check_mask_pins(fn, parent):
    mask, depth = fn(parent)
    N1 = len(parent)
    np.testing.assert_array_equal(mask, closure_mask(parent))
    np.testing.assert_array_equal(mask.sum(axis=1), depth + 1)
    assert depth[0] == 0
    for i in range(1, N1):
        expect = mask[parent[i]].copy()
        expect[i] = 1
        np.testing.assert_array_equal(mask[i], expect)
        assert depth[i] == depth[parent[i]] + 1


def test_mask_golden_figure():
    fx = _fixture("tree_mask_draft_tree_figure.json")
    assert fx["source"] and fx["derivation"]
    mask, depth = oracle.tree_attention_mask(np.asarray([fx["parent"]]))
    np.testing.assert_array_equal(mask[0], np.asarray(fx["expected"]["mask"], dtype=np.uint8))
    np.testing.assert_array_equal(depth[0], fx["expected"]["depth"])


@pytest.mark.parametrize("N1", [1, 2, 7, 33])
def test_mask_chain_is_causal(N1):
    mask, depth = tio.tree_attention_mask_sequence(np.arange(-1, N1 - 1))
    np.testing.assert_array_equal(mask, np.tril(np.ones((N1, N1), dtype=np.uint8)))
    np.testing.assert_array_equal(depth, np.arange(N1))


@pytest.mark.parametrize("N1", [2, 9, 40])
def test_mask_star_sees_root_and_self(N1):
    mask, depth = tio.tree_attention_mask_sequence(random_tree(None, N1, "star"))
    expect = np.eye(N1, dtype=np.uint8)
    expect[:, 0] = 1
    np.testing.assert_array_equal(mask, expect)
    np.testing.assert_array_equal(depth, [0] + [1] * (N1 - 1))


@pytest.mark.parametrize("seed", range(6))
def test_mask_random_trees_match_closure(seed):
    rng = np.random.default_rng(seed)
    for N1 in (3, 17, 64):
        check_mask_pins(tio.tree_attention_mask_sequence, random_tree(rng, N1))


@pytest.mark.parametrize("parent", [[0, 0, 1], [-1, 1, 1], [-1, 0, 3, 1], [-1, -1, 0], [-1, 0, 2]])
def test_mask_bad_topology_is_zero(parent):
    mask, depth = tio.tree_attention_mask_sequence(np.asarray(parent))
    assert not mask.any()
    assert (depth == -1).all()


# ---------------------------------------------------------------- commit pins
def entries_with_ids(planes, B, N1, W):
    """kv_nodes[p, b, i, :] encodes (p, b, i) so every copied entry names its source."""
    kv = np.zeros((planes, B, N1, W), dtype=np.int64)
    for p in range(planes):
        for b in range(B):
            for i in range(N1):
                kv[p, b, i, :] = ((p * 1000 + b) * 1000 + i) * 10 + np.arange(W) % 10
    return kv


def test_commit_golden_branch_a():
    fx = _fixture("tree_commit_branch_a.json")
    assert fx["source"] and fx["derivation"]
    rows = np.zeros((len(fx["parent"]), fx["V"]), dtype=np.float32)
    for i, a in enumerate(fx["row_argmax"]):
        rows[i, a] = 5.0
    res = oracle.verify_tree_greedy(rows[None], "f32", np.asarray([fx["parent"]]),
                                    np.asarray([fx["node_token"]]), fx["max_depth"])
    exp = fx["expected"]
    assert int(res.accept_len[0]) == exp["accept_len"]
    assert res.path_nodes[0].tolist() == exp["path_nodes"]
    assert res.tokens[0].tolist() == exp["emitted"]
    # the cache entry of node i is its token, so the cache reads the committed tokens
    kv = np.asarray(fx["node_token"], dtype=np.int64).reshape(1, 1, -1, 1)
    cache = np.full((1, 1, fx["L_cap"], 1), -7, dtype=np.int64)
    new_len = oracle.commit_path(kv, res.path_nodes, res.accept_len, np.asarray([fx["cache_len"]]), cache)
    assert new_len.tolist() == [exp["new_cache_len"]]
    c0 = fx["cache_len"]
    assert cache[0, 0, c0: exp["new_cache_len"], 0].tolist() == exp["cache_tokens"]
    assert (cache[0, 0, :c0] == -7).all() and (cache[0, 0, exp["new_cache_len"]:] == -7).all()


def check_commit_pins(fn, seed):
    rng = np.random.default_rng(seed)
    planes, B, N1, W, L_cap, P = 3, 6, 12, 5, 20, 6
    kv = entries_with_ids(planes, B, N1, W)
    path = np.full((B, P), -1, dtype=np.int64)
    acc = np.zeros(B, dtype=np.int64)
    for b in range(B):
        n = int(rng.integers(0, P + 1))
        acc[b] = n
        path[b, :n] = np.sort(rng.choice(np.arange(1, N1), size=n, replace=False))
    cache_len = rng.integers(0, L_cap - P, size=B)
    cache = np.full((planes, B, L_cap, W), -1, dtype=np.int64)
    new_len = fn(kv, path, acc, cache_len, cache)
    for b in range(B):
        n, c0 = int(acc[b]), int(cache_len[b])
        assert new_len[b] == c0 + n + 1
        nodes = [0] + path[b, :n].tolist()
        for k, v in enumerate(nodes):
            for p in range(planes):
                got = cache[p, b, c0 + k]
                assert (got // 10 == (p * 1000 + b) * 1000 + v).all()
                assert (got % 10 == np.arange(W) % 10).all()
        assert (cache[:, b, :c0] == -1).all() and (cache[:, b, c0 + n + 1:] == -1).all()


@pytest.mark.parametrize("seed", range(4))
def test_commit_copies_root_then_path(seed):
    check_commit_pins(oracle.commit_path, seed)


def test_commit_chain_reading_is_identity_path():
    kv = entries_with_ids(2, 3, 6, 4)
    acc = np.array([0, 5, 2])
    cl = np.array([0, 3, 9])
    a = np.full((2, 3, 16, 4), -1)
    b = a.copy()
    la = oracle.commit_path(kv, None, acc, cl, a)
    path = np.tile(np.arange(1, 6), (3, 1))
    lb = oracle.commit_path(kv, path, acc, cl, b)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


@pytest.mark.parametrize("acc,cl,path", [
    (-1, 0, [1, 2, -1]),   # verification flagged the sequence invalid
    (2, 14, [1, 2, -1]),   # 14 + 3 > capacity 16
    (2, -1, [1, 2, -1]),   # negative cache length
    (2, 0, [1, 6, -1]),    # node out of range (N1 = 6)
    (4, 0, [1, 2, 3]),     # more accepted nodes than the path row holds
])
def test_commit_invalid_writes_nothing(acc, cl, path):
    kv = entries_with_ids(1, 1, 6, 4)
    cache = np.full((1, 1, 16, 4), -1)
    new_len = oracle.commit_path(kv, np.asarray([path]), np.asarray([acc]), np.asarray([cl]), cache)
    assert new_len.tolist() == [-1]
    assert (cache == -1).all()


# ------------------------------------------------------------ planted mistakes
def _mask_without_self(parent):
    m, d = tio.tree_attention_mask_sequence(parent)
    m = m.copy()
    np.fill_diagonal(m, 0)
    return m, d


def _mask_without_root(parent):
    m, d = tio.tree_attention_mask_sequence(parent)
    m = m.copy()
    m[1:, 0] = 0
    return m, d - 1 * (np.arange(len(d)) > 0)


def _mask_transposed(parent):
    m, d = tio.tree_attention_mask_sequence(parent)
    return m.T.copy(), d


def _mask_parent_only(parent):
    m = np.eye(len(parent), dtype=np.uint8)
    for i in range(1, len(parent)):
        m[i, parent[i]] = 1
    return m, np.asarray([0] + [1] * (len(parent) - 1))


@pytest.mark.parametrize("mutant", [_mask_without_self, _mask_without_root, _mask_transposed, _mask_parent_only])
def test_mask_mutants_are_caught(mutant):
    parent = random_tree(np.random.default_rng(5), 17)
    with pytest.raises(AssertionError):
        check_mask_pins(mutant, parent)


def _commit_skipping_root(kv, path, acc, cl, cache):
    cache_shift = np.full_like(cache, -1)
    nl = oracle.commit_path(kv, path, acc, cl, cache_shift)
    cache[:, :, :-1] = cache_shift[:, :, 1:]
    return nl


def _commit_off_by_one(kv, path, acc, cl, cache):
    return oracle.commit_path(kv, path, acc, cl + 1, cache)


def _commit_one_short(kv, path, acc, cl, cache):
    return oracle.commit_path(kv, path, np.maximum(acc - 1, 0), cl, cache)


@pytest.mark.parametrize("mutant", [_commit_skipping_root, _commit_off_by_one, _commit_one_short])
def test_commit_mutants_are_caught(mutant):
    with pytest.raises(AssertionError):
        for seed in range(4):
            check_commit_pins(mutant, seed)
