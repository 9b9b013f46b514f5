"""Pins of the greedy-tree and n-gram oracles by brute force on tiny inputs and hand cases."""

import numpy as np
import pytest

import oracle


# ---------------------------------------------------------------- greedy tree: brute force over all root paths


def _brute_argmax(row):
    best = max(row)
    for i, v in enumerate(row):
        if v == best:
            return i


def _brute_tree(rows, parent, token):
    """Every node's root path is checked edge by edge; the deepest fully matching node wins
    (smallest index among equally deep ones)."""
    N1 = len(parent)
    amax = [_brute_argmax(list(rows[i])) for i in range(N1)]
    best, best_depth, best_path = 0, 0, []
    for v in range(1, N1):
        path = []
        u = v
        ok = True
        while u != 0:
            path.append(u)
            if token[u] != amax[parent[u]]:
                ok = False
            u = parent[u]
        if ok and len(path) > best_depth:
            best, best_depth, best_path = v, len(path), path[::-1]
    return best_depth, [int(token[u]) for u in best_path] + [amax[best]], best_path


def _random_tree(rng, N1, V):
    parent = [-1] + [int(rng.integers(0, i)) for i in range(1, N1)]
    token = [0] + [int(rng.integers(0, V)) for _ in range(1, N1)]
    rows = rng.integers(-2, 3, size=(N1, V)).astype(np.float32)   # small integers: many argmax ties
    return np.asarray(parent), np.asarray(token), rows


@pytest.mark.parametrize("seed", range(300))
def test_tree_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    N1 = int(rng.integers(1, 13))
    V = int(rng.integers(1, 7))
    parent, token, rows = _random_tree(rng, N1, V)
    # force some matches so that deep paths exist
    for i in range(1, N1):
        if rng.random() < 0.6:
            token[i] = _brute_argmax(list(rows[parent[i]]))
    depth, toks, path = _brute_tree(rows, parent, token)
    res = oracle.verify_tree_greedy(rows[None], "f32", parent[None], token[None], max_depth=N1)
    assert int(res.accept_len[0]) == depth
    assert res.tokens[0, : depth + 1].tolist() == toks
    assert (res.tokens[0, depth + 1:] == -1).all()
    assert res.path_nodes[0, :depth].tolist() == path


def test_tree_root_only_emits_root_argmax():
    rows = np.array([[0.0, 3.0, 3.0, 1.0]], dtype=np.float32)   # tie: smallest index 1
    res = oracle.verify_tree_greedy(rows[None], "f32", np.array([[-1]]), np.array([[0]]), max_depth=2)
    assert res.accept_len[0] == 0 and res.tokens[0].tolist() == [1, -1, -1]


def test_tree_equal_depth_tie_takes_smallest_node_index():
    # root -> 1 and root -> 2 both carry the root argmax token (duplicate siblings)
    rows = np.zeros((3, 4), dtype=np.float32)
    rows[0, 2] = 1.0
    rows[1, 3] = 1.0
    rows[2, 0] = 1.0
    res = oracle.verify_tree_greedy(rows[None], "f32", np.array([[-1, 0, 0]]), np.array([[0, 2, 2]]), max_depth=1)
    assert res.path_nodes[0].tolist() == [1, -1] and res.tokens[0].tolist() == [2, 3]


def test_tree_rejects_bad_topology():
    rows = np.zeros((3, 4), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.verify_tree_greedy(rows[None], "f32", np.array([[-1, 2, 0]]), np.array([[0, 1, 1]]), max_depth=3)


# ---------------------------------------------------------------- n-gram lookup: brute force over all (n, j)


def _brute_ngram(c, n_min, n_max, K):
    L = len(c)
    for n in range(n_max, n_min - 1, -1):
        for j in range(L):
            if j + n > L - 1:
                break
            if all(c[j + i] == c[L - n + i] for i in range(n)):
                return list(c[j + n: min(j + n + K, L)]), n
    return [], 0


@pytest.mark.parametrize("seed", range(300))
def test_ngram_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 41))
    V = int(rng.integers(1, 5))
    c = rng.integers(0, V, L).tolist()
    n_min = int(rng.integers(1, 3))
    n_max = int(rng.integers(n_min, 6))
    K = int(rng.integers(1, 7))
    toks, n = _brute_ngram(c, n_min, n_max, K)
    res = oracle.ngram_propose(np.asarray([c]), np.asarray([L]), n_min, n_max, K)
    assert int(res.match_n[0]) == n
    assert int(res.draft_len[0]) == len(toks)
    assert res.draft[0, : len(toks)].tolist() == toks
    assert (res.draft[0, len(toks):] == -1).all()


def test_ngram_hand_cases():
    # no earlier occurrence of the last token: no draft
    r = oracle.ngram_propose(np.array([[1, 2, 3, 4]]), np.array([4]), 1, 4, 5)
    assert r.draft_len[0] == 0 and r.match_n[0] == 0
    # suffix (7, 8) occurred at j = 1; continuation 9, 5, 7, 8 (truncated by K = 3)
    r = oracle.ngram_propose(np.array([[5, 7, 8, 9, 5, 7, 8]]), np.array([7]), 1, 4, 3)
    assert r.match_n[0] == 3 and r.draft[0].tolist() == [9, 5, 7]   # (5, 7, 8) matches at j = 0 first
    # overlapping occurrence of a repeated token: 'a a a a' -> suffix (a, a, a) at j = 0, continuation a
    r = oracle.ngram_propose(np.array([[6, 6, 6, 6]]), np.array([4]), 1, 4, 5)
    assert r.match_n[0] == 3 and r.draft[0].tolist() == [6, -1, -1, -1, -1]
    # continuation truncated at the end of the context
    r = oracle.ngram_propose(np.array([[1, 2, 9, 1, 2]]), np.array([5]), 1, 4, 5)
    assert r.match_n[0] == 2 and r.draft[0].tolist() == [9, 1, 2, -1, -1]
    # context of one token: nothing to match
    r = oracle.ngram_propose(np.array([[3, 0, 0]]), np.array([1]), 1, 4, 5)
    assert r.draft_len[0] == 0
    # padding beyond context_len is ignored
    r = oracle.ngram_propose(np.array([[4, 5, 4, 7, 7, 7]]), np.array([3]), 1, 4, 2)
    assert r.match_n[0] == 1 and r.draft[0].tolist() == [5, 4]
