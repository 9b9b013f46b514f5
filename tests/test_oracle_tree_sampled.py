"""Pins of the stochastic tree-verification oracle (CPU only).

  * A chain-shaped tree is chain verification: same accepted count and tokens as the
    (separately pinned) chain oracle, on random inputs with the same uniforms.
  * Invariance theorem by exact enumeration on tiny trees: every joint draw of the
    children's tokens (each child i.i.d. from q at its parent, weight prod q), every
    accept/reject branch (driven through the oracle itself with uniforms in the middle
    of each branch, weighted by the alpha the oracle reports) and every final token
    (weighted by the oracle's final weights).  Then, within 1e-9,
      (I1) P(first emitted token = v) = p_root(v),
      (I2) P(second emitted token = v | first step accepted child c) = p_c(v).
    The reference distributions are exp(l/T)/sum exp(l/T) computed here directly.
  * The pages' tree example with sampling (golden): B1 rejected, B2 accepted against the
    residual, B2 -> C2, bonus.
  * Planted mistakes in the residual or acceptance rule fail a pin.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import oracle.tree_sampled as ts

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _direct_softmax(l, T):
    e = np.array([0.0 if v == -np.inf else math.exp(v / T) for v in l])
    return e / math.fsum(e)


# ------------------------------------------------------------- chain-shaped trees
@pytest.mark.parametrize("seed", range(8))
def test_chain_shaped_tree_is_chain_verification(seed):
    rng = np.random.default_rng(seed)
    K, V, T = int(rng.integers(1, 6)), int(rng.integers(2, 40)), float(rng.choice([0.5, 1.0, 1.7]))
    target = rng.normal(0, 2.0, (K + 1, V))
    draft = target[:K] + rng.normal(0, 1.0, (K, V))
    if seed % 3 == 0:
        draft[:, 0] = -np.inf
    q = [_direct_softmax(draft[k], T) for k in range(K)]
    toks = np.array([int(rng.choice(V, p=q[k])) for k in range(K)])
    ua = rng.uniform(0.01, 1.0, K)
    uf = float(rng.uniform(0.01, 1.0))
    ch = oracle.verify_chain_sequence(target, draft, toks, K, T, ua, uf)
    parent = np.arange(-1, K)
    node_tok = np.concatenate([[0], toks])
    d_rows = np.concatenate([draft, np.zeros((1, V))])   # the leaf's draft row is unused
    u_nodes = np.concatenate([[0.5], ua])
    tr = ts.verify_tree_sampled_sequence(target, d_rows, parent, node_tok, T, u_nodes, uf, K)
    assert tr.accept_len == ch.num_accepted
    assert tr.tokens == ch.tokens
    assert tr.path_nodes == list(range(1, ch.num_accepted + 1))


# ------------------------------------------------------------- exact enumeration
def enumerate_tree(target, draft, parent, T):
    """Returns (first[v], second[c][v], reach[c]) summed over every branch."""
    N1, V = target.shape
    kids = [[] for _ in range(N1)]
    for i in range(1, N1):
        kids[parent[i]].append(i)
    q = [_direct_softmax(draft[i], T) for i in range(N1)]
    first = np.zeros(V)
    second = {c: np.zeros(V) for c in kids[0]}
    total = 0.0
    nodes = list(range(1, N1))
    for toks in itertools.product(range(V), repeat=N1 - 1):
        wq = 1.0
        for i, x in zip(nodes, toks):
            wq *= q[parent[i]][x]
        if wq <= 0.0:
            continue
        node_tok = np.array([0] + list(toks))

        def run(assign):
            u = np.array([assign.get(i, 0.5) for i in range(N1)])
            return u

        stack = [({}, wq)]
        while stack:
            assign, w = stack.pop()
            u = run(assign)
            res = ts.verify_tree_sampled_sequence(target, draft, parent, node_tok, T, u, 0.5, N1)
            branch = None
            for node, alpha, ok in res.tests:
                if node not in assign:
                    branch = (node, alpha)
                    break
                # the oracle must have taken the branch the uniform was chosen for
                assert ok == (assign[node] <= alpha), (node, alpha, assign)
            if branch is not None:
                node, alpha = branch
                if alpha > 0.0:
                    stack.append(({**assign, node: alpha / 2.0}, w * alpha))
                if alpha < 1.0:
                    stack.append(({**assign, node: (1.0 + alpha) / 2.0}, w * (1.0 - alpha)))
                continue
            fw = res.final_weights
            C = np.cumsum(fw)
            W = C[-1]
            for v in range(V):
                if fw[v] <= 0.0:
                    continue
                lo = C[v - 1] / W if v > 0 else 0.0
                uf = 0.5 * (lo + C[v] / W)
                r2 = ts.verify_tree_sampled_sequence(target, draft, parent, node_tok, T, u, uf, N1)
                assert r2.tokens[-1] == v and r2.path_nodes == res.path_nodes
                wb = w * fw[v] / W
                total += wb
                first[r2.tokens[0]] += wb
                if r2.path_nodes:
                    c = r2.path_nodes[0]
                    second[c][r2.tokens[1]] += wb
    return first, second, total


TREES = [
    # (parent, V, T, seed)
    ([-1, 0, 0], 3, 1.0, 0),            # root with two children
    ([-1, 0, 0, 0], 3, 0.8, 1),         # three children
    ([-1, 0, 0, 1], 3, 1.3, 2),         # two children, the first with a child
    ([-1, 0, 0, 1, 1, 2], 3, 1.0, 3),   # depth 2 with branching at both levels
    ([-1, 0, 0, 0, 1], 4, 1.0, 4),
]


@pytest.mark.parametrize("parent,V,T,seed", TREES)
def test_invariance_by_enumeration(parent, V, T, seed):
    rng = np.random.default_rng(seed)
    N1 = len(parent)
    target = rng.normal(0, 1.5, (N1, V))
    draft = rng.normal(0, 1.5, (N1, V))
    if seed % 2:
        draft[0, V - 1] = -np.inf   # a token the draft never proposes at the root
    parent = np.array(parent)
    first, second, total = enumerate_tree(target, draft, parent, T)
    assert abs(total - 1.0) < 1e-9
    p_root = _direct_softmax(target[0], T)
    assert np.max(np.abs(first - p_root)) < 1e-9                               # (I1)
    for c, dist in second.items():                                             # (I2)
        reach = dist.sum()
        if reach > 1e-12:
            assert np.max(np.abs(dist / reach - _direct_softmax(target[c], T))) < 1e-9, c


# ------------------------------------------------------------- golden
def _golden():
    with open(os.path.join(GOLDEN, "tree_sampled_b1_rejected_b2_accepted.json")) as f:
        return json.load(f)


def golden_inputs(fx):
    tgt = np.log(np.asarray(fx["target_probs"], dtype=np.float64))
    dft = np.log(np.asarray(fx["draft_probs"], dtype=np.float64))
    return tgt, dft


def test_golden_b1_rejected_b2_accepted():
    fx = _golden()
    assert fx["source"] and fx["derivation"]
    tgt, dft = golden_inputs(fx)
    r = ts.verify_tree_sampled_sequence(tgt, dft, np.array(fx["parent"]), np.array(fx["node_token"]),
                                        fx["temperature"], np.array(fx["u_accept"]), fx["u_final"], fx["max_depth"])
    exp = fx["expected"]
    assert r.accept_len == exp["accept_len"]
    assert r.path_nodes + [-1] * (fx["max_depth"] + 1 - len(r.path_nodes)) == exp["path_nodes"]
    assert r.tokens == exp["tokens"]
    assert [t[0] for t in r.tests] == [t[0] for t in exp["tests"]]
    for (_, a, _), (_, ea) in zip(r.tests, exp["tests"]):
        assert a == pytest.approx(ea, rel=1e-12)


def test_invalid_inputs_are_flagged():
    fx = _golden()
    tgt, dft = golden_inputs(fx)
    par, tok = np.array(fx["parent"]), np.array(fx["node_token"])
    ua = np.array(fx["u_accept"])
    for kw in (dict(parent=np.array([-1, 0, 2, 1, 2, 3])), dict(node_token=np.array([0, 0, 1, 9, 3, 3])),
               dict(T=0.0), dict(T=float("nan")), dict(ua=np.array([0.5, 0.5, 0.0, 0.5, 0.5, 0.3])),
               dict(uf=1.5), dict(max_depth=2)):
        r = ts.verify_tree_sampled_sequence(tgt, dft, kw.get("parent", par), kw.get("node_token", tok),
                                            kw.get("T", 1.0), kw.get("ua", ua), kw.get("uf", 0.5),
                                            kw.get("max_depth", 3))
        assert r.accept_len == -1, kw


# ------------------------------------------------------------- planted mistakes
@pytest.mark.parametrize("mutant", [
    lambda r, q: r,                          # siblings all tested against p (no residual update)
    lambda r, q: np.abs(r - q),              # max(0, .) dropped
    lambda r, q: np.maximum(0.0, q - r),     # operands swapped
])
def test_planted_residual_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(ts, "residual_weights", mutant)
    caught = 0
    for parent, V, T, seed in TREES[:2]:
        try:
            test_invariance_by_enumeration(parent, V, T, seed)
        except AssertionError:
            caught += 1
    try:
        test_golden_b1_rejected_b2_accepted()
    except AssertionError:
        caught += 1
    assert caught >= 1


def test_planted_ratio_inversion_is_caught(monkeypatch):
    monkeypatch.setattr(ts, "acceptance_probability", lambda p, q: min(1.0, q / p) if p > 0 else 1.0)
    with pytest.raises(AssertionError):
        test_invariance_by_enumeration(*TREES[0])
