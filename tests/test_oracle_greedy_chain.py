"""Greedy (temperature 0) chain verification in the oracle, pinned three ways:

* the page's cascade example under greedy decoding (tests/golden/chain_greedy_cascade.json);
* agreement with the greedy tree oracle on chain-shaped trees (an independent walk:
  accept along parent links, deepest accepted node), including many tied maxima;
* the limit of the sampled verification as temperature -> 0 on tie-free rows, where p
  becomes one-hot at the argmax, so alpha is 1 for the argmax and 0 otherwise and every
  draw (residual or bonus) lands on the argmax, whatever the uniforms and the draft.
"""

import numpy as np
import pytest

import oracle
from test_golden import load_fixtures


@pytest.mark.parametrize("fx", load_fixtures("chain_greedy"), ids=lambda f: f["_name"])
def test_greedy_chain_fixture(fx):
    assert fx["source"] and fx["derivation"] and fx["temperature"] == 0.0
    target = np.asarray(fx["target"], dtype=np.float64)
    K = target.shape[0] - 1
    r = oracle.verify_chain_greedy_sequence(target, np.asarray(fx["tokens"]), K)
    assert r.num_accepted == fx["expected"]["num_accepted"]
    assert r.tokens + [-1] * (K + 1 - len(r.tokens)) == fx["expected"]["tokens"]
    # the batched entry point takes the greedy path for temperature 0
    res = oracle.verify_chain(target[None].astype(np.float32), None, "f32", np.asarray([fx["tokens"]]),
                              np.zeros(1, np.float32), np.full((1, K), 0.5, np.float32), np.full(1, 0.5, np.float32))
    assert res.tokens[0].tolist() == fx["expected"]["tokens"]


@pytest.mark.parametrize("seed", range(40))
def test_greedy_chain_equals_greedy_tree_on_chains(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(2, 6))
    K = int(rng.integers(1, 5))
    kb = int(rng.integers(0, K + 1))
    rows = rng.integers(0, 3, (K + 1, V)).astype(np.float32)  # small integers: many ties
    amax = [int(np.argmax(r)) for r in rows]
    tokens = np.array([amax[k] if rng.random() < 0.6 else int(rng.integers(0, V)) for k in range(K)])
    r = oracle.verify_chain_greedy_sequence(rows.astype(np.float64), tokens, kb)
    # the same chain as a tree: node i (1..kb) carries draft i-1, row i-1 scores it
    parent = np.array([-1] + list(range(kb)), dtype=np.int32)
    node_tok = np.array([0] + [int(t) for t in tokens[:kb]], dtype=np.int32)
    t = oracle.verify_tree_greedy(rows[None, : kb + 1], "f32", parent[None], node_tok[None], max_depth=kb)
    assert r.num_accepted == int(t.accept_len[0])
    assert r.tokens == t.tokens[0, : r.num_accepted + 1].tolist()


@pytest.mark.parametrize("seed", range(30))
def test_greedy_chain_is_the_zero_temperature_limit(seed):
    rng = np.random.default_rng(100 + seed)
    V = int(rng.integers(2, 7))
    K = int(rng.integers(1, 5))
    # tie-free rows with gaps of at least 1 between sorted values
    target = np.stack([rng.permutation(V).astype(np.float64) * 1.5 for _ in range(K + 1)])
    draft = rng.normal(0, 1, (K, V))
    amax = target.argmax(axis=1)
    tokens = np.array([amax[k] if rng.random() < 0.7 else int(rng.integers(0, V)) for k in range(K)])
    g = oracle.verify_chain_greedy_sequence(target, tokens, K)
    for _ in range(3):
        s = oracle.verify_chain_sequence(target, draft, tokens, K, 1e-3, rng.uniform(1e-6, 1.0, K),
                                         float(rng.uniform(1e-6, 1.0)))
        assert s.num_accepted == g.num_accepted
        assert s.tokens == g.tokens


def test_greedy_chain_planted_mistake_is_caught(monkeypatch):
    # a greedy rule that takes the smallest logit instead of the largest fails a pin
    import oracle.chain as chain

    monkeypatch.setattr(chain, "argmax_first", lambda row: int(np.argmin(row)))
    with pytest.raises(AssertionError):
        for seed in range(10):
            test_greedy_chain_equals_greedy_tree_on_chains(seed)
