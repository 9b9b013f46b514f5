"""The pages' worked examples (tests/golden/*.json) against the oracle.

Each fixture names its page and section, the fact the page states, and the hand
derivation of the expected result; no expected value comes from the oracle.
The same fixtures are replayed on the GPU in test_gpu_edge_cases.py.
"""

import glob
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_fixtures(kind):
    out = []
    for path in sorted(glob.glob(os.path.join(GOLDEN, "*.json"))):
        with open(path) as f:
            fx = json.load(f)
        if fx["kind"] == kind:
            fx["_name"] = os.path.basename(path)
            out.append(fx)
    return out


def tree_rows(fx):
    V = fx["V"]
    rows = np.zeros((len(fx["parent"]), V), dtype=np.float32)
    for i, a in enumerate(fx["row_argmax"]):
        rows[i, a] = 5.0
    return rows


@pytest.mark.parametrize("fx", load_fixtures("chain"), ids=lambda f: f["_name"])
def test_chain_fixture(fx):
    assert fx["source"] and fx["derivation"]
    target = np.asarray(fx["target"], dtype=np.float64)
    draft = np.asarray(fx["draft"], dtype=np.float64)
    K = target.shape[0] - 1
    r = oracle.verify_chain_sequence(target, draft, np.asarray(fx["tokens"]), K, fx["temperature"],
                                     np.asarray(fx["u_accept"], dtype=np.float64), fx["u_final"])
    exp = fx["expected"]
    assert r.num_accepted == exp["num_accepted"]
    padded = r.tokens + [-1] * (K + 1 - len(r.tokens))
    assert padded == exp["tokens"]


@pytest.mark.parametrize("fx", load_fixtures("tree"), ids=lambda f: f["_name"])
def test_tree_fixture(fx):
    assert fx["source"] and fx["derivation"]
    rows = tree_rows(fx)
    res = oracle.verify_tree_greedy(rows[None], "f32", np.asarray([fx["parent"]]), np.asarray([fx["node_token"]]),
                                    fx["max_depth"])
    exp = fx["expected"]
    assert int(res.accept_len[0]) == exp["accept_len"]
    assert res.path_nodes[0].tolist() == exp["path_nodes"]
    assert res.tokens[0].tolist() == exp["tokens"]
    assert res.argmax[0].tolist() == fx["row_argmax"]
