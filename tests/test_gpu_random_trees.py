"""GPU parity of tree verification on seeded random shapes.

Greedy cases: random parents-first trees (random windows, chains, stars), target rows
N(0, sigma^2), and node tokens that copy their parent row's argmax with probability 0.7 (so
accepted paths run deep), in fp32 or bf16 over vocabularies ragged against every slice and
chunk size.  Both greedy designs (every row's argmax, and the walk over the accepted rows)
must equal the oracle bit for bit.  Stochastic cases: the same topologies with the sampled
tree recipe at random temperatures, checked on every sequence with the near-tie rule.
"""

import numpy as np
import pytest

import synth
from test_gpu_tree_sampled import compare as compare_sampled
from test_gpu_tree_walk import compare as compare_greedy

pytestmark = pytest.mark.gpu

VOCABS = [2, 100, 2047, 2049, 8193, 16385, 40000, 65537]


def _depth(parent_row):
    d = np.zeros(len(parent_row), dtype=np.int64)
    for i in range(1, len(parent_row)):
        d[i] = d[parent_row[i]] + 1
    return int(d.max())


def _greedy_case(i):
    rng = np.random.default_rng(5000 + i)
    B = int(rng.integers(1, 7))
    N1 = int(rng.integers(2, 41))
    V = int(rng.choice(VOCABS))
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    parent = synth.random_parents(6000 + i, B=B, N1=N1, kind=str(rng.choice(["random", "chain", "star", "mixed"])))
    rows = rng.standard_normal((B, N1, V), dtype=np.float32) * np.float32(rng.choice([1.0, 2.0]))
    target = synth.bf16_bits_from_f32(rows) if dtype == "bf16" else rows
    values = synth.f32_from_bf16_bits(target) if dtype == "bf16" else target
    token = rng.integers(0, V, (B, N1)).astype(np.int32)
    for b in range(B):
        for n in range(1, N1):
            if rng.random() < 0.7:
                token[b, n] = int(np.argmax(values[b, parent[b, n]]))  # first index of the maximum
    token[:, 0] = 0
    depth = max(_depth(parent[b]) for b in range(B))
    return synth.TreeInputs(target=target, dtype=dtype, parent=parent, node_token=token, max_depth=depth,
                            name=f"random{i}_{dtype}_B{B}_N{N1 - 1}_V{V}")


@pytest.mark.parametrize("i", range(24))
def test_random_greedy_tree(i):
    compare_greedy(_greedy_case(i))


@pytest.mark.parametrize("i", range(16))
def test_random_sampled_tree(i):
    rng = np.random.default_rng(8000 + i)
    B = int(rng.integers(1, 7))
    N1 = int(rng.integers(2, 33))
    V = int(rng.choice(VOCABS[1:]))  # the sampled recipe plants peaks, so V > peaks
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    parent = synth.random_parents(9000 + i, B=B, N1=N1, kind=str(rng.choice(["random", "chain", "star", "mixed"])))
    depth = max(_depth(parent[b]) for b in range(B))
    x = synth.tree_sampled_inputs(9500 + i, B=B, n_nodes=N1 - 1, depth=depth, V=V, dtype=dtype, parent=parent,
                                  temperature=float(rng.choice([0.3, 0.8, 1.5])), peaks=min(20, V // 4),
                                  name=f"random{i}_{dtype}_B{B}_N{N1 - 1}_V{V}")
    compare_sampled(x)
