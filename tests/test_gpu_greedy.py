"""GPU parity of greedy (temperature 0) chain verification against the oracle."""

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import chain_on_gpu, chain_oracle, compare_chain, f32, i32, log, logits_to_device
from test_golden import load_fixtures

pytestmark = pytest.mark.gpu


def _with_greedy(inp, seed, every=2, argmax_prefix=True):
    """Temperature 0 for every `every`-th sequence; for half of those the drafts start with a
    random-length prefix of the target's own argmaxes (so that some are accepted)."""
    rng = np.random.default_rng(seed)
    inp.temperature = inp.temperature.copy()
    inp.tokens = np.array(inp.tokens, copy=True)
    for b in range(0, inp.B, every):
        inp.temperature[b] = 0.0
        if argmax_prefix and rng.random() < 0.5:
            rows = inp.target[b]
            if inp.dtype == "bf16":
                rows = synth.f32_from_bf16_bits(rows)
            m = int(rng.integers(0, inp.K + 1))
            for k in range(m):
                inp.tokens[b, k] = int(np.argmax(rows[k]))
    return inp


@pytest.mark.parametrize("seed", range(3))
def test_greedy_and_sampled_sequences_in_one_batch(seed):
    inp = _with_greedy(synth.chain_config_high_accept_bf16(30 + seed, B=24, V=50000), seed)
    log(f"[greedy] mixed batch B={inp.B} K={inp.K} V={inp.V}")
    rep = compare_chain(chain_on_gpu(inp), chain_oracle(inp), inp)
    log(f"[greedy]   {rep}")
    assert rep.ok(), rep.failures[:5]


def test_greedy_full_headline_shape():
    inp = _with_greedy(synth.chain_config_high_accept_bf16(40), 40, every=1)
    rep = compare_chain(chain_on_gpu(inp), chain_oracle(inp), inp)
    log(f"[greedy] all greedy B=64 K=5 V=128256: {rep}")
    assert rep.ok(), rep.failures[:5]
    assert rep.exact == inp.B


def test_greedy_ties_take_the_smallest_index():
    inp = _with_greedy(synth.chain_config_small_f32(5, B=8, K=4, V=3000), 5, every=1)
    inp.target = np.round(inp.target / 2.0).astype(np.float32)  # many tied maxima
    for b in range(inp.B):  # drafts: the first tied maximum, a later tied one, or anything
        for k in range(inp.K):
            row = inp.target[b, k]
            ties = np.flatnonzero(row == row.max())
            inp.tokens[b, k] = int(ties[0]) if (b + k) % 3 else int(ties[-1])
    rep = compare_chain(chain_on_gpu(inp), chain_oracle(inp), inp)
    assert rep.ok(), rep.failures[:5]


def test_greedy_one_hot_and_variable_length():
    inp = synth.chain_config_high_accept_bf16(44, B=16, V=30000)
    inp.draft = None
    inp.draft_len = np.random.default_rng(44).integers(0, inp.K + 1, inp.B).astype(np.int32)
    inp = _with_greedy(inp, 44)
    rep = compare_chain(chain_on_gpu(inp), chain_oracle(inp), inp)
    assert rep.ok(), rep.failures[:5]


@pytest.mark.parametrize("fx", load_fixtures("chain_greedy"), ids=lambda f: f["_name"])
def test_golden_greedy_chain_on_gpu(fx):
    import draft_token_verification_09_amd as sv

    target = np.asarray(fx["target"], dtype=np.float32)[None]
    K = target.shape[1] - 1
    res = sv.spec_verify_chain(logits_to_device(target, "f32"), None, i32([fx["tokens"]]), f32([0.0]),
                               f32(np.full((1, K), 0.5)), f32([0.5]))
    torch.cuda.synchronize()
    assert int(res.num_accepted.cpu()[0]) == fx["expected"]["num_accepted"]
    assert res.tokens.cpu()[0].tolist() == fx["expected"]["tokens"]
