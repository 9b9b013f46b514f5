"""The seeded workload generators: determinism, domains and the bf16 rounding rule."""

import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 3, 100000).astype(np.float32),
                        np.array([1.0, -1.0, 0.0, -0.0, 1e-40, 3.0e38, 1.00390625, 1.01171875], np.float32)])
    ours = synth.bf16_bits_from_f32(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    back = synth.f32_from_bf16_bits(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_uniforms_on_open_closed_grid():
    u = synth.uniforms_open_closed(synth.philox(0, "u_accept", 0), (200000,))
    assert u.dtype == np.float32 and u.min() > 0.0 and u.max() <= 1.0
    k = u.astype(np.float64) * 2.0**24
    assert np.array_equal(k, np.round(k))


def test_chain_generation_is_deterministic_and_per_sequence():
    a = synth.chain_config_high_accept_bf16(3, B=4, K=3, V=1000)
    b = synth.chain_config_high_accept_bf16(3, B=4, K=3, V=1000, threads=1)
    for f in ("target", "draft", "tokens", "u_accept", "u_final"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    # sequence b depends only on (seed, b): a larger batch has the same first sequences
    c = synth.chain_config_high_accept_bf16(3, B=6, K=3, V=1000)
    assert np.array_equal(c.target[:4], a.target) and np.array_equal(c.tokens[:4], a.tokens)
    assert a.tokens.min() >= 0 and a.tokens.max() < 1000


def test_high_accept_recipe_has_peaks():
    x = synth.chain_config_high_accept_bf16(0, B=2, K=2, V=5000)
    t = synth.f32_from_bf16_bits(x.target)
    # 20 peak tokens at +8 on N(0, 9): the row maximum sits well above the bulk
    assert (np.sort(t, axis=-1)[..., -20:] > 4.0).mean() > 0.8


def test_tree_generation_shape():
    tr = synth.tree_config_eagle_bf16(0, B=8, V=1000)
    assert tr.target.shape == (8, 61, 1000) and tr.max_depth == 6
    for b in range(8):
        par = tr.parent[b]
        assert par[0] == -1 and all(0 <= par[i] < i for i in range(1, 61))
        depth = np.zeros(61, int)
        for i in range(1, 61):
            depth[i] = depth[par[i]] + 1
        assert depth.max() == 6
        for i in range(61):   # branching at most 4
            assert (par == i).sum() <= 4


def test_ngram_prompts_recipe():
    pr = synth.ngram_config_prompts(0, B=4, L=4096, V=32000)
    assert pr.context.shape == (4, 4096) and pr.context.min() >= 0 and pr.context.max() < 32000
    # Zipf: token 0 (rank 1) is the most frequent
    counts = np.bincount(pr.context.ravel(), minlength=32000)
    assert counts.argmax() == 0
