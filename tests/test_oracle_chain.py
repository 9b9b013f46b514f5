"""Pins of the chain-verification oracle against closed forms and hand-evaluated cases.

Every expected value here is derived by hand from the method's definition
("Speculative Decoding in Production", section I.1: alpha = min(1, p/q),
accept iff r <= alpha, residual max(0, p - q) normalised) or from an
independent library routine -- never from the oracle itself.
"""

import math

import numpy as np
import pytest

import oracle
from oracle.chain import acceptance_probability, inverse_cdf_sample, residual_weights, softmax_at_temperature

NEG = -1000.0  # exp(-1000) underflows to exactly 0 in float64


# ---------------------------------------------------------------- softmax with temperature


def test_softmax_two_token_logistic_closed_form():
    for l0, l1, T in [(0.3, -1.2, 1.0), (2.0, 2.5, 0.8), (-4.0, 3.0, 1.7)]:
        p = softmax_at_temperature(np.array([l0, l1]), T)
        p0 = 1.0 / (1.0 + math.exp((l1 - l0) / T))
        assert abs(p[0] - p0) < 1e-15 and abs(p[1] - (1.0 - p0)) < 1e-15


def test_softmax_sums_to_one_and_is_shift_invariant():
    rng = np.random.default_rng(1)
    l = rng.normal(0, 3, 5000)
    for T in (0.5, 1.0, 2.0):
        p = softmax_at_temperature(l, T)
        assert abs(p.sum() - 1.0) < 1e-12
        assert np.allclose(softmax_at_temperature(l + 123.25, T), p, rtol=1e-12, atol=0)


def test_softmax_temperature_limits():
    l = np.array([1.0, -2.0, 0.5, 3.0])
    assert np.allclose(softmax_at_temperature(l, 1e9), 0.25, atol=1e-8)   # T -> inf: uniform
    p = softmax_at_temperature(l, 1e-3)                                    # T -> 0: one-hot at argmax
    assert p[3] == 1.0 and p[:3].max() < 1e-300


def test_softmax_neg_inf_gets_zero_probability():
    p = softmax_at_temperature(np.array([0.0, -np.inf, 0.0]), 1.0)
    assert p.tolist() == [0.5, 0.0, 0.5]


def test_softmax_matches_exp_ratio_directly():
    # independent evaluation without the max shift (small logits cannot overflow)
    l = np.array([0.1, -0.7, 1.3, 0.0, 2.2])
    T = 0.8
    e = np.array([math.exp(v / T) for v in l])
    assert np.allclose(softmax_at_temperature(l, T), e / math.fsum(e), rtol=1e-14, atol=0)


# ---------------------------------------------------------------- acceptance probability


def test_alpha_closed_forms():
    assert acceptance_probability(0.25, 0.5) == 0.5
    assert acceptance_probability(0.5, 0.25) == 1.0       # capped at 1
    assert acceptance_probability(0.0, 0.5) == 0.0
    assert acceptance_probability(0.3, 0.3) == 1.0
    assert acceptance_probability(0.2, 0.0) == 1.0        # q(x) = 0 reading
    assert acceptance_probability(0.0, 0.0) == 0.0


def _seq(target, draft, tokens, u_acc, u_fin, T=1.0, kb=None):
    t = np.asarray(target, dtype=np.float64)
    d = None if draft is None else np.asarray(draft, dtype=np.float64)
    K = t.shape[0] - 1
    return oracle.verify_chain_sequence(t, d, np.asarray(tokens), K if kb is None else kb, T,
                                        np.asarray(u_acc, dtype=np.float64), u_fin)


def test_accept_boundary_is_inclusive():
    # p = (1/2, 1/2), q = (1, 0): x = 0 has alpha = 1/2 exactly.
    target = [[0.0, 0.0], [0.0, 0.0]]
    draft = [[0.0, NEG]]
    r = _seq(target, draft, [0], [0.5], 0.5)
    assert r.alpha == [0.5] and r.num_accepted == 1          # r == alpha accepts
    r = _seq(target, draft, [0], [0.5 + 2.0**-24], 0.5)
    assert r.num_accepted == 0                               # r > alpha rejects
    # residual max(0, p - q) = (0, 1/2): the replacement must be token 1
    assert r.tokens == [1] and r.mode == "residual"


def test_alpha_one_accepts_u_equal_one_and_alpha_zero_rejects_smallest_u():
    target = [[0.0, NEG], [0.0, 0.0]]   # p = (1, 0)
    draft = [[0.0, 0.0]]                # q = (1/2, 1/2)
    r1 = _seq(target, draft, [0], [1.0], 0.3)
    assert r1.alpha == [1.0] and r1.num_accepted == 1                   # alpha = min(1, 2) = 1
    r = _seq(target, draft, [1], [2.0**-24], 0.3)                       # alpha = 0
    assert r.num_accepted == 0 and r.tokens == [0]                      # residual = (1/2, 0)


# ---------------------------------------------------------------- residual and its sampling


def test_residual_closed_form():
    p = np.array([0.25, 0.25, 0.25, 0.25])
    q = np.array([0.5, 0.5, 0.0, 0.0])
    assert residual_weights(p, q).tolist() == [0.0, 0.0, 0.25, 0.25]
    assert residual_weights(q, p).tolist() == [0.25, 0.25, 0.0, 0.0]


def test_inverse_cdf_hand_cases():
    w = np.array([0.1, 0.2, 0.3, 0.4])
    # C = (0.1, 0.3, 0.6, 1.0); smallest i with C_i >= u W
    assert inverse_cdf_sample(w, 0.05)[0] == 0
    assert inverse_cdf_sample(w, 0.25)[0] == 1
    assert inverse_cdf_sample(w, 0.61)[0] == 3
    assert inverse_cdf_sample(w, 1.0)[0] == 3
    # exact boundary: u W == C_i selects i (inclusive)
    w2 = np.array([0.25, 0.25, 0.5])
    assert inverse_cdf_sample(w2, 0.25)[0] == 0
    assert inverse_cdf_sample(w2, 0.5)[0] == 1
    # zero-weight entries are never selected, even at the smallest uniform
    w3 = np.array([0.0, 0.0, 0.5, 0.0, 0.5])
    assert inverse_cdf_sample(w3, 2.0**-24)[0] == 2
    assert inverse_cdf_sample(w3, 1.0)[0] == 4


def test_inverse_cdf_matches_searchsorted():
    rng = np.random.default_rng(7)
    for _ in range(200):
        V = int(rng.integers(1, 60))
        w = rng.random(V) * (rng.random(V) < 0.6)
        if w.sum() == 0:
            w[int(rng.integers(V))] = 1.0
        u = (int(rng.integers(0, 1 << 24)) + 1) * 2.0**-24
        C = np.cumsum(w)
        expect = int(np.searchsorted(C, u * C[-1], side="left"))
        assert inverse_cdf_sample(w, u)[0] == expect


def test_inverse_cdf_gap_measures_distance_to_boundary():
    w = np.array([1.0, 1.0, 2.0])   # C = 1, 2, 4
    i, gap, W = inverse_cdf_sample(w, 0.4)  # t = 1.6 in (1, 2]: gap = min(0.6, 0.4) / 4
    assert i == 1 and W == 4.0 and abs(gap - 0.1) < 1e-15


# ---------------------------------------------------------------- special cases of the whole chain


def test_draft_equal_target_accepts_everything_then_bonus_from_next_row():
    rng = np.random.default_rng(3)
    K, V = 4, 6
    target = rng.normal(0, 2, (K + 1, V))
    bonus_row = np.full(V, NEG)
    bonus_row[4] = 0.0                      # p_K is one-hot at token 4
    target[K] = bonus_row
    draft = target[:K].copy()
    for trial in range(20):
        toks = rng.integers(0, V, K)
        u = (rng.integers(0, 1 << 24, K) + 1) * 2.0**-24
        r = _seq(target, draft, toks, u, 0.77)
        assert r.alpha == [1.0] * K
        assert r.num_accepted == K and r.mode == "bonus"
        assert r.tokens == [int(t) for t in toks] + [4]


def test_vocabulary_of_one_always_accepts_and_emits_token_zero():
    r = _seq([[0.3], [1.0], [-2.0]], [[5.0], [0.1]], [0, 0], [1.0, 1.0], 1.0)
    assert r.num_accepted == 2 and r.tokens == [0, 0, 0]


def test_one_hot_draft_alpha_is_p_and_residual_excludes_the_draft_token():
    target = np.log(np.array([[0.1, 0.2, 0.3, 0.4], [0.25, 0.25, 0.25, 0.25]]))
    r = _seq(target, None, [3], [0.5], 0.4)
    assert abs(r.alpha[0] - 0.4) < 1e-15 and r.q_x == [1.0]
    assert r.num_accepted == 0
    # residual = p with token 3 removed: (0.1, 0.2, 0.3); t = 0.4 * 0.6 = 0.24 -> C = (0.1, 0.3, 0.6) -> index 1
    assert r.tokens == [1]
    r2 = _seq(target, None, [3], [0.39], 0.5)
    assert r2.num_accepted == 1 and r2.tokens == [3, 1]   # bonus from row 1 (uniform): t = 0.5 -> index 1


def test_draft_len_shorter_than_K_takes_bonus_from_row_draft_len():
    target = np.full((4, 3), NEG)
    target[0] = [0.0, NEG, NEG]
    target[1] = [NEG, NEG, 0.0]        # row k_b = 1 is one-hot at token 2
    target[2] = [NEG, 0.0, NEG]
    target[3] = [NEG, 0.0, NEG]
    draft = target[:3].copy()
    r = _seq(target, draft, [0, 1, 1], [0.9, 0.9, 0.9], 0.5, kb=1)
    assert r.num_accepted == 1 and r.tokens == [0, 2]
    r0 = _seq(target, draft, [0, 1, 1], [0.9, 0.9, 0.9], 0.5, kb=0)
    assert r0.num_accepted == 0 and r0.tokens == [0] and r0.mode == "bonus"


def test_expected_alpha_equals_overlap_mass():
    # E_{x~q}[alpha(x)] = sum_x min(p(x), q(x)): a consequence of alpha = min(1, p/q)
    rng = np.random.default_rng(11)
    for _ in range(20):
        V = int(rng.integers(2, 30))
        p = softmax_at_temperature(rng.normal(0, 2, V), 1.0)
        q = softmax_at_temperature(rng.normal(0, 2, V), 1.0)
        e_alpha = sum(q[x] * acceptance_probability(p[x], q[x]) for x in range(V))
        assert abs(e_alpha - np.minimum(p, q).sum()) < 1e-14


def test_invalid_inputs_raise():
    t = [[0.0, 0.0], [0.0, 0.0]]
    with pytest.raises(ValueError):
        _seq(t, [[0.0, 0.0]], [2], [0.5], 0.5)       # token out of range
    with pytest.raises(ValueError):
        _seq(t, [[0.0, 0.0]], [0], [0.0], 0.5)       # u = 0 outside (0, 1]
    with pytest.raises(ValueError):
        _seq(t, [[0.0, 0.0]], [0], [0.5], 1.5)
    with pytest.raises(ValueError):
        _seq(t, [[0.0, 0.0]], [0], [0.5], 0.5, T=0.0)


def test_batch_wrapper_reads_bf16_bits_exactly():
    # bf16 0x3F80 = 1.0, 0xBF80 = -1.0, 0x4000 = 2.0, 0xFF80 = -inf
    target = np.array([[[0x3F80, 0xBF80, 0x4000, 0xFF80], [0x3F80, 0x3F80, 0x3F80, 0x3F80]]], dtype=np.uint16)
    draft = np.array([[[0x3F80, 0x3F80, 0x3F80, 0x3F80]]], dtype=np.uint16)
    res = oracle.verify_chain(target, draft, "bf16", np.array([[2]]), np.array([1.0], np.float32),
                              np.array([[0.5]], np.float32), np.array([0.5], np.float32))
    e = np.exp([1.0, -1.0, 2.0])
    p2 = e[2] / e.sum()
    assert abs(res.probs[0, 0, 0] - p2) < 1e-15
    assert abs(res.probs[0, 0, 1] - 0.25) < 1e-15
    assert res.num_accepted[0] == 1
