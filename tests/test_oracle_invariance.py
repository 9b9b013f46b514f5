"""Exact-enumeration pin of the chain oracle against the invariance theorem.

"Speculative Decoding in Production" (blog.llmgo.top), section I.1, "The
Invariance Theorem": marginalising over the acceptance and residual branches
recovers the target distribution p exactly.

For tiny vocabularies every branch of the verification is enumerated: each draft
chain x ~ q (weight prod q_k(x_k)), each acceptance pattern (accept the first n,
reject the next one), and each replacement / bonus token v.  The oracle function
itself is driven with uniforms taken from the middle of each branch's interval,
and must return exactly that branch.  Summing branch weights must then give
  (I1) P(first emitted token = v) = p_0(v),
  (I2) P(token at position j = v | first j drafts accepted) = p_j(v) for j = 0..k_b
       (j = k_b exercises the bonus row),
  (I3) E[number accepted] = sum_{j=1..k_b} prod_{k<j} sum_x min(p_k(x), q_k(x)),
all within 1e-9.  The reference distributions below are computed directly as
exp(l/T) / sum exp(l/T), independently of the oracle's softmax.
"""

import itertools
import math

import numpy as np
import pytest

import oracle


def _direct_softmax(l, T):
    e = np.array([0.0 if v == -np.inf else math.exp(v / T) for v in l])
    return e / math.fsum(e)


def check_invariance(target, draft, T, kb=None, fixed_draft=None):
    """target [K+1, V], draft [K, V] or None (then fixed_draft gives the drafted tokens)."""
    K1, V = target.shape
    K = K1 - 1
    kb = K if kb is None else kb
    p = [_direct_softmax(target[k], T) for k in range(K + 1)]
    if draft is None:
        chains = [(tuple(int(v) for v in fixed_draft[:kb]), 1.0)]
    else:
        q_rows = [_direct_softmax(draft[k], T) for k in range(K)]
        chains = []
        for xs in itertools.product(range(V), repeat=kb):
            w = 1.0
            for k, x in enumerate(xs):
                w *= q_rows[k][x]
            if w > 0.0:
                chains.append((xs, w))

    def q_of(k, x):
        if draft is None:
            return 1.0 if x == chains[0][0][k] else 0.0
        return q_rows[k][x]

    emitted = np.zeros((kb + 1, V))     # emitted[j, v] = P(position j emits v and first j accepted)
    reach = np.zeros(kb + 1)            # P(first j accepted)
    e_n = 0.0
    total = 0.0
    for xs, wq in chains:
        alpha = []
        for k in range(kb):
            pk, qk = p[k][xs[k]], q_of(k, xs[k])
            alpha.append(min(1.0, pk / qk) if qk > 0 else (1.0 if pk > 0 else 0.0))
        for n in range(kb + 1):
            w_acc = wq
            for k in range(n):
                w_acc *= alpha[k]
            if n < kb:
                w_acc *= 1.0 - alpha[n]
            if w_acc <= 0.0:
                continue
            if n < kb:
                qn = np.array([q_of(n, x) for x in range(V)])
                wv = np.maximum(0.0, p[n] - qn)
                if wv.sum() <= 0.0:
                    wv = p[n].copy()
            else:
                wv = p[kb].copy()
            C = np.cumsum(wv)
            W = C[-1]
            u_acc = np.full(max(K, 1), 0.5)
            for k in range(n):
                u_acc[k] = alpha[k] / 2.0
            if n < kb:
                u_acc[n] = (1.0 + alpha[n]) / 2.0
            toks = np.zeros(K, dtype=np.int64)
            toks[:kb] = xs
            for v in range(V):
                if wv[v] <= 0.0:
                    continue
                lo = C[v - 1] / W if v > 0 else 0.0
                u_fin = 0.5 * (lo + C[v] / W)
                res = oracle.verify_chain_sequence(target, draft, toks, kb, T, u_acc[:K], u_fin)
                assert res.num_accepted == n, (xs, n, v)
                assert res.tokens == list(xs[:n]) + [v], (xs, n, v, res.tokens)
                wb = w_acc * wv[v] / W
                total += wb
                e_n += wb * n
                for j in range(n + 1):
                    reach[j] += wb
                    emitted[j, xs[j] if j < n else v] += wb
    assert abs(total - 1.0) < 1e-9
    assert np.max(np.abs(emitted[0] - p[0])) < 1e-9                       # (I1)
    for j in range(kb + 1):                                                # (I2)
        if reach[j] > 1e-12:
            assert np.max(np.abs(emitted[j] / reach[j] - p[j])) < 1e-9, j
    if draft is not None:                                                  # (I3)
        beta = [np.minimum(p[k], q_rows[k]).sum() for k in range(kb)]
        expect = sum(math.prod(beta[:j]) for j in range(1, kb + 1))
        assert abs(e_n - expect) < 1e-9


CASES = [
    # (V, K, T, seed, n_neg_inf)
    (2, 1, 1.0, 0, 0),
    (3, 2, 0.7, 1, 0),
    (4, 3, 1.0, 2, 0),
    (5, 2, 1.6, 3, 2),
    (5, 3, 0.9, 4, 3),
    (6, 2, 1.0, 5, 4),
    (8, 3, 1.2, 6, 0),
]


def _case(V, K, T, seed, n_neg):
    rng = np.random.default_rng(seed)
    target = rng.normal(0, 1.5, (K + 1, V))
    draft = rng.normal(0, 1.5, (K, V))
    # knock out some entries so that zero probabilities (alpha = 0, empty residual slots) appear
    for _ in range(n_neg):
        r, c = int(rng.integers(K)), int(rng.integers(V))
        if rng.random() < 0.5:
            target[r, c] = -np.inf
        else:
            draft[r, c] = -np.inf
    for r in range(K + 1):
        if not np.isfinite(target[r]).any():
            target[r, 0] = 0.0
    for r in range(K):
        if not np.isfinite(draft[r]).any():
            draft[r, 0] = 0.0
    return target, draft


@pytest.mark.parametrize("V,K,T,seed,n_neg", CASES)
def test_invariance_sampled_draft(V, K, T, seed, n_neg):
    target, draft = _case(V, K, T, seed, n_neg)
    check_invariance(target, draft, T)


@pytest.mark.parametrize("kb", [0, 1, 2])
def test_invariance_variable_draft_len(kb):
    target, draft = _case(5, 3, 1.0, 10 + kb, 1)
    check_invariance(target, draft, 1.0, kb=kb)


@pytest.mark.parametrize("seed", range(4))
def test_invariance_one_hot_draft(seed):
    rng = np.random.default_rng(100 + seed)
    V, K = 6, 3
    target = rng.normal(0, 1.5, (K + 1, V))
    fixed = rng.integers(0, V, K)
    check_invariance(target, None, 0.9, fixed_draft=fixed)


def test_identical_target_and_draft_never_rejects():
    target, _ = _case(4, 2, 1.0, 42, 0)
    check_invariance(target, target[:2].copy(), 1.0)
