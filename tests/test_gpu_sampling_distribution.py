"""The GPU's draws reproduce the target distribution ("Speculative Decoding in Production",
section I.1, "The Invariance Theorem": verifying drafts drawn from q by the modified rejection
rule emits tokens distributed as p).

Every other GPU test compares the HIP path with the oracle on the same uniforms.  This one
checks the claim itself, with no oracle decision in the loop: at a tiny vocabulary, batches of
sequences that share one set of rows, each with fresh drafts x_k ~ q_k and fresh uniforms,
are verified on the GPU, and the emitted tokens are tested against p by chi-square:

  * the first emitted token against p_0 (all sequences);
  * the token after one accepted draft against p_1 (sequences with n >= 1);
  * the bonus token after every draft is accepted against p_K (sequences with n = K);
  * the mean accepted count against its closed form sum_j prod_{k<j} sum_x min(p_k, q_k)
    (invariance, E[n]), by a normal approximation.

Cases: sampled drafts (fp32 and bf16 logits), one-hot drafts (q = the point mass at the
proposed token: alpha = p(x), residual = p without x), and a bonus-heavy batch (q close to
p).  Each case runs CALLS calls of B sequences (about 10^6 first tokens).  A histogram fails
when its p-value is below P_MIN (family-wise, about 1e-3 over the whole file); the tests stop
at the first failure.  Expected probabilities come from the oracle's float64 softmax of the
same stored logit values.
"""

import numpy as np
import pytest
import torch
from scipy import stats

import oracle
import synth
from gpu_helpers import chain_on_gpu, log

pytestmark = pytest.mark.gpu

B = 1 << 17
CALLS = 8
P_MIN = 1e-4
Z_MAX = 4.5


def _rows(case):
    rng = np.random.default_rng({"sampled": 1, "bf16": 2, "onehot": 3, "bonus": 4}[case])
    V, K = 7, 2
    t = (rng.standard_normal((K + 1, V)) * 0.8).astype(np.float32)
    if case == "bonus":
        d = t[:K] + (rng.standard_normal((K, V)) * 0.15).astype(np.float32)
    else:
        d = t[:K] + (rng.standard_normal((K, V)) * 1.0).astype(np.float32)
    if case == "bf16":
        return synth.bf16_bits_from_f32(t), synth.bf16_bits_from_f32(d), "bf16", 0.8
    if case == "onehot":
        return t, None, "f32", 1.0
    return t, d, "f32", 1.0


def _chisq(counts, probs, what):
    n = counts.sum()
    exp = probs * n
    assert exp.min() >= 50, f"{what}: expected counts too small ({exp.min():.1f})"
    chi, pv = stats.chisquare(counts, exp)
    log(f"[chi2] {what}: n={n} chi2={chi:.2f} dof={len(probs) - 1} p={pv:.4f}")
    assert pv >= P_MIN, f"{what}: p-value {pv:.2e} < {P_MIN}"


@pytest.mark.parametrize("case", ["sampled", "bf16", "onehot", "bonus"])
def test_emitted_tokens_follow_the_target_distribution(case):
    target, draft, dtype, T = _rows(case)
    widen = lambda r: oracle.widen_logits(r, dtype)  # noqa: E731
    K1, V = target.shape
    K = K1 - 1
    p = [oracle.softmax_at_temperature(widen(target[k]), T) for k in range(K1)]
    # one-hot drafts propose each row's most likely token, so that all three histograms fill
    onehot_tokens = np.array([int(np.argmax(widen(target[k]))) for k in range(K)], dtype=np.int32)
    if draft is None:
        # q_k is the point mass at x_k: E[n] = sum_j prod_{k<j} p_k(x_k)
        beta = [float(p[k][onehot_tokens[k]]) for k in range(K)]
    else:
        q = [oracle.softmax_at_temperature(widen(draft[k]), T) for k in range(K)]
        beta = [float(np.minimum(p[k], q[k]).sum()) for k in range(K)]
    first = np.zeros(V, np.int64)
    second = np.zeros(V, np.int64)
    bonus = np.zeros(V, np.int64)
    n_sum = 0
    n_sq = 0
    for call in range(CALLS):
        inp = synth.chain_shared_rows(900 + call, call, target=target, draft=draft, dtype=dtype, B=B, temperature=T,
                                      tokens=onehot_tokens, name=case)
        g = chain_on_gpu(inp, want_packed=False)
        tok = g.tokens.cpu().numpy()
        n = g.num_accepted.cpu().numpy().astype(np.int64)
        torch.cuda.synchronize()
        assert (n >= 0).all() and (n <= K).all()
        first += np.bincount(tok[:, 0], minlength=V)
        second += np.bincount(tok[n >= 1, 1], minlength=V)
        bonus += np.bincount(tok[n == K, K], minlength=V)
        n_sum += int(n.sum())
        n_sq += int((n * n).sum())
    total = B * CALLS
    log(f"[chi2] {case}: {total} sequences, {CALLS} calls of {B}; accept rates {np.round(beta, 4).tolist()}")
    _chisq(first, p[0], f"{case}: first token vs p_0")
    _chisq(second, p[1], f"{case}: token after one accepted draft vs p_1")
    _chisq(bonus, p[K], f"{case}: bonus token after {K} accepted drafts vs p_{K}")
    expect = sum(float(np.prod(beta[:j])) for j in range(1, K + 1))
    mean = n_sum / total
    var = n_sq / total - mean * mean
    z = (mean - expect) / np.sqrt(var / total)
    log(f"[chi2] {case}: mean accepted {mean:.5f}, closed form {expect:.5f}, z = {z:.2f}")
    assert abs(z) <= Z_MAX
