"""Planted mistakes in the oracle (CPU only): each must be caught by a pin.

These show that the pins are strong enough: a dropped max(0, .), swapped
operands, the wrong prefix convention or a flipped comparison each fail one of
the invariance / closed-form checks.
"""

import numpy as np
import pytest

import oracle.chain as chain
from test_oracle_invariance import _case, check_invariance


def _real_inverse_cdf():
    return chain.inverse_cdf_sample


@pytest.mark.parametrize("mutant", [
    lambda p, q: np.abs(p - q),               # max(0, .) dropped
    lambda p, q: np.maximum(0.0, q - p),      # operands swapped
    lambda p, q: p,                           # residual replaced by p
])
def test_wrong_residual_is_caught(monkeypatch, mutant):
    monkeypatch.setattr(chain, "residual_weights", mutant)
    target, draft = _case(4, 2, 1.0, 2, 0)
    with pytest.raises(AssertionError):
        check_invariance(target, draft, 1.0)


@pytest.mark.parametrize("mutant", [
    lambda p, q: min(1.0, q / p) if p > 0 else 1.0,   # ratio inverted
    lambda p, q: min(1.0, p),                         # q ignored
])
def test_wrong_acceptance_is_caught(monkeypatch, mutant):
    monkeypatch.setattr(chain, "acceptance_probability", mutant)
    target, draft = _case(4, 2, 1.0, 2, 0)
    with pytest.raises(AssertionError):
        check_invariance(target, draft, 1.0)


def test_exclusive_prefix_convention_is_caught(monkeypatch):
    real = _real_inverse_cdf()

    def shifted(w, u):
        i, gap, W = real(w, u)
        return min(i + 1, len(w) - 1), gap, W

    monkeypatch.setattr(chain, "inverse_cdf_sample", shifted)
    target, draft = _case(4, 2, 1.0, 2, 0)
    with pytest.raises(AssertionError):
        check_invariance(target, draft, 1.0)


def test_strict_accept_comparison_is_caught(monkeypatch):
    # accept iff r < alpha (instead of r <= alpha) flips the exact-boundary hand case
    import test_oracle_chain as hand

    monkeypatch.setattr(chain, "accept_test", lambda r, alpha: r < alpha)
    with pytest.raises(AssertionError):
        hand.test_accept_boundary_is_inclusive()


def test_dropped_cap_is_caught(monkeypatch):
    # alpha = p/q without min(1, .) decides identically for r <= 1 but reports alpha > 1
    import test_oracle_chain as hand

    monkeypatch.setattr(chain, "acceptance_probability", lambda p, q: p / q if q > 0 else 1.0)
    with pytest.raises(AssertionError):
        hand.test_alpha_one_accepts_u_equal_one_and_alpha_zero_rejects_smallest_u()
