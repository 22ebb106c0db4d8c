"""The fp64 oracle against closed forms, invariants, brute force, finite differences
and torch's CPU float64 attention (see tests/oracle_pins.py for what pins what)."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.FORWARD_PINS, ids=lambda f: f.__name__)
def test_forward_pin(pin):
    if pin is pins.pin_two_key_example:
        pin(oracle.forward, oracle.backward)
    else:
        pin(oracle.forward)


@pytest.mark.parametrize("pin", [p for p in pins.BACKWARD_PINS if p is not pins.pin_two_key_example],
                         ids=lambda f: f.__name__)
def test_backward_pin(pin):
    pin(oracle.forward, oracle.backward)


def test_probabilities_are_a_distribution():
    """Every row of P is non-negative, sums to 1, and is exactly 0 above the diagonal if causal."""
    rng = np.random.default_rng(41)
    q, k = rng.standard_normal((40, 16)) * 3, rng.standard_normal((40, 16))
    for causal in (False, True):
        p, m, l = oracle.probabilities(q, k, 0.25, causal)
        assert np.all(p >= 0)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        if causal:
            assert np.all(p[np.triu_indices(40, 1)] == 0.0)
            assert np.all(p[np.diag_indices(40)] > 0.0)


def test_forward_rows_matches_forward():
    """Evaluating selected rows equals the same rows of the full forward."""
    rng = np.random.default_rng(43)
    B, H, N, d = 2, 3, 50, 8
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    rows = np.stack([np.stack([np.sort(rng.choice(N, 9, replace=False)) for _ in range(H)]) for _ in range(B)])
    for causal in (False, True):
        o, lse = oracle.forward(q, k, v, 0.3, causal)
        o_r, lse_r = oracle.forward_rows(q, k, v, 0.3, causal, rows)
        np.testing.assert_allclose(o_r, np.take_along_axis(o, rows[..., None], axis=2), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse_r, np.take_along_axis(lse, rows, axis=2), rtol=0, atol=1e-13)


def test_d_identity():
    """D_i = sum_j P_ij dP_ij equals rowsum(dO * O) (the form a recomputing backward uses)."""
    rng = np.random.default_rng(47)
    q, k, v, do = (rng.standard_normal((31, 8)) for _ in range(4))
    for causal in (False, True):
        p, _, _ = oracle.probabilities(q, k, 0.5, causal)
        o = p @ v
        dp = do @ v.T
        np.testing.assert_allclose(np.sum(p * dp, axis=1), np.sum(do * o, axis=1), rtol=0, atol=1e-12)


def test_large_logits_do_not_overflow():
    """Logits far beyond exp's range stay finite (the max is subtracted first)."""
    rng = np.random.default_rng(53)
    q, k, v = (rng.standard_normal((1, 1, 16, 4)) for _ in range(3))
    o, lse = oracle.forward(q * 1e3, k, v, 1.0, True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert np.max(np.abs(o)) <= np.max(np.abs(v)) + 1e-12
