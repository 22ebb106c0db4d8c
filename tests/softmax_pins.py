"""Pins for a row-softmax implementation ``fn(x) -> (y, lse)`` (x 2-D): closed forms,
invariants, a library routine and the pages' online (running max, running sum) merge.
Each pin raises AssertionError on a mismatch.  ``tests/test_softmax_pins.py`` applies them
to the oracle; ``tests/test_oracle_mutants.py`` applies them to planted mistakes."""
from __future__ import annotations

import numpy as np
import scipy.special

import oracle


def pin_constant_row(fn):
    """A constant row c of length C: every output 1/C, lse = c + ln C."""
    for c, n in ((0.0, 1), (2.5, 7), (-40.0, 1000)):
        y, lse = fn(np.full((1, n), c))
        np.testing.assert_allclose(y, 1.0 / n, rtol=1e-15, atol=0)
        assert abs(lse[0] - (c + np.log(n))) < 1e-12


def pin_two_entries(fn):
    """softmax([a, b]) = (sigmoid(a - b), sigmoid(b - a)); lse = ln(e^a + e^b)."""
    a, b = 1.75, -0.5
    y, lse = fn(np.array([[a, b]]))
    s = 1.0 / (1.0 + np.exp(-(a - b)))
    np.testing.assert_allclose(y[0], [s, 1.0 - s], rtol=1e-15)
    assert abs(lse[0] - np.log(np.exp(a) + np.exp(b))) < 1e-14


def pin_scipy(fn):
    """scipy.special.softmax and logsumexp over rows of a non-square array."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((9, 333)) * 4
    y, lse = fn(x)
    np.testing.assert_allclose(y, scipy.special.softmax(x, axis=1), rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(x, axis=1), rtol=1e-14)


def pin_invariants(fn):
    """Rows sum to 1; shifting a row by c leaves y and adds c to lse; no overflow at 1e3."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 64)) * 3
    y, lse = fn(x)
    np.testing.assert_allclose(y.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    y2, lse2 = fn(x + 1000.0)
    assert np.all(np.isfinite(y2))
    np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(lse2, lse + 1000.0, rtol=1e-15)


def pin_minus_infinity(fn):
    """-inf entries get exactly 0 and leave a softmax of the finite entries; an all -inf
    row is NaN throughout (0 / 0)."""
    x = np.array([[0.0, -np.inf, 1.0, -np.inf], [-np.inf] * 4])
    y, lse = fn(x)
    assert y[0, 1] == 0.0 and y[0, 3] == 0.0
    np.testing.assert_allclose(y[0, [0, 2]], scipy.special.softmax([0.0, 1.0]), rtol=1e-15)
    assert np.all(np.isnan(y[1])) and np.isnan(lse[1])


def pin_online_merge(fn):
    """Folding a row chunk by chunk with the pages' (max, sum) merge gives the same lse."""
    rng = np.random.default_rng(5)
    row = rng.standard_normal(1000) * 5
    m, l = -np.inf, 0.0
    for c in range(0, 1000, 96):
        m, l = oracle.chunk_merge(m, l, row[c:c + 96])
    _, lse = fn(row[None, :])
    assert abs((m + np.log(l)) - lse[0]) < 1e-12


SOFTMAX_PINS = [pin_constant_row, pin_two_entries, pin_scipy, pin_invariants, pin_minus_infinity,
                pin_online_merge]
