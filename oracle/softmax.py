"""Plain fp64 CPU oracle for the row-wise softmax (and its logsumexp) -- test infrastructure.

TEST INFRASTRUCTURE ONLY (same rule as ``oracle.attention``: only ``tests/``, the smoke
check and the bench's CPU baseline may use it; the HIP library never does, and this module
imports nothing from it).

What it computes is the definition, per row r of a [R, C] array x:

    m_r   = max_c x[r, c]
    y[r]  = exp(x[r] - m_r) / sum_c exp(x[r, c] - m_r)
    lse_r = m_r + ln sum_c exp(x[r, c] - m_r)

Sources (page title -- section):
  * "Breaking the Memory Wall: A Deep Dive into FlashAttention" -- "2. The Incremental
    Softmax Trick" states the softmax e^{x_i} / sum_j e^{x_j} of a row.
  * "How FlashAttention Actually Works" -- "The Secret Weapon: Online Softmax": the row
    maximum is subtracted before exponentiating so nothing overflows, and the running
    (max, sum) pair can be built block by block; the standalone kernel this oracle checks
    computes that pair in one pass and then normalises, which reaches this definition up
    to floating-point summation order.

Readings where the pages are silent: -inf entries are
allowed and give exact zeros; a row whose entries are all -inf has no softmax (0 / 0)
and yields NaN in every output of the row and in its lse, as the definition evaluates;
lse is the natural-log logsumexp.  All arithmetic is float64; inputs are upcast exactly.
"""
from __future__ import annotations

import numpy as np

__all__ = ["softmax_rows"]


def softmax_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """Row-wise softmax of a 2-D array and the natural-log logsumexp of each row.

    Returns (y [R, C] float64, lse [R] float64).
    """
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("x must be 2-D [rows, cols]")
    with np.errstate(invalid="ignore"):
        m = np.max(x, axis=1)
        e = np.exp(x - m[:, None])        # all -inf row: -inf - -inf = nan, as the definition
        l = np.sum(e, axis=1)
        return e / l[:, None], m + np.log(l)
