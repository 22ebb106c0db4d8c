"""Online-softmax re-derivations used to pin the exactness claim (fp64, CPU).

TEST INFRASTRUCTURE ONLY (same rule as ``oracle.attention``: only tests, the smoke
check and the bench's CPU baseline may use it; the HIP library never does).

Two pieces, both written from the pages' description, in their order and notation:

* ``chunk_merge`` -- one step of the running (max, sum) update for a chunk of
  logits: m2 = max(m1, max(chunk)), l2 = e^{m1 - m2} l1 + sum(e^{chunk - m2}).
  "How does FlashAttention optimize memory and speed via tiling?" -- "Core
  Technical Innovations in FlashAttention", item 2 (the merge equation; the page
  writes the running sum as d, here l) and "Example" (the chunk function).

* ``tiled_forward`` -- the block-by-block forward of "Breaking the Memory Wall: A
  Deep Dive into FlashAttention" -- "Implementation: Simulating FlashAttention in
  PyTorch": outer loop over K/V blocks, inner loop over Q blocks, running m, l and
  unnormalised O kept per query row, final O / l.  The exponentials are taken
  against the *updated running* maximum (``exp_reference="running"``), which is
  what the merge equation above states.  The page's listing instead exponentiates
  each block against that block's own maximum while rescaling the history by
  e^{m_old - m_new}; ``exp_reference="block"`` reproduces that reading so a test
  can show it misses the page's own 1e-5 check, which is why the running reading
  is the one taken.

Both exist to show, in fp64, that tiling plus online rescaling reproduces the
plain definition in ``oracle.attention`` (the pages' "exact" claim), not to serve
as the parity reference.
"""
from __future__ import annotations

import numpy as np

__all__ = ["chunk_merge", "tiled_forward"]


def chunk_merge(prev_max: float, prev_sum: float, chunk) -> tuple[float, float]:
    """Merge one chunk of logits into a running (max, sum) pair (scalar row)."""
    chunk = np.asarray(chunk, dtype=np.float64)
    new_max = max(float(prev_max), float(np.max(chunk)))
    # e^{prev_max - new_max} rescales the history; prev_max = -inf contributes 0.
    carry = 0.0 if prev_sum == 0.0 else np.exp(prev_max - new_max) * prev_sum
    return new_max, float(carry + np.sum(np.exp(chunk - new_max)))


def tiled_forward(q, k, v, scale: float, block_size: int, causal: bool = False,
                  exp_reference: str = "running"):
    """Block-tiled forward with online softmax; q, k, v are [Bt, N, d] (Bt = batch*heads).

    Returns O [Bt, N, d] (float64).  ``exp_reference`` selects which maximum each
    block's exponentials use (see the module docstring).
    """
    if exp_reference not in ("running", "block"):
        raise ValueError(exp_reference)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    bt, n, _ = q.shape
    acc = np.zeros((bt, n, v.shape[-1]))
    run_max = np.full((bt, n), -np.inf)
    run_sum = np.zeros((bt, n))
    for j0 in range(0, n, block_size):
        kb = k[:, j0:j0 + block_size]
        vb = v[:, j0:j0 + block_size]
        for i0 in range(0, n, block_size):
            qb = q[:, i0:i0 + block_size]
            s = scale * np.einsum("bid,bjd->bij", qb, kb)
            if causal:
                qi = np.arange(i0, i0 + qb.shape[1])[:, None]
                kj = np.arange(j0, j0 + kb.shape[1])[None, :]
                s = np.where(kj > qi, -np.inf, s)
            blk_max = np.max(s, axis=-1)
            m_old = run_max[:, i0:i0 + qb.shape[1]]
            m_new = np.maximum(m_old, blk_max)
            # Rows with nothing visible yet keep m = -inf; use 0 as their exponent base.
            safe_new = np.where(np.isneginf(m_new), 0.0, m_new)
            alpha = np.where(np.isneginf(m_old), 0.0, np.exp(m_old - safe_new))
            if exp_reference == "running":
                ref = safe_new
            else:
                ref = np.where(np.isneginf(blk_max), 0.0, blk_max)
            p = np.exp(s - ref[..., None])
            run_sum[:, i0:i0 + qb.shape[1]] = alpha * run_sum[:, i0:i0 + qb.shape[1]] + p.sum(-1)
            acc[:, i0:i0 + qb.shape[1]] = (alpha[..., None] * acc[:, i0:i0 + qb.shape[1]]
                                           + np.einsum("bij,bjd->bid", p, vb))
            run_max[:, i0:i0 + qb.shape[1]] = m_new
    return acc / run_sum[..., None]
