"""Online-softmax re-derivations used to pin the exactness claim (fp64, CPU).

TEST INFRASTRUCTURE ONLY (same rule as ``oracle.attention``: only tests, the smoke
check and the bench's CPU baseline may use it; the HIP library never does).

Both pieces come from one equation, the merge of two running (max, sum) pairs in
"How does FlashAttention optimize memory and speed via tiling?" -- "Core Technical
Innovations in FlashAttention", item 2 (the page writes the running sum as d, here l):
    m = max(m1, m2),   l = e^{m1 - m} l1 + e^{m2 - m} l2.

* ``chunk_merge`` -- that merge for one new chunk of logits of a single row, whose own
  pair is (max(chunk), sum(e^{chunk - max(chunk)})).  The same page's "Example" names
  this step for a chunk.

* ``tiled_forward`` -- attention over key blocks.  Each key block j yields, for every
  query row, its own triple (m_j, l_j, O_j): the block's row maximum, the sum of
  e^{s - m_j} over the block, and the unnormalised output sum of e^{s - m_j} v.  The
  triples are folded left to right with the merge above, the output carried with the
  same two factors as the sum; the result is O / l.  Tiling into blocks and rescaling
  earlier partial results when the maximum grows is "Breaking the Memory Wall: A Deep
  Dive into FlashAttention" -- "The Solution: IO-Awareness & Tiling", items 1-2.

  ``exp_reference="block"`` drops the merge's factor e^{m_j - m} on the incoming block,
  leaving its exponentials against the block's own maximum while the history is still
  rescaled.  That is how the printed simulation on "Breaking the Memory Wall" --
  "Implementation" reads, and a test shows it misses that page's own 1e-5 check; the
  merge equation (``"running"``) is the reading taken.

Both exist to show, in fp64, that tiling plus online rescaling reproduces the plain
definition in ``oracle.attention`` (the pages' "exact" claim), not to serve as the
parity reference.
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


def _block_triple(q, kb, vb, scale, causal, j0):
    """(m_j, l_j, O_j) of one key block starting at key j0, for every query row; rows that
    see no key of the block get (-inf, 0, 0)."""
    s = scale * np.einsum("bid,bjd->bij", q, kb)
    if causal:
        s = np.where(np.arange(j0, j0 + kb.shape[1])[None, None, :] > np.arange(q.shape[1])[None, :, None],
                     -np.inf, s)
    m = np.max(s, axis=-1)
    e = np.exp(s - np.where(np.isneginf(m), 0.0, m)[..., None])  # exp(-inf) = 0 where masked
    return m, e.sum(-1), np.einsum("bij,bjd->bid", e, vb)


def tiled_forward(q, k, v, scale: float, block_size: int, causal: bool = False,
                  exp_reference: str = "running"):
    """Attention by folding per-key-block (max, sum, output) triples with the merge
    equation; q, k, v are [Bt, N, d] (Bt = batch*heads).  Returns O [Bt, N, d] (float64).
    ``exp_reference`` selects the merge ("running") or the page listing's slip ("block");
    see the module docstring."""
    if exp_reference not in ("running", "block"):
        raise ValueError(exp_reference)
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    n = k.shape[1]
    m = l = o = None
    for j0 in range(0, n, block_size):
        mj, lj, oj = _block_triple(q, k[:, j0:j0 + block_size], v[:, j0:j0 + block_size], scale, causal, j0)
        if m is None:
            m, l, o = mj, lj, oj
            continue
        m_new = np.maximum(m, mj)
        base = np.where(np.isneginf(m_new), 0.0, m_new)
        f_old = np.where(np.isneginf(m), 0.0, np.exp(m - base))
        if exp_reference == "running":
            f_blk = np.where(np.isneginf(mj), 0.0, np.exp(mj - base))
        else:
            f_blk = np.ones_like(mj)
        l = f_old * l + f_blk * lj
        o = f_old[..., None] * o + f_blk[..., None] * oj
        m = m_new
    return o / l[..., None]
