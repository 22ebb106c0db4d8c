"""Plain fp64 CPU oracle for exact self-attention (forward and backward).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from it.

What it computes is the plain definition of attention, with the N x N score
matrix S and probability matrix P materialised explicitly, per (batch, head):

    S = scale * Q K^T                       (masked to -inf above the diagonal if causal)
    P = softmax_rows(S)                     exp(S - rowmax) / rowsum
    O = P V,   lse = rowmax + ln(rowsum)

Sources (page title -- section):
  * "Breaking the Memory Wall: A Deep Dive into FlashAttention" -- "The Problem:
    The Memory Wall" defines P = softmax(Q K^T / sqrt(d)); "2. The Incremental
    Softmax Trick" gives the softmax definition e^{x_i} / sum_j e^{x_j};
    "3. Backward Pass Recomputation" says the backward keeps only the
    normalisation factors (here the per-row logsumexp, lse) and recomputes P.
  * "How does FlashAttention optimize memory and speed via tiling?" -- "Detail"
    names S = Q K^T and P = softmax(S) as the matrices standard attention
    materialises; "Interview tips" and every page's summary state that the
    tiled method is exact, so the tiled GPU result must equal this definition
    up to floating-point summation order.
  * "How FlashAttention Actually Works" -- "The Secret Weapon: Online Softmax":
    the max is subtracted before exponentiation to avoid overflow.

Readings where the pages are silent:
  * causal: key j > query i is masked (square, top-left aligned; diagonal kept);
  * lse is the natural-log logsumexp of the *scaled* logits, lse = m + ln l;
  * gradients for the loss L = sum(O * dO) come from the softmax Jacobian
    diag(p) - p p^T (the pages give no gradient formulas):
        dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,
        dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.

All arithmetic is float64; inputs are upcast exactly (bf16 and fp32 values are
representable in fp64).  Arrays are numpy, layout [B, H, N, d].
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "scores",
    "probabilities",
    "forward",
    "forward_rows",
    "backward",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def scores(q: np.ndarray, k: np.ndarray, scale: float, causal: bool) -> np.ndarray:
    """S = scale * q k^T for one head (q [N, d], k [N, d]); causal entries j > i are -inf.

    "Breaking the Memory Wall" -- "The Problem: The Memory Wall" (the QK^T / sqrt(d)
    inside the softmax); the causal mask is the reading stated in the module header.
    """
    q = _f64(q)
    k = _f64(k)
    s = float(scale) * (q @ k.T)
    if causal:
        n_q, n_k = s.shape
        above = np.triu(np.ones((n_q, n_k), dtype=bool), k=1)
        s = np.where(above, -np.inf, s)
    return s


def probabilities(q: np.ndarray, k: np.ndarray, scale: float, causal: bool):
    """Row softmax of the scores for one head: returns (P, m, l).

    m_i = max_j S_ij and l_i = sum_j exp(S_ij - m_i), so P = exp(S - m) / l.
    "Breaking the Memory Wall" -- "2. The Incremental Softmax Trick" (softmax
    definition); "How FlashAttention Actually Works" -- "The Secret Weapon:
    Online Softmax" (the running maximum guards the exponential).
    """
    s = scores(q, k, scale, causal)
    m = np.max(s, axis=1)
    e = np.exp(s - m[:, None])  # exp(-inf) == 0 for masked entries
    l = np.sum(e, axis=1)
    return e / l[:, None], m, l


def forward(q, k, v, scale: float, causal: bool):
    """O = softmax(scale q k^T) v and lse = m + ln l for every (b, h); [B,H,N,d] -> (O, lse).

    "Breaking the Memory Wall" -- "The Problem: The Memory Wall" (P and the weighted
    sum); "3. Backward Pass Recomputation" (the saved normalisation factor, read as lse).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    bsz, heads, n, d = q.shape
    o = np.empty((bsz, heads, n, v.shape[-1]), dtype=np.float64)
    lse = np.empty((bsz, heads, n), dtype=np.float64)
    for b in range(bsz):
        for h in range(heads):
            p, m, l = probabilities(q[b, h], k[b, h], scale, causal)
            o[b, h] = p @ v[b, h]
            lse[b, h] = m + np.log(l)
    return o, lse


def forward_rows(q, k, v, scale: float, causal: bool, rows):
    """The same definition evaluated only at selected query rows.

    ``rows`` is an int array [B, H, R] of query indices.  Returns (O_rows [B,H,R,d],
    lse_rows [B,H,R]).  Each row i uses every key (or keys 0..i when causal) exactly
    as ``forward`` does; restricting to rows changes no arithmetic, it only avoids
    materialising rows nobody compares.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    rows = np.asarray(rows)
    bsz, heads, r = rows.shape
    o = np.empty((bsz, heads, r, v.shape[-1]), dtype=np.float64)
    lse = np.empty((bsz, heads, r), dtype=np.float64)
    for b in range(bsz):
        for h in range(heads):
            idx = rows[b, h]
            s = float(scale) * (q[b, h, idx] @ k[b, h].T)  # [R, N]
            if causal:
                s = np.where(np.arange(s.shape[1])[None, :] > idx[:, None], -np.inf, s)
            m = np.max(s, axis=1)
            e = np.exp(s - m[:, None])
            l = np.sum(e, axis=1)
            o[b, h] = (e / l[:, None]) @ v[b, h]
            lse[b, h] = m + np.log(l)
    return o, lse


def backward(q, k, v, do, scale: float, causal: bool):
    """Gradients of L = sum(O * dO) with respect to q, k, v, by the explicit formulas.

    P is recomputed from q and k ("How FlashAttention Actually Works" -- "The Backward
    Pass: Recomputation"; "Breaking the Memory Wall" -- "3. Backward Pass
    Recomputation").  The gradient formulas themselves are not on the pages; they are
    the softmax Jacobian written out (module header).  Returns (dQ, dK, dV), [B,H,N,d].
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    bsz, heads = q.shape[:2]
    for b in range(bsz):
        for h in range(heads):
            p, _, _ = probabilities(q[b, h], k[b, h], scale, causal)
            g = do[b, h]
            dv[b, h] = p.T @ g
            dp = g @ v[b, h].T
            dd = np.sum(p * dp, axis=1)
            ds = p * (dp - dd[:, None])
            dq[b, h] = float(scale) * (ds @ k[b, h])
            dk[b, h] = float(scale) * (ds.T @ q[b, h])
    return dq, dk, dv
