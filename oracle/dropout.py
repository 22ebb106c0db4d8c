"""fp64 CPU oracle for attention with dropout on the probabilities -- test infrastructure.

TEST INFRASTRUCTURE ONLY (same rule as ``oracle.attention``: only tests, the smoke check
and the bench's CPU baseline may use it; the HIP library never does, and this module
imports nothing from it).

"How FlashAttention Actually Works" -- "The GPU Memory Wall: HBM vs. SRAM" lists dropout
among the steps of standard attention (matmul, mask, softmax, dropout, matmul) that a fused
kernel runs on chip.  The pages define neither the random numbers nor where the mask applies;
this module fixes them as follows:

  * Random numbers: Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and
    Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011): a 128-bit counter
    (c0, c1, c2, c3) and a 64-bit key (k0, k1); ten rounds of
        (hi0, lo0) = 0xD2511F53 * c0,  (hi1, lo1) = 0xCD9E8D57 * c2   (32 x 32 -> 64 bits)
        (c0, c1, c2, c3) <- (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0)
    with the key bumped by (0x9E3779B9, 0xBB67AE85) between rounds.
  * Mask: for head bh = b * H + h, query i and key j, one call with counter
    (j >> 2, i >> 2, bh, offset) and key (seed mod 2^32, seed >> 32) covers the 4 x 4 block
    of (query, key) pairs; element (i, j) reads byte (j & 3) of output word (i & 3) as an
    8-bit integer u and is kept iff u >= t, t = round(256 p) clamped to [0, 256].
  * Keep scale: an element is kept with probability (256 - t) / 256 exactly, so kept values
    are scaled by s = 256 / (256 - t) (s = 0 when t = 256 and nothing is kept), which makes
    E[Z] = 1 exactly (inverted dropout); 1 / (1 - p) would be biased by the rounding of t.
  * Where it applies: O = (P o Z) V with Z = keep * s; lse stays the logsumexp of
    the undropped scores (the softmax is not renormalised after dropout).  Gradients of
    L = sum(O * dO) then follow with dP = Z o (dO V^T): dV = (P o Z)^T dO,
    D_i = sum_j P_ij dP_ij = rowsum(dO * O)_i, dS = P o (dP - D), dQ = scale dS K,
    dK = scale dS^T Q.
"""
from __future__ import annotations

import numpy as np

from .attention import probabilities

__all__ = ["philox4x32_10", "keep_mask", "keep_scale", "forward_dropout", "backward_dropout"]

_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = np.uint32(0x9E3779B9), np.uint32(0xBB67AE85)
_LO = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with ten rounds on arrays of 32-bit counters (broadcast) and a 32-bit key
    pair.  Returns the four 32-bit output words as uint32 arrays."""
    c = [np.asarray(x, dtype=np.uint32) for x in np.broadcast_arrays(c0, c1, c2, c3)]
    k0, k1 = np.uint32(k0), np.uint32(k1)
    with np.errstate(over="ignore"):
        for r in range(10):
            p0 = _M0 * c[0].astype(np.uint64)
            p1 = _M1 * c[2].astype(np.uint64)
            hi0, lo0 = (p0 >> np.uint64(32)).astype(np.uint32), (p0 & _LO).astype(np.uint32)
            hi1, lo1 = (p1 >> np.uint64(32)).astype(np.uint32), (p1 & _LO).astype(np.uint32)
            c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
            if r < 9:
                k0, k1 = np.uint32(k0 + _W0), np.uint32(k1 + _W1)
    return c


def threshold(p: float) -> int:
    """The 8-bit threshold of dropout probability p: round(256 p), clamped to [0, 256]."""
    return int(min(256, max(0, int(np.floor(256.0 * float(p) + 0.5)))))


def keep_scale(p: float) -> float:
    """The factor s of kept values: the reciprocal of the exact keep probability (256 - t) / 256
    of the 8-bit threshold t, or 0 when t = 256 (nothing is kept)."""
    t = threshold(p)
    return 0.0 if t == 256 else 256.0 / (256 - t)


def keep_mask(bh: int, n_q: int, n_k: int, p: float, seed: int, offset: int) -> np.ndarray:
    """Boolean [n_q, n_k] keep mask of head bh (see the module docstring)."""
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    words = philox4x32_10(j >> 2, i >> 2, np.uint32(bh), np.uint32(offset),
                          np.uint32(seed & 0xFFFFFFFF), np.uint32((seed >> 32) & 0xFFFFFFFF))
    w = np.choose(i & 3, words)  # word (i & 3)
    u = (w >> (8 * (j & 3)).astype(np.uint32)) & np.uint32(0xFF)
    return u >= threshold(p)


def forward_dropout(q, k, v, scale: float, causal: bool, p: float, seed: int, offset: int = 0, bh0: int = 0):
    """O = (P o Z) V and the undropped lse, per (batch, head); arrays [B, H, N, d].

    The mask of array head (b, h) is that of head index bh0 + b * H + h (bh0 places a slice
    of heads inside a larger batch)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, N, _ = q.shape
    o = np.empty_like(v)
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            pr, m, l = probabilities(q[b, h], k[b, h], scale, causal)
            z = keep_mask(bh0 + b * H + h, N, N, p, seed, offset) * keep_scale(p)
            o[b, h] = (pr * z) @ v[b, h]
            lse[b, h] = m + np.log(l)
    return o, lse


def backward_dropout(q, k, v, do, scale: float, causal: bool, p: float, seed: int, offset: int = 0, bh0: int = 0):
    """(dQ, dK, dV) of L = sum(O * dO) for the forward above; arrays [B, H, N, d] (bh0 as
    in ``forward_dropout``)."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, H, N, _ = q.shape
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    for b in range(B):
        for h in range(H):
            pr, _, _ = probabilities(q[b, h], k[b, h], scale, causal)
            z = keep_mask(bh0 + b * H + h, N, N, p, seed, offset) * keep_scale(p)
            g = do[b, h]
            dv[b, h] = (pr * z).T @ g
            dp = z * (g @ v[b, h].T)
            dd = np.sum(pr * dp, axis=1)
            ds = pr * (dp - dd[:, None])
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
    return dq, dk, dv
