"""Pins for the fp64 oracle: checks against facts that do not come from the oracle itself.

Each ``pin_*`` function takes the functions under test (a forward ``fwd(q, k, v, scale,
causal) -> (O, lse)`` and/or a backward ``bwd(q, k, v, do, scale, causal) -> (dQ, dK, dV)``,
numpy [B, H, N, d]) and raises AssertionError on a mismatch.  The real oracle must pass
all of them (test_oracle_pins.py); copies of it with a planted mistake must fail at least
one (test_oracle_mutants.py).

What pins what:
  * closed forms: Q = 0 gives the (prefix) mean of V and lse = ln(#visible keys); causal
    row 0 gives V[0]; a one-hot dominant logit selects one V row and gives
    lse = ln(e^c + N - 1); a hand-solved 2-key example with rational probabilities
    (forward and backward);
  * invariants: linearity in V, (K, V) row permutation (non-causal), K shift invariance,
    backward column sums;
  * brute force: pure-Python loops with math.fsum on tiny inputs (no max subtraction,
    no numpy);
  * finite differences of sum(O * dO) for the backward;
  * a library special case: torch CPU float64 scaled_dot_product_attention and autograd.
"""
from __future__ import annotations

import math

import numpy as np

RNG_SEED = 1234


def _rng(seed=RNG_SEED):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------------------- forward
def pin_q_zero(fwd):
    """Q = 0: every visible logit is 0, so P is uniform over the visible keys."""
    rng = _rng()
    B, H, N, d = 2, 3, 37, 8
    q = np.zeros((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    o, lse = fwd(q, k, v, 0.3, False)
    _close(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), 1e-12, "Q=0 non-causal O")
    _close(lse, np.full((B, H, N), math.log(N)), 1e-12, "Q=0 non-causal lse")
    o, lse = fwd(q, k, v, 0.3, True)
    prefix = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    _close(o, prefix, 1e-12, "Q=0 causal O (prefix mean)")
    _close(lse, np.broadcast_to(np.log(np.arange(1, N + 1)), (B, H, N)), 1e-12, "Q=0 causal lse")


def pin_causal_row0(fwd):
    """Causal row 0 sees only key 0: O[0] = V[0] and lse[0] = scale * q0 . k0."""
    rng = _rng(7)
    B, H, N, d = 2, 2, 19, 16
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    o, lse = fwd(q, k, v, 0.25, True)
    _close(o[:, :, 0], v[:, :, 0], 0.0, "causal row 0 O")
    _close(lse[:, :, 0], 0.25 * np.sum(q[:, :, 0] * k[:, :, 0], axis=-1), 1e-13, "causal row 0 lse")


def pin_dominant_logit(fwd):
    """Orthonormal key rows and q_i = c k_pi(i): logits are c*scale at pi(i) and 0 elsewhere.

    Then P_i,pi(i) = e^{cs} / (e^{cs} + N - 1), so O_i -> V_pi(i) and lse_i = ln(e^{cs} + N - 1).
    """
    rng = _rng(11)
    N, d = 12, 16
    basis, _ = np.linalg.qr(rng.standard_normal((d, d)))
    k = basis[:N][None, None]                        # rows orthonormal
    perm = rng.permutation(N)
    c, scale = 40.0, 0.5                             # logit c*scale = 20
    q = c * k[:, :, perm]
    v = rng.standard_normal((1, 1, N, d))
    o, lse = fwd(q, k, v, scale, False)
    cs = c * scale
    w_hit = math.exp(cs) / (math.exp(cs) + N - 1)
    expected = w_hit * v[:, :, perm] + (1 - w_hit) * (v.sum(axis=2, keepdims=True) - v[:, :, perm]) / (N - 1)
    _close(o, expected, 1e-9, "dominant logit O")
    assert np.max(np.abs(o - v[:, :, perm])) < 2 * (N - 1) * math.exp(-cs) * np.max(np.abs(v)) + 1e-12
    _close(lse, np.full((1, 1, N), math.log(math.exp(cs) + N - 1)), 1e-9, "dominant logit lse")


def pin_two_key_example(fwd, bwd=None):
    """Hand-solved example with d = 1, N = 2, scale = 1 (non-causal and causal).

    q = [1, 2], k = [0, ln 3], v = [4, 8].  Logits: row 0 [0, ln 3] -> P = [1/4, 3/4];
    row 1 [0, 2 ln 3 = ln 9] -> P = [1/10, 9/10].  O = [1 + 6, 0.4 + 7.2] = [7, 7.6],
    lse = [ln 4, ln 10].  Causal: row 0 sees key 0 only -> O0 = 4, lse0 = 0.
    Backward with dO = [1, 1]: dV = P^T dO = [0.35, 1.65]; dP = dO v^T = [[4, 8], [4, 8]];
    D = [7, 7.6]; dS = P * (dP - D) = [[-0.75, 0.75], [-0.36, 0.36]];
    dQ = dS k = [0.75 ln 3, 0.36 ln 3]; dK = dS^T q = [-0.75 - 0.72, 0.75 + 0.72].
    Causal backward: P = [[1, 0], [1/10, 9/10]], D = [4, 7.6], dS row 0 = 0;
    dV = [1.1, 0.9], dQ = [0, 0.36 ln 3], dK = [-0.72, 0.72].
    """
    l3 = math.log(3.0)
    q = np.array([1.0, 2.0]).reshape(1, 1, 2, 1)
    k = np.array([0.0, l3]).reshape(1, 1, 2, 1)
    v = np.array([4.0, 8.0]).reshape(1, 1, 2, 1)
    o, lse = fwd(q, k, v, 1.0, False)
    _close(o.ravel(), [7.0, 7.6], 1e-13, "2-key O")
    _close(lse.ravel(), [math.log(4.0), math.log(10.0)], 1e-13, "2-key lse")
    o, lse = fwd(q, k, v, 1.0, True)
    _close(o.ravel(), [4.0, 7.6], 1e-13, "2-key causal O")
    _close(lse.ravel(), [0.0, math.log(10.0)], 1e-13, "2-key causal lse")
    if bwd is None:
        return
    do = np.ones((1, 1, 2, 1))
    dq, dk, dv = bwd(q, k, v, do, 1.0, False)
    _close(dv.ravel(), [0.35, 1.65], 1e-13, "2-key dV")
    _close(dq.ravel(), [0.75 * l3, 0.36 * l3], 1e-13, "2-key dQ")
    _close(dk.ravel(), [-1.47, 1.47], 1e-13, "2-key dK")
    dq, dk, dv = bwd(q, k, v, do, 1.0, True)
    _close(dv.ravel(), [1.1, 0.9], 1e-13, "2-key causal dV")
    _close(dq.ravel(), [0.0, 0.36 * l3], 1e-13, "2-key causal dQ")
    _close(dk.ravel(), [-0.72, 0.72], 1e-13, "2-key causal dK")


def pin_constant_v(fwd):
    """All V rows equal to one vector v: O = v for every row, causal or not."""
    rng = _rng(3)
    B, H, N, d = 1, 2, 23, 8
    q, k = rng.standard_normal((B, H, N, d)) * 2, rng.standard_normal((B, H, N, d))
    row = rng.standard_normal(d)
    v = np.broadcast_to(row, (B, H, N, d)).copy()
    for causal in (False, True):
        o, _ = fwd(q, k, v, 0.4, causal)
        _close(o, v, 1e-12, f"constant V causal={causal}")


def pin_invariants(fwd):
    """Linearity in V; (K, V) row permutation (non-causal); K shift invariance."""
    rng = _rng(5)
    B, H, N, d = 1, 2, 29, 8
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    a = rng.standard_normal((d, d))
    for causal in (False, True):
        o, lse = fwd(q, k, v, 0.35, causal)
        o2, _ = fwd(q, k, v @ a, 0.35, causal)
        _close(o2, o @ a, 1e-11, f"linearity in V causal={causal}")
        u = rng.standard_normal(d)
        o3, lse3 = fwd(q, k + u, v, 0.35, causal)
        _close(o3, o, 1e-11, f"K shift O causal={causal}")
        _close(lse3, lse + 0.35 * (q @ u), 1e-11, f"K shift lse causal={causal}")
    perm = rng.permutation(N)
    o, lse = fwd(q, k, v, 0.35, False)
    o4, lse4 = fwd(q, k[:, :, perm], v[:, :, perm], 0.35, False)
    _close(o4, o, 1e-12, "(K,V) permutation O")
    _close(lse4, lse, 1e-12, "(K,V) permutation lse")
    # Q-row permutation commutes with the (non-causal) output.
    o5, lse5 = fwd(q[:, :, perm], k, v, 0.35, False)
    _close(o5, o[:, :, perm], 1e-12, "Q permutation O")


def _brute_row(qi, keys, vals, scale):
    """Pure-Python attention for one query row: no numpy, no max subtraction, fsum sums."""
    logits = [scale * math.fsum(a * b for a, b in zip(qi, kj)) for kj in keys]
    w = [math.exp(x) for x in logits]
    z = math.fsum(w)
    out = [math.fsum(w[j] * vals[j][c] for j in range(len(keys))) / z for c in range(len(vals[0]))]
    return out, math.log(z)


def pin_bruteforce(fwd):
    """Tiny inputs against pure-Python loops (N <= 6, d <= 3), causal and not."""
    rng = _rng(17)
    for (N, d) in [(1, 1), (2, 3), (5, 2), (6, 3)]:
        q, k, v = (rng.standard_normal((1, 2, N, d)) for _ in range(3))
        for causal in (False, True):
            o, lse = fwd(q, k, v, 0.7, causal)
            for h in range(2):
                for i in range(N):
                    last = i + 1 if causal else N
                    ref_o, ref_lse = _brute_row(list(q[0, h, i]), [list(x) for x in k[0, h, :last]],
                                                [list(x) for x in v[0, h, :last]], 0.7)
                    _close(o[0, h, i], ref_o, 1e-13, f"brute O N={N} d={d} causal={causal}")
                    _close(lse[0, h, i], ref_lse, 1e-13, f"brute lse N={N} d={d} causal={causal}")


def pin_torch_sdpa(fwd):
    """torch CPU float64 scaled_dot_product_attention (a library special case)."""
    import torch
    import torch.nn.functional as F
    rng = _rng(23)
    B, H, N, d = 2, 2, 70, 16
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    for causal in (False, True):
        o, lse = fwd(q, k, v, 0.2, causal)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                             is_causal=causal, scale=0.2).numpy()
        _close(o, ref, 1e-12, f"sdpa O causal={causal}")
        s = 0.2 * torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2)
        if causal:
            s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
        _close(lse, torch.logsumexp(s, dim=-1).numpy(), 1e-12, f"torch logsumexp causal={causal}")


# ---------------------------------------------------------------------------- backward
def _loss(fwd, q, k, v, do, scale, causal):
    o, _ = fwd(q, k, v, scale, causal)
    return float(np.sum(o * do))


def pin_finite_differences(fwd, bwd):
    """Central differences of L = sum(O * dO) in fp64 on tiny inputs (relative err <= 1e-6)."""
    rng = _rng(29)
    h = 1e-6
    for (N, d) in [(1, 2), (3, 2), (5, 4), (8, 3)]:
        q, k, v, do = (rng.standard_normal((1, 1, N, d)) for _ in range(4))
        for causal in (False, True):
            grads = bwd(q, k, v, do, 0.6, causal)
            for which, g in enumerate(grads):
                num = np.zeros_like(g)
                base = [q, k, v]
                for idx in np.ndindex(g.shape):
                    plus = [x.copy() for x in base]
                    minus = [x.copy() for x in base]
                    plus[which][idx] += h
                    minus[which][idx] -= h
                    num[idx] = (_loss(fwd, *plus, do, 0.6, causal) - _loss(fwd, *minus, do, 0.6, causal)) / (2 * h)
                scale_ref = max(1.0, float(np.max(np.abs(num))))
                err = float(np.max(np.abs(num - g))) / scale_ref
                assert err <= 1e-6, f"finite differences {'qkv'[which]} N={N} d={d} causal={causal}: {err:.2e}"


def pin_backward_invariants(fwd, bwd):
    """Column sums and degenerate cases of the backward."""
    rng = _rng(31)
    B, H, N, d = 1, 2, 27, 8
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, v, do, 0.3, causal)
        # sum_j dS_ij = 0 for every row, hence sum_j dK_j = scale * sum_i (sum_j dS_ij) q_i = 0.
        _close(dk.sum(axis=2), np.zeros((B, H, d)), 1e-11, f"sum dK causal={causal}")
        # P rows sum to 1, hence sum_j dV_j = sum_i dO_i.
        _close(dv.sum(axis=2), do.sum(axis=2), 1e-11, f"sum dV causal={causal}")
        # dQ is unchanged by shifting all keys (softmax shift invariance in the K direction).
        dq2, _, _ = bwd(q, k + rng.standard_normal(d), v, do, 0.3, causal)
        _close(dq2, dq, 1e-10, f"dQ under K shift causal={causal}")
    vconst = np.broadcast_to(rng.standard_normal(d), (B, H, N, d)).copy()
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, vconst, do, 0.3, causal)
        _close(dq, np.zeros_like(dq), 1e-12, f"constant V dQ causal={causal}")
        _close(dk, np.zeros_like(dk), 1e-12, f"constant V dK causal={causal}")
    dq, dk, dv = bwd(np.zeros_like(q), k, v, do, 0.3, False)
    _close(dv, np.broadcast_to(do.mean(axis=2, keepdims=True), dv.shape), 1e-12, "Q=0 dV = mean dO")
    # Causal: key N-1 is seen only by query N-1, so dV[N-1] = P[N-1, N-1] dO[N-1].
    dq, dk, dv = bwd(q, k, v, do, 0.3, True)
    o, lse = fwd(q, k, v, 0.3, True)
    p_last = np.exp(0.3 * np.sum(q[:, :, -1] * k[:, :, -1], axis=-1) - lse[:, :, -1])
    _close(dv[:, :, -1], p_last[..., None] * do[:, :, -1], 1e-12, "causal dV of the last key")


def pin_torch_autograd(fwd, bwd):
    """torch CPU float64 autograd through scaled_dot_product_attention (library special case)."""
    import torch
    import torch.nn.functional as F
    rng = _rng(37)
    B, H, N, d = 1, 2, 33, 8
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    for causal in (False, True):
        tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
        out = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.45)
        out.backward(torch.from_numpy(do))
        dq, dk, dv = bwd(q, k, v, do, 0.45, causal)
        _close(dq, tq.grad.numpy(), 1e-12, f"autograd dQ causal={causal}")
        _close(dk, tk.grad.numpy(), 1e-12, f"autograd dK causal={causal}")
        _close(dv, tv.grad.numpy(), 1e-12, f"autograd dV causal={causal}")


FORWARD_PINS = [pin_q_zero, pin_causal_row0, pin_dominant_logit, pin_two_key_example, pin_constant_v,
                pin_invariants, pin_bruteforce, pin_torch_sdpa]
BACKWARD_PINS = [pin_two_key_example, pin_finite_differences, pin_backward_invariants, pin_torch_autograd]
