"""Helpers for the GPU parity tests: move seeded cases to the device, read results back,
and compare with the oracle under the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np

# fp32 inputs: max-abs <= 1e-4.  bf16 inputs with fp32 accumulation: max-abs <= 2e-2 and
# mean-abs <= 2e-3.  Applied to every compared output (O, lse, dQ, dK, dV).
TOL = {"f32": {"max_abs": 1e-4, "mean_abs": None}, "bf16": {"max_abs": 2e-2, "mean_abs": 2e-3}}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def to_device(case: dict, name: str):
    import torch
    t = case[name]
    if case["dtype"] == "bf16":
        host = torch.from_numpy(t["bits"].view(np.int16)).view(torch.bfloat16)
    else:
        host = torch.from_numpy(np.ascontiguousarray(t["values"]))
    return host.to("cuda").contiguous()


def to_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if not np.all(np.isfinite(got)):
        return float("inf"), float("inf")
    d = np.abs(got - ref)
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0


# Unit roundoff of bfloat16 (8 significant bits, round to nearest even): storing x in bf16
# moves it by at most BF16_U * |x|.
BF16_U = 2.0 ** -8


def bwd_condition(q, k, v, do, scale: float, causal: bool):
    """Per-element condition sums of the three gradient products of one head, in fp64.

    Each gradient is a sum of products whose left factor the kernels round to bf16 before
    the MFMA: dV = P^T dO (P rounded), dK = scale dS^T Q and dQ = scale dS K (dS rounded).
    Rounding a_i to bf16 moves sum_i a_i b_i by at most BF16_U * sum_i |a_i| |b_i|, and
    storing the result in bf16 moves it by at most BF16_U * |result|, itself at most the
    same sum.  Returns (cond_dQ, cond_dK, cond_dV) = (scale |dS| |K|, scale |dS|^T |Q|,
    |P|^T |dO|), each [N, d], with P and dS from the oracle's recomputation.
    """
    from oracle import attention as oracle
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    p, _, _ = oracle.probabilities(q, k, scale, causal)
    dp = do @ v.T
    ads = np.abs(p * (dp - np.sum(p * dp, axis=1)[:, None]))
    return scale * (ads @ np.abs(k)), scale * (ads.T @ np.abs(q)), p.T @ np.abs(do)


def assert_parity(what: str, got, ref, dtype: str, cond=None, mean_cond: bool = False) -> tuple[float, float]:
    """Element-wise comparison under the stated tolerance.

    ``cond`` (same shape as ``ref``) widens the element-wise bound to
    max_abs + 2 * BF16_U * cond: the first-order rounding bound of a bf16-rounded factor
    plus a bf16-stored output (see ``bwd_condition``).  It is passed only where the
    gradients grow past 8 in magnitude, where half a bf16 ulp (>= 1/32) alone already
    exceeds the 2e-2 bound.  The mean-abs bound is unchanged unless ``mean_cond`` adds the
    mean of the same first-order rounding, BF16_U * mean(cond).
    """
    mx, mean = errors(got, ref)
    tol = TOL[dtype]
    log(f"  {what}: max-abs {mx:.3e} mean-abs {mean:.3e} (tol {tol['max_abs']:.0e}"
        f"{'' if tol['mean_abs'] is None else ' / %.0e' % tol['mean_abs']}"
        f"{' + 2^-7 cond' if cond is not None else ''})")
    if cond is not None:
        g, r = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
        c = np.asarray(cond, dtype=np.float64).reshape(r.shape)
        excess = np.abs(g - r) - (tol["max_abs"] + 2 * BF16_U * c)
        log(f"  {what}: worst (err - {tol['max_abs']:.0e}) / cond = "
            f"{np.max((np.abs(g - r) - tol['max_abs']) / np.maximum(c, 1e-30)):.3e} (bound {2 * BF16_U:.3e})")
        assert np.all(np.isfinite(g)) and excess.max() <= 0, \
            f"{what}: exceeds {tol['max_abs']:.0e} + 2^-7 cond by {excess.max():.3e}"
    else:
        assert mx <= tol["max_abs"], f"{what}: max-abs {mx:.3e} > {tol['max_abs']:.1e}"
    if tol["mean_abs"] is not None:
        # mean_cond: the mean bound also carries the mean first-order rounding, 2^-8 mean(cond).
        mb = tol["mean_abs"] + (BF16_U * float(np.mean(cond)) if (mean_cond and cond is not None) else 0.0)
        assert mean <= mb, f"{what}: mean-abs {mean:.3e} > {mb:.3e}"
    return mx, mean


def fp8_forward_bounds(q, k, v, scale: float, causal: bool, rows=None):
    """Per-element error bounds of the FP8 forward for one head, in fp64 from oracle values.

    The kernel rounds each probability P~_k (in [0, 256]) to E4M3 for the P V product and
    the row sum: a normal value moves by at most 2^-4 P~_k, a subnormal one (below 2^-6) by
    at most 2^-10.  With l~ = sum_k P~_k, the first-order change of O = sum P8 V / sum P8 is
    sum_k dP~_k (V_k - O) / l~.  The kernel's reference maximum never exceeds the row's true
    maximum, so l~ >= l, the sum of exp(s - max) the oracle computes, and
        |dO_c| <= sum_k (2^-4 P_k + 2^-10 / l) |V_kc - O_c|,
        |dlse| <= sum_k (2^-4 P_k + 2^-10 / l)   (lse = m + ln sum P8).
    The bf16 store adds BF16_U |O_c| = 2^-8 |O_c|.  Returned: (bound_O, sigma_O, bound_lse) for the given
    query rows (default all), where sigma_O is the standard deviation of the same error
    under independent roundings uniform in their half-ulp intervals (a mean-error scale).
    """
    from oracle import attention as oracle
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    idx = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    s = scale * (q[idx] @ k.T)
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] > idx[:, None], -np.inf, s)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    o = p @ v
    vis = np.isfinite(s)
    c = np.where(vis, 2.0 ** -4 * p + 2.0 ** -10 / l, 0.0)  # [R, N] per-key coefficient
    bound = np.empty_like(o)
    var = np.empty_like(o)
    for col in range(v.shape[1]):
        dv = np.abs(v[None, :, col] - o[:, col:col + 1])  # [R, N]
        bound[:, col] = (c * dv).sum(axis=1)
        var[:, col] = ((c * dv) ** 2).sum(axis=1) / 3.0
    var += (BF16_U * np.abs(o)) ** 2 / 3.0
    return bound + BF16_U * np.abs(o), np.sqrt(var), c.sum(axis=1)


def dropout_conditions(q, k, v, do, scale: float, causal: bool, p: float, seed: int, offset: int, bh: int):
    """Condition sums of the dropout forward and backward products of one head (fp64), as
    in ``bwd_condition`` with the keep factor Z = keep * keep_scale(p) included, plus the effect
    on dQ and dK of D computed from the bf16-stored O:
    (cond_O, cond_dQ, cond_dK, cond_dV) = (|P Z| |V|, scale |dS| |K|, scale |dS|^T |Q|,
    |P Z|^T |dO|) with dS = P (Z (dO V^T) - D)."""
    from oracle import attention as oracle
    from oracle.dropout import keep_mask, keep_scale
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    pr, _, _ = oracle.probabilities(q, k, scale, causal)
    z = keep_mask(bh, q.shape[0], k.shape[0], p, seed, offset) * keep_scale(p)
    pz = np.abs(pr * z)
    dp = z * (do @ v.T)
    ds = np.abs(pr * (dp - np.sum(pr * dp, axis=1)[:, None]))
    # The kernels take D = rowsum(dO * O) from the bf16-stored O: |dD_i| <= 2^-8 sum_c |dO O|,
    # and dS_ij moves by P_ij dD_i.
    dd = np.sum(np.abs(do) * np.abs((pr * z) @ v), axis=1)
    cond_dq = scale * (ds @ np.abs(k) + dd[:, None] * (np.abs(pr) @ np.abs(k)))
    cond_dk = scale * (ds.T @ np.abs(q) + np.abs(pr).T @ (dd[:, None] * np.abs(q)))
    return pz @ np.abs(v), cond_dq, cond_dk, pz.T @ np.abs(do)


def host_workers() -> int:
    """Threads for running the oracle head by head: the host cores this process may use, at
    most 12 (each thread holds a few N x N fp64 arrays at a time)."""
    import os
    return max(1, min(12, len(os.sched_getaffinity(0))))


def parity_by_head(label: str, heads, got, ref_fn, dtype: str) -> dict:
    """Compare every element of several outputs with the oracle, one head at a time.

    ``got`` maps an output name to the GPU result as an fp64 array indexed [b, h, ...];
    ``ref_fn(b, h)`` returns the oracle's values of head (b, h) as a dict of the same names.
    A value may be a pair (ref, cond): the element-wise bound is then max_abs + BF16_U * cond,
    a first-order rounding bound derived for the arithmetic of the path under test.
    The oracle runs in a thread pool (NumPy releases the GIL in its kernels; BLAS is held to
    one thread per call), so host memory stays bounded by a few heads.  Max-abs and mean-abs
    are taken over all compared elements of each output and checked against the stated
    tolerance of ``dtype``."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    heads = list(heads)

    def one(bh):
        b, h = bh
        ref = ref_fn(b, h)
        out = {}
        for name, r in ref.items():
            r, cond = r if isinstance(r, tuple) else (r, None)
            g = np.asarray(got[name][b, h], dtype=np.float64)
            assert g.shape == r.shape, (name, g.shape, r.shape)
            d = np.abs(g - r)
            # excess over the element-wise bound (<= 0 when within it)
            over = float((d - BF16_U * cond).max()) if cond is not None else float(d.max())
            out[name] = (bool(np.all(np.isfinite(g))), float(d.max()), float(d.sum()), d.size, over,
                         cond is not None)
        return out

    with threadpool_limits(1), ThreadPoolExecutor(host_workers()) as ex:
        results = list(ex.map(one, heads))
    tol = TOL[dtype]
    summary = {}
    for name in results[0]:
        finite = all(r[name][0] for r in results)
        mx = max(r[name][1] for r in results)
        mean = sum(r[name][2] for r in results) / sum(r[name][3] for r in results)
        over = max(r[name][4] for r in results)
        with_cond = results[0][name][5]
        summary[name] = (mx, mean)
        log(f"  {label} {name}: {len(heads)} heads, every element: max-abs {mx:.3e} mean-abs {mean:.3e} "
            f"(tol {tol['max_abs']:.0e}{' + 2^-8 cond' if with_cond else ''}"
            f"{'' if tol['mean_abs'] is None else ' / %.0e' % tol['mean_abs']})")
        assert finite, f"{label} {name}: non-finite output"
        assert over <= tol["max_abs"], f"{label} {name}: exceeds the element-wise bound ({over:.3e} > {tol['max_abs']:.1e})"
        if tol["mean_abs"] is not None:
            assert mean <= tol["mean_abs"], f"{label} {name}: mean-abs {mean:.3e} > {tol['mean_abs']:.1e}"
    return summary


def std_forward_condition(q, k, v, scale: float, causal: bool):
    """Per-element condition sum of the standard path's forward for one head (fp64): it stores
    S in bf16 (|dS_ij| <= BF16_U |S_ij|), which moves O_ic by sum_j P_ij dS_ij (V_jc - O_ic) to
    first order, and rounds P before the P V product (BF16_U sum_j P_ij |V_jc|); the bf16 output
    adds BF16_U |O_ic|, at most the second sum.  Returns
    cond = sum_j P_ij (|S_ij| |V_jc - O_ic| + |V_jc|), [N, d]."""
    from oracle import attention as oracle
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    s = oracle.scores(q, k, scale, causal)
    p, _, _ = oracle.probabilities(q, k, scale, causal)
    o = p @ v
    ps = p * np.where(np.isfinite(s), np.abs(s), 0.0)
    # sum_j ps_ij |v_jc - o_ic| per column c
    cond = np.empty_like(o)
    for c in range(v.shape[1]):
        cond[:, c] = (ps * np.abs(v[None, :, c] - o[:, c:c + 1])).sum(axis=1)
    return cond + p @ np.abs(v)


def std_backward_condition(q, k, v, do, scale: float, causal: bool):
    """Per-element condition sums of the standard path's backward for one head (fp64), the
    first-order effect of every bf16 store it makes, each moving a value x by at most
    BF16_U |x|:
      * S stored (forward) and P stored: |dP~_ij| <= u a_ij, a_ij = P_ij (|S_ij| + sum_k P_ik |S_ik| + 1)
        (a perturbation s of S moves P_ij by P_ij (s_ij - sum_k P_ik s_ik));
      * dP stored: u |dP_ij|;  D = rowsum(P~ dP~): |dD_i| <= u e_i, e_i = sum_j (a_ij + P_ij) |dP_ij|;
      * dS stored: dS_ij = P~ (dP~ - D~) moves by u c_ij,
        c_ij = a_ij |dP_ij - D_i| + P_ij (|dP_ij| + e_i) + |dS_ij|;
      * the gradients stored: dQ = scale dS K moves by u scale sum_j (c_ij + |dS_ij|) |K_jc|, and
        alike dK = scale dS^T Q; dV = P~^T dO by u sum_i (a_ij + P_ij) |dO_ic|.
    Returns (cond_dQ, cond_dK, cond_dV), each [N, d]: the bound is 2e-2 + BF16_U * cond."""
    from oracle import attention as oracle
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    s = oracle.scores(q, k, scale, causal)
    p, _, _ = oracle.probabilities(q, k, scale, causal)
    s_abs = np.where(np.isfinite(s), np.abs(s), 0.0)
    a = p * (s_abs + np.sum(p * s_abs, axis=1, keepdims=True) + 1.0)
    dp = do @ v.T
    dd = np.sum(p * dp, axis=1, keepdims=True)
    ds = p * (dp - dd)
    e = np.sum((a + p) * np.abs(dp), axis=1, keepdims=True)
    c = a * np.abs(dp - dd) + p * (np.abs(dp) + e) + np.abs(ds)
    w = c + np.abs(ds)
    return scale * (w @ np.abs(k)), scale * (w.T @ np.abs(q)), (a + p).T @ np.abs(do)


def bwd_condition_full(q, k, v, do, scale: float, causal: bool):
    """Per-element condition sums of the backward for one head (fp64) that also carry what the
    backward inherits from the forward, each rounding moving a value x by at most BF16_U |x|:
      * lse: the forward's row sum adds up the bf16-rounded probabilities, so lse is off by at
        most BF16_U and the recomputed P_ij by at most BF16_U P_ij;
      * D = rowsum(dO * O) from the bf16-stored O, itself off by the forward's rounding of P
        before P V and of its output: |dD_i| <= BF16_U e_i,
        e_i = sum_c |dO_ic| (2 |O_ic| + (P |V|)_ic);
      * dS = P (dP - D) rounded to bf16: it moves by BF16_U c_ij, c_ij = 2 |dS_ij| + P_ij e_i;
      * dQ = scale dS K and dK = scale dS^T Q, stored in bf16: moved by
        BF16_U scale sum (c + |dS|) |K| (and alike for dK);
      * dV = P^T dO with P off by the lse error and rounded before the product, stored in bf16:
        moved by BF16_U 3 (P^T |dO|).
    Returns (cond_dQ, cond_dK, cond_dV), each [N, d]: the bound is 2e-2 + BF16_U * cond."""
    from oracle import attention as oracle
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    p, _, _ = oracle.probabilities(q, k, scale, causal)
    o = p @ v
    dp = do @ v.T
    dd = np.sum(p * dp, axis=1, keepdims=True)
    ds = np.abs(p * (dp - dd))
    e = np.sum(np.abs(do) * (2.0 * np.abs(o) + p @ np.abs(v)), axis=1, keepdims=True)
    w = 3.0 * ds + p * e
    return scale * (w @ np.abs(k)), scale * (w.T @ np.abs(q)), 3.0 * (p.T @ np.abs(do))
