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


def assert_parity(what: str, got, ref, dtype: str, cond=None) -> tuple[float, float]:
    """Element-wise comparison under the stated tolerance.

    ``cond`` (same shape as ``ref``) widens the element-wise bound to
    max_abs + 2 * BF16_U * cond: the first-order rounding bound of a bf16-rounded factor
    plus a bf16-stored output (see ``bwd_condition``).  It is passed only where the
    gradients grow past 8 in magnitude, where half a bf16 ulp (>= 1/32) alone already
    exceeds the 2e-2 bound.  The mean-abs bound is unchanged.
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
        assert mean <= tol["mean_abs"], f"{what}: mean-abs {mean:.3e} > {tol['mean_abs']:.1e}"
    return mx, mean
