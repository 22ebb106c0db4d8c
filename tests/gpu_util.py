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


def assert_parity(what: str, got, ref, dtype: str) -> tuple[float, float]:
    mx, mean = errors(got, ref)
    tol = TOL[dtype]
    log(f"  {what}: max-abs {mx:.3e} mean-abs {mean:.3e} (tol {tol['max_abs']:.0e}"
        f"{'' if tol['mean_abs'] is None else ' / %.0e' % tol['mean_abs']})")
    assert mx <= tol["max_abs"], f"{what}: max-abs {mx:.3e} > {tol['max_abs']:.1e}"
    if tol["mean_abs"] is not None:
        assert mean <= tol["mean_abs"], f"{what}: mean-abs {mean:.3e} > {tol['mean_abs']:.1e}"
    return mx, mean
