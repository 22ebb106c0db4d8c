"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no attention arithmetic: it only draws Gaussian tensors, rounds
them to the storage dtype and samples row indices.  Both the HIP path and the
oracle consume its output; neither is imported here.

Workloads (Gaussian Q/K/V, as in the verification block of "Breaking the Memory
Wall: A Deep Dive into FlashAttention" -- "Implementation: Simulating
FlashAttention in PyTorch", which draws q, k, v with randn):

  name                              pass  dtype  B  H   N      d    causal  seed
  fwd_f32_b2h1_n512_d64             fwd   f32    2  1   512    64   no      1
  fwd_bf16_b8h16_n2048_d64          fwd   bf16   8  16  2048   64   no      2
  fwd_bf16_causal_b4h32_n8192_d128  fwd   bf16   4  32  8192   128  yes     3  (Q drawn x3)
  fwd_bf16_causal_b1h32_n16384_d128 fwd   bf16   1  32  16384  128  yes     4  (rows seed 1004)
  bwd_bf16_causal_b4h16_n4096_d128  bwd   bf16   4  16  4096   128  yes     5

Row-softmax workloads (the softmax step of attention on its own: logits of unit
Gaussian q and k scaled by 1/sqrt(d) are N(0, 1)):

  name                          dtype  rows    cols  seed
  softmax_bf16_r65536_c8192     bf16   65536   8192  11   (8 heads' score rows at N = 8192)
  softmax_f32_r8192_c2048       f32    8192    2048  12

Tensors past 2^31 elements (the 64-bit offset case: B=1, H=4104, N=4096, d=128,
4.3 GB per bf16 tensor) are drawn on the GPU by ``device_normal_bf16``: torch's
seeded device generator, N(0, 1) in fp32, rounded to bf16.  Tests copy the heads they
check back to the host, so the oracle still sees the stored values.

Recipe: ``np.random.default_rng(seed).standard_normal(shape, dtype=float32)`` drawn
in the order Q, K, V (then dO for backward cases); Q multiplied by ``q_scale`` in
fp32; then rounded to the storage dtype (bf16 with round-to-nearest-even).  The
scale passed to attention is 1/sqrt(d).
"""
from __future__ import annotations

import math

import numpy as np

CONFIGS = {
    "fwd_f32_b2h1_n512_d64": dict(pass_="fwd", dtype="f32", B=2, H=1, N=512, d=64,
                                  causal=False, seed=1, q_scale=1.0),
    "fwd_bf16_b8h16_n2048_d64": dict(pass_="fwd", dtype="bf16", B=8, H=16, N=2048, d=64,
                                     causal=False, seed=2, q_scale=1.0),
    "fwd_bf16_causal_b4h32_n8192_d128": dict(pass_="fwd", dtype="bf16", B=4, H=32, N=8192,
                                             d=128, causal=True, seed=3, q_scale=3.0),
    "fwd_bf16_causal_b1h32_n16384_d128": dict(pass_="fwd", dtype="bf16", B=1, H=32, N=16384,
                                              d=128, causal=True, seed=4, q_scale=1.0,
                                              row_seed=1004, rows_per_head=256),
    "bwd_bf16_causal_b4h16_n4096_d128": dict(pass_="bwd", dtype="bf16", B=4, H=16, N=4096,
                                             d=128, causal=True, seed=5, q_scale=1.0),
}

FP8_CONFIGS = {
    # The bf16 bench workload's draws (same seed and Q scale), quantised to E4M3 per head.
    "fwd_fp8_causal_b4h32_n8192_d128": dict(B=4, H=32, N=8192, d=128, causal=True, seed=3, q_scale=3.0),
    "fwd_fp8_b4h8_n2048_d128": dict(B=4, H=8, N=2048, d=128, causal=False, seed=6, q_scale=1.0),
}

SOFTMAX_CONFIGS = {
    "softmax_bf16_r65536_c8192": dict(dtype="bf16", rows=65536, cols=8192, seed=11, x_scale=1.0),
    "softmax_f32_r8192_c2048": dict(dtype="f32", rows=8192, cols=2048, seed=12, x_scale=1.0),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 value of bfloat16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw(shape, seed: int, names=("q", "k", "v"), q_scale: float = 1.0) -> dict:
    """Draw float32 N(0,1) tensors of ``shape`` in the order given (default Q, K, V)."""
    rng = np.random.default_rng(seed)
    out = {}
    for name in names:
        out[name] = rng.standard_normal(shape, dtype=np.float32)
    if "q" in out and q_scale != 1.0:
        out["q"] *= np.float32(q_scale)
    return out


def make_case(B: int, H: int, N: int, d: int, dtype: str, seed: int, q_scale: float = 1.0,
              with_grad: bool = False) -> dict:
    """Inputs of one case, as stored values.

    Returns ``{"dtype", "scale", name: {"bits" or None, "values": float32 array}}`` for
    names q, k, v (and "do" if ``with_grad``).  For bf16, ``values`` holds the exact
    float32 value of the stored bf16 bits; for f32 it is the drawn array itself.
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"unknown dtype {dtype!r}")
    names = ("q", "k", "v", "do") if with_grad else ("q", "k", "v")
    raw = draw((B, H, N, d), seed, names, q_scale)
    case = {"dtype": dtype, "scale": 1.0 / math.sqrt(d), "shape": (B, H, N, d)}
    for name, arr in raw.items():
        if dtype == "bf16":
            bits = bf16_bits(arr)
            case[name] = {"bits": bits, "values": bf16_bits_to_f32(bits)}
        else:
            case[name] = {"bits": None, "values": arr}
    return case


def make_config(name: str) -> dict:
    """The case for one named workload in ``CONFIGS``."""
    c = CONFIGS[name]
    return make_case(c["B"], c["H"], c["N"], c["d"], c["dtype"], c["seed"], c["q_scale"],
                     with_grad=(c["pass_"] == "bwd"))


def sample_rows(B: int, H: int, N: int, rows_per_head: int, seed: int) -> np.ndarray:
    """Per (b, h), ``rows_per_head`` distinct query rows drawn uniformly without replacement.

    Returns int64 [B, H, R], each row sorted ascending.
    """
    rng = np.random.default_rng(seed)
    r = min(rows_per_head, N)
    out = np.empty((B, H, r), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            out[b, h] = np.sort(rng.choice(N, size=r, replace=False))
    return out


def make_softmax_case(rows: int, cols: int, dtype: str, seed: int, x_scale: float = 1.0,
                      mask: str | None = None) -> dict:
    """Logits of one row-softmax case, as stored values.

    ``x_scale`` multiplies the N(0, 1) draw (float32) before rounding to the storage
    dtype.  ``mask="causal"`` sets entry (r, c) to -inf for c > r mod cols (the visible
    keys of a causal score row); ``mask="empty-rows"`` also makes every 7th row all -inf.
    Returns ``{"dtype", "shape", "bits" or None, "values": float32 [rows, cols]}``.
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"unknown dtype {dtype!r}")
    x = np.random.default_rng(seed).standard_normal((rows, cols), dtype=np.float32)
    if x_scale != 1.0:
        x *= np.float32(x_scale)
    if mask in ("causal", "empty-rows"):
        r = np.arange(rows)[:, None] % cols
        x[np.arange(cols)[None, :] > r] = -np.inf
        if mask == "empty-rows":
            x[::7] = -np.inf
    elif mask is not None:
        raise ValueError(f"unknown mask {mask!r}")
    if dtype == "bf16":
        bits = bf16_bits(x)
        return {"dtype": dtype, "shape": (rows, cols), "bits": bits, "values": bf16_bits_to_f32(bits)}
    return {"dtype": dtype, "shape": (rows, cols), "bits": None, "values": x}


def e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Round float32 values to OCP E4M3 (nearest, ties to even) and return the uint8 codes.

    Input preparation only: the conversion is torch's float8_e4m3fn cast on the CPU."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def make_fp8_case(B: int, H: int, N: int, d: int, seed: int, q_scale: float = 1.0) -> dict:
    """Inputs of one FP8 forward case: Q, K, V drawn as in ``make_case`` (float32), then each
    (b, h) of each tensor scaled so its largest magnitude maps to 448 (the largest E4M3
    value) and rounded to E4M3.  Returns ``{"shape", "scale", name: {"codes": uint8
    [B,H,N,d], "descale": float32 [B,H]}}``; the value of a code is decode(code) * descale."""
    raw = draw((B, H, N, d), seed, ("q", "k", "v"), q_scale)
    case = {"shape": (B, H, N, d), "scale": 1.0 / math.sqrt(d)}
    for name, x in raw.items():
        amax = np.abs(x).reshape(B, H, -1).max(axis=2)
        sc = (np.float32(448.0) / np.maximum(amax, np.float32(1e-30))).astype(np.float32)
        codes = e4m3_codes(x * sc[:, :, None, None])
        case[name] = {"codes": codes, "descale": (np.float32(1.0) / sc).astype(np.float32)}
    return case


def device_normal_bf16(shape, generator, device="cuda"):
    """A bf16 tensor of N(0, 1) draws made on the GPU by ``generator`` (a seeded
    ``torch.Generator`` on ``device``): fp32 draws rounded to bf16 (RNE).  For inputs too
    large to draw on the host; successive calls continue the generator's stream."""
    import torch
    return torch.randn(tuple(shape), generator=generator, device=device, dtype=torch.float32).to(torch.bfloat16)
