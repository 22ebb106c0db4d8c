"""fp64 CPU oracle for attention over OCP FP8 (E4M3) inputs -- test infrastructure only.

TEST INFRASTRUCTURE ONLY (same rule as ``oracle.attention``: only tests, the smoke check
and the bench's CPU baseline may use it; the HIP library never does, and this module
imports nothing from it).

The FP8 forward takes Q, K, V as E4M3 codes with one float descale per (batch, head) and
tensor: the value of code c of head (b, h) of tensor X is decode(c) * X_descale[b, h].
What it computes is then plain attention of those values, so the oracle decodes the codes
exactly (every E4M3 value is a dyadic rational, exact in fp64) and calls the plain
definition in ``oracle.attention.forward``.  The pages name FP8 support only as a feature
added by FlashAttention-3 ("How does FlashAttention optimize memory and speed via
tiling?" -- "Interview tips"); the format and the per-head scaling below are readings, not
the pages' text.

E4M3 (the OCP 8-bit floating-point format, "FN" variant): 1 sign bit, 4 exponent bits
with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals (m/8) * 2^-6; the
all-ones exponent with all-ones mantissa is NaN; there are no infinities; the largest
finite value is 1.75 * 2^8 = 448.
"""
from __future__ import annotations

import numpy as np

from .attention import forward

__all__ = ["decode_e4m3", "forward_fp8"]


def decode_e4m3(codes) -> np.ndarray:
    """Exact fp64 values of E4M3 codes (uint8 array); NaN codes decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32))
    sub = sign * np.ldexp(m / 8.0, -6)
    out = np.where(e == 0, sub, normal)
    return np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, out)


def forward_fp8(q8, k8, v8, q_descale, k_descale, v_descale, scale: float, causal: bool):
    """Attention of decoded, descaled FP8 inputs: codes [B, H, N, d], descales [B, H].

    Returns (O [B, H, N, d], lse [B, H, N]) in fp64, from ``oracle.attention.forward``.
    """
    def values(codes, descale):
        return decode_e4m3(codes) * np.asarray(descale, dtype=np.float64)[:, :, None, None]
    return forward(values(q8, q_descale), values(k8, k_descale), values(v8, v_descale), scale, causal)
