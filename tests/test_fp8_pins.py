"""The FP8 oracle pinned: E4M3 decoding against torch's float8_e4m3fn (every code) and
the format's landmark values; the FP8 forward against the plain forward on the same
values; the seeded quantiser's scaling."""
import numpy as np
import pytest
import torch

import fa_inputs
import oracle


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode_e4m3(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


@pytest.mark.parametrize("code,value", [(0x00, 0.0), (0x80, -0.0), (0x38, 1.0), (0xB8, -1.0), (0x7E, 448.0),
                                        (0xFE, -448.0), (0x08, 2.0 ** -6), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),
                                        (0x3C, 1.5), (0x40, 2.0)])
def test_decode_landmarks(code, value):
    """Zero, one, the largest finite value 448, the smallest normal 2^-6, the smallest
    subnormal 2^-9, and a few exact values, from the format's definition."""
    got = oracle.decode_e4m3(np.array([code], dtype=np.uint8))[0]
    assert got == value and np.signbit(got) == np.signbit(value)


def test_nan_codes():
    assert np.isnan(oracle.decode_e4m3(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def test_forward_fp8_is_plain_attention_of_the_decoded_values():
    """Descaled decoding followed by the plain forward: checked against torch's float8
    decoding and CPU float64 attention on the same values."""
    rng = np.random.default_rng(9)
    B, H, N, d = 1, 2, 40, 16
    codes = [rng.integers(0, 256, (B, H, N, d), dtype=np.uint8) for _ in range(3)]
    codes = [np.where((c & 0x7F) == 0x7F, 0x3C, c).astype(np.uint8) for c in codes]  # no NaN codes
    ds = [rng.uniform(0.001, 0.01, (B, H)).astype(np.float32) for _ in range(3)]
    o, lse = oracle.forward_fp8(*codes, *ds, 0.25, True)
    vals = [torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64) * torch.from_numpy(s).double()[:, :, None, None]
            for c, s in zip(codes, ds)]
    s = 0.25 * vals[0] @ vals[1].transpose(-1, -2)
    s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    ref = torch.softmax(s, dim=-1) @ vals[2]
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12)


def test_quantiser_uses_the_full_range_per_head():
    """Each (b, h) of each tensor is scaled so its largest magnitude maps to 448 (or just
    below, after rounding), and decode * descale reproduces the drawn values to E4M3
    precision (relative 2^-4 for normal values)."""
    case = fa_inputs.make_fp8_case(2, 3, 50, 32, seed=4, q_scale=3.0)
    raw = fa_inputs.draw((2, 3, 50, 32), 4, ("q", "k", "v"), 3.0)
    for name in ("q", "k", "v"):
        vals = oracle.decode_e4m3(case[name]["codes"])
        amax = np.abs(vals).reshape(2, 3, -1).max(axis=2)
        assert np.all(amax <= 448.0) and np.all(amax >= 416.0)
        back = vals * case[name]["descale"].astype(np.float64)[:, :, None, None]
        x = raw[name].astype(np.float64)
        big = np.abs(x) >= 2.0 ** -6 * case[name]["descale"][:, :, None, None]
        assert np.all(np.abs(back - x)[big] <= 2.0 ** -4 * np.abs(x)[big] + 1e-12)
