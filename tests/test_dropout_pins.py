"""The dropout oracle pinned: Philox4x32-10 against its published known-answer vectors,
the mask's index convention and keep rate, p = 0 reducing to plain attention, O unbiased
over seeds, and the dropout backward against finite differences of the dropout forward."""
import os

import numpy as np
import pytest

import oracle
from oracle.dropout import keep_scale, threshold

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def test_philox_known_answers():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        c = [int(x, 16) for x in r[:4]]
        k = [int(x, 16) for x in r[4:6]]
        want = [int(x, 16) for x in r[6:10]]
        got = [int(x) for x in oracle.philox4x32_10(*c, *k)]
        assert got == want, (r, [hex(x) for x in got])


def test_mask_index_convention():
    """Element (i, j) of head bh is byte (j & 3) of word (i & 3) of the call with counter
    (j >> 2, i >> 2, bh, offset) and key (seed lo, seed hi)."""
    seed, offset, bh, p = 0x1234_5678_9ABC_DEF0, 7, 5, 0.3
    m = oracle.keep_mask(bh, 13, 11, p, seed, offset)
    for i, j in [(0, 0), (5, 6), (12, 10), (3, 9)]:
        w = oracle.philox4x32_10(j >> 2, i >> 2, bh, offset, seed & 0xFFFFFFFF, seed >> 32)[i & 3]
        u = (int(w) >> (8 * (j & 3))) & 0xFF
        assert m[i, j] == (u >= threshold(p))


def test_keep_rate_and_extremes():
    m = oracle.keep_mask(0, 512, 512, 0.25, seed=99, offset=0)
    rate = m.mean()
    # 262144 draws: the standard deviation of the rate is about 0.00085
    assert abs(rate - 0.75) < 0.005
    assert oracle.keep_mask(1, 64, 64, 0.0, 1, 0).all()
    assert not oracle.keep_mask(1, 64, 64, 1.0, 1, 0).any()
    assert threshold(0.3) == 77 and threshold(0.5) == 128


@pytest.mark.parametrize("p", [0.0, 0.001, 0.1, 0.2, 0.3, 0.5, 0.9, 0.999])
def test_keep_factor_has_mean_one_exactly(p):
    """Over the 256 equally likely byte values u, the keep factor Z = [u >= t] * s has mean
    exactly 1 whenever anything is kept (inverted dropout with the 8-bit threshold t); at
    p = 0.1 the factor 1 / (1 - p) would give 0.998."""
    t = threshold(p)
    z = np.array([(u >= t) * keep_scale(p) for u in range(256)])
    if t < 256:
        assert abs(z.mean() - 1.0) <= 1e-15
    else:
        assert not z.any()
    assert keep_scale(0.1) == 256 / 230 and threshold(0.1) == 26


def _case(seed=11, N=24, d=8):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((1, 2, N, d)) for _ in range(4)]


@pytest.mark.parametrize("causal", [False, True])
def test_p_zero_is_plain_attention(causal):
    q, k, v, do = _case()
    o, lse = oracle.forward_dropout(q, k, v, 0.3, causal, 0.0, seed=5)
    o_ref, lse_ref = oracle.forward(q, k, v, 0.3, causal)
    np.testing.assert_allclose(o, o_ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-14)
    for a, b in zip(oracle.backward_dropout(q, k, v, do, 0.3, causal, 0.0, seed=5),
                    oracle.backward(q, k, v, do, 0.3, causal)):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def pin_unbiased(fwd_d):
    """E[O] over masks equals the undropped O (the keep scale): the mean of 400 seeds is
    within a few standard errors."""
    q, k, v, _ = _case(N=16)
    o_ref, _ = oracle.forward(q, k, v, 0.4, False)
    outs = np.stack([fwd_d(q, k, v, 0.4, False, 0.2, s)[0] for s in range(400)])
    se = outs.std(axis=0) / np.sqrt(len(outs))
    assert np.all(np.abs(outs.mean(axis=0) - o_ref) <= 5 * se + 1e-12)


def pin_finite_differences(fwd_d, bwd_d, causal=True):
    """With the mask fixed by (seed, offset), L = sum(O * dO) is smooth in q, k, v."""
    q, k, v, do = _case(seed=12, N=12, d=4)
    p, seed, off = 0.35, 2024, 3
    grads = bwd_d(q, k, v, do, 0.5, causal, p, seed, off)

    def loss(q_, k_, v_):
        return float(np.sum(fwd_d(q_, k_, v_, 0.5, causal, p, seed, off)[0] * do))
    eps = 1e-6
    rng = np.random.default_rng(3)
    for which, g in zip(range(3), grads):
        for _ in range(6):
            idx = tuple(rng.integers(0, s) for s in q.shape)
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += eps
            up = loss(*args)
            args[which][idx] -= 2 * eps
            dn = loss(*args)
            assert abs((up - dn) / (2 * eps) - g[idx]) < 1e-6


def test_delta_identity_with_dropout():
    """rowsum(dO * O) = rowsum(P * dP) with dP = Z o (dO V^T): the D the kernels compute
    from O is the one the dropout gradient needs."""
    q, k, v, do = _case(seed=13)
    p, seed = 0.3, 77
    o, _ = oracle.forward_dropout(q, k, v, 0.25, True, p, seed)
    pr, _, _ = oracle.probabilities(q[0, 1], k[0, 1], 0.25, True)
    z = oracle.keep_mask(1, 24, 24, p, seed, 0) * keep_scale(p)
    dp = z * (do[0, 1] @ v[0, 1].T)
    np.testing.assert_allclose(np.sum(do[0, 1] * o[0, 1], axis=1), np.sum(pr * dp, axis=1), rtol=1e-12)


def test_output_is_unbiased_over_seeds():
    pin_unbiased(oracle.forward_dropout)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences(causal):
    pin_finite_differences(oracle.forward_dropout, oracle.backward_dropout, causal)


def _mutant(mistake):
    """Copies of the dropout forward / backward with one planted mistake."""
    from oracle.dropout import keep_mask

    def fwd_d(q, k, v, scale, causal, p, seed, offset=0):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        o = np.empty_like(v)
        for b in range(q.shape[0]):
            for h in range(q.shape[1]):
                pr, _, _ = oracle.probabilities(q[b, h], k[b, h], scale, causal)
                z = keep_mask(b * q.shape[1] + h, q.shape[2], q.shape[2], p, seed, offset)
                z = z if mistake == "no keep scale" else z * keep_scale(p)
                o[b, h] = (pr * z) @ v[b, h]
        return o, None

    def bwd_d(q, k, v, do, scale, causal, p, seed, offset=0):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
        for b in range(q.shape[0]):
            for h in range(q.shape[1]):
                pr, _, _ = oracle.probabilities(q[b, h], k[b, h], scale, causal)
                z = keep_mask(b * q.shape[1] + h, q.shape[2], q.shape[2], p, seed, offset) * keep_scale(p)
                g = do[b, h]
                dv[b, h] = (pr if mistake == "dV without the mask" else pr * z).T @ g
                dp = g @ v[b, h].T
                if mistake != "dP without the mask":
                    dp = z * dp
                ds = pr * (dp - np.sum(pr * dp, axis=1)[:, None])
                dq[b, h] = scale * (ds @ k[b, h])
                dk[b, h] = scale * (ds.T @ q[b, h])
        return dq, dk, dv
    return fwd_d, bwd_d


@pytest.mark.parametrize("mistake", ["no keep scale", "dP without the mask", "dV without the mask", None])
def test_planted_mistakes_are_caught(mistake):
    fwd_d, bwd_d = _mutant(mistake)
    caught = 0
    for pin in (lambda: pin_unbiased(fwd_d), lambda: pin_finite_differences(fwd_d, bwd_d, True),
                lambda: pin_finite_differences(fwd_d, bwd_d, False)):
        try:
            pin()
        except AssertionError:
            caught += 1
    assert (caught > 0) == (mistake is not None), (mistake, caught)


def test_head_offset_places_a_slice():
    """A slice of heads with bh0 gives the same result as the full batch."""
    q, k, v, do = _case(seed=14, N=10)
    full = oracle.forward_dropout(q, k, v, 0.4, True, 0.3, 9, 2)[0]
    part = oracle.forward_dropout(q[:, 1:2], k[:, 1:2], v[:, 1:2], 0.4, True, 0.3, 9, 2, bh0=1)[0]
    np.testing.assert_array_equal(full[:, 1:2], part)
    g_full = oracle.backward_dropout(q, k, v, do, 0.4, True, 0.3, 9, 2)
    g_part = oracle.backward_dropout(q[:, 1:2], k[:, 1:2], v[:, 1:2], do[:, 1:2], 0.4, True, 0.3, 9, 2, bh0=1)
    for a, b in zip(g_full, g_part):
        np.testing.assert_array_equal(a[:, 1:2], b)
