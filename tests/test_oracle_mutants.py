"""Planted mistakes in copies of the oracle (on the CPU) must each fail at least one pin.

This shows that the pins in tests/oracle_pins.py are strong enough: a dropped term, a
wrong sign or index, or a transposed operand anywhere in the forward or backward does
not slip through."""
import numpy as np
import pytest

from tests import oracle_pins as pins


def _make_fwd(scores_fn=None, norm_axis=1, lse_with_max=True, transpose_p=False):
    def scores(q, k, scale, causal):
        s = scale * (q @ k.T)
        if causal:
            s = np.where(np.triu(np.ones(s.shape, dtype=bool), 1), -np.inf, s)
        return s

    sf = scores_fn or scores

    def fwd(q, k, v, scale, causal):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, H, N, _ = q.shape
        o = np.empty_like(v)
        lse = np.empty((B, H, N))
        with np.errstate(all="ignore"):
            for b in range(B):
                for h in range(H):
                    s = sf(q[b, h], k[b, h], scale, causal)
                    m = np.max(s, axis=norm_axis, keepdims=True)
                    e = np.exp(s - m)
                    l = np.sum(e, axis=norm_axis, keepdims=True)
                    p = e / l
                    o[b, h] = (p.T if transpose_p else p) @ v[b, h]
                    mm, ll = np.max(s, axis=1), np.sum(np.exp(s - np.max(s, axis=1, keepdims=True)), axis=1)
                    lse[b, h] = (mm if lse_with_max else 0.0) + np.log(ll)
        return o, lse
    return fwd


def _no_scale(q, k, scale, causal):
    s = q @ k.T
    return np.where(np.triu(np.ones(s.shape, dtype=bool), 1), -np.inf, s) if causal else s


def _transposed(q, k, scale, causal):
    s = scale * (k @ q.T)
    return np.where(np.triu(np.ones(s.shape, dtype=bool), 1), -np.inf, s) if causal else s


def _mask_flipped(q, k, scale, causal):
    s = scale * (q @ k.T)
    return np.where(np.tril(np.ones(s.shape, dtype=bool), -1), -np.inf, s) if causal else s


def _mask_strict(q, k, scale, causal):
    s = scale * (q @ k.T)
    return np.where(np.triu(np.ones(s.shape, dtype=bool), 0), -np.inf, s) if causal else s


FWD_MUTANTS = {
    "scale dropped": _make_fwd(scores_fn=_no_scale),
    "scores transposed": _make_fwd(scores_fn=_transposed),
    "causal mask flipped": _make_fwd(scores_fn=_mask_flipped),
    "diagonal masked": _make_fwd(scores_fn=_mask_strict),
    "softmax over columns": _make_fwd(norm_axis=0),
    "lse without the max": _make_fwd(lse_with_max=False),
    "P transposed in PV": _make_fwd(transpose_p=True),
}


@pytest.mark.parametrize("name", list(FWD_MUTANTS))
def test_forward_mutant_is_caught(name):
    fwd = FWD_MUTANTS[name]
    failures = 0
    for pin in pins.FORWARD_PINS:
        try:
            pin(fwd)
        except AssertionError:
            failures += 1
    assert failures > 0, f"no forward pin caught the planted mistake: {name}"


def _make_bwd(mistake):
    fwd = _make_fwd()

    def bwd(q, k, v, do, scale, causal):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
        B, H = q.shape[:2]
        for b in range(B):
            for h in range(H):
                s = scale * (q[b, h] @ k[b, h].T)
                if causal:
                    s = np.where(np.triu(np.ones(s.shape, dtype=bool), 1), -np.inf, s)
                e = np.exp(s - s.max(axis=1, keepdims=True))
                p = e / e.sum(axis=1, keepdims=True)
                g = do[b, h]
                dv[b, h] = (p @ g) if mistake == "dV not transposed" else (p.T @ g)
                dp = g @ v[b, h].T
                dd = np.sum(p * dp, axis=1, keepdims=True)
                if mistake == "D term dropped":
                    ds = p * dp
                elif mistake == "dS sign flipped":
                    ds = p * (dd - dp)
                else:
                    ds = p * (dp - dd)
                dq[b, h] = scale * ((ds.T if mistake == "dS transposed in dQ" else ds) @ k[b, h])
                dk[b, h] = (1.0 if mistake == "dK scale dropped" else scale) * (ds.T @ q[b, h])
                if mistake == "dK uses K":
                    dk[b, h] = scale * (ds.T @ k[b, h])
        return dq, dk, dv
    return fwd, bwd


BWD_MUTANTS = ["dV not transposed", "D term dropped", "dS sign flipped", "dS transposed in dQ",
               "dK scale dropped", "dK uses K"]


@pytest.mark.parametrize("name", BWD_MUTANTS)
def test_backward_mutant_is_caught(name):
    fwd, bwd = _make_bwd(name)
    failures = 0
    for pin in pins.BACKWARD_PINS:
        try:
            if pin is pins.pin_two_key_example:
                pin(fwd, bwd)
            else:
                pin(fwd, bwd)
        except AssertionError:
            failures += 1
    assert failures > 0, f"no backward pin caught the planted mistake: {name}"


def test_unmutated_copies_pass():
    """The mutant builders themselves are right when no mistake is planted."""
    fwd, bwd = _make_bwd(None)
    for pin in pins.FORWARD_PINS:
        pin(fwd) if pin is not pins.pin_two_key_example else pin(fwd, bwd)
    for pin in pins.BACKWARD_PINS:
        pin(fwd, bwd)


def _make_softmax(mistake):
    def fn(x):
        x = np.asarray(x, dtype=np.float64)
        with np.errstate(all="ignore"):
            m = np.zeros(x.shape[0]) if mistake == "max not subtracted" else np.max(x, axis=1)
            if mistake == "max over columns":
                m = np.broadcast_to(np.max(x), x.shape[:1])
            e = np.exp(x - m[:, None])
            l = np.sum(e, axis=1)
            if mistake == "normalised over the whole array":
                l = np.full(x.shape[0], np.sum(e))
            y = e / l[:, None]
            lse = (0.0 if mistake == "lse without the max" else m) + (
                np.log10(l) if mistake == "lse in log10" else np.log(l))
        return y, lse
    return fn


SOFTMAX_MUTANTS = ["max not subtracted", "max over columns", "normalised over the whole array", "lse without the max",
                   "lse in log10"]


@pytest.mark.parametrize("name", SOFTMAX_MUTANTS)
def test_softmax_mutant_is_caught(name):
    from tests import softmax_pins
    fn = _make_softmax(name)
    failures = 0
    for pin in softmax_pins.SOFTMAX_PINS:
        try:
            pin(fn)
        except AssertionError:
            failures += 1
    assert failures > 0, f"no softmax pin caught the planted mistake: {name}"


def test_unmutated_softmax_copy_passes():
    from tests import softmax_pins
    fn = _make_softmax(None)
    for pin in softmax_pins.SOFTMAX_PINS:
        pin(fn)
