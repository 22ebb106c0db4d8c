"""The widened backward bound (``gpu_util.bwd_condition``) checked on the CPU: emulating
the kernels' bf16 roundings in numpy must stay inside it, and dropping a term of the
condition sum must make the emulation break it somewhere."""
import numpy as np
import torch

import oracle
from tests.gpu_util import BF16_U, bwd_condition


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def _emulated_grads(q, k, v, do, scale, causal):
    """dQ, dK, dV with dS and P rounded to bf16 before the products and the results
    stored in bf16; everything else in fp64."""
    p, _, _ = oracle.probabilities(q, k, scale, causal)
    dp = do @ v.T
    ds = p * (dp - np.sum(p * dp, axis=1)[:, None])
    dsr = _bf16(ds)
    return _bf16(scale * dsr @ k), _bf16(scale * dsr.T @ q), _bf16(_bf16(p).T @ do)


def test_bf16_rounding_within_condition_bound():
    rng = np.random.default_rng(7)
    n, d, scale = 96, 32, 32 ** -0.5
    for causal in (False, True):
        q, k, v, do = (_bf16(rng.standard_normal((n, d)) * s) for s in (4.0, 1.0, 1.0, 1.0))
        ref = oracle.backward(q[None, None], k[None, None], v[None, None], do[None, None], scale, causal)
        got = _emulated_grads(q, k, v, do, scale, causal)
        conds = bwd_condition(q, k, v, do, scale, causal)
        for g, r, c in zip(got, ref, conds):
            err = np.abs(g - r[0, 0])
            assert np.all(err <= 2 * BF16_U * c + 1e-12), float(np.max(err - 2 * BF16_U * c))


def test_condition_bound_is_not_vacuous():
    """The emulated error exceeds u*cond somewhere in each gradient: both roundings (the
    factor and the output) matter, and a bound that dropped either term, or a condition
    sum missing its scale factor, would be broken."""
    rng = np.random.default_rng(8)
    n, d, scale = 96, 32, 32 ** -0.5
    q, k, v, do = (_bf16(rng.standard_normal((n, d)) * s) for s in (4.0, 1.0, 1.0, 1.0))
    ref = oracle.backward(q[None, None], k[None, None], v[None, None], do[None, None], scale, True)
    got = _emulated_grads(q, k, v, do, scale, True)
    conds = bwd_condition(q, k, v, do, scale, True)
    for g, r, c in zip(got, ref, conds):
        ratio = np.max(np.abs(g - r[0, 0]) / np.maximum(c, 1e-30))
        assert ratio > BF16_U, ratio / BF16_U
