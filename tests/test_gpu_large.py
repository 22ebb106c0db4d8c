"""GPU parity when each tensor holds more than 2^31 elements.

B=1, H=4104, N=4096, d=128: every bf16 tensor has 4104 * 2^19 = 2.15e9 elements (4.3 GB),
so the heads from 4096 on start at or past element 2^31, and the kernels' per-head offsets
must be 64-bit.  Forward and backward run over all heads; the fp64 oracle checks the
first head, the head ending at element 2^31, the first head starting at it, and the last
one, with the stated bf16 tolerances.  Inputs are seeded N(0, 1) drawn on the GPU
(fa_inputs.device_normal_bf16); the checked heads are copied back for the oracle."""
import math

import numpy as np
import pytest

import fa_inputs
import oracle
from tests.gpu_util import assert_parity, gpu_available, log, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

B, H, N, D = 1, 4104, 4096, 128


def test_fwd_bwd_tensors_past_2e31_elements():
    import torch
    import exact_io_aware_70_amd as fa
    assert B * H * N * D > 2 ** 31 and 4096 * N * D == 2 ** 31
    log(f"[large] B={B} H={H} N={N} d={D} causal: {B * H * N * D:.3e} elements per tensor")
    gen = torch.Generator(device="cuda").manual_seed(2031)
    q, k, v, do = (fa_inputs.device_normal_bf16((B, H, N, D), gen) for _ in range(4))
    scale = 1.0 / math.sqrt(D)
    o, lse = fa.fa_fwd(q, k, v, scale=scale, causal=True)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, lse, do, scale=scale, causal=True)
    torch.cuda.synchronize()
    for t in (o, lse, dq, dk, dv):
        assert bool(t.isfinite().all())
    for h in (0, 4095, 4096, H - 1):
        log(f"  head {h}: first element {h * N * D}")

        def host(t):
            return t[:, h:h + 1].float().cpu().numpy().astype(np.float64)

        qh, kh, vh, doh = host(q), host(k), host(v), host(do)
        ref_o, ref_lse = oracle.forward(qh, kh, vh, scale, True)
        assert_parity("O", host(o), ref_o, "bf16")
        assert_parity("lse", to_f64(lse[:, h:h + 1]), ref_lse, "bf16")
        for nm, got, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), oracle.backward(qh, kh, vh, doh, scale, True)):
            assert_parity(nm, host(got), r, "bf16")
