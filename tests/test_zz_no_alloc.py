"""fa_bwd_noalloc (the backward with its workspace in the library's static per-GPU scratch)
against fa_bwd, through the C ABI: two calls in a row, the second on a smaller input, each
bitwise equal to fa_bwd on the same input (the same kernels), the smaller one also against
the fp64 oracle; torch's allocator is untouched across the calls."""
import pytest

import fa_inputs
import oracle
from tests.gpu_util import assert_parity, gpu_available, log, to_device, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _inputs(B, H, N, d, seed, causal):
    import torch
    import exact_io_aware_70_amd as fa
    case = fa_inputs.make_case(B, H, N, d, "bf16", seed=seed, with_grad=True)
    q, k, v, do = (to_device(case, n) for n in ("q", "k", "v", "do"))
    o, lse = fa.fa_fwd(q, k, v, scale=case["scale"], causal=causal)
    outs = [torch.empty_like(q) for _ in range(3)]
    torch.cuda.synchronize()
    return case, (q, k, v, o, lse, do), outs


def test_noalloc_matches_fa_bwd_twice_shrinking():
    import torch
    import exact_io_aware_70_amd as fa
    # First a larger call (4 heads x 3000 rows), then a smaller one (3 heads x 517 rows): the
    # second reads only scratch its own first kernel wrote.
    for (B, H, N, d, causal, seed) in [(2, 2, 3000, 128, True, 501), (1, 3, 517, 64, False, 502)]:
        log(f"[noalloc] B={B} H={H} N={N} d={d} causal={causal}")
        case, (q, k, v, o, lse, do), (dq, dk, dv) = _inputs(B, H, N, d, seed, causal)
        before = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        fa.fa_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, scale=case["scale"], causal=causal)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before and torch.cuda.max_memory_allocated() == before
        ref = fa.fa_bwd(q, k, v, o, lse, do, scale=case["scale"], causal=causal)
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
            assert torch.equal(a, b), f"{name} differs from fa_bwd"
        if N < 1000:
            r = oracle.backward(case["q"]["values"], case["k"]["values"], case["v"]["values"],
                                case["do"]["values"], case["scale"], causal)
            for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), r):
                assert_parity(name, to_f64(got), want, "bf16")
