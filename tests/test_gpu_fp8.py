"""GPU parity of fa_fwd_fp8 against the fp64 oracle on the same E4M3 codes and descales.

The bound is derived from the arithmetic (``gpu_util.fp8_forward_bounds``): every output
element within 1.1x the first-order effect of rounding the probabilities to E4M3 plus the
bf16 store, plus 1e-5 for fp32 arithmetic; lse likewise; and the mean error no larger
than the mean standard deviation of that rounding under independent roundings."""
import numpy as np
import pytest

import fa_inputs
import oracle
from tests.gpu_util import fp8_forward_bounds, gpu_available, log, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def to_dev(case):
    import torch
    out = {}
    for n in ("q", "k", "v"):
        out[n] = torch.from_numpy(case[n]["codes"]).cuda()
        out[n + "d"] = torch.from_numpy(case[n]["descale"]).cuda()
    return out


def run(case, causal):
    import torch
    import exact_io_aware_70_amd as fa
    t = to_dev(case)
    o, lse = fa.fa_fwd_fp8(t["q"], t["k"], t["v"], t["qd"], t["kd"], t["vd"], scale=case["scale"], causal=causal)
    torch.cuda.synchronize()
    return to_f64(o), to_f64(lse)


def values(case, name, b, h):
    return oracle.decode_e4m3(case[name]["codes"][b, h]) * float(case[name]["descale"][b, h])


def check_head(case, causal, b, h, got_o, got_lse, rows=None, label=""):
    qv, kv, vv = (values(case, n, b, h) for n in ("q", "k", "v"))
    idx = np.arange(qv.shape[0]) if rows is None else np.asarray(rows)
    ref_o, ref_lse = oracle.forward(qv[None, None], kv[None, None], vv[None, None], case["scale"], causal)
    ref_o, ref_lse = ref_o[0, 0][idx], ref_lse[0, 0][idx]
    bound, sigma, bound_lse = fp8_forward_bounds(qv, kv, vv, case["scale"], causal, idx)
    err = np.abs(got_o - ref_o)
    excess = err - (1.1 * bound + 1e-5)
    lerr = np.abs(got_lse - ref_lse)
    log(f"  {label} head ({b},{h}): O max-abs {err.max():.3e} (bound max {bound.max():.3e}), mean-abs "
        f"{err.mean():.3e} (sigma mean {sigma.mean():.3e}); lse max-abs {lerr.max():.3e}")
    assert np.all(np.isfinite(got_o)) and excess.max() <= 0, f"O exceeds its bound by {excess.max():.3e}"
    assert err.mean() <= sigma.mean(), f"O mean-abs {err.mean():.3e} > {sigma.mean():.3e}"
    assert np.all(lerr <= 1.1 * bound_lse + 1e-5), "lse exceeds its bound"


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 100, 129, 300, 1000])
def test_fp8_small(causal, N):
    case = fa_inputs.make_fp8_case(2, 2, N, 128, seed=700 + N, q_scale=2.0)
    log(f"[fp8] small N={N} causal={causal}")
    o, lse = run(case, causal)
    for b in range(2):
        for h in range(2):
            check_head(case, causal, b, h, o[b, h], lse[b, h], label=f"N={N}")


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_odd_head_count(causal):
    """Five heads of several query tiles each: paired-head work order, last head alone."""
    case = fa_inputs.make_fp8_case(1, 5, 700, 128, seed=750, q_scale=2.0)
    log(f"[fp8] odd heads H=5 N=700 causal={causal}")
    o, lse = run(case, causal)
    for h in range(5):
        check_head(case, causal, 0, h, o[0, h], lse[0, h], label=f"H=5 h={h}")


def test_fp8_config_b4h8_n2048():
    c = fa_inputs.FP8_CONFIGS["fwd_fp8_b4h8_n2048_d128"]
    case = fa_inputs.make_fp8_case(c["B"], c["H"], c["N"], c["d"], c["seed"], c["q_scale"])
    log("[fp8] fwd_fp8_b4h8_n2048_d128 (all outputs of 4 heads, finite everywhere)")
    o, lse = run(case, c["causal"])
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    for b, h in [(0, 0), (1, 3), (2, 5), (3, 7)]:
        check_head(case, c["causal"], b, h, o[b, h], lse[b, h], label="n2048")


def test_fp8_bench_workload_sampled_rows():
    """The FP8 bench workload at full size (B=4 H=32 N=8192 d=128 causal, the bf16 bench
    draws quantised per head): 128 seeded rows of 4 heads against the oracle."""
    c = fa_inputs.FP8_CONFIGS["fwd_fp8_causal_b4h32_n8192_d128"]
    case = fa_inputs.make_fp8_case(c["B"], c["H"], c["N"], c["d"], c["seed"], c["q_scale"])
    log("[fp8] fwd_fp8_causal_b4h32_n8192_d128 (sampled rows)")
    o, lse = run(case, c["causal"])
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    rows = fa_inputs.sample_rows(c["B"], c["H"], c["N"], 128, seed=2003)
    for b, h in [(0, 0), (1, 17), (2, 9), (3, 31)]:
        r = rows[b, h]
        check_head(case, c["causal"], b, h, o[b, h][r], lse[b, h][r], rows=r, label="n8192")
