"""GPU parity of the standard (materialising) attention baseline, fa_std_fwd / fa_std_bwd,
against the fp64 oracle, through the C ABI.

The baseline stores the probability matrix itself, so P is compared too (the oracle's P,
with P = 0 in the padding columns).  Small cases span several 128-row and 128-column tiles
with ragged tails, causal and not, d 64 and 128; the two workloads the baseline is timed on
(B=8 H=16 N=2048 d=64 non-causal forward, B=4 H=16 N=4096 d=128 causal backward) are
compared in full, one head of the oracle at a time."""
import numpy as np
import pytest

import fa_inputs
import oracle
from tests.gpu_util import assert_parity, gpu_available, log, parity_by_head, to_device, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def run_std(case, causal, grads=True):
    import torch
    import exact_io_aware_70_amd as fa
    q, k, v = (to_device(case, n) for n in ("q", "k", "v"))
    o, lse, p = fa.fa_std_fwd(q, k, v, scale=case["scale"], causal=causal)
    out = {"O": o, "lse": lse, "P": p}
    if grads:
        do = to_device(case, "do")
        out["dQ"], out["dK"], out["dV"] = fa.fa_std_bwd(q, k, v, do, p, scale=case["scale"], causal=causal)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 100, 129, 300])
def test_std_small(d, causal, N):
    log(f"[std] small d={d} causal={causal} N={N}")
    case = fa_inputs.make_case(2, 2, N, d, "bf16", seed=600 + N + d, with_grad=True)
    out = run_std(case, causal)
    qv, kv, vv, dov = (case[n]["values"] for n in ("q", "k", "v", "do"))
    ref_o, ref_lse = oracle.forward(qv, kv, vv, case["scale"], causal)
    assert_parity("O", to_f64(out["O"]), ref_o, "bf16")
    assert_parity("lse", to_f64(out["lse"]), ref_lse, "bf16")
    p = to_f64(out["P"])
    ref_p = np.stack([np.stack([oracle.probabilities(qv[b, h], kv[b, h], case["scale"], causal)[0]
                                for h in range(2)]) for b in range(2)])
    assert_parity("P", p[..., :N], ref_p, "bf16")
    assert np.all(p[..., N:] == 0.0), "padding columns of P must be 0"
    for name, r in zip(("dQ", "dK", "dV"), oracle.backward(qv, kv, vv, dov, case["scale"], causal)):
        assert_parity(name, to_f64(out[name]), r, "bf16")


def test_std_matches_flash_on_a_medium_case():
    """Both paths against the oracle on one causal case with several tiles each way."""
    import exact_io_aware_70_amd as fa
    case = fa_inputs.make_case(1, 3, 1000, 128, "bf16", seed=611, with_grad=True)
    out = run_std(case, True)
    q, k, v, do = (to_device(case, n) for n in ("q", "k", "v", "do"))
    o, lse = fa.fa_fwd(q, k, v, scale=case["scale"], causal=True)
    grads = fa.fa_bwd(q, k, v, o, lse, do, scale=case["scale"], causal=True)
    qv, kv, vv, dov = (case[n]["values"] for n in ("q", "k", "v", "do"))
    ref_o, ref_lse = oracle.forward(qv, kv, vv, case["scale"], True)
    for label, got_o in (("std O", out["O"]), ("flash O", o)):
        assert_parity(label, to_f64(got_o), ref_o, "bf16")
    ref = oracle.backward(qv, kv, vv, dov, case["scale"], True)
    for name, std_g, fl_g, r in zip(("dQ", "dK", "dV"), (out["dQ"], out["dK"], out["dV"]), grads, ref):
        assert_parity("std " + name, to_f64(std_g), r, "bf16")
        assert_parity("flash " + name, to_f64(fl_g), r, "bf16")


def test_std_large_logits_within_the_score_rounding_bound():
    """Q drawn x3 (logits up to ~15): the standard path stores S in bf16, and rounding S_ij
    moves O_i by sum_j P_ij dS_ij (V_j - O_i) to first order, |dS_ij| <= 2^-8 |S_ij|.  With the
    rounding of P before P V and of the bf16 output this gives the element-wise bound
    2e-2 + 2^-7 cond, cond = sum_j P_ij (|S_ij| |V_jc - O_ic| + |V_jc|) (``std_forward_condition``);
    the stated 2e-2 alone is not reachable by any bf16 store of S there (the flash path keeps S
    in fp32 registers and meets it, ``test_fwd_large_logits_bf16``)."""
    from tests.gpu_util import std_forward_condition
    case = fa_inputs.make_case(1, 3, 1000, 128, "bf16", seed=612, q_scale=3.0, with_grad=False)
    out = run_std(case, True, grads=False)
    qv, kv, vv = (case[n]["values"] for n in ("q", "k", "v"))
    ref_o, ref_lse = oracle.forward(qv, kv, vv, case["scale"], True)
    cond = np.stack([std_forward_condition(qv[0, h], kv[0, h], vv[0, h], case["scale"], True) for h in range(3)])[None]
    assert_parity("std O (Q x3)", to_f64(out["O"]), ref_o, "bf16", cond=cond, mean_cond=True)


def test_std_forward_workload_b8h16_n2048_d64():
    """The non-causal d = 64 forward workload at full size: every element of O, lse and P."""
    name = "fwd_bf16_b8h16_n2048_d64"
    cfg = fa_inputs.CONFIGS[name]
    case = fa_inputs.make_config(name)
    log(f"[std] {name} forward (all heads, every output)")
    out = run_std(case, cfg["causal"], grads=False)
    N = cfg["N"]
    got = {"O": to_f64(out["O"]), "lse": to_f64(out["lse"]), "P": to_f64(out["P"][..., :N])}
    del out
    vals = [case[n]["values"] for n in ("q", "k", "v")]

    def ref(b, h):
        sl = (slice(b, b + 1), slice(h, h + 1))
        r_o, r_lse = oracle.forward(*(x[sl] for x in vals), case["scale"], cfg["causal"])
        p, _, _ = oracle.probabilities(vals[0][b, h], vals[1][b, h], case["scale"], cfg["causal"])
        return {"O": r_o[0, 0], "lse": r_lse[0, 0], "P": p}
    parity_by_head("std " + name, [(b, h) for b in range(cfg["B"]) for h in range(cfg["H"])], got, ref, "bf16")


def test_std_backward_workload_b4h16_n4096_d128():
    """The causal backward workload at full size: every element of dQ, dK, dV of all 64 heads.

    The standard path stores S, P, dP and dS in bf16, and |dP| reaches ~40 here, so its
    gradients carry more rounding than the flash path's (which keeps S, P and dP in fp32
    registers): dQ reaches 3e-2.  The element-wise bound is 2e-2 + 2^-8 cond with cond the
    first-order effect of those stores (``std_backward_condition``, checked against an
    emulation of the same roundings in ``tests/test_tolerance.py``); the mean-abs bound stays
    2e-3."""
    from tests.gpu_util import std_backward_condition
    name = "bwd_bf16_causal_b4h16_n4096_d128"
    cfg = fa_inputs.CONFIGS[name]
    case = fa_inputs.make_config(name)
    log(f"[std] {name} (all heads, every output)")
    out = run_std(case, cfg["causal"])
    got = {n: to_f64(out[n]) for n in ("dQ", "dK", "dV")}
    del out
    vals = [case[n]["values"] for n in ("q", "k", "v", "do")]

    def ref(b, h):
        sl = (slice(b, b + 1), slice(h, h + 1))
        r = oracle.backward(*(x[sl] for x in vals), case["scale"], cfg["causal"])
        c = std_backward_condition(*(x[b, h] for x in vals), case["scale"], cfg["causal"])
        return {"dQ": (r[0][0, 0], c[0]), "dK": (r[1][0, 0], c[1]), "dV": (r[2][0, 0], c[2])}
    parity_by_head("std " + name, [(b, h) for b in range(cfg["B"]) for h in range(cfg["H"])], got, ref, "bf16")
