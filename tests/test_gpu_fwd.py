"""GPU parity of fa_fwd against the fp64 oracle (element by element), through the C ABI.

Small cases span several query and key tiles with ragged tails and are compared in full;
the named workloads run at their full sizes in the launch configuration the bench times and
are compared in full, except the N = 16384 workload, whose definition compares a seeded
sample of 256 rows per head (the oracle computes those rows one by one)."""
import numpy as np
import pytest

import fa_inputs
import oracle
from tests.gpu_util import assert_parity, gpu_available, log, parity_by_head, to_device, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def run_fwd(case, causal):
    import exact_io_aware_70_amd as fa
    q, k, v = (to_device(case, n) for n in ("q", "k", "v"))
    o, lse = fa.fa_fwd(q, k, v, scale=case["scale"], causal=causal)
    import torch
    torch.cuda.synchronize()
    return q, k, v, o, lse


def check_full(case, causal, label):
    log(f"[fwd] {label}")
    _, _, _, o, lse = run_fwd(case, causal)
    ref_o, ref_lse = oracle.forward(case["q"]["values"], case["k"]["values"], case["v"]["values"],
                                    case["scale"], causal)
    assert_parity("O", to_f64(o), ref_o, case["dtype"])
    assert_parity("lse", to_f64(lse), ref_lse, case["dtype"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 100, 129, 300, 1000])
def test_fwd_small(dtype, d, causal, N):
    case = fa_inputs.make_case(2, 2, N, d, dtype, seed=100 + N + d)
    check_full(case, causal, f"small {dtype} d={d} causal={causal} N={N}")


@pytest.mark.parametrize("B,H", [(1, 3), (1, 5), (3, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_odd_head_counts(B, H, causal):
    """Odd head counts with several query tiles per head: the workgroup order pairs heads
    when a head has few tiles, and an odd count leaves the last head on its own."""
    case = fa_inputs.make_case(B, H, 700, 128, "bf16", seed=300 + 10 * B + H)
    check_full(case, causal, f"bf16 B={B} H={H} N=700 causal={causal}")


@pytest.mark.parametrize("B,H", [(1, 3), (1, 4), (3, 2)])
def test_fwd_head_parts(B, H):
    """Head counts that do not divide by 8, at 64 query tiles per head: the work order cuts
    each head into 8 / gcd(B*H, 8) parts of equal causal work, one XCD's worth each.  Every
    element of O and lse, causal, one head of the oracle at a time."""
    N = 8192
    case = fa_inputs.make_case(B, H, N, 128, "bf16", seed=320 + 10 * B + H)
    log(f"[fwd] head parts B={B} H={H} N={N}")
    _, _, _, o, lse = run_fwd(case, True)
    got = {"O": to_f64(o), "lse": to_f64(lse)}
    vals = [case[n]["values"] for n in ("q", "k", "v")]

    def ref(b, h):
        sl = (slice(b, b + 1), slice(h, h + 1))
        r_o, r_lse = oracle.forward(*(x[sl] for x in vals), case["scale"], True)
        return {"O": r_o[0, 0], "lse": r_lse[0, 0]}
    parity_by_head(f"head parts B={B} H={H}", [(b, h) for b in range(B) for h in range(H)], got, ref, "bf16")


@pytest.mark.parametrize("B,H,N,causal,q_scale", [(1, 2, 8192, True, 3.0), (1, 1, 5000, False, 1.0), (2, 3, 1500, True, 1.0)])
def test_fwd_key_groups(B, H, N, causal, q_scale):
    """Grids of at most 512 tiles run with two key groups per tile whose partial (m, l, O)
    merge on chip; every element of O and lse, including a Q x3 case (rescales in both
    groups) and ragged lengths."""
    case = fa_inputs.make_case(B, H, N, 128, "bf16", seed=340 + N + H, q_scale=q_scale)
    log(f"[fwd] key groups B={B} H={H} N={N} causal={causal} q x{q_scale:g}")
    _, _, _, o, lse = run_fwd(case, causal)
    got = {"O": to_f64(o), "lse": to_f64(lse)}
    vals = [case[n]["values"] for n in ("q", "k", "v")]

    def ref(b, h):
        sl = (slice(b, b + 1), slice(h, h + 1))
        r_o, r_lse = oracle.forward(*(x[sl] for x in vals), case["scale"], causal)
        return {"O": r_o[0, 0], "lse": r_lse[0, 0]}
    parity_by_head(f"key groups B={B} H={H} N={N}", [(b, h) for b in range(B) for h in range(H)], got, ref, "bf16")


@pytest.mark.parametrize("B,H,N", [(8, 16, 1024), (3, 67, 1000)])
def test_fwd_head_groups(B, H, N):
    """Few tiles per head on grids past the key-group split: heads go in groups of up to 8
    whose tiles are taken heaviest first across the group (201 heads leave a last group of
    one).  Every element of O and lse, causal."""
    case = fa_inputs.make_case(B, H, N, 128, "bf16", seed=350 + H)
    log(f"[fwd] head groups B={B} H={H} N={N}")
    _, _, _, o, lse = run_fwd(case, True)
    got = {"O": to_f64(o), "lse": to_f64(lse)}
    vals = [case[n]["values"] for n in ("q", "k", "v")]

    def ref(b, h):
        sl = (slice(b, b + 1), slice(h, h + 1))
        r_o, r_lse = oracle.forward(*(x[sl] for x in vals), case["scale"], True)
        return {"O": r_o[0, 0], "lse": r_lse[0, 0]}
    parity_by_head(f"head groups B={B} H={H}", [(b, h) for b in range(B) for h in range(H)], got, ref, "bf16")


def test_fwd_large_logits_bf16():
    """Q drawn x3 (logits std ~3) with a long causal row: the online rescale is exercised."""
    case = fa_inputs.make_case(1, 4, 2000, 128, "bf16", seed=77, q_scale=3.0)
    check_full(case, True, "bf16 causal q x3 N=2000")


def test_fwd_config_f32_b2h1_n512_d64():
    case = fa_inputs.make_config("fwd_f32_b2h1_n512_d64")
    check_full(case, False, "fwd_f32_b2h1_n512_d64 (all outputs)")


def test_fwd_config_bf16_b8h16_n2048_d64():
    case = fa_inputs.make_config("fwd_bf16_b8h16_n2048_d64")
    check_full(case, False, "fwd_bf16_b8h16_n2048_d64 (all outputs)")


def _check_rows(name, rows):
    cfg = fa_inputs.CONFIGS[name]
    case = fa_inputs.make_config(name)
    log(f"[fwd] {name} (sampled rows: {rows.shape[-1]} per head)")
    _, _, _, o, lse = run_fwd(case, cfg["causal"])
    import torch
    idx = torch.from_numpy(rows).to("cuda")
    o_rows = torch.gather(o, 2, idx[..., None].expand(-1, -1, -1, o.shape[-1]))
    lse_rows = torch.gather(lse, 2, idx)
    ref_o, ref_lse = oracle.forward_rows(case["q"]["values"], case["k"]["values"], case["v"]["values"],
                                         case["scale"], cfg["causal"], rows)
    assert_parity("O rows", to_f64(o_rows), ref_o, case["dtype"])
    assert_parity("lse rows", to_f64(lse_rows), ref_lse, case["dtype"])
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


def test_fwd_config_bf16_causal_b4h32_n8192_d128():
    """Q x3 stress config at full size: every element of O and lse of all 128 heads against
    the oracle, which runs one head at a time (the definition with S and P materialised)."""
    name = "fwd_bf16_causal_b4h32_n8192_d128"
    cfg = fa_inputs.CONFIGS[name]
    case = fa_inputs.make_config(name)
    log(f"[fwd] {name} (all {cfg['B'] * cfg['H']} heads, every output)")
    _, _, _, o, lse = run_fwd(case, cfg["causal"])
    got = {"O": to_f64(o), "lse": to_f64(lse)}
    del o, lse
    vals = [case[n]["values"] for n in ("q", "k", "v")]

    def ref(b, h):
        sl = (slice(b, b + 1), slice(h, h + 1))
        r_o, r_lse = oracle.forward(*(x[sl] for x in vals), case["scale"], cfg["causal"])
        return {"O": r_o[0, 0], "lse": r_lse[0, 0]}
    parity_by_head(name, [(b, h) for b in range(cfg["B"]) for h in range(cfg["H"])], got, ref, case["dtype"])


def test_fwd_config_bf16_causal_b1h32_n16384_d128():
    """Long context: the seeded 256 rows per head (plus row 0 and row N-1)."""
    cfg = fa_inputs.CONFIGS["fwd_bf16_causal_b1h32_n16384_d128"]
    rows = fa_inputs.sample_rows(cfg["B"], cfg["H"], cfg["N"], cfg["rows_per_head"], cfg["row_seed"])
    rows = np.concatenate([rows, np.broadcast_to(np.array([0, cfg["N"] - 1]), (cfg["B"], cfg["H"], 2))], axis=2)
    _check_rows("fwd_bf16_causal_b1h32_n16384_d128", rows)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fwd_deterministic(dtype):
    """No atomics in the forward: two runs are bitwise identical."""
    import torch
    case = fa_inputs.make_case(2, 4, 777, 128, dtype, seed=5)
    _, _, _, o1, l1 = run_fwd(case, True)
    _, _, _, o2, l2 = run_fwd(case, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fwd_allocates_nothing():
    """With outputs preallocated, fa_fwd leaves torch's allocator untouched: no N x N buffer."""
    import torch
    import exact_io_aware_70_amd as fa
    case = fa_inputs.make_case(1, 2, 4096, 128, "bf16", seed=9)
    q, k, v = (to_device(case, n) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    fa.fa_fwd(q, k, v, o, lse, causal=True)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.cuda.max_memory_allocated() == before


def test_fwd_closed_forms_on_gpu():
    """Q = 0: O is the (prefix) mean of V and lse = ln(#visible keys), on the GPU path."""
    import torch
    import exact_io_aware_70_amd as fa
    N, d = 333, 64
    v = torch.randn(1, 2, N, d, device="cuda", dtype=torch.float32)
    q = torch.zeros_like(v)
    k = torch.randn_like(v)
    o, lse = fa.fa_fwd(q, k, v, causal=True)
    prefix = torch.cumsum(v.double(), dim=2) / torch.arange(1, N + 1, device="cuda", dtype=torch.float64)[:, None]
    assert (o.double() - prefix).abs().max().item() < 1e-5
    assert (lse.double() - torch.log(torch.arange(1, N + 1, device="cuda", dtype=torch.float64))).abs().max().item() < 1e-5
    o, lse = fa.fa_fwd(q, k, v, causal=False)
    assert (o.double() - v.double().mean(dim=2, keepdim=True)).abs().max().item() < 1e-5
