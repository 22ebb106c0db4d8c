"""Every output is written under each branch of the work order, forward and backward.

The kernels take their tiles through an order that depends on the number of heads and of
tiles per head: one head at a time (64 tiles or more per head), groups of up to 8 heads
whose tiles alternate (fewer), equal-work parts of each head when the head count does not
divide by 8, and two groups of waves per tile on grids of at most 512 tiles.  Outputs are
filled with NaN before each call, so a tile that no workgroup took would show as a
non-finite value.  Three heads of each shape are also compared with the oracle (forward:
rows 0, N - 1 and 30 seeded rows; backward: every element, for N <= 4100)."""
import numpy as np
import pytest

import fa_inputs
import oracle
from tests.gpu_util import assert_parity, bwd_condition_full, gpu_available, log, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

# (B, H, N, d, causal): 1 to 128 tiles per head, head counts that divide by 8 and that do
# not, grids on both sides of 512 tiles, and lengths that are not multiples of the tile.
SHAPES = [
    (1, 1, 128, 128, True),
    (1, 3, 300, 64, False),
    (2, 5, 1024, 128, True),
    (1, 7, 2000, 128, True),
    (1, 6, 4100, 128, True),
    (1, 12, 8064, 128, True),
    (1, 9, 8192, 128, True),
    (1, 5, 8320, 128, True),
    (1, 24, 8320, 128, False),
    (1, 3, 16384, 128, True),
    (1, 40, 2048, 64, True),
    (2, 67, 256, 128, True),
]


@pytest.mark.parametrize("B,H,N,d,causal", SHAPES)
def test_work_order_covers_every_tile(B, H, N, d, causal):
    import torch
    import exact_io_aware_70_amd as fa
    log(f"[order] B={B} H={H} N={N} d={d} causal={causal}")
    g = torch.Generator(device="cuda")
    g.manual_seed(500 + N + H + d)
    q, k, v, do = (fa_inputs.device_normal_bf16((B, H, N, d), g) for _ in range(4))
    scale = 1.0 / float(np.sqrt(d))
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), device=q.device)
    fa.fa_fwd(q, k, v, o=o, lse=lse, scale=scale, causal=causal)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    fa.fa_bwd(q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, scale=scale, causal=causal)
    torch.cuda.synchronize()
    for name, t in (("O", o), ("lse", lse), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert torch.isfinite(t).all(), f"{name}: some elements were never written"
    rng = np.random.default_rng(N + H)
    for b, h in sorted({(0, 0), (B // 2, H // 2), (B - 1, H - 1)}):
        qh, kh, vh, doh = (to_f64(x[b:b + 1, h:h + 1]) for x in (q, k, v, do))
        rows = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 30)]))
        ro, rl = oracle.forward_rows(qh, kh, vh, scale, causal, rows[None, None])
        idx = torch.from_numpy(rows).to(q.device)
        assert_parity(f"O rows ({b},{h})", to_f64(o[b, h][idx]), ro[0, 0], "bf16")
        assert_parity(f"lse rows ({b},{h})", to_f64(lse[b, h][idx]), rl[0, 0], "bf16")
        if N <= 4100:
            r = oracle.backward(qh, kh, vh, doh, scale, causal)
            c = bwd_condition_full(qh[0, 0], kh[0, 0], vh[0, 0], doh[0, 0], scale, causal)
            for i, (name, t) in enumerate((("dQ", dq), ("dK", dk), ("dV", dv))):
                assert_parity(f"{name} ({b},{h})", to_f64(t[b, h]), r[i][0, 0], "bf16", cond=c[i])
