"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = the whole hot path over one batch: fa_fwd (tiled online-softmax forward,
writing O and lse) followed by fa_bwd (delta, dK/dV and dQ by recomputation) for the
upstream gradient dO.  Inputs are seeded synthetic Gaussians already resident in HBM.
The default workload is the bf16 causal forward stress case: B=4, H=32, N=8192, d=128,
Q drawn x3, scale 1/sqrt(d).

FLOPs follow the metric: forward 4 B H N^2 d, halved for causal; the backward counts its
five products, 10 B H N^2 d, halved for causal (the dQ kernel's recomputation is not
counted).  `value` = step FLOPs / wall time per step.  The JSON line also carries the
forward and backward separately (HIP events on the launch stream), the roofline of the
dominant kernel, and the fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="fwd_bf16_causal_b4h32_n8192_d128")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-heads", type=int, default=16, help="heads of the workload the CPU oracle runs")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="before the steps, copy this many MiB once with a plain device copy: the reference "
                        "kernel whose FETCH_SIZE / WRITE_SIZE counters calibrate the HBM byte counts")
    return p.parse_args()


def flops(B, H, N, d, causal):
    f = 0.5 if causal else 1.0
    return 4.0 * B * H * N * N * d * f, 10.0 * B * H * N * N * d * f


def cpu_baseline(case, causal, heads):
    """The fp64 oracle (as it stands) on `heads` heads of the workload: forward + backward."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    sl = (slice(0, 1), slice(0, heads))
    q, k, v, do = (case[n]["values"][sl] for n in ("q", "k", "v", "do"))
    t0 = time.perf_counter()
    oracle.forward(q, k, v, case["scale"], causal)
    oracle.backward(q, k, v, do, case["scale"], causal)
    dt = time.perf_counter() - t0
    B, H, N, d = q.shape
    ff, fb = flops(B, H, N, d, causal)
    return {"value": round((ff + fb) / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{heads} of {case['shape'][0] * case['shape'][1]} heads (b=0), full N={N}, d={d}: "
                      f"fp64 forward + backward with explicit S and P, {dt:.1f} s",
            "seconds": round(dt, 3)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(heads shard across GPUs with no exchange, so one GPU runs one share).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import exact_io_aware_70_amd as fa
    import fa_inputs

    cfg = fa_inputs.CONFIGS[args.workload]
    B, H, N, d, causal = cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["causal"]
    case = fa_inputs.make_case(B, H, N, d, cfg["dtype"], cfg["seed"], cfg["q_scale"], with_grad=True)
    dev = torch.device("cuda:0")

    def to_dev(name):
        if case["dtype"] == "bf16":
            return torch.from_numpy(case[name]["bits"].view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(case[name]["values"]).to(dev)

    q, k, v, do = (to_dev(n) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    code = fa.FA_BF16 if case["dtype"] == "bf16" else fa.FA_F32
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d, code), dtype=torch.uint8, device=dev)
    sc = case["scale"]
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fa.fa_fwd(q, k, v, o, lse, scale=sc, causal=causal, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, scale=sc, causal=causal, workspace=ws, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    if args.copy_mib > 0:
        n = args.copy_mib * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    fwd_ms = [e[0].elapsed_time(e[1]) for e in events]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in events]
    ms_step = wall * 1e3 / args.steps
    ff, fb = flops(B, H, N, d, causal)
    fwd_avg, bwd_avg = float(np.mean(fwd_ms)), float(np.mean(bwd_ms))
    fwd_tf, bwd_tf = ff / (fwd_avg * 1e-3) / 1e12, fb / (bwd_avg * 1e-3) / 1e12
    value = (ff + fb) / (ms_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if case["dtype"] == "bf16" else PEAK_F32_TFLOPS
    elt = 2 if case["dtype"] == "bf16" else 4
    tensor_bytes = B * H * N * d * elt

    # Dominant kernel: the forward kernel is one launch per fa_fwd, so its average launch
    # duration is the fwd event interval.  Its algorithmic units: 4 B H N^2 d (x1/2 causal)
    # FLOPs; its compulsory bytes: Q, K, V read and O written once, lse written.
    roofline = {"kernel": "fwd_bf16_kernel" if code == fa.FA_BF16 else "fwd_f32_kernel",
                "bound": "mfma", "achieved": round(fwd_tf, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(fwd_tf / peak, 4), "traffic": None,
                "launch_ms": round(fwd_avg, 4),
                "compulsory_bytes": 4 * tensor_bytes + 4 * B * H * N}

    out = {
        "metric": "attention fwd/bwd TFLOP/s (4*B*H*N^2*d fwd, 10*B*H*N^2*d bwd, causal halved)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case["dtype"],
        "data": "synthetic (seeded N(0,1) Q/K/V/dO, Q x%g)" % cfg["q_scale"],
        "config": {"workload": args.workload, "B": B, "H": H, "N": N, "d": d, "causal": causal,
                   "pass": "fwd+bwd", "step_flops": ff + fb},
        "pct_peak": round(100 * value / peak, 2),
        "fwd": {"ms": round(fwd_avg, 4), "ms_min": round(min(fwd_ms), 4), "tflops": round(fwd_tf, 2),
                "pct_peak": round(100 * fwd_tf / peak, 2), "flops": ff},
        "bwd": {"ms": round(bwd_avg, 4), "ms_min": round(min(bwd_ms), 4), "tflops": round(bwd_tf, 2),
                "pct_peak": round(100 * bwd_tf / peak, 2), "flops": fb,
                "tflops_literal_4x": round(fb * 0.4 / (bwd_avg * 1e-3) / 1e12, 2)},
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(case, causal, args.cpu_heads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
