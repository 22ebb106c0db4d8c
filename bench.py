"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --workload softmax_bf16_r65536_c8192   (the row-softmax kernel on its own)
    python bench.py --workload fwd_fp8_causal_b4h32_n8192_d128   (the E4M3 forward)
    python bench.py --dropout 0.1   (the same step with dropout on the probabilities)
    python bench.py --summarize-pmc FETCH_DIR WRITE_DIR [--copy-mib M] [--workload NAME]
    python bench.py --summarize-sq STATS_CSV PMC_DIR [PMC_DIR ...] [--workload NAME]

One step = the whole hot path over one batch: fa_fwd (tiled online-softmax forward,
writing O and lse) followed by fa_bwd (D = rowsum(dO * O), dK/dV and dQ by recomputation)
for the upstream gradient dO.  Inputs are seeded synthetic Gaussians already resident in
HBM.  The default workload is the bf16 causal stress case: B=4, H=32, N=8192, d=128, Q
drawn x3, scale 1/sqrt(d).

FLOPs follow the metric: forward 4 B H N^2 d, halved for causal; the backward counts its
five products, 10 B H N^2 d, halved for causal (the dQ kernel's recomputation of S and dP
is not counted).  `value` = step FLOPs / wall time per step.

Every kernel is timed live with HIP events recorded on the launch stream (fa_bwd_timed
records them between its own launches).  `roofline` is the dominant kernel's: its
algorithmic units per launch over its average duration, against the MI355X peak for its
bound.  `traffic` comes from the committed rocprofv3 counter summary
(profiles/hbm_traffic_<workload>.txt, made by --summarize-pmc) and is null when the kernel
sources have changed since those counters were taken.  `cpu_baseline` is the fp64 oracle
timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
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
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA (published)
# What a workload's counter summaries are keyed to: its kernel sources and the build script
# (compiler flags change the code as much as the sources do).
BUILD_SCRIPT = "exact_io_aware_70_amd/build.py"
KERNEL_SOURCES = ["exact_io_aware_70_amd/csrc/fa_fwd.hip", "exact_io_aware_70_amd/csrc/fa_bwd.hip",
                  "exact_io_aware_70_amd/csrc/fa_device.h", "exact_io_aware_70_amd/csrc/fa_dropout.h", BUILD_SCRIPT]
SOFTMAX_SOURCES = ["exact_io_aware_70_amd/csrc/fa_softmax.hip", "exact_io_aware_70_amd/csrc/fa_device.h",
                   BUILD_SCRIPT]
FP8_SOURCES = ["exact_io_aware_70_amd/csrc/fa_fwd_fp8.hip", "exact_io_aware_70_amd/csrc/fa_device.h", BUILD_SCRIPT]


DEFAULT_WORKLOAD = "fwd_bf16_causal_b4h32_n8192_d128"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-heads", type=int, default=16, help="heads of the workload the CPU oracle runs")
    p.add_argument("--dropout", type=float, default=0.0,
                   help="attention workloads: dropout probability of the probabilities (fa_fwd_dropout / "
                        "fa_bwd_dropout, seed 1234, offset 0); 0 runs the plain path")
    p.add_argument("--cpu-rows", type=int, default=65536,
                   help="rows of a row-softmax workload the CPU oracle runs")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="before the steps, copy this many MiB once with a plain device copy: the reference "
                        "kernel whose FETCH_SIZE / WRITE_SIZE counters calibrate the HBM byte counts")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE, both with "
                        "--copy-mib) into profiles/hbm_traffic_<workload>.txt, then exit")
    p.add_argument("--summarize-sq", nargs="+", metavar="PATH",
                   help="a rocprofv3 kernel_stats.csv followed by the output folders of rocprofv3 --pmc runs "
                        "of this script with SQ_* / GRBM_GUI_ACTIVE counters: write "
                        "profiles/mfma_util_<workload>.md (MFMA, VALU and LDS use per kernel), then exit")
    return p.parse_args()


def flops(B, H, N, d, causal):
    f = 0.5 if causal else 1.0
    return 4.0 * B * H * N * N * d * f, 10.0 * B * H * N * N * d * f


def is_softmax(workload) -> bool:
    return workload.startswith("softmax_")


def is_fp8(workload) -> bool:
    return workload.startswith("fwd_fp8_")


def sources_digest(workload="") -> str:
    """SHA-256 of the kernel sources a workload runs (the counter summaries record it)."""
    h = hashlib.sha256()
    if is_std(workload):
        paths = KERNEL_SOURCES + STD_SOURCES_EXTRA
    else:
        paths = SOFTMAX_SOURCES if is_softmax(workload) else FP8_SOURCES if is_fp8(workload) else KERNEL_SOURCES
    for path in paths:
        with open(os.path.join(ROOT, path), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def kernel_table(dtype, B, H, N, d, causal):
    """Algorithmic units per launch of each kernel of one step (name -> (bound, units, unit))."""
    cf = 0.5 if causal else 1.0
    sfx = "bf16" if dtype == "bf16" else "f32"
    n2d = B * H * N * N * d * cf
    # In launch order: fa_fwd, then fa_bwd's two launches (dQ, then dK/dV).
    return {
        # two products (S = Q K^T, O = P V), 2 N^2 d flops each per head
        f"fwd_{sfx}_kernel": ("mfma", 4.0 * n2d, "flop"),
        # one product of the method: dQ += dS K.  The kernel also recomputes S and dP, the
        # price of a backward without atomics; those flops are not algorithmic units and are
        # reported apart (EXECUTED_FACTOR).  It also forms D = rowsum(dO o O) of its rows (a
        # reduction with no matrix work, whose extra bytes are O read and D, lse written)
        f"dq_{sfx}_kernel": ("mfma", 2.0 * n2d, "flop"),
        # four products: S, dP, dV += P^T dO, dK += dS^T Q
        f"dkdv_{sfx}_kernel": ("mfma", 8.0 * n2d, "flop"),
    }


# Executed over algorithmic flops, for kernels that recompute products: the dQ kernel runs
# three products (S, dP, dQ) for the one it contributes.
EXECUTED_FACTOR = {"dq_bf16_kernel": 3.0, "dq_f32_kernel": 3.0}


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt")


def load_traffic(workload):
    """Measured HBM bytes per launch from the committed counter summary, if still current."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    if data.get("source_sha256") != sources_digest(workload):
        return None  # the kernels changed since the counters were taken
    return data["kernels"]


def util_file(workload):
    return os.path.join(ROOT, "profiles", f"mfma_util_{workload}.json")


def load_util(workload):
    """MFMA busy share and clock per kernel from the committed SQ counter summary, if still current."""
    path = util_file(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    if data.get("source_sha256") != sources_digest(workload):
        return None
    return data["kernels"]


def add_measured(entry, name, traffic, util):
    """Add to one kernel entry what the counters measured for it: HBM GB/s (counter bytes over
    the live launch time, against the 8 TB/s peak) and the matrix cores' busy share at the
    clock the kernel ran; null where no current counter summary exists."""
    tb = traffic.get(name, {}).get("bytes") if traffic else None
    entry["traffic"] = tb
    gbs = tb / (entry["ms"] * 1e-3) / 1e9 if tb else None
    entry["hbm_gbs"] = round(gbs, 1) if gbs else None
    entry["hbm_frac"] = round(gbs / PEAK_HBM_GBS, 4) if gbs else None
    u = util.get(name) if util else None
    if entry.get("bound") == "mfma":
        entry["mfma_busy"] = u["mfma_busy"] if u else None
        entry["clock_ghz"] = u["clock_ghz"] if u else None
    return entry


def summarize_pmc(args):
    """Average FETCH_SIZE / WRITE_SIZE per dispatch of each kernel, scaled by the copy kernel."""
    def read(dirname, counter):
        per = {}
        for dp, _, files in os.walk(dirname):
            for fn in files:
                if fn.endswith("counter_collection.csv"):
                    with open(os.path.join(dp, fn)) as f:
                        for r in csv.DictReader(f):
                            if r["Counter_Name"] != counter:
                                continue
                            key = (r["Dispatch_Id"], r["Kernel_Name"])
                            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        return per

    fetch, write = read(args.summarize_pmc[0], "FETCH_SIZE"), read(args.summarize_pmc[1], "WRITE_SIZE")
    copy_bytes = args.copy_mib * (1 << 20)

    def calib(per):
        # The calibration copy is the largest copy kernel of the run (uploads of the inputs
        # may also run as small copy kernels).
        vals = [v for (_, name), v in per.items() if "copyBuffer" in name]
        if not vals or copy_bytes <= 0:
            raise SystemExit("no copy kernel in the counter runs (run them with --copy-mib)")
        return copy_bytes / (max(vals) * 1024.0)

    ff, fw = calib(fetch), calib(write)
    names = ["fwd_bf16_kernel", "fwd_f32_kernel", "dkdv_bf16_kernel", "dkdv_f32_kernel",
             "dq_bf16_kernel", "dq_f32_kernel", "softmax_rows_kernel", "fwd_fp8_kernel"] + STD_KERNELS
    out = {}
    for short in names:
        fv = [v for (_, n), v in fetch.items() if short in n]
        wv = [v for (_, n), v in write.items() if short in n]
        if fv and wv:
            fb = sum(fv) / len(fv) * 1024.0 * ff
            wb = sum(wv) / len(wv) * 1024.0 * fw
            out[short] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "bytes": round(fb + wb),
                          "dispatches": len(fv)}
    data = {"workload": args.workload, "source_sha256": sources_digest(args.workload),
            "fetch_scale": ff, "write_scale": fw, "copy_mib": args.copy_mib,
            "commands": [f"rocprofv3 --pmc FETCH_SIZE -d <FETCH_DIR> -f csv -- python3 bench.py --steps 1 --warmup 1 "
                         f"--no-cpu-baseline --copy-mib {args.copy_mib} --workload {args.workload}",
                         f"rocprofv3 --pmc WRITE_SIZE -d <WRITE_DIR> -f csv -- python3 bench.py --steps 1 --warmup 1 "
                         f"--no-cpu-baseline --copy-mib {args.copy_mib} --workload {args.workload}",
                         f"python3 bench.py --summarize-pmc <FETCH_DIR> <WRITE_DIR> --copy-mib {args.copy_mib} "
                         f"--workload {args.workload}"],
            "kernels": out}
    os.makedirs(os.path.dirname(traffic_file(args.workload)), exist_ok=True)
    with open(traffic_file(args.workload), "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")
    print(json.dumps(data, indent=1))


def read_counters(dirs):
    """Mean per dispatch of every counter, per kernel (short name), over rocprofv3 --pmc folders."""
    names = ["fwd_bf16_kernel", "dkdv_bf16_kernel", "dq_bf16_kernel", "fwd_fp8_kernel"]
    per = {}  # (short, counter) -> {dispatch: value}
    for d in dirs:
        for dp, _, files in os.walk(d):
            for fn in files:
                if not fn.endswith("counter_collection.csv"):
                    continue
                with open(os.path.join(dp, fn)) as f:
                    for r in csv.DictReader(f):
                        short = next((n for n in names if n in r["Kernel_Name"]), None)
                        if short is None:
                            continue
                        slot = per.setdefault((short, r["Counter_Name"]), {})
                        key = (d, r["Dispatch_Id"])
                        slot[key] = slot.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (short, counter), vals in per.items():
        out.setdefault(short, {})[counter] = sum(vals.values()) / len(vals)
    return out


def counter_names(d):
    """Counter names of one rocprofv3 --pmc output folder, in first-seen order."""
    seen = []
    for dp, _, files in os.walk(d):
        for fn in files:
            if fn.endswith("counter_collection.csv"):
                with open(os.path.join(dp, fn)) as f:
                    for r in csv.DictReader(f):
                        if r["Counter_Name"] not in seen:
                            seen.append(r["Counter_Name"])
    return seen


def summarize_sq(args):
    """MFMA, VALU and LDS use per kernel from SQ counters, as a short markdown table.

    The chip has 256 CUs of 4 SIMDs in 8 XCDs; GRBM_GUI_ACTIVE is summed over the XCDs, so
    one XCD's busy cycles are an eighth of it, and the clock is those cycles over the kernel's
    average duration (from the kernel-trace statistics given first).  A 32x32x16 bf16 MFMA
    keeps its SIMD's matrix core busy for 32 cycles and a 32x32x64 fp8 one for 64
    (SQ_VALU_MFMA_BUSY_CYCLES counts exactly that), so MFMA busy = busy cycles / (1024 SIMDs
    x cycles)."""
    stats_csv, dirs = args.summarize_sq[0], args.summarize_sq[1:]
    dur = {}
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            for n in ("fwd_bf16_kernel", "dkdv_bf16_kernel", "dq_bf16_kernel", "fwd_fp8_kernel"):
                if n in r["Name"]:
                    dur[n] = float(r["AverageNs"]) * 1e-9
    c = read_counters(dirs)
    import fa_inputs
    if is_fp8(args.workload):
        w = fa_inputs.FP8_CONFIGS[args.workload]
        table = {"fwd_fp8_kernel": ("mfma", flops(w["B"], w["H"], w["N"], w["d"], w["causal"])[0], "flop")}
    else:
        w = fa_inputs.CONFIGS[args.workload]
        table = kernel_table(w["dtype"], w["B"], w["H"], w["N"], w["d"], w["causal"])
    # flops of one MFMA instruction: 32x32x16 bf16, 32x32x64 fp8
    per_instr = {"fwd_fp8_kernel": 131072.0}
    trace_dir = os.path.dirname(stats_csv)
    wl = "" if args.workload == DEFAULT_WORKLOAD else f" --workload {args.workload}"
    lines = [f"# MFMA, VALU and LDS use per kernel: {args.workload}", "",
             "Commands (from the repository root, on one MI355X; the kernel-trace statistics come from",
             f"`rocprofv3 --kernel-trace --stats -T -d {trace_dir} -o run -f csv -- python3 bench.py --steps 5 "
             f"--warmup 1 --no-cpu-baseline{wl}`; one `--pmc` run per counter group):", ""]
    for d in dirs:
        lines.append(f"    rocprofv3 --pmc {' '.join(counter_names(d)) or '<none found>'} -d {d} -f csv -- "
                     f"python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline --workload {args.workload}")
    lines += [f"    python3 bench.py --summarize-sq {stats_csv} {' '.join(dirs)} --workload {args.workload}", "",
              "Counter values are means per dispatch (one warm-up and one timed step).  Durations come from "
              "the kernel-trace statistics named above.", ""]
    if not is_fp8(args.workload):
        lines += ["The dQ kernel's algorithmic work is the one product dQ = scale dS K; it also recomputes S and dP "
                  "(the price of a backward without atomics), hence about 3 MFMA instructions per algorithmic one.", ""]
    if is_fp8(args.workload):
        lines += ["The FP8 kernel issues 9 MFMAs per 8 of the attention products (the ninth, with an all-ones "
                  "operand, sums the rounded probabilities), hence about 1.13 MFMA instructions per algorithmic one.",
                  ""]
    lines += [
              "| kernel | ms | clock (GHz) | MFMA instr. / algorithmic | MFMA busy | MFMA busy with VALU co-issue "
              "| other VALU instr. per MFMA (exp included) | exp per MFMA | LDS instr. per MFMA | CU busy |",
              "|---|---|---|---|---|---|---|---|---|---|"]
    summary = {}
    for n in ("fwd_bf16_kernel", "dkdv_bf16_kernel", "dq_bf16_kernel", "fwd_fp8_kernel"):
        k = c.get(n, {})
        if "GRBM_GUI_ACTIVE" not in k or n not in dur:
            continue
        cyc = k["GRBM_GUI_ACTIVE"] / 8.0
        clock = cyc / dur[n] / 1e9
        mfma = k.get("SQ_INSTS_MFMA", float("nan"))
        if n not in table:
            continue
        algo = table[n][1] / per_instr.get(n, 32768.0)
        busy = k.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / (1024.0 * cyc)
        coex = k.get("SQ_VALU_MFMA_COEXEC_CYCLES", float("nan")) / k.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan"))
        valu = (k.get("SQ_INSTS_VALU", float("nan")) - mfma) / mfma
        trans = k.get("SQ_INSTS_VALU_TRANS_F32", float("nan")) / mfma
        lds = k.get("SQ_INSTS_LDS", float("nan")) / mfma
        cu = k.get("SQ_BUSY_CU_CYCLES", float("nan")) / (256.0 * cyc)
        lines.append(f"| {n} | {dur[n] * 1e3:.3f} | {clock:.2f} | {mfma / algo:.3f} | {busy:.1%} | {coex:.1%} "
                     f"| {valu:.2f} | {trans:.2f} | {lds:.2f} | {cu:.1%} |")
        summary[n] = {"mfma_busy": round(busy, 4), "clock_ghz": round(clock, 3), "valu_coissue": round(coex, 4)}
    lines += ["", "Raw means per dispatch:", "", "| kernel | counter | value |", "|---|---|---|"]
    for n in sorted(c):
        for counter in sorted(c[n]):
            lines.append(f"| {n} | {counter} | {c[n][counter]:.4g} |")
    path = os.path.join(ROOT, "profiles", f"mfma_util_{args.workload}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(util_file(args.workload), "w") as f:
        json.dump({"workload": args.workload, "source_sha256": sources_digest(args.workload),
                   "from": os.path.basename(path), "kernels": summary}, f, indent=1)
        f.write("\n")
    print("\n".join(lines))


def host_info():
    """Threads the oracle's BLAS uses, and what the host is: CPU model and BLAS library."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, cores = "unknown", len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if pools:
            cores = max(i.get("num_threads", 1) for i in pools)
            blas = ", ".join(f"{i.get('internal_api', '?')} {i.get('version', '?')}" for i in pools)
    except Exception:
        pass
    return cores, {"cpu_model": model, "blas": blas}


def cpu_baseline(case, causal, heads):
    """The fp64 oracle (as it stands) on `heads` heads of the workload: forward + backward."""
    import numpy as np
    import oracle
    cores, host = host_info()
    B0, H0 = case["shape"][:2]
    heads = min(heads, B0 * H0)
    sel = [(b, h) for b in range(B0) for h in range(H0)][:heads]
    t_total = 0.0
    for b, h in sel:
        sl = (slice(b, b + 1), slice(h, h + 1))
        q, k, v, do = (case[n]["values"][sl] for n in ("q", "k", "v", "do"))
        t0 = time.perf_counter()
        oracle.forward(q, k, v, case["scale"], causal)
        oracle.backward(q, k, v, do, case["scale"], causal)
        t_total += time.perf_counter() - t0
    _, _, N, d = case["shape"]
    ff, fb = flops(1, heads, N, d, causal)
    # The oracle materialises all of S and P: 2 + 5 products of 2 N^2 d flops per head, causal or not.
    executed = 14.0 * heads * N * N * d
    return {"value": round((ff + fb) / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{heads} of {B0 * H0} heads, full N={N}, d={d}: fp64 forward + backward with explicit S and P "
                      f"({t_total:.1f} s); same flop formula as value",
            "seconds": round(t_total, 3), "executed_tflops": round(executed / t_total / 1e12, 6), **host}


def softmax_bytes(rows, cols, dtype):
    """Algorithmic HBM bytes of one row-softmax launch: x read once, y and lse written once."""
    return 2.0 * rows * cols * (2 if dtype == "bf16" else 4) + 4.0 * rows


def cpu_softmax_baseline(case, rows):
    """The fp64 oracle (as it stands) on the first `rows` rows of the workload."""
    import oracle
    cores, host = host_info()
    R, C = case["shape"]
    rows = min(rows, R)
    x = case["values"][:rows]
    t0 = time.perf_counter()
    oracle.softmax_rows(x)
    t = time.perf_counter() - t0
    return {"value": round(softmax_bytes(rows, C, case["dtype"]) / t / 1e9, 4), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle", "sample": f"{rows} of {R} rows, cols={C}: fp64 softmax and logsumexp ({t:.1f} s); "
                                        f"same byte formula as value", "seconds": round(t, 3), **host}


def cpu_fp8_baseline(case, causal, heads):
    """The fp64 FP8 oracle (as it stands) on `heads` heads of the workload: decode + forward."""
    import oracle
    cores, host = host_info()
    B0, H0, N, d = case["shape"]
    heads = min(heads, B0 * H0)
    sel = [(b, h) for b in range(B0) for h in range(H0)][:heads]
    t = 0.0
    for b, h in sel:
        sl = (slice(b, b + 1), slice(h, h + 1))
        args = [case[n]["codes"][sl] for n in ("q", "k", "v")] + [case[n]["descale"][sl] for n in ("q", "k", "v")]
        t0 = time.perf_counter()
        oracle.forward_fp8(*args, case["scale"], causal)
        t += time.perf_counter() - t0
    ff, _ = flops(1, heads, N, d, causal)
    executed = 4.0 * heads * N * N * d  # the oracle computes all of S and P
    return {"value": round(ff / t / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{heads} of {B0 * H0} heads, full N={N}, d={d}: fp64 decode + forward with explicit S and P "
                      f"({t:.1f} s); same flop formula as value", "seconds": round(t, 3),
            "executed_tflops": round(executed / t / 1e12, 6), **host}


def bench_fp8(args):
    """One step = one fa_fwd_fp8 launch (E4M3 Q, K, V with per-head descales; bf16 O)."""
    import numpy as np
    import torch

    import exact_io_aware_70_amd as fa
    import fa_inputs

    c = fa_inputs.FP8_CONFIGS[args.workload]
    B, H, N, d, causal = c["B"], c["H"], c["N"], c["d"], c["causal"]
    case = fa_inputs.make_fp8_case(B, H, N, d, c["seed"], c["q_scale"])
    dev = torch.device("cuda:0")
    t = {n: torch.from_numpy(case[n]["codes"]).to(dev) for n in ("q", "k", "v")}
    ds = {n: torch.from_numpy(case[n]["descale"]).to(dev) for n in ("q", "k", "v")}
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib * (1 << 20), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step():
        fa.fa_fwd_fp8(t["q"], t["k"], t["v"], ds["q"], ds["k"], ds["v"], o, lse, scale=case["scale"],
                      causal=causal, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for ev in events:
        for e in ev:
            e.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for ev in events:
        ev[0].record(stream)
        step()
        ev[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [ev[0].elapsed_time(ev[1]) for ev in events]
    avg = float(np.mean(ms))
    ff, _ = flops(B, H, N, d, causal)
    ms_step = wall * 1e3 / args.steps
    ach = ff / (avg * 1e-3) / 1e12
    traffic = load_traffic(args.workload)
    kd8 = add_measured({"ms": round(avg, 4), "ms_min": round(min(ms), 4), "bound": "mfma", "achieved": round(ach, 2),
                        "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_FP8_TFLOPS, 4),
                        "units_per_launch": ff}, "fwd_fp8_kernel", traffic, load_util(args.workload))
    tb = kd8["traffic"]
    out = {
        "metric": "attention fwd TFLOP/s (4*B*H*N^2*d, causal halved), E4M3 inputs",
        "value": round(ff / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic (seeded N(0,1) Q/K/V, Q x%g, quantised to E4M3 per head)" % c["q_scale"],
        "config": {"workload": args.workload, "B": B, "H": H, "N": N, "d": d, "causal": causal, "pass": "fwd",
                   "step_flops": ff},
        "kernels": {"fwd_fp8_kernel": kd8},
        "roofline": {"kernel": "fwd_fp8_kernel", "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ach / PEAK_FP8_TFLOPS, 4), "traffic": tb,
                     "launch_ms": round(avg, 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_fp8_baseline(case, causal, args.cpu_heads)
    print(json.dumps(out), flush=True)


def bench_softmax(args):
    """One step = one fa_softmax_rows launch over the whole [rows, cols] array."""
    import numpy as np
    import torch

    import exact_io_aware_70_amd as fa
    import fa_inputs

    c = fa_inputs.SOFTMAX_CONFIGS[args.workload]
    case = fa_inputs.make_softmax_case(c["rows"], c["cols"], c["dtype"], c["seed"], c["x_scale"])
    dev = torch.device("cuda:0")
    if case["dtype"] == "bf16":
        x = torch.from_numpy(case["bits"].view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        x = torch.from_numpy(case["values"]).to(dev)
    y = torch.empty_like(x)
    lse = torch.empty((c["rows"],), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib * (1 << 20), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        fa.fa_softmax_rows(x, y, lse, stream=stream)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for ev in events:
        for e in ev:
            e.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for ev in events:
        ev[0].record(stream)
        fa.fa_softmax_rows(x, y, lse, stream=stream)
        ev[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [ev[0].elapsed_time(ev[1]) for ev in events]
    avg = float(np.mean(ms))
    nbytes = softmax_bytes(c["rows"], c["cols"], c["dtype"])
    ms_step = wall * 1e3 / args.steps
    ach = nbytes / (avg * 1e-3) / 1e9
    traffic = load_traffic(args.workload)
    tb = traffic.get("softmax_rows_kernel", {}).get("bytes") if traffic else None
    out = {
        "metric": "row softmax + logsumexp GB/s (algorithmic bytes: x read once, y and lse written once)",
        "value": round(nbytes / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c["dtype"],
        "data": "synthetic (seeded N(0,1) logits)",
        "config": {"workload": args.workload, "rows": c["rows"], "cols": c["cols"], "bytes_per_step": nbytes},
        "kernels": {"softmax_rows_kernel": add_measured(
            {"ms": round(avg, 4), "ms_min": round(min(ms), 4), "bound": "hbm", "achieved": round(ach, 2),
             "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "units_per_launch": nbytes},
            "softmax_rows_kernel", traffic, None)},
        "roofline": {"kernel": "softmax_rows_kernel", "bound": "hbm", "achieved": round(ach, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": tb,
                     "launch_ms": round(avg, 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_softmax_baseline(case, args.cpu_rows)
    print(json.dumps(out), flush=True)


def is_std(workload) -> bool:
    return workload.startswith("std_")


STD_SOURCES_EXTRA = ["exact_io_aware_70_amd/csrc/fa_std.hip", "exact_io_aware_70_amd/csrc/fa_softmax.hip"]


def std_bytes(B, H, N, d, elt=2):
    """Algorithmic HBM bytes of the standard method per step (the N x N terms counted once per
    pass the method makes over them; matrices are N x ld, ld = N rounded up to 128):
    forward  S write, S read + P write (softmax), P read (P V); Q, K, V read, O written, lse;
    backward P read (dV), dP write, P and dP read + dS write (softmax backward), dS read twice
    (dQ, dK); Q, K, V, dO read, dQ, dK, dV written."""
    ld = (N + 127) // 128 * 128
    nn = B * H * N * ld * elt
    nd = B * H * N * d * elt
    fwd = 4 * nn + 4 * nd + 4 * B * H * N
    bwd = 7 * nn + 7 * nd
    return fwd, bwd


def flash_bytes(B, H, N, d, elt=2):
    """Algorithmic HBM bytes of the flash path per step: fwd Q, K, V read, O and lse written;
    bwd Q, K, V, O, dO, lse read, dQ, dK, dV written, D and lse*log2(e) written and read."""
    nd = B * H * N * d * elt
    return 4 * nd + 4 * B * H * N, 8 * nd + 20 * B * H * N


STD_KERNELS = ["std_scores_kernel", "softmax_rows_kernel", "std_pv_kernel", "std_dv_kernel", "std_dp_kernel",
               "softmax_grad_rows_kernel", "std_dq_kernel", "std_dk_kernel"]


def bench_std(args):
    """One step = the standard (materialising) forward and backward on the workload's inputs;
    the flash path runs the same step in the same process for the ratios."""
    import numpy as np
    import torch

    import exact_io_aware_70_amd as fa
    import fa_inputs

    base = args.workload[len("std_"):]
    cfg = fa_inputs.CONFIGS[base]
    B, H, N, d, causal = cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["causal"]
    case = fa_inputs.make_case(B, H, N, d, cfg["dtype"], cfg["seed"], cfg["q_scale"], with_grad=True)
    dev = torch.device("cuda:0")
    q, k, v, do = (torch.from_numpy(case[n]["bits"].view(np.int16)).view(torch.bfloat16).to(dev)
                   for n in ("q", "k", "v", "do"))
    o, lse = torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ld = fa.fa_std_ld(N)
    p = torch.empty((B, H, N, ld), dtype=torch.bfloat16, device=dev)
    dp = torch.empty_like(p)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d, fa.FA_BF16), dtype=torch.uint8, device=dev)
    sc = case["scale"]
    stream = torch.cuda.current_stream(dev)
    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib * (1 << 20), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def std_step(ev=None):
        if ev:
            ev[0].record(stream)
        fa.fa_std_fwd(q, k, v, o, lse, p, scale=sc, causal=causal, stream=stream)
        if ev:
            ev[1].record(stream)
        fa.fa_std_bwd(q, k, v, do, p, dq, dk, dv, dp, scale=sc, causal=causal, stream=stream)
        if ev:
            ev[2].record(stream)

    def flash_step(ev=None):
        if ev:
            ev[0].record(stream)
        fa.fa_fwd(q, k, v, o, lse, scale=sc, causal=causal, stream=stream)
        if ev:
            ev[1].record(stream)
        fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, scale=sc, causal=causal, workspace=ws, stream=stream)
        if ev:
            ev[2].record(stream)

    def timed(step):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        for ev in events:
            for e in ev:
                e.record(stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for ev in events:
            step(ev)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        f = float(np.mean([ev[0].elapsed_time(ev[1]) for ev in events]))
        b = float(np.mean([ev[1].elapsed_time(ev[2]) for ev in events]))
        return wall * 1e3 / args.steps, f, b

    std_ms, std_f, std_b = timed(std_step)
    fl_ms, fl_f, fl_b = timed(flash_step)
    ff, fb = flops(B, H, N, d, causal)
    sbf, sbb = std_bytes(B, H, N, d)
    fbf, fbb = flash_bytes(B, H, N, d)
    value = (ff + fb) / (std_ms * 1e-3) / 1e12
    ach = (sbf + sbb) / (std_ms * 1e-3) / 1e9
    traffic = load_traffic(args.workload)
    out = {
        "metric": "attention fwd/bwd TFLOP/s (4*B*H*N^2*d fwd, 10*B*H*N^2*d bwd, causal halved): standard "
                  "materialising attention",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(std_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V/dO, Q x%g)" % cfg["q_scale"],
        "config": {"workload": args.workload, "B": B, "H": H, "N": N, "d": d, "causal": causal,
                   "pass": "fwd+bwd", "step_flops": ff + fb, "matrix_ld": ld},
        "std": {"fwd_ms": round(std_f, 4), "bwd_ms": round(std_b, 4), "fwd_bytes": sbf, "bwd_bytes": sbb,
                "fwd_hbm_floor_ms": round(sbf / 8e12 * 1e3, 4), "bwd_hbm_floor_ms": round(sbb / 8e12 * 1e3, 4)},
        "flash": {"fwd_ms": round(fl_f, 4), "bwd_ms": round(fl_b, 4), "step_ms": round(fl_ms, 4),
                  "fwd_bytes": fbf, "bwd_bytes": fbb},
        "speedup": {"fwd": round(std_f / fl_f, 3), "bwd": round(std_b / fl_b, 3), "step": round(std_ms / fl_ms, 3)},
        "kernels": ({n: traffic[n] for n in STD_KERNELS if n in traffic} if traffic else None),
        "roofline": {"kernel": "standard step (all launches)", "bound": "hbm", "achieved": round(ach, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                     "traffic": (sum(t["bytes"] for t in traffic.values()) if traffic else None),
                     "launch_ms": round(std_ms, 4)},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    if args.summarize_sq:
        summarize_sq(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(heads shard across GPUs with no exchange, so one GPU runs one share).", file=sys.stderr)
        sys.exit(2)

    if is_softmax(args.workload):
        bench_softmax(args)
        return
    if is_std(args.workload):
        bench_std(args)
        return
    if is_fp8(args.workload):
        bench_fp8(args)
        return

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
    kinds = kernel_table(case["dtype"], B, H, N, d, causal)
    knames = list(kinds)

    drop = args.dropout

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if drop > 0.0:
            fa.fa_fwd_dropout(q, k, v, drop, 1234, 0, o, lse, scale=sc, causal=causal, stream=stream)
            fa.fa_bwd_dropout(q, k, v, o, lse, do, drop, 1234, 0, dq, dk, dv, scale=sc, causal=causal, workspace=ws,
                              stream=stream, events=None if ev is None else ev[1:])
        else:
            fa.fa_fwd(q, k, v, o, lse, scale=sc, causal=causal, stream=stream)
            fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, scale=sc, causal=causal, workspace=ws, stream=stream,
                      events=None if ev is None else ev[1:])

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

    # ev[0]: before fa_fwd; ev[1..]: recorded by fa_bwd_timed before each of its launches and after.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2 + fa.FA_BWD_LAUNCHES)]
              for _ in range(args.steps)]
    for ev in events:  # create the underlying events before the timed region
        for e in ev:
            e.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # fwd = ev0 -> ev1 (fa_fwd is one launch); then dQ (with D) and dK/dV between ev1..ev3.
    per = {name: [ev[j].elapsed_time(ev[j + 1]) for ev in events] for j, name in enumerate(knames)}
    avg = {name: float(np.mean(ts)) for name, ts in per.items()}
    ms_step = wall * 1e3 / args.steps
    ff, fb = flops(B, H, N, d, causal)
    fwd_ms = avg[knames[0]]
    bwd_ms = sum(avg[n] for n in knames[1:])
    value = (ff + fb) / (ms_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if case["dtype"] == "bf16" else PEAK_F32_TFLOPS
    traffic = load_traffic(args.workload) if drop == 0.0 else None  # counters cover the plain kernels
    util = load_util(args.workload) if drop == 0.0 else None

    kernels = {}
    for name in knames:
        bound, units, unit = kinds[name]
        rate = units / (avg[name] * 1e-3)
        if unit == "flop":
            ach, pk, u = rate / 1e12, peak, "TFLOP/s"
        else:
            ach, pk, u = rate / 1e9, PEAK_HBM_GBS, "GB/s"
        kernels[name] = add_measured({"ms": round(avg[name], 4), "ms_min": round(min(per[name]), 4),
                                      "bound": bound, "achieved": round(ach, 2), "peak": pk, "unit": u,
                                      "frac": round(ach / pk, 4), "units_per_launch": units}, name, traffic, util)
        if name in EXECUTED_FACTOR:
            ex = EXECUTED_FACTOR[name] * units
            kernels[name]["executed_flops"] = ex
            kernels[name]["executed_tflops"] = round(ex / (avg[name] * 1e-3) / 1e12, 2)
    dom = max(knames, key=lambda n: avg[n])
    kd = kernels[dom]
    roofline = {"kernel": dom, "bound": kd["bound"], "achieved": kd["achieved"], "peak": kd["peak"],
                "unit": kd["unit"], "frac": kd["frac"], "traffic": kd["traffic"], "launch_ms": kd["ms"]}

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
                   "pass": "fwd+bwd", "step_flops": ff + fb, **({"dropout_p": drop} if drop > 0.0 else {})},
        "pct_peak": round(100 * value / peak, 2),
        "fwd": {"ms": round(fwd_ms, 4), "tflops": round(ff / (fwd_ms * 1e-3) / 1e12, 2),
                "pct_peak": round(100 * ff / (fwd_ms * 1e-3) / 1e12 / peak, 2), "flops": ff},
        "bwd": {"ms": round(bwd_ms, 4), "tflops": round(fb / (bwd_ms * 1e-3) / 1e12, 2),
                "pct_peak": round(100 * fb / (bwd_ms * 1e-3) / 1e12 / peak, 2), "flops": fb,
                "tflops_literal_4x": round(fb * 0.4 / (bwd_ms * 1e-3) / 1e12, 2)},
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(case, causal, args.cpu_heads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
