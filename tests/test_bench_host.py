"""bench.py's host logic on the CPU: the one-GPU guard, the algorithmic units, and the
rocprofv3 counter summaries (synthetic CSVs)."""
import csv
import json
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_kernel_units_at_the_bench_workload():
    """B=4 H=32 N=8192 d=128 causal: the forward counts 4 B H N^2 d / 2 = 2.199e12 flops;
    the backward kernels count their own products, listed in launch order (fa_fwd, then
    fa_bwd's dQ and dK/dV)."""
    t = bench.kernel_table("bf16", 4, 32, 8192, 128, True)
    assert t["fwd_bf16_kernel"][1] == pytest.approx(2.199023e12, rel=1e-6)
    assert t["dkdv_bf16_kernel"][1] == 2 * t["fwd_bf16_kernel"][1]
    # dQ counts only dQ = scale dS K (2 N^2 d per head, causal halved); its recomputed S and
    # dP are executed flops, reported apart
    assert t["dq_bf16_kernel"][1] == 0.5 * t["fwd_bf16_kernel"][1]
    assert bench.EXECUTED_FACTOR["dq_bf16_kernel"] * t["dq_bf16_kernel"][1] == 1.5 * t["fwd_bf16_kernel"][1]
    # frac at the measured dQ time of 2.889 ms: 1.0995e12 / 2.889e-3 / 2.5e15 = 0.152
    assert t["dq_bf16_kernel"][1] / 2.889e-3 / 2.5e15 == pytest.approx(0.1522, abs=1e-3)
    assert list(t) == ["fwd_bf16_kernel", "dq_bf16_kernel", "dkdv_bf16_kernel"]
    f = bench.kernel_table("f32", 2, 1, 512, 64, False)
    assert f["fwd_f32_kernel"][1] == 4 * 2 * 512 * 512 * 64


def _write_counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], r)))


def test_counter_means_sum_instances_per_dispatch(tmp_path):
    """Rows of one dispatch (one per XCD or SE instance) add up; dispatches are averaged."""
    name = "void fa::(anonymous namespace)::fwd_bf16_kernel<128, 4, 1, true>(...)"
    _write_counters(str(tmp_path / "a"), [
        (1, name, "SQ_INSTS_MFMA", 10), (1, name, "SQ_INSTS_MFMA", 30),
        (7, name, "SQ_INSTS_MFMA", 20), (7, name, "SQ_INSTS_MFMA", 20),
        (2, "some_other_kernel", "SQ_INSTS_MFMA", 999)])
    _write_counters(str(tmp_path / "b"), [(1, name, "GRBM_GUI_ACTIVE", 8), (7, name, "GRBM_GUI_ACTIVE", 16)])
    c = bench.read_counters([str(tmp_path / "a"), str(tmp_path / "b")])
    assert set(c) == {"fwd_bf16_kernel"}
    assert c["fwd_bf16_kernel"]["SQ_INSTS_MFMA"] == 40.0
    assert c["fwd_bf16_kernel"]["GRBM_GUI_ACTIVE"] == 12.0


def test_traffic_is_scaled_by_the_copy_kernel(tmp_path, monkeypatch):
    """A 1 MiB copy whose FETCH_SIZE reads 512 KiB fixes a factor 2 for every kernel."""
    fwd = "fwd_bf16_kernel<128, 4, 1, true>"
    copy = "__amd_rocclr_copyBuffer"
    _write_counters(str(tmp_path / "fetch"), [(1, copy, "FETCH_SIZE", 512), (2, fwd, "FETCH_SIZE", 100),
                                              (3, fwd, "FETCH_SIZE", 300)])
    _write_counters(str(tmp_path / "write"), [(1, copy, "WRITE_SIZE", 1024), (2, fwd, "WRITE_SIZE", 50),
                                              (3, fwd, "WRITE_SIZE", 50)])
    out = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "traffic_file", lambda w: str(out))
    args = types.SimpleNamespace(summarize_pmc=[str(tmp_path / "fetch"), str(tmp_path / "write")],
                                 copy_mib=1, workload="synthetic")
    bench.summarize_pmc(args)
    data = json.loads(out.read_text())
    assert data["fetch_scale"] == 2.0 and data["write_scale"] == 1.0
    k = data["kernels"]["fwd_bf16_kernel"]
    assert k["fetch_bytes"] == 200 * 1024 * 2 and k["write_bytes"] == 50 * 1024 and k["dispatches"] == 2
    # Current sources: the summary is used; any other digest: traffic is unknown.
    assert bench.load_traffic("synthetic") == data["kernels"]
    data["source_sha256"] = "0" * 64
    out.write_text(json.dumps(data))
    assert bench.load_traffic("synthetic") is None


def test_softmax_units_and_digest():
    """The row softmax moves x once and y once (plus one float of lse per row); its counter
    summary is keyed to its own sources, so editing the attention kernels does not stale it."""
    assert bench.softmax_bytes(65536, 8192, "bf16") == 2 * 65536 * 8192 * 2 + 4 * 65536
    assert bench.softmax_bytes(3, 5, "f32") == 2 * 3 * 5 * 4 + 12
    assert bench.is_softmax("softmax_bf16_r65536_c8192") and not bench.is_softmax("fwd_bf16_causal_b4h32_n8192_d128")
    assert bench.sources_digest("softmax_bf16_r65536_c8192") != bench.sources_digest("fwd_bf16_causal_b4h32_n8192_d128")


def test_measured_rates_come_from_current_summaries_only(tmp_path, monkeypatch):
    """A kernel entry gains HBM GB/s (counter bytes over the live launch time) and the MFMA
    busy share and clock of the committed SQ summary; with a stale digest both are null."""
    util = tmp_path / "util.json"
    monkeypatch.setattr(bench, "util_file", lambda w: str(util))
    util.write_text(json.dumps({"source_sha256": bench.sources_digest("synthetic"),
                                "kernels": {"dq_bf16_kernel": {"mfma_busy": 0.5, "clock_ghz": 1.7}}}))
    traffic = {"dq_bf16_kernel": {"bytes": 2_000_000_000}}
    e = bench.add_measured({"ms": 2.0, "bound": "mfma"}, "dq_bf16_kernel", traffic, bench.load_util("synthetic"))
    assert e["traffic"] == 2_000_000_000 and e["hbm_gbs"] == 1000.0 and e["hbm_frac"] == 0.125
    assert e["mfma_busy"] == 0.5 and e["clock_ghz"] == 1.7
    util.write_text(json.dumps({"source_sha256": "0" * 64, "kernels": {}}))
    e = bench.add_measured({"ms": 2.0, "bound": "mfma"}, "dq_bf16_kernel", None, bench.load_util("synthetic"))
    assert e["traffic"] is None and e["hbm_gbs"] is None and e["mfma_busy"] is None
    h = bench.add_measured({"ms": 1.0, "bound": "hbm"}, "softmax_rows_kernel", {"softmax_rows_kernel": {"bytes": 8e9}},
                           None)
    assert h["hbm_gbs"] == 8000.0 and "mfma_busy" not in h
