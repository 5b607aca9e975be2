"""Host logic of bench.py and the committed measurement files: the one-GPU guard, the JSON line's
contract in the committed run, the kernel trace agreeing with the bench's own timing, and the committed
HBM-traffic table being current for the kernel sources it was measured on."""
from __future__ import annotations

import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
import bench  # noqa: E402  (torch is imported lazily there, so this runs without a GPU)

PROFILES = os.path.join(ROOT, "profiles")


def load(name):
    with open(os.path.join(PROFILES, name)) as f:
        return json.load(f)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip())["error"]


def traffic_keys():
    with open(os.path.join(ROOT, "bench.py")) as f:
        return re.findall(r'measured_traffic\("(\w+)", "([\w.]+)"', f.read())


def test_committed_traffic_is_current():
    # every traffic figure the bench reports comes from counters taken on the kernel source as it is now
    table = load("traffic.json")
    pairs = traffic_keys()
    assert len(pairs) >= 8
    for key, src in pairs:
        assert key in table, key
        e = table[key]
        assert e["source_sha"] == bench.source_sha(src), f"{key}: counters taken on another {src}"
        assert e["bytes_per_launch"] == pytest.approx(e["read_bytes"] + e["write_bytes"])
        assert bench.measured_traffic(key, src) == pytest.approx(e["bytes_per_launch"])
    assert bench.measured_traffic("no_such_kernel", "gemm_mxfp4_ring.hip") is None


def test_committed_bench_line_contract():
    d = load("bench_prefill_mx.json")
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["metric"] == bench.METRIC and d["unit"] == "TFLOP/s" and d["n_gpus"] == 1
    assert d["higher_is_better"] is True and d["data"] == "synthetic"
    cfg = d["config"]
    assert cfg["workload"].startswith("prefill_mx") and (cfg["M"], cfg["K"], cfg["N"]) == (2048, 4096, 14336)
    flops = 2.0 * cfg["M"] * cfg["N"] * cfg["K"]
    # value: whole-step throughput over the wall-clock step time
    assert d["value"] == pytest.approx(flops / (d["ms_per_step"] * 1e-3) / 1e12, rel=1e-9)
    r = d["roofline"]
    assert (r["bound"], r["unit"], r["peak"]) == ("mfma", "TFLOP/s", bench.MFMA_FP4_PEAK_TFLOPS)
    assert r["algorithmic_flops"] == pytest.approx(flops)
    assert r["achieved"] == pytest.approx(flops / (r["avg_launch_us"] * 1e-6) / 1e12, rel=1e-9)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-9)
    assert r["traffic"] == pytest.approx(load("traffic.json")["gemm_mxfp4_ring"]["bytes_per_launch"])
    rq = d["roofline_rotate_quantize"]
    assert (rq["bound"], rq["unit"], rq["peak"]) == ("hbm", "GB/s", bench.HBM_PEAK_GBS)
    assert rq["algorithmic_bytes"] == 16384 * 8192 * (2 + 0.5 + 1 / 32)
    assert rq["frac"] == pytest.approx(rq["achieved"] / rq["peak"], rel=1e-9)
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["unit"] == "TFLOP/s" and c["cores"] >= 1 and c["sample"]
    assert c["value"] == pytest.approx(flops / c["seconds"] / 1e12, rel=1e-6)


def trace_line(kernel, grid):
    with open(os.path.join(PROFILES, "bench_default_kernel_stats.txt")) as f:
        text = f.read()
    m = re.search(re.escape(kernel) + r" grid " + str(grid) + r": (\d+) calls, median ([\d.]+) us, mean ([\d.]+) us",
                  text)
    assert m, (kernel, grid)
    return int(m.group(1)), float(m.group(2)), float(m.group(3))


def test_kernel_trace_agrees_with_the_bench():
    # the rocprofv3 trace of the same command times the headline GEMM within a few percent of the
    # bench's own HIP-event average (the trace also holds the untimed ramp launches)
    d = load("bench_prefill_mx.json")
    calls, median, mean = trace_line("gemm_mxfp4_ring<true>", 256 * 1024)  # 512 workgroups x 512 threads
    assert calls > 100
    avg = d["roofline"]["avg_launch_us"]
    assert abs(median - avg) / avg < 0.1 and abs(mean - avg) / avg < 0.1
    _, median_nv, _ = trace_line("gemm_nvfp4_ring<true>", 256 * 1024)
    assert abs(median_nv - d["other_rows"]["gemm_nvfp4"]["us"]) / median_nv < 0.1
