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


def test_committed_traffic_is_current():
    # every traffic figure the bench reports comes from counters taken on the kernel source as it is now
    import bench_profiles

    table = load("traffic.json")
    assert len(bench_profiles.TRAFFIC_MAP) >= 10
    for kernel, grid, key, src, *_ in bench_profiles.TRAFFIC_MAP:
        assert key in table, key
        e = table[key]
        assert (e["kernel"], e["grid"]) == (kernel, grid)
        assert e["source_sha"] == bench.source_sha(src), f"{key}: counters taken on another {src}"
        assert e["bytes_per_launch"] == pytest.approx(e["read_bytes"] + e["write_bytes"])
        assert bench.measured_traffic(key, src) == pytest.approx(e["bytes_per_launch"])
    assert bench.measured_traffic("no_such_kernel", "gemm_mxfp4_ring.hip") is None


def test_bench_traffic_lookups_are_in_the_map():
    # the literal keys bench.py looks up are ones the profiling pipeline measures
    import bench_profiles

    keys = {e[2] for e in bench_profiles.TRAFFIC_MAP}
    with open(os.path.join(ROOT, "bench.py")) as f:
        lits = re.findall(r'measured_traffic\("([\w@]+)",', f.read())
    assert len(lits) >= 6
    assert set(lits) <= keys, set(lits) - keys
    assert {"gemm_mxfp4_ring@prefill_mx", "rotate_quant_mx@stress_mx32", "gemm_mxfp4_decode@decode",
            "gemm_mxfp4_decode@decode_wide"} <= keys
    # the decode rows' table: every key measured, on the source it names
    srcs = {e[2]: e[3] for e in bench_profiles.TRAFFIC_MAP}
    for name, (key, src) in bench.DECODE_TRAFFIC_KEY.items():
        assert srcs.get(key) == src, (name, key, src)


def test_roofline_kernel_follows_the_library_dispatch():
    # the kernel fp4_linear runs for each workload (16-byte-aligned scales): decode kernel for M <= 16
    # with K % 512 == 0 (up to 64 rows when K <= 8192, except MXFP4 with 33-64 rows against N >= 8192,
    # which takes the 128-row ring tiles), the 256-row-tile kernels for M, N >= 256, the general
    # kernels otherwise
    from microscaling_fp4_quantized_amd import workloads as WL

    want = {"tiny": "gemm_mxfp4_kernel", "decode1": "gemm_mxfp4_decode", "decode4": "gemm_mxfp4_decode",
            "decode16": "gemm_mxfp4_decode", "decode_wide1": "gemm_mxfp4_decode",
            "decode_wide4": "gemm_mxfp4_decode", "decode_wide16": "gemm_mxfp4_decode",
            "decode_wide32": "gemm_mxfp4_decode", "decode_wide64": "gemm_mxfp4_ring_skinny",
            "decode_nv_wide1": "gemm_nvfp4_decode", "decode_nv_wide16": "gemm_nvfp4_decode",
            "decode_nv_wide64": "gemm_nvfp4_decode", "decode_wide128": "gemm_mxfp4_ring_skinny",
            "decode_nv_wide128": "gemm_nvfp4_ring_skinny",
            "prefill_nv": "gemm_nvfp4_ring", "prefill_mx": "gemm_mxfp4_ring", "prefill_mx_m4096": "gemm_mxfp4_ring",
            "large": "gemm_mxfp4_ring"}
    for name, w in WL.WORKLOADS.items():
        if w.N == 0:
            continue
        src, kern = bench.gemm_kernel_for(w.fmt, w.M, w.N, w.K)
        assert kern == want[name], name
        assert os.path.exists(os.path.join(ROOT, "microscaling_fp4_quantized_amd", "csrc", src))
    assert bench.gemm_kernel_for("mxfp4", 16, 4096, 4224)[1] == "gemm_mxfp4_kernel"   # K % 512 != 0
    assert bench.gemm_kernel_for("mxfp4", 17, 4096, 4096)[1] == "gemm_mxfp4_decode"   # up to 64 tokens
    assert bench.gemm_kernel_for("mxfp4", 64, 4096, 8192)[1] == "gemm_mxfp4_decode"
    assert bench.gemm_kernel_for("mxfp4", 64, 8191, 4096)[1] == "gemm_mxfp4_decode"
    assert bench.gemm_kernel_for("mxfp4", 33, 8192, 4096)[1] == "gemm_mxfp4_ring_skinny"  # 128 x 64 tiles
    assert bench.gemm_kernel_for("mxfp4", 32, 14336, 4096)[1] == "gemm_mxfp4_decode"
    assert bench.gemm_kernel_for("mxfp4", 48, 14336, 8704)[1] == "gemm_mxfp4_ring_skinny"
    assert bench.gemm_kernel_for("nvfp4", 48, 14336, 4096)[1] == "gemm_nvfp4_decode"
    assert bench.gemm_kernel_for("mxfp4", 64, 4096, 8704)[1] == "gemm_mxfp4_kernel"   # K past the slices
    assert bench.gemm_kernel_for("mxfp4", 65, 4096, 4096)[1] == "gemm_mxfp4_ring_skinny"  # 256 x 64 tiles
    assert bench.gemm_kernel_for("mxfp4", 65, 1000, 4096)[1] == "gemm_mxfp4_kernel"   # too few columns
    assert bench.gemm_kernel_for("nvfp4", 100, 2048, 768)[1] == "gemm_nvfp4_ring_skinny"
    assert bench.gemm_kernel_for("nvfp4", 16, 4096, 4096)[1] == "gemm_nvfp4_decode"
    assert bench.gemm_kernel_for("nvfp4", 16, 4096, 8704)[1] == "gemm_nvfp4_kernel"    # K past the slices
    assert bench.gemm_kernel_for("nvfp4", 64, 4096, 4096)[1] == "gemm_nvfp4_decode"
    assert bench.gemm_kernel_for("nvfp4", 65, 1000, 4096)[1] == "gemm_nvfp4_kernel"
    assert bench.gemm_kernel_for("nvfp4", 256, 256, 256)[1] == "gemm_nvfp4_ring"
    assert bench.gemm_kernel_for("nvfp4", 256, 256, 384)[1] == "gemm_nvfp4_kernel"    # K % 256 != 0
    assert bench.gemm_kernel_for("mxfp4", 16, 4096, 1 << 28)[1] == "gemm_mxfp4_kernel"  # K past the decode bound


def test_split_runs_separates_consecutive_rows(tmp_path):
    # two bench rows launch the same kernel and grid one after the other, with other launches
    # between them: the counter values of each row come back separately, in order
    import bench_profiles

    d = tmp_path / "fetch"
    d.mkdir()
    rows = [(i, "k<1>", 512, 10.0) for i in (3, 4, 6, 7)] + [(i, "k<1>", 512, 30.0) for i in (40, 41, 43)] + \
        [(5, "other", 512, 99.0), (20, "k<1>", 1024, 7.0)]
    with open(d / "run_counter_collection.csv", "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Grid_Size,Counter_Name,Counter_Value\n")
        for i, n, g, v in rows:
            f.write(f"{i},{n},{g},FETCH_SIZE,{v}\n")
    assert bench_profiles.split_runs(str(d), "FETCH_SIZE", ("k<1>", 512), 2) == [(10.0, 4), (30.0, 3)]
    assert bench_profiles.split_runs(str(d), "FETCH_SIZE", ("k<1>", 512), 1) == [(pytest.approx(130 / 7), 7)]


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
    assert r["traffic"] == pytest.approx(load("traffic.json")["gemm_mxfp4_ring@prefill_mx"]["bytes_per_launch"])
    h = r["w_from_hbm"]
    assert h["frac"] == pytest.approx(flops / (h["avg_launch_us"] * 1e-6) / 1e12 / r["peak"], rel=1e-9)
    rq = d["roofline_rotate_quantize"]
    assert (rq["bound"], rq["unit"], rq["peak"]) == ("hbm", "GB/s", bench.HBM_PEAK_GBS)
    assert rq["algorithmic_bytes"] == 16384 * 8192 * (2 + 0.5 + 1 / 32)
    assert rq["frac"] == pytest.approx(rq["achieved"] / rq["peak"], rel=1e-9)
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["unit"] == "TFLOP/s" and c["cores"] >= 1 and c["sample"]
    assert c["value"] == pytest.approx(flops / c["seconds"] / 1e12, rel=1e-6)
    assert c["host"]["cpu_model"] and c["host"]["cpu_count"] >= 1
    q = c["rotate_quantize"]
    assert q["unit"] == "GB/s" and q["cores"] >= 1 and q["GB/s"] == pytest.approx(
        q["algorithmic_bytes"] / q["seconds"] / 1e9, rel=1e-9)
    for name, p in c["parity_counts"].items():  # the bench input's sampled rows: no unflagged difference
        assert p["rows_checked"] > 0 and p["code_mismatch_unflagged"] == 0 and p["scale_mismatch_unflagged"] == 0


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
