#!/usr/bin/env python3
"""rocprofv3 evidence for bench.py's default run: the commands, and the summaries made from them.

    python bench_profiles.py commands OUT    print the profiling commands (run them on the GPU
                                             machine from /tmp with TMPDIR=/tmp); raw output goes
                                             under OUT/{trace,fetch,write,copy_fetch,copy_write,sq1,sq2,
                                             nvsq1,nvsq2}
    python bench_profiles.py summarize OUT   read that raw output and write profiles/*.txt and
                                             profiles/traffic.json

HBM traffic per launch is FETCH_SIZE and WRITE_SIZE (KiB per dispatch, one counter per run), each
scaled by what the same counter reads for a plain device copy of 256 MiB (bench.py --copy-probe).
Every entry of traffic.json carries a hash of its kernel's source and the shared headers, and
bench.py reports the entry only while the hash still matches.
"""
from __future__ import annotations

import csv
import glob
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
PROFILES = os.path.join(ROOT, "profiles")

BENCH_ARGS = "--steps 3 --warmup 1 --ramp-ms 0 --no-cpu"
TRACE_ARGS = "--steps 20 --warmup 5 --no-cpu"
SQ_PASSES = {
    "sq1": "SQ_BUSY_CU_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_LDS_IDX_ACTIVE SQ_LDS_DATA_FIFO_FULL SQ_LDS_CMD_FIFO_FULL "
           "SQ_VMEM_TA_ADDR_FIFO_FULL SQ_VMEM_TA_CMD_FIFO_FULL SQ_LDS_BANK_CONFLICT",
    "sq2": "SQ_INSTS_LDS_LOAD_BANDWIDTH SQ_INSTS_LDS_STORE_BANDWIDTH SQ_WAIT_INST_LDS SQ_WAIT_INST_ANY SQ_WAVE_CYCLES "
           "SQ_INSTS_MFMA SQ_ACTIVE_INST_LDS SQ_CYCLES",
}

# (kernel name as rocprofv3 prints it, grid in work-items on the 256-CU MI355X, traffic key, source,
#  workload[, (run, runs)]) for every kernel launch the default bench run reports HBM traffic for. With
# (run, runs), the launches of that kernel and grid come from `runs` bench rows, one after the other,
# and the entry takes row number `run` of them (split_runs).
TRAFFIC_MAP = [
    ("gemm_mxfp4_ring<true>", 262144, "gemm_mxfp4_ring@prefill_mx", "gemm_mxfp4_ring.hip",
     "prefill_mx M=2048 K=4096 N=14336 bf16 Y"),
    ("gemm_mxfp4_ring<true>", 524288, "gemm_mxfp4_ring@prefill_mx_m4096", "gemm_mxfp4_ring.hip",
     "prefill_mx_m4096 M=4096 K=4096 N=14336 bf16 Y"),
    ("gemm_mxfp4_ring<false>", 1835008, "gemm_mxfp4_ring@large", "gemm_mxfp4_ring.hip",
     "large M=8192 K=8192 N=28672 fp32 Y"),
    ("gemm_nvfp4_ring<true>", 262144, "gemm_nvfp4_ring@prefill_nv", "gemm_nvfp4_ring.hip",
     "prefill_nv M=2048 K=4096 N=14336 bf16 Y"),
    ("gemm_mxfp4_decode<false, 1, 1>", 131072, "gemm_mxfp4_decode@decode", "gemm_decode.hip",
     "decode M in {1,4,16} K=4096 N=4096 fp32 Y, one 16-row tile per workgroup, W from HBM"),
    ("gemm_mxfp4_decode<false, 2, 1>", 229376, "gemm_mxfp4_decode@decode_wide", "gemm_decode.hip",
     "decode_wide M in {1,4,16} K=4096 N=14336 fp32 Y, two 16-row tiles per workgroup, W from HBM"),
    ("gemm_mxfp4_decode<false, 2, 2>", 229376, "gemm_mxfp4_decode@decode_wide32", "gemm_decode.hip",
     "decode_wide32 M=32 K=4096 N=14336 fp32 Y, two 16-row tiles and two X fragments per workgroup, W from HBM"),
    ("gemm_mxfp4_ring_skinny<false, Tile<64, 4, 2, 128, 3>>", 114688, "gemm_mxfp4_ring_skinny@decode_wide64",
     "gemm_mxfp4_ring.hip", "decode_wide64 M=64 K=4096 N=14336 fp32 Y, 128x64 tiles (rows past 64 repeat row 63), "
     "W from HBM", (0, 2)),
    ("gemm_mxfp4_ring_skinny<false, Tile<64, 4, 2, 128, 3>>", 114688, "gemm_mxfp4_ring_skinny@decode_wide128",
     "gemm_mxfp4_ring.hip", "decode_wide128 M=128 K=4096 N=14336 fp32 Y, 128x64 tiles, W from HBM", (1, 2)),
    ("gemm_nvfp4_ring_skinny<false, Tile<64, 4, 2, 128, 2>>", 114688, "gemm_nvfp4_ring_skinny@decode_nv_wide128",
     "gemm_nvfp4_ring.hip", "decode_nv_wide128 M=128 K=4096 N=14336 NVFP4 block 16 fp32 Y, 128x64 tiles, W from HBM"),
    ("gemm_nvfp4_decode<false, 2, 1>", 229376, "gemm_nvfp4_decode@decode_nv_wide", "gemm_decode.hip",
     "decode_nv_wide M in {1,16} K=4096 N=14336 NVFP4 block 16 fp32 Y, two 16-row tiles per workgroup, W from HBM"),
    ("gemm_nvfp4_decode<false, 2, 4>", 229376, "gemm_nvfp4_decode@decode_nv_wide64", "gemm_decode.hip",
     "decode_nv_wide64 M=64 K=4096 N=14336 NVFP4 block 16 fp32 Y, two 16-row tiles and four X fragments per "
     "workgroup, W from HBM"),
    ("rotate_quant_mx<32, 0>", 4194304, "rotate_quant_mx@stress_mx32", "rotate_quant.hip",
     "stress_mx32 16384x8192 block 32"),
    ("rotate_quant_mx<128, 0>", 4194304, "rotate_quant_mx@stress_mx128", "rotate_quant.hip",
     "stress_mx128 16384x8192 block 128"),
    ("rotate_amax<32>", 262144, "rotate_amax@stress_nv32", "rotate_quant.hip",
     "stress_nv32 16384x8192 block 32, max pass"),
    ("rotate_quant_nv<32, 0>", 4194304, "rotate_quant_nv@stress_nv32", "rotate_quant.hip",
     "stress_nv32 16384x8192 block 32, quantize pass"),
    ("rotate_amax<128>", 262144, "rotate_amax@stress_nv128", "rotate_quant.hip",
     "stress_nv128 16384x8192 block 128, max pass"),
    ("rotate_quant_nv<128, 0>", 4194304, "rotate_quant_nv@stress_nv128", "rotate_quant.hip",
     "stress_nv128 16384x8192 block 128, quantize pass"),
]
# SQ counter passes: (raw-output prefix, bench workload, (kernel, grid), summary file, description)
SQ_TARGETS = [
    ("sq", "prefill_mx", ("gemm_mxfp4_ring<true>", 262144), "gemm_mxfp4_ring_prefill_sq_counters.txt",
     "prefill_mx: M=2048 K=4096 N=14336, MXFP4 block 32, bf16 Y"),
    ("nvsq", "prefill_nv", ("gemm_nvfp4_ring<true>", 262144), "gemm_nvfp4_ring_prefill_nv_sq_counters.txt",
     "prefill_nv: M=2048 K=4096 N=14336, NVFP4 block 16, bf16 Y"),
]


def commands(out):
    py = "python3 $REPO/bench.py"
    lines = ["cd /tmp && export TMPDIR=/tmp REPO=$GRAFT_REPO_ROOT",
             f"timeout -k 10 300 rocprofv3 --kernel-trace --stats --output-format csv -d $REPO/{out}/trace -o run "
             f"-- {py} {TRACE_ARGS}"]
    for c, d in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        lines.append(f"timeout -s KILL 300 rocprofv3 --pmc {c} --output-format csv -d $REPO/{out}/{d} -o run "
                     f"-- {py} {BENCH_ARGS}")
        lines.append(f"timeout -s KILL 120 rocprofv3 --pmc {c} --output-format csv -d $REPO/{out}/copy_{d} -o run "
                     f"-- {py} --copy-probe 256 --no-cpu")
    for prefix, wl, _, _, _ in SQ_TARGETS:
        wl_arg = "" if wl == "prefill_mx" else f" --workload {wl}"
        for d, cs in SQ_PASSES.items():
            lines.append(f"timeout -s KILL 300 rocprofv3 --pmc {cs} --output-format csv "
                         f"-d $REPO/{out}/{prefix}{d[2:]} -o run -- {py} {BENCH_ARGS} --no-extra --stress ''{wl_arg}")
    return lines


def _rows(path_glob):
    files = sorted(glob.glob(path_glob, recursive=True))
    if not files:
        raise SystemExit(f"no file matches {path_glob}")
    out = []
    for fn in files:
        with open(fn, newline="") as f:
            out += list(csv.DictReader(f))
    return out


def _grid(r):
    if "Grid_Size" in r:
        return int(r["Grid_Size"])
    return int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y", 1) or 1) * int(r.get("Grid_Size_Z", 1) or 1)


def _name(r):
    n = r["Kernel_Name"].replace("void ", "").replace("fp4::(anonymous namespace)::", "")
    return n.split("(")[0].strip().replace("> >", ">>")


def split_runs(d, counter, kern, runs):
    """Means per dispatch of one counter for the launches of kern = (kernel, grid), split into `runs`
    groups at the runs - 1 widest gaps between their dispatch ids (bench rows that use the same
    kernel and grid run one after the other, with other launches between them); [(mean, count)]."""
    per_dispatch = {}
    for r in _rows(os.path.join(d, "**", "*counter_collection.csv")):
        if r["Counter_Name"] != counter or (_name(r), _grid(r)) != kern:
            continue
        i = int(r.get("Dispatch_Id", r.get("Correlation_Id")))
        per_dispatch[i] = per_dispatch.get(i, 0.0) + float(r["Counter_Value"])
    ids = sorted(per_dispatch)
    cuts = sorted(sorted(range(1, len(ids)), key=lambda j: ids[j] - ids[j - 1])[-(runs - 1):]) if runs > 1 else []
    bounds = [0] + cuts + [len(ids)]
    return [(statistics.fmean(per_dispatch[i] for i in ids[a:b]), b - a) for a, b in zip(bounds, bounds[1:])]


def counter_means(d, counter):
    """Mean value per dispatch of one counter, by (kernel, grid)."""
    acc = {}
    per_dispatch = {}
    for r in _rows(os.path.join(d, "**", "*counter_collection.csv")):
        if r["Counter_Name"] != counter:
            continue
        k = (_name(r), _grid(r), r.get("Dispatch_Id", r.get("Correlation_Id")))
        per_dispatch[k] = per_dispatch.get(k, 0.0) + float(r["Counter_Value"])
    for (n, g, _), v in per_dispatch.items():
        acc.setdefault((n, g), []).append(v)
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def summarize(out):
    out = os.path.join(ROOT, out) if not os.path.isabs(out) else out
    cmds = commands(os.path.relpath(out, ROOT))
    # each summary is written only when its raw output is present, so a partial run (say, the SQ
    # passes alone) leaves the other summaries as they are
    if os.path.isdir(os.path.join(out, "trace")):
        _summarize_trace_and_traffic(out, cmds)
    _summarize_sq(out, cmds)


def _summarize_trace_and_traffic(out, cmds):
    import bench

    # kernel trace: per (kernel, grid) medians and means
    trace = _rows(os.path.join(out, "trace", "**", "*kernel_trace.csv"))
    durs = {}
    for r in trace:
        durs.setdefault((_name(r), _grid(r)), []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    stats_rows = _rows(os.path.join(out, "trace", "**", "*kernel_stats.csv"))
    lines = ["# rocprofv3 kernel statistics of the bench.py run below (prefill_mx step, the rotate+quantize stress",
             "# workloads and variants, the NVFP4 and large GEMMs, the decode rows and the offline weight quantizations)",
             "# command:", "#   " + cmds[0], "#   " + cmds[1],
             "# per-grid medians and means from the kernel trace (the --stats table below pools every grid of a kernel):"]
    for (n, g), v in sorted(durs.items()):
        lines.append(f"#   {n} grid {g}: {len(v)} calls, median {statistics.median(v):.1f} us, "
                     f"mean {statistics.fmean(v):.1f} us")
    lines.append("# Name | Calls | TotalDurationNs | AverageNs | Percentage | MinNs | MaxNs")
    for r in stats_rows:
        lines.append(" | ".join(str(r.get(c, "")) for c in ("Name", "Calls", "TotalDurationNs", "AverageNs",
                                                           "Percentage", "MinNs", "MaxNs")))
    with open(os.path.join(PROFILES, "bench_default_kernel_stats.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")

    # HBM traffic
    cal = 256 << 20
    cf = counter_means(os.path.join(out, "copy_fetch"), "FETCH_SIZE")
    cw = counter_means(os.path.join(out, "copy_write"), "WRITE_SIZE")
    copy_f = max(v for (n, g), (v, c) in cf.items() if "copy" in n.lower() or "elementwise" in n)
    copy_w = max(v for (n, g), (v, c) in cw.items() if "copy" in n.lower() or "elementwise" in n)
    sf, sw = cal / (copy_f * 1024), cal / (copy_w * 1024)
    fetch = counter_means(os.path.join(out, "fetch"), "FETCH_SIZE")
    write = counter_means(os.path.join(out, "write"), "WRITE_SIZE")
    lines = ["# HBM traffic per dispatch from rocprofv3 counters of the bench.py run below, one counter per run",
             "# commands:"] + ["#   " + c for c in cmds[0:1] + cmds[2:6]] + [
        f"# calibration: the same counters on a plain 256 MiB device copy: read scale {sf:.4f}, write scale {sw:.4f}",
        "# (HBM bytes = counter KiB * 1024 * scale)",
        "# kernel | grid | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB | HBM write MB | trace median us"]
    for k in sorted(set(fetch) | set(write)):
        fv, fc = fetch.get(k, (float("nan"), 0))
        wv, _ = write.get(k, (float("nan"), 0))
        med = statistics.median(durs[k]) if k in durs else float("nan")
        lines.append(f"{k[0]} | {k[1]} | {fc} | {fv:.1f} | {wv:.1f} | {fv * 1024 * sf / 1e6:.2f} | "
                     f"{wv * 1024 * sw / 1e6:.2f} | {med:.1f}")
    with open(os.path.join(PROFILES, "bench_default_hbm_counters.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    table = {"_comment": "HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per dispatch), "
                         "each scaled by the same counter's reading for a plain 256 MiB device copy; valid only while "
                         "the hash of the kernel source and the shared headers matches (bench_profiles.py)",
             "copy_scale_fetch": sf, "copy_scale_write": sw}
    for n, g, key, src, wl, *part in TRAFFIC_MAP:
        if (n, g) not in fetch or (n, g) not in write:
            print(f"warning: no counters for {n} grid {g} ({key})", file=sys.stderr)
            continue
        (fv, fc), (wv, _) = fetch[(n, g)], write[(n, g)]
        if part:
            run, runs = part[0]
            fr = split_runs(os.path.join(out, "fetch"), "FETCH_SIZE", (n, g), runs)
            wr = split_runs(os.path.join(out, "write"), "WRITE_SIZE", (n, g), runs)
            # the rows sharing a kernel and grid launch it equally often; anything else means the
            # widest gaps did not fall between rows (say, a row was left out of the run)
            if len({c for _, c in fr}) != 1 or len({c for _, c in wr}) != 1:
                print(f"warning: {key}: launches of {n} grid {g} do not split into {runs} equal rows", file=sys.stderr)
                continue
            (fv, fc), (wv, _) = fr[run], wr[run]
        rb, wb = fv * 1024 * sf, wv * 1024 * sw
        table[key] = {"workload": wl, "kernel": n, "grid": g, "source_sha": bench.source_sha(src),
                      "bytes_per_launch": rb + wb, "read_bytes": rb, "write_bytes": wb, "dispatches": fc}
    with open(os.path.join(PROFILES, "traffic.json"), "w") as f:
        json.dump(table, f, indent=1)
        f.write("\n")


def _summarize_sq(out, cmds):
    # SQ counters of the GEMMs
    for prefix, wl, kern, fname, desc in SQ_TARGETS:
        dirs = [prefix + d[2:] for d in SQ_PASSES]
        if not all(os.path.isdir(os.path.join(out, d)) for d in dirs):
            continue
        vals = {}
        for d, (pd, cs) in zip(dirs, SQ_PASSES.items()):
            for c in cs.split():
                m = counter_means(os.path.join(out, d), c)
                if kern in m:
                    vals[c] = m[kern]
        lines = [f"# SQ counters of {kern[0]} grid {kern[1]} ({desc}), averages per dispatch summed",
                 "# over the chip. SQ_WAVE_CYCLES and SQ_WAIT_* are sampled every 4 cycles. commands:"]
        lines += ["#   " + cmds[0]] + ["#   " + c for c in cmds if any(f"/{d} " in c for d in dirs)]
        for c, (v, n) in vals.items():
            extra = ""
            if c.startswith("SQ_WAIT") and "SQ_WAVE_CYCLES" in vals:
                extra = f"   ({v / vals['SQ_WAVE_CYCLES'][0]:.1%} of wave cycles)"
            lines.append(f"{c:<32}{v:>16.0f}  over {n} dispatches{extra}")
        with open(os.path.join(PROFILES, fname), "w") as f:
            f.write("\n".join(lines) + "\n")


def main():
    if len(sys.argv) != 3 or sys.argv[1] not in ("commands", "summarize"):
        raise SystemExit(__doc__)
    if sys.argv[1] == "commands":
        print(" &&\n".join(commands(sys.argv[2])))
    else:
        summarize(sys.argv[2])


if __name__ == "__main__":
    main()
