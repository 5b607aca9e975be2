#!/usr/bin/env python3
"""Benchmark of the online FP4 linear-layer path on one MI355X.

A step is one pass of the whole online path over one batch of synthetic input:
block-Hadamard rotate + MXFP4 quantize of the bf16 activations
(fp4_rotate_quantize), then the W4A4 GEMM against weights rotated and
quantized offline (fp4_linear). The default workload is the prefill linear
layer K=4096, N=14336 with M=2048 tokens, MXFP4, Hadamard block 32, float32
accumulation and bf16 output. Weights are quantized once, before timing (offline
in the method).

Printed: ONE JSON line with the step throughput (TFLOP/s of the linear layer,
2*M*N*K per step), the GEMM's roofline (MFMA FP4 peak), the rotate+quantize
roofline on the full-size bandwidth-stress workload (16384 x 8192 bf16, HBM
peak), and the CPU oracle timed on the host as a baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense MXFP4 MFMA
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "MXFP4 W4A4 linear TFLOP/s + rotate-quantize GB/s (% roofline), K=4096"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# headers every kernel source includes: a change in them changes the kernels too
SHARED_HEADERS = ("common.hpp", "quant_device.hpp")


def source_sha(name: str) -> str:
    """Hash of a kernel source and the shared headers it is compiled with."""
    h = hashlib.sha256()
    for n in (name,) + SHARED_HEADERS:
        with open(os.path.join(ROOT, "microscaling_fp4_quantized_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key: str, source: str, launches_per_unit: float = 1.0):
    """HBM bytes per launch from committed rocprofv3 --pmc counters, or None if the
    kernel source changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kernel_key)
    if not e or e.get("source_sha") != source_sha(source):
        return None
    return e["bytes_per_launch"] * launches_per_unit


def gemm_kernel_for(fmt: str, M: int, N: int, K: int):
    """(source file, kernel name) of the kernel fp4_linear runs for this shape when the scale
    buffers are 16-byte aligned (torch's allocations are): the library's dispatch predicates, in
    its order."""
    if fmt == "mxfp4":
        ring = K % 512 == 0 and K < (1 << 25) and ((M >= 256 and N >= 256) or (M > 64 and N >= 1024) or
                                                   (M > 32 and N >= 8192))
        if not (ring and M > 32) and K % 512 == 0 and (K < (1 << 28) if M <= 16 else (M <= 64 and K <= 8192)):
            return "gemm_decode.hip", "gemm_mxfp4_decode"
        if ring:
            return ("gemm_mxfp4_ring.hip", "gemm_mxfp4_ring" if M >= 256 else "gemm_mxfp4_ring_skinny")
        return "gemm_mxfp4.hip", "gemm_mxfp4_kernel"
    if M <= 64 and K % 512 == 0 and K <= 8192:
        return "gemm_decode.hip", "gemm_nvfp4_decode"
    if K % 256 == 0 and K < (1 << 25) and M >= 256 and N >= 256:
        return "gemm_nvfp4_ring.hip", "gemm_nvfp4_ring"
    if K % 256 == 0 and K < (1 << 25) and M > 64 and N >= 1024:
        return "gemm_nvfp4_ring.hip", "gemm_nvfp4_ring_skinny"
    return "gemm_nvfp4.hip", "gemm_nvfp4_kernel"


def bf16_dev(bits, dev):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def time_batch(fn, iters, torch):
    """Average device time (ms) per launch of fn(i), i = 0..iters-1, issued back to back on the
    current stream (the one the library launches on) between one pair of HIP events, so that
    neither event overhead nor host launch gaps are counted per launch."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(iters):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / iters


def ramp(fn, torch, seconds=0.1):
    """Untimed calls of fn(i) for about `seconds`, so that the batch timed next runs at this
    kernel's own steady clocks (the GPU sets its clock by the load it carries: right after a
    different kernel, or after idling, the same kernel runs at another speed)."""
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            fn(i)
            i += 1
        torch.cuda.synchronize()


def time_graph(fn, iters, torch):
    """Average device time (ms) per call of fn(i) with `iters` calls captured in one HIP graph and
    replayed between two events, so the host's launch rate does not bound kernels that run for a
    few microseconds. The library launches on torch's current stream, which is the capture stream
    inside torch.cuda.graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(iters):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / iters


def time_cold(fn, iters, torch, dev):
    """Per-launch device time (us) of fn(i) with a 1 GiB buffer read before each launch, so that the
    256 MB Infinity Cache and the L2s hold only clean lines of that buffer (a written flush would
    leave dirty lines whose write-back the timed kernel would pay for); returns the median and the
    10th / 90th percentiles."""
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    ts = []
    for i in range(iters):
        torch.sum(flush, dim=(0,), out=sink)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn(i)
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    del flush
    ts.sort()
    return {"median_us": ts[len(ts) // 2], "p10_us": ts[len(ts) // 10], "p90_us": ts[(9 * len(ts)) // 10],
            "launches": iters}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rq_worker(args):
    """One pool worker of the CPU rotate+quantize baseline: the oracle on a block of rows."""
    lo, hi = args
    from oracle import fp4_oracle as O

    O.rotate_quantize(_CPU_RQ["x"][lo:hi], _CPU_RQ["block"], _CPU_RQ["fmt"])
    return hi - lo


_CPU_RQ = {}


def cpu_rotate_quantize(wl, rows_per_worker=1024, max_workers=16):
    """The oracle's rotate+quantize (float32 FWHT, exact scale and rounding, NumPy) on the first
    rows of a workload's X, split by rows over a pool of host processes, one per core up to
    max_workers. Runs before the GPU is touched (the pool forks), and reports GB/s of the same
    algorithmic bytes as the GPU figure."""
    import multiprocessing as mp

    from microscaling_fp4_quantized_amd import workloads as WL

    P = max(1, min(max_workers, os.cpu_count() or 1))
    rows = min(wl.M, rows_per_worker * P)
    _CPU_RQ.update(x=WL.draw_x(wl, M=rows), block=wl.block, fmt=wl.fmt)
    bounds = [(rows * i // P, rows * (i + 1) // P) for i in range(P)]
    with mp.get_context("fork").Pool(P) as pool:
        pool.map(abs, range(P))  # every worker is up before the clock starts
        t0 = time.perf_counter()
        done = sum(pool.map(_oracle_rq_worker, bounds))
        dt = time.perf_counter() - t0
    _CPU_RQ.clear()
    g = 32 if wl.fmt == "mxfp4" else 16
    nbytes = done * wl.K * (2 + 0.5 + 1.0 / g)
    return {"GB/s": nbytes / dt / 1e9, "unit": "GB/s", "cores": P, "seconds": dt, "algorithmic_bytes": nbytes,
            "sample": f"the first {done} rows of {wl.name} ({wl.M}x{wl.K} bf16, block {wl.block}, "
                      f"{wl.fmt.upper()}), {P} processes of {done // P} rows each, oracle rotate+quantize "
                      f"(single-threaded NumPy per process)"}


def quant_parity_counts(O, x_bits, block, fmt, codes, scales, rows):
    """Near-boundary and mismatch counts of the GPU's codes and scales on sampled rows against the
    oracle (MXFP4; the rule of the parity tests: differences at flagged elements are reported apart
    from the others)."""
    xr = x_bits[rows]
    o_packed, o_scales, o_ts = O.rotate_quantize(xr, block, fmt)
    y32 = O.rotate_fwht_f32(O.widen_bf16(xr), block)
    flags = O.near_boundary_flags(y32, o_scales, fmt, o_ts)
    diff = O.unpack_nibbles(o_packed) != O.unpack_nibbles(codes[rows])
    g = 32 if fmt == "mxfp4" else 16
    gflags = flags.reshape(flags.shape[0], -1, g).any(axis=2)
    sdiff = o_scales != scales[rows]
    return {"rows_checked": int(len(rows)), "elements": int(diff.size), "flagged": int(flags.sum()),
            "code_mismatch_flagged": int((diff & flags).sum()), "code_mismatch_unflagged": int((diff & ~flags).sum()),
            "scale_mismatch_flagged": int((sdiff & gflags).sum()),
            "scale_mismatch_unflagged": int((sdiff & ~gflags).sum())}


def cpu_baseline(wl, x_bits, w_bits, rq_cpu=None, parity=None):
    """The oracle (plain NumPy, untuned) on whole steps of the workload, with the rotate+quantize
    baseline in GB/s and the parity counts measured beside it."""
    from threadpoolctl import threadpool_info

    from oracle import fp4_oracle as O

    wq, ws, wts = O.rotate_quantize(w_bits, wl.block, wl.fmt)  # offline, untimed (as on the GPU)
    # whole steps until about 10 s of CPU work (at most 12), averaged
    steps, t0 = 0, time.perf_counter()
    while steps < 12 and (steps == 0 or time.perf_counter() - t0 < 10.0):
        xq, xs, xts = O.rotate_quantize(x_bits, wl.block, wl.fmt)
        O.linear_f64(xq, xs, wq, ws, wl.fmt, xts, wts)
        steps += 1
    dt = (time.perf_counter() - t0) / steps
    blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    flops = 2.0 * wl.M * wl.N * wl.K
    out = {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(max(blas) if blas else 1),
        "kind": "oracle",
        "sample": f"{steps} full steps of {wl.name} (M={wl.M}, K={wl.K}, N={wl.N}), averaged: oracle "
                  f"rotate+quantize of X (float32 FWHT, single-threaded NumPy) + float64 dequantized product "
                  f"(BLAS dgemm on the BLAS threads counted in cores); {dt:.2f} s per step",
        "seconds": dt,
        "host": {"cpu_model": cpu_model(), "cpu_count": os.cpu_count()},
    }
    if rq_cpu is not None:
        out["rotate_quantize"] = rq_cpu
    if parity is not None:
        out["parity_counts"] = parity
    return out


EXTRA_ROWS = ("nv_stress", "variants", "block128", "nv_gemm", "large", "m4096", "decode")


def extra_rows(B, WL, torch, dev, groups=EXTRA_ROWS):
    """The other rows of the path, each timed over back-to-back launches on the library's stream
    (groups: nv_stress, variants, block128 on the 16384x8192 stress input; nv_gemm, large, m4096
    GEMMs; decode, see decode_rows)."""
    out = {}
    sw = WL.WORKLOADS["stress_nv32"]
    if {"nv_stress", "variants", "block128"} & set(groups):
        sx = WL.draw_x(sw)
        bufs = [bf16_dev(sx, dev) for _ in range(3)]
        del sx
        flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        torch.sum(flush, dim=(0,))
        del flush
        o = (torch.empty((sw.M, sw.K // 2), dtype=torch.uint8, device=dev),
             torch.empty((sw.M, sw.K // 16), dtype=torch.uint8, device=dev),
             torch.empty((1,), dtype=torch.float32, device=dev))
        for i in range(3):
            B.fp4_rotate_quantize(bufs[i % 3], sw.block, "nvfp4", out=o)
    if "nv_stress" in groups:
        # NVFP4 rotate+quantize, 16384 x 8192, block 32: the max pass and the quantize pass
        ramp(lambda i: B.fp4_rotate_quantize(bufs[i % 3], sw.block, "nvfp4", out=o), torch)
        ms = time_batch(lambda i: B.fp4_rotate_quantize(bufs[i % 3], sw.block, "nvfp4", out=o), 21, torch)
        nbytes = sw.M * sw.K * (2 + 2 + 0.5 + 1.0 / 16) + 8
        t_max = measured_traffic("rotate_amax@stress_nv32", "rotate_quant.hip")
        t_nv = measured_traffic("rotate_quant_nv@stress_nv32", "rotate_quant.hip")
        out["rotate_quantize_nvfp4"] = {
            "workload": "stress_nv32: X 16384x8192 bf16, block 32, NVFP4 (max pass + quantize pass)",
            "us": ms * 1e3, "GB/s": nbytes / (ms * 1e-3) / 1e9,
            "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": nbytes,
            "traffic": None if t_max is None or t_nv is None else t_max + t_nv}
        log(f"[bench] NVFP4 stress rotate+quantize {ms * 1e3:.1f} us = {out['rotate_quantize_nvfp4']['GB/s']:.0f} GB/s")
    if "variants" in groups:
        # quantizer variants on the same 16384 x 8192 input (block 32)
        signs = torch.from_numpy(WL.draw_signs(sw.K, 1)).to(dev)
        var = {}
        given = torch.tensor([float(o[2].item())], dtype=torch.float32, device=dev)  # the computed s_t, reused
        for fmt, rule, sg in (("nvfp4", "fit", None), ("nvfp4", "given_scale", None), ("mxfp4", "oas", None),
                              ("mxfp4", "ocp_floor", None), ("mxfp4", "fit", None), ("mxfp4", "standard", signs)):
            g = 32 if fmt == "mxfp4" else 16
            oo = (torch.empty((sw.M, sw.K // 2), dtype=torch.uint8, device=dev),
                  torch.empty((sw.M, sw.K // g), dtype=torch.uint8, device=dev),
                  torch.empty((1,), dtype=torch.float32, device=dev) if fmt == "nvfp4" else None)

            def call(i, fmt=fmt, rule=rule, sg=sg, oo=oo):
                if rule == "given_scale":
                    B.fp4_rotate_quantize(bufs[i % 3], sw.block, fmt, out=oo, tensor_scale=given)
                else:
                    B.fp4_rotate_quantize(bufs[i % 3], sw.block, fmt, out=oo, rule=rule, signs=sg)

            ramp(call, torch)
            ms = time_batch(call, 12, torch)
            nb = sw.M * sw.K * ((2 if fmt == "nvfp4" and rule != "given_scale" else 0) + 2 + 0.5 + 1.0 / g)
            name = f"{fmt}_{rule}" + ("_signs" if sg is not None else "")
            var[name] = {"us": ms * 1e3, "GB/s": nb / (ms * 1e-3) / 1e9,
                         "frac_hbm": nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
            log(f"[bench] variant {name}: {ms * 1e3:.1f} us = {var[name]['GB/s']:.0f} GB/s")
        out["rotate_quantize_variants"] = {"workload": "16384x8192 bf16, block 32 (stress_nv32 input)", **var}
    if "block128" in groups:
        # the same input with the 128-element Hadamard block, both formats
        b128 = {}
        for fmt in ("mxfp4", "nvfp4"):
            g = 32 if fmt == "mxfp4" else 16
            oo = (torch.empty((sw.M, sw.K // 2), dtype=torch.uint8, device=dev),
                  torch.empty((sw.M, sw.K // g), dtype=torch.uint8, device=dev),
                  torch.empty((1,), dtype=torch.float32, device=dev) if fmt == "nvfp4" else None)

            def call128(i, fmt=fmt, oo=oo):
                B.fp4_rotate_quantize(bufs[i % 3], 128, fmt, out=oo)

            ramp(call128, torch)
            ms = time_batch(call128, 21, torch)
            nb = sw.M * sw.K * ((2 if fmt == "nvfp4" else 0) + 2 + 0.5 + 1.0 / g) + (8 if fmt == "nvfp4" else 0)
            if fmt == "mxfp4":
                tr = measured_traffic("rotate_quant_mx@stress_mx128", "rotate_quant.hip")
            else:
                t1 = measured_traffic("rotate_amax@stress_nv128", "rotate_quant.hip")
                t2 = measured_traffic("rotate_quant_nv@stress_nv128", "rotate_quant.hip")
                tr = None if t1 is None or t2 is None else t1 + t2
            b128[fmt] = {"us": ms * 1e3, "GB/s": nb / (ms * 1e-3) / 1e9,
                         "frac_hbm": nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": nb, "traffic": tr}
            log(f"[bench] block 128 {fmt} stress rotate+quantize {ms * 1e3:.1f} us = {b128[fmt]['GB/s']:.0f} GB/s "
                f"({b128[fmt]['frac_hbm']:.1%} of HBM)")
        out["rotate_quantize_block128"] = {
            "workload": "stress_mx128 / stress_nv128: X 16384x8192 bf16 (the stress_nv32 input), block 128; NVFP4 "
                        "counts its max pass as a second read of X", **b128}
    if {"nv_stress", "variants", "block128"} & set(groups):
        del bufs, o
    if "nv_gemm" in groups:
        # NVFP4 prefill GEMM, M=2048 K=4096 N=14336, Y bf16
        wl = WL.WORKLOADS["prefill_nv"]
        xq, xs, xts = B.fp4_rotate_quantize(bf16_dev(WL.draw_x(wl), dev), wl.block, "nvfp4")
        wq, ws, wts = B.fp4_quantize_weights(bf16_dev(WL.draw_w(wl), dev), wl.block, "nvfp4")
        y = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device=dev)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.25:  # 250 ms of this kernel first, at its own steady clocks
            for _ in range(10):
                B.fp4_linear(xq, xs, wq, ws, "nvfp4", x_ts=xts, w_ts=wts, out_dtype=torch.bfloat16, out=y)
            torch.cuda.synchronize()
        ms = time_batch(lambda i: B.fp4_linear(xq, xs, wq, ws, "nvfp4", x_ts=xts, w_ts=wts,
                                               out_dtype=torch.bfloat16, out=y), 20, torch)
        tf = 2.0 * wl.M * wl.N * wl.K / (ms * 1e-3) / 1e12
        out["gemm_nvfp4"] = {"workload": "prefill_nv: M=2048 K=4096 N=14336, block 16, Y bf16",
                             "us": ms * 1e3, "TFLOP/s": tf, "frac_bf16_mfma_peak": tf / MFMA_BF16_PEAK_TFLOPS,
                             "frac_fp4_mfma_peak": tf / MFMA_FP4_PEAK_TFLOPS,
                             "traffic": measured_traffic("gemm_nvfp4_ring@prefill_nv", "gemm_nvfp4_ring.hip")}
        log(f"[bench] NVFP4 GEMM {ms * 1e3:.1f} us = {tf:.0f} TFLOP/s ({tf / MFMA_BF16_PEAK_TFLOPS:.1%} of the 16-bit peak)")
        del xq, xs, wq, ws, y
    if "large" in groups:
        # the large MXFP4 configuration: M=8192 K=8192 N=28672, block 128, Y fp32 (whole rounds of tiles)
        wl = WL.WORKLOADS["large"]
        xq, xs, _ = B.fp4_rotate_quantize(bf16_dev(WL.draw_x(wl), dev), wl.block, "mxfp4")
        wq, ws, _ = B.fp4_quantize_weights(bf16_dev(WL.draw_w(wl), dev), wl.block, "mxfp4")
        y = torch.empty((wl.M, wl.N), dtype=torch.float32, device=dev)
        ramp(lambda i: B.fp4_linear(xq, xs, wq, ws, "mxfp4", out=y), torch, 0.25)
        ms = time_batch(lambda i: B.fp4_linear(xq, xs, wq, ws, "mxfp4", out=y), 10, torch)
        tf = 2.0 * wl.M * wl.N * wl.K / (ms * 1e-3) / 1e12
        out["gemm_mxfp4_large"] = {"workload": "large: M=8192 K=8192 N=28672, block 128, Y fp32",
                                   "us": ms * 1e3, "TFLOP/s": tf, "frac_fp4_mfma_peak": tf / MFMA_FP4_PEAK_TFLOPS,
                                   "algorithmic_bytes": (wl.M + wl.N) * wl.K * (0.5 + 1.0 / 32) + wl.M * wl.N * 4,
                                   "traffic": measured_traffic("gemm_mxfp4_ring@large", "gemm_mxfp4_ring.hip")}
        log(f"[bench] large MXFP4 GEMM {ms * 1e3:.1f} us = {tf:.0f} TFLOP/s ({tf / MFMA_FP4_PEAK_TFLOPS:.1%} of peak)")
        del xq, xs, wq, ws, y
    if "m4096" in groups:
        # the headline layer at twice the tokens: M=4096 K=4096 N=14336, MXFP4 block 32, Y bf16
        wl = WL.WORKLOADS["prefill_mx_m4096"]
        xq, xs, _ = B.fp4_rotate_quantize(bf16_dev(WL.draw_x(wl), dev), wl.block, "mxfp4")
        wq, ws, _ = B.fp4_quantize_weights(bf16_dev(WL.draw_w(wl), dev), wl.block, "mxfp4")
        y = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device=dev)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.25:  # 250 ms of this kernel first, as the headline step's ramp
            for _ in range(20):
                B.fp4_linear(xq, xs, wq, ws, "mxfp4", out_dtype=torch.bfloat16, out=y)
            torch.cuda.synchronize()
        ms = time_batch(lambda i: B.fp4_linear(xq, xs, wq, ws, "mxfp4", out_dtype=torch.bfloat16, out=y), 20, torch)
        tf = 2.0 * wl.M * wl.N * wl.K / (ms * 1e-3) / 1e12
        out["gemm_mxfp4_m4096"] = {"workload": "prefill_mx_m4096: M=4096 K=4096 N=14336, block 32, Y bf16",
                                   "us": ms * 1e3, "TFLOP/s": tf, "frac_fp4_mfma_peak": tf / MFMA_FP4_PEAK_TFLOPS,
                                   "algorithmic_bytes": (wl.M + wl.N) * wl.K * (0.5 + 1.0 / 32) + wl.M * wl.N * 2,
                                   "traffic": measured_traffic("gemm_mxfp4_ring@prefill_mx_m4096",
                                                               "gemm_mxfp4_ring.hip")}
        log(f"[bench] M=4096 MXFP4 GEMM {ms * 1e3:.1f} us = {tf:.0f} TFLOP/s ({tf / MFMA_FP4_PEAK_TFLOPS:.1%} of peak)")
        del xq, xs, wq, ws, y
    if "decode" in groups:
        out.update(decode_rows(B, WL, torch, dev))
        out.update(nv_decode_rows(B, WL, torch, dev))
    return out


# traffic-table key and kernel source of each decode row (the kernel and its launch differ with N and M)
DECODE_TRAFFIC_KEY = {
    "decode1": ("gemm_mxfp4_decode@decode", "gemm_decode.hip"),
    "decode4": ("gemm_mxfp4_decode@decode", "gemm_decode.hip"),
    "decode16": ("gemm_mxfp4_decode@decode", "gemm_decode.hip"),
    "decode_wide1": ("gemm_mxfp4_decode@decode_wide", "gemm_decode.hip"),
    "decode_wide4": ("gemm_mxfp4_decode@decode_wide", "gemm_decode.hip"),
    "decode_wide16": ("gemm_mxfp4_decode@decode_wide", "gemm_decode.hip"),
    "decode_wide32": ("gemm_mxfp4_decode@decode_wide32", "gemm_decode.hip"),
    "decode_wide64": ("gemm_mxfp4_ring_skinny@decode_wide64", "gemm_mxfp4_ring.hip"),
    "decode_wide128": ("gemm_mxfp4_ring_skinny@decode_wide128", "gemm_mxfp4_ring.hip"),
    "decode_nv_wide1": ("gemm_nvfp4_decode@decode_nv_wide", "gemm_decode.hip"),
    "decode_nv_wide16": ("gemm_nvfp4_decode@decode_nv_wide", "gemm_decode.hip"),
    "decode_nv_wide64": ("gemm_nvfp4_decode@decode_nv_wide64", "gemm_decode.hip"),
    "decode_nv_wide128": ("gemm_nvfp4_ring_skinny@decode_nv_wide128", "gemm_nvfp4_ring.hip"),
}


def decode_rows(B, WL, torch, dev, names=("decode1", "decode4", "decode16", "decode_wide1", "decode_wide4",
                                            "decode_wide16", "decode_wide32", "decode_wide64", "decode_wide128")):
    """Decode-shaped MXFP4 layers (M in {1, 4, 16} tokens, K=4096; W 4096x4096 or 14336x4096; and
    batches of 32, 64 and 128 tokens against the wide W), bound by reading W from HBM. Each row is timed as a HIP graph of calls that cycle over copies of
    W totalling more than 512 MB, so that no call finds its W in the 256 MB Infinity Cache (as in a
    model whose weights do not fit in it); the graph's result is checked against an eager call. The
    same call with one W, resident in the cache, is reported as warm_us. The whole decode step from
    bf16 X (two calls, or for M <= 16 the one-launch fused call) is timed the same way."""
    import math

    out = {}
    for name in names:
        wl = WL.WORKLOADS[name]
        xb = bf16_dev(WL.draw_x(wl), dev)
        wq, ws, _ = B.fp4_quantize_weights(bf16_dev(WL.draw_w(wl), dev), wl.block, "mxfp4")
        wbytes = wl.N * wl.K * (0.5 + 1.0 / 32)
        n_sets = int(math.ceil(512e6 / wbytes))
        sets = [(wq.clone(), ws.clone()) for _ in range(n_sets)]
        xq, xs, _ = B.fp4_rotate_quantize(xb, wl.block, "mxfp4")
        y = torch.empty((wl.M, wl.N), dtype=torch.float32, device=dev)
        B.fp4_linear(xq, xs, wq, ws, "mxfp4", out=y)
        ref = y.clone()
        calls = 2 * n_sets

        def gemm(i):
            w_i = sets[i % n_sets]
            B.fp4_linear(xq, xs, w_i[0], w_i[1], "mxfp4", out=y)

        y.zero_()
        ms = time_graph(gemm, calls, torch)
        graph_ok = bool(torch.equal(y, ref))
        ms_warm = time_graph(lambda i: B.fp4_linear(xq, xs, wq, ws, "mxfp4", out=y), 50, torch)
        ms_call = time_batch(lambda i: B.fp4_linear(xq, xs, wq, ws, "mxfp4", out=y), 50, torch)
        nbytes = wbytes + wl.M * wl.K * (0.5 + 1.0 / 32) + wl.M * wl.N * 4
        row = {"workload": f"{name}: M={wl.M} K={wl.K} N={wl.N} MXFP4, Y fp32",
               "us": ms * 1e3, "GB/s": nbytes / (ms * 1e-3) / 1e9,
               "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": nbytes,
               "w_copies": n_sets, "graph_replay_matches_eager": graph_ok,
               "warm_us": ms_warm * 1e3, "warm_GB/s": nbytes / (ms_warm * 1e-3) / 1e9,
               "us_per_python_call": ms_call * 1e3,
               "traffic": measured_traffic(*DECODE_TRAFFIC_KEY[name]),
               "note": f"{calls} calls in one HIP graph over {n_sets} copies of W ({n_sets * wbytes / 1e6:.0f} MB), "
                       "so W comes from HBM; warm_us: one W, resident in the Infinity Cache"}
        log(f"[bench] {name} GEMM {ms * 1e3:.2f} us with W from HBM = {row['GB/s']:.0f} GB/s "
            f"({row['frac_hbm']:.1%} of HBM); W in cache {ms_warm * 1e3:.2f} us; graph matches eager: {graph_ok}")
        # the whole decode step from bf16 X: two calls, or the one-launch fused kernel
        xqo = (torch.empty((wl.M, wl.K // 2), dtype=torch.uint8, device=dev),
               torch.empty((wl.M, wl.K // 32), dtype=torch.uint8, device=dev), None)
        y2 = torch.empty_like(y)

        def two_calls(i):
            w_i = sets[i % n_sets]
            B.fp4_rotate_quantize(xb, wl.block, "mxfp4", out=xqo)
            B.fp4_linear(xqo[0], xqo[1], w_i[0], w_i[1], "mxfp4", out=y2)

        ws_buf = torch.empty(B.linear_workspace_bytes(wl.M, wl.K), dtype=torch.uint8, device=dev)

        def fused(i):
            w_i = sets[i % n_sets]
            B.fp4_rotate_quantize_linear(xb, w_i[0], w_i[1], wl.block, out=y, workspace=ws_buf)

        ms_two = time_graph(two_calls, calls, torch)
        if wl.M <= 16:
            ms_fused = time_graph(fused, calls, torch)
            same = bool(torch.equal(y, y2))
            row["step_from_bf16_x"] = {"two_calls_us": ms_two * 1e3, "fused_us": ms_fused * 1e3,
                                       "fused_equals_two_calls": same}
            log(f"[bench] {name} step from bf16 X, W from HBM: two calls {ms_two * 1e3:.2f} us, "
                f"fused {ms_fused * 1e3:.2f} us (same result: {same})")
        else:  # the fused call takes at most 16 tokens
            row["step_from_bf16_x"] = {"two_calls_us": ms_two * 1e3}
            log(f"[bench] {name} step from bf16 X, W from HBM: two calls {ms_two * 1e3:.2f} us")
        out[f"gemm_{name}"] = row
        del sets, wq, ws
    return out


def nv_decode_rows(B, WL, torch, dev, names=("decode_nv_wide1", "decode_nv_wide16", "decode_nv_wide64",
                                               "decode_nv_wide128")):
    """NVFP4 decode-shaped layers (1, 16, 64 and 128 tokens, K=4096, W 14336x4096, block 16), timed as
    decode_rows times the MXFP4 ones: a HIP graph of calls over copies of W totalling more than
    512 MB (W from HBM), and warm_us with one W resident in the Infinity Cache."""
    import math

    out = {}
    for name in names:
        wl = WL.WORKLOADS[name]
        xq, xs, xt = B.fp4_rotate_quantize(bf16_dev(WL.draw_x(wl), dev), wl.block, "nvfp4")
        wq, ws, wt = B.fp4_quantize_weights(bf16_dev(WL.draw_w(wl), dev), wl.block, "nvfp4")
        wbytes = wl.N * wl.K * (0.5 + 1.0 / 16)
        n_sets = int(math.ceil(512e6 / wbytes))
        sets = [(wq.clone(), ws.clone()) for _ in range(n_sets)]
        y = torch.empty((wl.M, wl.N), dtype=torch.float32, device=dev)
        B.fp4_linear(xq, xs, wq, ws, "nvfp4", x_ts=xt, w_ts=wt, out=y)
        ref = y.clone()
        calls = 2 * n_sets

        def gemm(i):
            w_i = sets[i % n_sets]
            B.fp4_linear(xq, xs, w_i[0], w_i[1], "nvfp4", x_ts=xt, w_ts=wt, out=y)

        y.zero_()
        ms = time_graph(gemm, calls, torch)
        graph_ok = bool(torch.equal(y, ref))
        ms_warm = time_graph(lambda i: B.fp4_linear(xq, xs, wq, ws, "nvfp4", x_ts=xt, w_ts=wt, out=y), 50, torch)
        nbytes = wbytes + wl.M * wl.K * (0.5 + 1.0 / 16) + wl.M * wl.N * 4 + 8
        out[f"gemm_{name}"] = {
            "workload": f"{name}: M={wl.M} K={wl.K} N={wl.N} NVFP4 block {wl.block}, Y fp32",
            "us": ms * 1e3, "GB/s": nbytes / (ms * 1e-3) / 1e9, "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes": nbytes, "w_copies": n_sets, "graph_replay_matches_eager": graph_ok,
            "warm_us": ms_warm * 1e3,
            "traffic": measured_traffic(*DECODE_TRAFFIC_KEY[name]),
            "note": f"{calls} calls in one HIP graph over {n_sets} copies of W ({n_sets * wbytes / 1e6:.0f} MB), "
                    "so W comes from HBM; warm_us: one W, resident in the Infinity Cache"}
        log(f"[bench] {name} NVFP4 GEMM {ms * 1e3:.2f} us with W from HBM = {nbytes / (ms * 1e-3) / 1e9:.0f} GB/s; "
            f"W in cache {ms_warm * 1e3:.2f} us; graph matches eager: {graph_ok}")
        del sets, wq, ws
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--ramp-ms", type=float, default=250.0,
                    help="untimed steps run for this long before the warm-up steps (clock ramp)")
    ap.add_argument("--workload", default="prefill_mx")
    ap.add_argument("--stress", default="stress_mx32", help="rotate+quantize HBM workload ('' to skip)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the NVFP4 and decode-shaped measurements reported beside the headline")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--rows", default=",".join(EXTRA_ROWS),
                    help="comma-separated groups of other rows to run (default: all of %s)" % ",".join(EXTRA_ROWS))
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    from microscaling_fp4_quantized_amd import workloads as WL

    # CPU baseline of rotate+quantize first: its process pool forks before anything touches the GPU
    rq_cpu = None
    if not args.no_cpu and not args.copy_probe:
        log("[bench] CPU oracle rotate+quantize baseline ...")
        rq_cpu = cpu_rotate_quantize(WL.WORKLOADS[args.stress or "stress_mx32"])
        log(f"[bench] CPU oracle rotate+quantize: {rq_cpu['GB/s']:.3f} GB/s on {rq_cpu['cores']} processes")

    import numpy as np
    import torch

    from microscaling_fp4_quantized_amd import binding as B

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B.load_library()

    if args.copy_probe:
        n = args.copy_probe << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n}), flush=True)
        return

    wl = WL.WORKLOADS[args.workload]
    log(f"[bench] workload {wl.name}: M={wl.M} K={wl.K} N={wl.N} {wl.fmt} block {wl.block}")
    x_bits, w_bits = WL.draw_x(wl), WL.draw_w(wl)
    x = bf16_dev(x_bits, dev)
    w = bf16_dev(w_bits, dev)
    wq, ws, wts = B.fp4_quantize_weights(w, wl.block, wl.fmt)  # offline
    del w
    out_dtype = torch.bfloat16 if wl.out_dtype == "bf16" else torch.float32
    g = B.group_size(wl.fmt)
    xq = torch.empty((wl.M, wl.K // 2), dtype=torch.uint8, device=dev)
    xs = torch.empty((wl.M, wl.K // g), dtype=torch.uint8, device=dev)
    xts = torch.empty((1,), dtype=torch.float32, device=dev) if wl.fmt == "nvfp4" else None
    y = torch.empty((wl.M, wl.N), dtype=out_dtype, device=dev)

    ev = {k: [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)] for k in ("a", "b", "c")}

    def step(i=None):
        if i is not None:
            ev["a"][i].record()
        B.fp4_rotate_quantize(x, wl.block, wl.fmt, out=(xq, xs, xts))
        if i is not None:
            ev["b"][i].record()
        B.fp4_linear(xq, xs, wq, ws, wl.fmt, x_ts=xts, w_ts=wts, out_dtype=out_dtype, out=y)
        if i is not None:
            ev["c"][i].record()

    # The GPU raises its clocks only under sustained load: right after setup, back-to-back steps
    # run 15-20% slower than after ~100 ms of them. A serving loop runs in that steady state, so
    # untimed steps run first for --ramp-ms; the roofline's cold figure is measured separately.
    t_ramp = time.perf_counter()
    ramp_steps = 0
    while (time.perf_counter() - t_ramp) * 1e3 < args.ramp_ms:
        for _ in range(20):
            step()
        ramp_steps += 20
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    # per-kernel breakdown from a separate pass: events inside the timed loop would add gaps to it
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    step_codes, step_scales = xq.cpu().numpy(), xs.cpu().numpy()
    rq_ms = sum(a.elapsed_time(b) for a, b in zip(ev["a"], ev["b"])) / args.steps
    gemm_ms = sum(b.elapsed_time(c) for b, c in zip(ev["b"], ev["c"])) / args.steps
    flops = 2.0 * wl.M * wl.N * wl.K
    step_tflops = flops / (ms_step * 1e-3) / 1e12
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    peak = MFMA_FP4_PEAK_TFLOPS if wl.fmt == "mxfp4" else MFMA_BF16_PEAK_TFLOPS
    gemm_src, gemm_kernel = gemm_kernel_for(wl.fmt, wl.M, wl.N, wl.K)
    rq_bytes = wl.M * wl.K * (2 + 0.5 + 1.0 / g) + (8 if wl.fmt == "nvfp4" else 0)
    if wl.fmt == "nvfp4":
        rq_bytes += wl.M * wl.K * 2  # the tensor-maximum pass reads X a second time
    y_bytes = wl.M * wl.N * (2 if out_dtype == torch.bfloat16 else 4)
    gemm_alg_bytes = (wl.M + wl.N) * wl.K * (0.5 + 1.0 / g) + y_bytes
    log(f"[bench] step {ms_step * 1e3:.1f} us (events: rotate+quantize {rq_ms * 1e3:.1f} us, "
        f"GEMM {gemm_ms * 1e3:.1f} us = {gemm_tflops:.0f} TFLOP/s)")

    # Roofline of the GEMM: the kernel's average duration over back-to-back launches.
    def gemm_only(i):
        B.fp4_linear(xq, xs, wq, ws, wl.fmt, x_ts=xts, w_ts=wts, out_dtype=out_dtype, out=y)

    roof_ms = time_batch(gemm_only, max(args.steps, 20), torch)
    roof_tflops = flops / (roof_ms * 1e-3) / 1e12
    log(f"[bench] GEMM back-to-back {roof_ms * 1e3:.1f} us = {roof_tflops:.0f} TFLOP/s ({roof_tflops / peak:.1%} of peak)")
    # the same, back to back, with W read from HBM: calls cycle over copies of W totalling more than
    # 512 MB (a model's layers do not share one W that stays in the 256 MB Infinity Cache)
    w_bytes = wq.numel() + ws.numel()
    n_w = -(-512 * 10 ** 6 // w_bytes)
    w_sets = [(wq.clone(), ws.clone(), None if wts is None else wts.clone()) for _ in range(n_w)]

    def gemm_w_hbm(i):
        q, sc, t = w_sets[i % n_w]
        B.fp4_linear(xq, xs, q, sc, wl.fmt, x_ts=xts, w_ts=t, out_dtype=out_dtype, out=y)

    for i in range(n_w):
        gemm_w_hbm(i)
    hbm_ms = time_batch(gemm_w_hbm, 2 * n_w, torch)
    hbm_tflops = flops / (hbm_ms * 1e-3) / 1e12
    del w_sets
    log(f"[bench] GEMM back-to-back, W from HBM ({n_w} copies): {hbm_ms * 1e3:.1f} us = {hbm_tflops:.0f} TFLOP/s "
        f"({hbm_tflops / peak:.1%} of peak)")
    cold = time_cold(gemm_only, 30, torch, dev)
    log(f"[bench] GEMM cold (1 GiB read between launches): median {cold['median_us']:.1f} us "
        f"(p10 {cold['p10_us']:.1f}, p90 {cold['p90_us']:.1f})")

    result = {
        "metric": METRIC,
        "value": step_tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ramp": {"ms": args.ramp_ms, "steps": ramp_steps,
                 "note": "untimed steps before the warm-up, so that the timed steps run at steady-state clocks"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.fmt,
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: prefill linear layer, X {wl.M}x{wl.K} bf16 (Student-t(5), 1% outlier "
                        f"channels x30) -> block-{wl.block} Hadamard + {wl.fmt.upper()} -> W4A4 GEMM "
                        f"vs W {wl.N}x{wl.K} (pre-rotated, quantized offline), Y {wl.out_dtype}",
            "M": wl.M, "K": wl.K, "N": wl.N, "block": wl.block, "format": wl.fmt,
            "out_dtype": wl.out_dtype, "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": gemm_kernel,
            "bound": "mfma",
            "achieved": roof_tflops,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": roof_tflops / peak,
            "traffic": measured_traffic(f"{gemm_kernel}@{wl.name}", gemm_src),
            "algorithmic_flops": flops,
            "algorithmic_bytes": gemm_alg_bytes,
            "avg_launch_us": roof_ms * 1e3,
            "w_from_hbm": {"avg_launch_us": hbm_ms * 1e3, "achieved": hbm_tflops, "frac": hbm_tflops / peak,
                           "w_copies": n_w,
                           "note": "back-to-back launches cycling over copies of W totalling more than 512 MB, "
                                   "so every launch reads its W from HBM"},
            "cold": {**cold, "TFLOP/s_median": flops / (cold["median_us"] * 1e-6) / 1e12,
                     "note": "each launch timed alone after reading a 1 GiB buffer, so W and X come from HBM "
                             "instead of the 256 MB Infinity Cache"},
        },
        "components": {
            "rotate_quantize_step_input": {
                "us": rq_ms * 1e3,
                "GB/s": rq_bytes / (rq_ms * 1e-3) / 1e9,
                "note": "X of the step (16 MiB) stays resident in the 256 MB Infinity Cache between steps",
            },
            "gemm": {"us": gemm_ms * 1e3, "TFLOP/s": gemm_tflops},
        },
    }

    if args.stress:
        sw = WL.WORKLOADS[args.stress]
        log(f"[bench] rotate+quantize stress {sw.name}: {sw.M}x{sw.K} {sw.fmt} block {sw.block}")
        sx = WL.draw_x(sw)
        # three input buffers in rotation, and a 1 GiB read after uploading them, so that no launch
        # finds its X in the 256 MB Infinity Cache (streaming loads may leave lines that were
        # resident before the first launch in place)
        bufs = [bf16_dev(sx, dev) for _ in range(3)]
        stress_rows = np.unique(np.random.default_rng(17).choice(sw.M, 64, replace=False))
        stress_x_rows = sx[stress_rows].copy()
        del sx
        flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        torch.sum(flush, dim=(0,))
        del flush
        sg = B.group_size(sw.fmt)
        outs = (torch.empty((sw.M, sw.K // 2), dtype=torch.uint8, device=dev),
                torch.empty((sw.M, sw.K // sg), dtype=torch.uint8, device=dev),
                torch.empty((1,), dtype=torch.float32, device=dev) if sw.fmt == "nvfp4" else None)

        def rq(i):
            B.fp4_rotate_quantize(bufs[i % 3], sw.block, sw.fmt, out=outs)

        ramp(rq, torch)
        s_ms = time_batch(rq, 42, torch)
        s_cold = time_cold(rq, 20, torch, dev)
        s_bytes = sw.M * sw.K * (2 + 0.5 + 1.0 / sg)
        if sw.fmt == "nvfp4":
            s_bytes += sw.M * sw.K * 2
        gbs = s_bytes / (s_ms * 1e-3) / 1e9
        log(f"[bench] stress rotate+quantize {s_ms * 1e3:.1f} us = {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of HBM)")
        cold_gbs = s_bytes / (s_cold["median_us"] * 1e-6) / 1e9
        log(f"[bench] stress rotate+quantize cold (1 GiB read before each launch): median {s_cold['median_us']:.1f} us "
            f"= {cold_gbs:.0f} GB/s ({cold_gbs / HBM_PEAK_GBS:.1%} of HBM)")
        result["roofline_rotate_quantize"] = {
            "kernel": "rotate_quant_mx" if sw.fmt == "mxfp4" else "rotate_amax + rotate_quant_nv",
            "workload": f"{sw.name}: X {sw.M}x{sw.K} bf16 Student-t(3) x log-normal channel scales, "
                        f"block {sw.block}, {sw.fmt.upper()}",
            "bound": "hbm",
            "achieved": gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS,
            "traffic": measured_traffic(f"rotate_quant_mx@{sw.name}", "rotate_quant.hip")
            if sw.fmt == "mxfp4" else None,
            "algorithmic_bytes": s_bytes,
            "avg_launch_us": s_ms * 1e3,
            "cold": {**s_cold, "GB/s_median": cold_gbs, "frac_median": cold_gbs / HBM_PEAK_GBS,
                     "note": "each launch timed alone after reading a 1 GiB buffer (no Infinity Cache residency)"},
        }
        stress_out = (sw, stress_rows, stress_x_rows, outs[0].cpu().numpy()[stress_rows],
                      outs[1].cpu().numpy()[stress_rows])
        del bufs, outs

    if not args.no_extra:
        result["other_rows"] = extra_rows(B, WL, torch, dev, [r for r in args.rows.split(",") if r])

    if not args.no_cpu:
        log("[bench] CPU oracle baseline ...")
        from oracle import fp4_oracle as O

        parity = {}
        if wl.fmt == "mxfp4":
            rows = np.unique(np.random.default_rng(19).choice(wl.M, min(wl.M, 64), replace=False))
            parity[wl.name] = quant_parity_counts(O, x_bits, wl.block, wl.fmt, step_codes, step_scales, rows)
        if args.stress and stress_out[0].fmt == "mxfp4":
            sw, srows, sxr, scodes, sscales = stress_out
            parity[sw.name] = quant_parity_counts(O, sxr, sw.block, sw.fmt, scodes, sscales, np.arange(len(srows)))
            parity[sw.name]["rows"] = "64 rows drawn with seed 17"
        log(f"[bench] parity counts on sampled rows: {parity}")
        result["cpu_baseline"] = cpu_baseline(wl, x_bits, w_bits, rq_cpu, parity)
        log(f"[bench] CPU oracle: {result['cpu_baseline']['seconds']:.2f} s per step")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
