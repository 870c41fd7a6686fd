#!/usr/bin/env python3
"""Throughput of the MX block-scaled NT GEMM on one MI355X.

One step = one mx_gemm call (C = A * B^T, MX block-scaled) over a synthetic,
already-quantized workload resident in HBM; quantization is outside the
timed region, as in the measurements the FlyDSL article reports (section
"Performance numbers need their baselines").  The default workload is the
largest one: the MXFP4 Llama-3.3-70B MLP down projection at M=2048
(N=8192, K=28672, BF16 out, 962 GFLOP per call).

Prints one JSON line: whole-job TFLOP/s over exactly --steps timed steps
(cycling through operand copies, so no step finds its data in the
last-level cache), the kernel's roofline position from the cold median of
60 launches each timed alone (HIP events on the launch stream) against the
MI355X dense MX MFMA peak and against the measured MFMA ceiling of the same
device, and the CPU oracle's rate on a bounded row sample of the workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--all]
    python bench.py --ceiling         (the HBM read ceiling, the MFMA ceiling of both formats)
    python bench.py --quantize | --grouped | --mixed | --bf16
        (the quantizer / grouped GEMM / mixed-format GEMM / dense BF16 GEMM)
"""
import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import mxinputs  # noqa: E402

DEFAULT_WORKLOAD = "mxfp4_llama70b_down_m2048"
METRIC = "MX GEMM TFLOPS and % of MI355X dense MXFP4/MXFP8 MFMA peak per shape"
# MI355X published dense peaks: MXFP4 10.1 PFLOP/s, MXFP8 5.0 PFLOP/s; HBM3E 8 TB/s.
PEAK_TFLOPS = {mxinputs.FMT_E2M1: 10100.0, mxinputs.FMT_E4M3: 5000.0}
PEAK_HBM_GBS = 8000.0
# Ridge points (FLOP per byte) above which the MFMA, not HBM, bounds a shape.
RIDGE = {f: PEAK_TFLOPS[f] * 1e12 / (PEAK_HBM_GBS * 1e9) for f in PEAK_TFLOPS}
CSRC = os.path.join(ROOT, "microscaled_block_scaled_amd", "csrc")
# The device code of each kernel family: a counter summary taken on other
# device code is stale.
GEMM_SOURCES = [os.path.join(CSRC, "mx_kernels.h")]
DECODE_SOURCES = GEMM_SOURCES + [os.path.join(CSRC, "mx_decode.h")]
QUANT_SOURCES = [os.path.join(CSRC, "mx_quant.h")]
QUANT6_SOURCES = [os.path.join(CSRC, "mx_quant.h"), os.path.join(CSRC, "mx_quant6.h")]


def algorithmic_bytes(fmt, M, N, K, out):
    """Compulsory HBM traffic: A, B and their scales read once, C written once."""
    eb = K // 2 if fmt == mxinputs.FMT_E2M1 else K
    return (M + N) * eb + (M + N) * (K // 32) + M * N * (4 if out == mxinputs.OUT_FP32 else 2)


def kernel_source_hash(sources=None):
    h = hashlib.sha256()
    for p in (GEMM_SOURCES if sources is None else sources):
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def gemm_sources(plan):
    """The device code a GEMM plan runs: the tile kernel, or the decode kernel
    (which also uses the tile kernel's helpers)."""
    import microscaled_block_scaled_amd as mxg
    return DECODE_SOURCES if plan["variant"] == mxg.VARIANT_DECODE else GEMM_SOURCES


def measured_traffic(workload, sources=None, plan=None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current device code (and, for the GEMM, the same launch
    plan); else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.txt" % workload)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash(sources):
        return None
    if plan is not None and kv.get("plan") != plan:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def host_cores():
    """(cores this process may run on, cores the host reports)."""
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return usable, os.cpu_count() or usable


def cpu_baseline(case, target_s=10.0, single_s=6.0):
    """The CPU oracle on a row sample of the same workload (all N columns):
    about target_s seconds on up to 16 threads, then about single_s seconds
    on one thread."""
    import numpy as np
    import oracle
    threads = cpu_threads()
    M, N, K, fmt = case["M"], case["N"], case["K"], case["fmt"]

    def run(rows, nthreads):
        t0 = time.perf_counter()
        oracle.gemm(fmt, case["A"], case["A_scale"], case["B"], case["B_scale"], K,
                    rows=rows, threads=nthreads)
        return time.perf_counter() - t0

    def sample(nthreads, budget):
        r0 = min(M, max(1, nthreads // 4))
        t0 = run(np.arange(r0), nthreads)
        nrows = int(max(r0, min(M, r0 * budget / max(t0, 1e-6))))
        rows = np.linspace(0, M - 1, nrows).astype(np.int64)
        return nrows, run(rows, nthreads)

    nrows, t = sample(threads, target_s)
    n1, t1 = sample(1, single_s)
    usable, reported = host_cores()
    flop_row = 2.0 * N * K
    return {"value": round(nrows * flop_row / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d of %d rows of A (all %d columns, K=%d), %.1f s on %d threads; "
                      "single thread: %d rows in %.1f s" % (nrows, M, N, K, t, threads, n1, t1),
            "single_thread_value": round(n1 * flop_row / t1 / 1e12, 6),
            "host_cores_usable": usable, "host_cores_reported": reported}


def mfma_ceiling(fmt, target_s=0.05, reps=3):
    """The block-scaled MFMA's sustained rate on this device with no memory
    traffic (mx_mfma_ceiling, the tile kernel's launch shape), on random and
    on constant operands: TFLOP/s, median of `reps` launches of about
    target_s seconds each, after one warm-up launch."""
    import torch
    import microscaled_block_scaled_amd as mxg
    dev = torch.device("cuda", 0)
    out = torch.empty(mxg.CEILING_WORKGROUPS * mxg.CEILING_THREADS, dtype=torch.float32,
                      device=dev)
    stream = torch.cuda.current_stream(dev)
    nominal = PEAK_TFLOPS[fmt] * 1e12
    steps = int(target_s * nominal / mxg.ceiling_flops(1)) // 2 * 2
    res = {}
    for random_data in (1, 0):
        ts = []
        for i in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = mxg.ceiling_ptr(fmt, steps, random_data, out.data_ptr(), stream.cuda_stream)
            if rc != 0:
                raise RuntimeError("mx_mfma_ceiling failed: %s" % mxg.strerror(rc))
            e1.record(stream)
            e1.synchronize()
            if i:
                ts.append(e0.elapsed_time(e1) / 1e3)
        ts.sort()
        res["random" if random_data else "constant"] = round(
            mxg.ceiling_flops(steps) / ts[len(ts) // 2] / 1e12, 1)
    return res


_HBM_CEILING = []


def hbm_ceiling(nbytes=1 << 30, reps=5):
    """The rate at which this device streams HBM into the CUs
    (mx_hbm_read_ceiling, a plain read of every byte): GB/s, median of
    `reps` launches over one of two 1 GiB buffers, alternated so that the
    buffer read is never in the 256 MB last-level cache.  Each launch is
    timed alone, with the stream kept busy by an untimed launch on the other
    buffer while its event pair is enqueued.  Measured once per process."""
    if _HBM_CEILING:
        return _HBM_CEILING[0]
    import torch
    import microscaled_block_scaled_amd as mxg
    dev = torch.device("cuda", 0)
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(2)]
    out = torch.empty(mxg.HBM_CEILING_WORKGROUPS * mxg.HBM_CEILING_THREADS, dtype=torch.int32,
                      device=dev)
    stream = torch.cuda.current_stream(dev)

    def launch(buf):
        rc = mxg.hbm_ceiling_ptr(buf.data_ptr(), nbytes, out.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError("mx_hbm_read_ceiling failed: %s" % mxg.strerror(rc))

    ts = []
    for i in range(reps + 1):
        launch(bufs[(i + 1) % 2])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        launch(bufs[i % 2])
        e1.record(stream)
        e1.synchronize()
        if i:
            ts.append(e0.elapsed_time(e1) / 1e3)
    del bufs
    ts.sort()
    _HBM_CEILING.append(round(nbytes / ts[len(ts) // 2] / 1e9, 1))
    return _HBM_CEILING[0]


def hbm_fields(roof):
    """For an HBM-bound line: the measured read ceiling and the fraction of it
    reached."""
    if roof["bound"] == "hbm":
        hbm = hbm_ceiling()
        roof["hbm_read_ceiling_gbs"] = hbm
        roof["frac_of_measured_hbm"] = round(roof["achieved"] / hbm, 4)
    return roof


def _percentiles(ts):
    ts = sorted(ts)
    q = lambda f: ts[min(len(ts) - 1, int(f * len(ts)))]
    return {"median_us": round(q(0.5), 2), "p10_us": round(q(0.1), 2), "p90_us": round(q(0.9), 2)}


def bench_one(name, steps, warmup, with_cpu, cold_launches=60, with_ceiling=True):
    """One workload.  The timed region is `steps` back-to-back mx_gemm calls
    cycling through enough copies of the operands and output that no call
    finds its data in the 256 MB last-level cache (each copy was last
    touched at least 768 MB of traffic earlier).  Then, for the roofline,
    `cold_launches` calls each timed alone between its own event pair after
    a 512 MiB read that evicts the caches (median, p10, p90), and the same
    with no eviction (warm)."""
    import torch
    import microscaled_block_scaled_amd as mxg

    case = mxinputs.make_case(name)
    fmt, M, N, K, out = case["fmt"], case["M"], case["N"], case["K"], case["out"]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    tdt = torch.float32 if out == mxinputs.OUT_FP32 else torch.bfloat16
    nbytes = algorithmic_bytes(fmt, M, N, K, out)
    ncopies = max(2, min(64, -(-(768 << 20) // nbytes)))
    host = [torch.from_numpy(case[k]) for k in ("A", "A_scale", "B", "B_scale")]
    sets = []
    for _ in range(ncopies):
        A, As, B, Bs = (h.to(dev) for h in host)
        C = torch.empty((M, N), dtype=tdt, device=dev)
        sets.append((A, As, B, Bs, C))
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    argsets = [(fmt, M, N, K, A.data_ptr(), As.data_ptr(), B.data_ptr(), Bs.data_ptr(),
                C.data_ptr(), out, sh) for (A, As, B, Bs, C) in sets]

    def call(i):
        rc = mxg.gemm_ptr(*argsets[i % ncopies])
        if rc != 0:
            raise RuntimeError("mx_gemm failed: %s" % mxg.strerror(rc))

    for i in range(warmup):
        call(i)
    # The timed region: an event pair on the launch stream around the same
    # launches gives their average duration too.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        call(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    rotating_us = e0.elapsed_time(e1) / steps * 1e3

    flush = torch.ones(512 << 20, dtype=torch.uint8, device=dev).view(torch.float32)

    def per_launch(evict):
        # The stream is kept busy (the evicting read, or an untimed call on
        # the same operands) while the event pair and the timed call are
        # enqueued, so the host's launch latency stays outside the pair.
        ts = []
        for i in range(5 + cold_launches):
            if evict:
                flush.amax()
            else:
                call(0)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            call(0)
            b.record(stream)
            b.synchronize()
            if i >= 5:
                ts.append(a.elapsed_time(b) * 1e3)
        return _percentiles(ts)

    cold, warm = per_launch(True), per_launch(False)
    del flush
    ceiling = mfma_ceiling(fmt) if with_ceiling else None

    flops = 2.0 * M * N * K
    tflops = flops * steps / wall / 1e12
    bound = "mfma" if flops / nbytes >= RIDGE[fmt] else "hbm"
    plan = mxg.plan(fmt, M, N, K, out)
    plan_str = "variant %d tile %dx%d split %d, %d workgroups" % (
        plan["variant"], plan["tile_m"], plan["tile_n"], plan["split_k"], plan["workgroups"])
    traffic = measured_traffic(name, gemm_sources(plan), plan_str)
    launch_s = cold["median_us"] * 1e-6
    if bound == "mfma":
        achieved = flops / launch_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS[fmt],
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS[fmt], 4)}
    else:
        achieved = nbytes / launch_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["traffic"] = traffic
    roof["algorithmic_bytes"] = nbytes
    roof["launch_us"] = cold["median_us"]
    roof["timing"] = "cold median of %d launches, each alone after a 512 MiB cache-evicting read" \
        % cold_launches
    roof["cold"] = cold
    roof["warm"] = warm
    roof["rotating_avg_us"] = round(rotating_us, 2)
    roof["mfma_ceiling_tflops"] = ceiling
    roof["tflops"] = round(flops / launch_s / 1e12, 2)
    roof["frac_of_measured_ceiling"] = (round(flops / launch_s / 1e12 / ceiling["random"], 4)
                                        if ceiling else None)
    if with_ceiling:
        hbm_fields(roof)
    res = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(wall / steps * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp8_e4m3" if fmt == mxinputs.FMT_E4M3 else "mxfp4_e2m1",
        "data": "synthetic",
        "config": {"workload": name, "M": M, "N": N, "K": K,
                   "format": mxinputs.fmt_name(fmt),
                   "out": "fp32" if out == mxinputs.OUT_FP32 else "bf16",
                   "accumulate": "fp32", "peak_frac": round(tflops / PEAK_TFLOPS[fmt], 4),
                   "plan": plan_str, "operand_copies": ncopies,
                   "kernel_source_sha256": kernel_source_hash(gemm_sources(plan))},
        "roofline": roof,
    }
    if with_cpu:
        res["cpu_baseline"] = cpu_baseline(case)
    return res


def bench_quantize(steps, warmup, fmt, in_dtype):
    """MX quantization of the fused-QKV operands (A and B stacked: 8192 x
    4096 values) from FP32 or BF16: HBM-bound, reported against 8 TB/s."""
    import torch
    import microscaled_block_scaled_amd as mxg
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    rows, K = 8192, 4096
    g = torch.Generator(device="cpu").manual_seed(1234)
    x = torch.randn((rows, K), generator=g, dtype=torch.float32)
    tdt = torch.float32 if in_dtype == mxg.IN_FP32 else torch.bfloat16
    x = x.to(tdt).to(dev)
    q = torch.empty((rows, mxinputs.row_bytes(fmt, K)), dtype=torch.uint8, device=dev)
    srcs = QUANT6_SOURCES if fmt in (mxinputs.FMT_E2M3, mxinputs.FMT_E3M2) else QUANT_SOURCES
    qs = torch.empty((rows, K // 32), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    args = (fmt, in_dtype, rows, K, x.data_ptr(), q.data_ptr(), qs.data_ptr(), stream.cuda_stream)
    for _ in range(warmup):
        if mxg.quantize_ptr(*args) != 0:
            raise RuntimeError("mx_quantize failed")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        mxg.quantize_ptr(*args)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_s = e0.elapsed_time(e1) / steps / 1e3
    nbytes = rows * K * x.element_size() + q.numel() + qs.numel()
    achieved = nbytes / launch_s / 1e9
    return {"metric": "MX quantize GB/s (HBM bytes read + written)",
            "value": round(nbytes * steps / wall / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
            "steps": steps, "warmup": warmup, "ms_per_step": round(wall / steps * 1e3, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f32" if in_dtype == mxg.IN_FP32 else "bf16", "data": "synthetic",
            "config": {"workload": "quantize_%s_from_%s_8192x4096" % (
                mxinputs.fmt_name(fmt), "f32" if in_dtype == mxg.IN_FP32 else "bf16"),
                "rows": rows, "K": K, "kernel_source_sha256": kernel_source_hash(srcs)},
            "roofline": hbm_fields({
                "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic("quantize_%s_from_%s_8192x4096" % (
                    mxinputs.fmt_name(fmt), "f32" if in_dtype == mxg.IN_FP32 else "bf16"), srcs),
                "algorithmic_bytes": nbytes,
                "launch_us": round(launch_s * 1e6, 2)})}


# Eight experts of a mixture-of-experts layer: token counts of one 4096-token
# batch (uneven load), each expert's weight N x K.
GROUPED_ROWS = [704, 320, 512, 896, 128, 640, 448, 448]
GROUPED_N, GROUPED_K = 4096, 2048


def bench_grouped(steps, warmup, fmt):
    """mx_gemm_grouped (fmt an MX format) or mx_gemm_grouped_bf16 (fmt
    "bf16") over eight uneven experts (4096 tokens in all, N=4096, K=2048,
    BF16 out): TFLOP/s of the useful products, roofline by the same ridge
    rule as the plain GEMM."""
    import numpy as np
    import torch
    import microscaled_block_scaled_amd as mxg
    rows, N, K = GROUPED_ROWS, GROUPED_N, GROUPED_K
    G, M, out = len(rows), sum(rows), mxinputs.OUT_BF16
    dense = fmt == "bf16"
    # (fa, fb): E4M3 activations with E2M1 expert weights
    fa, fb = fmt if isinstance(fmt, tuple) else (fmt, fmt)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    if dense:
        A = torch.from_numpy(mxinputs.make_bf16(M, K, seed=2030).view(np.int16)).to(dev)
        B = torch.from_numpy(mxinputs.make_bf16(G * N, K, seed=2030, tensor=1).view(np.int16)).to(dev)
        args = (rows, N, K, A.data_ptr(), B.data_ptr(), C.data_ptr(), out, stream.cuda_stream)
        run = mxg.grouped_bf16_ptr
        peak = PEAK_BF16_TFLOPS
    else:
        ca = mxinputs.make_random(fa, M, 1, K, seed=2024 + fa)
        cb = mxinputs.make_random(fb, 1, G * N, K, seed=2024 + fb)
        A, As = torch.from_numpy(ca["A"]).to(dev), torch.from_numpy(ca["A_scale"]).to(dev)
        B, Bs = torch.from_numpy(cb["B"]).to(dev), torch.from_numpy(cb["B_scale"]).to(dev)
        args = (fa, rows, N, K, A.data_ptr(), As.data_ptr(), B.data_ptr(), Bs.data_ptr(),
                C.data_ptr(), out, stream.cuda_stream, fb)
        run = mxg.grouped_ptr
        # an 8-bit operand runs the MFMA at the 8-bit rate
        peak = PEAK_TFLOPS[mxinputs.FMT_E4M3 if mxinputs.FMT_E4M3 in (fa, fb) else fa]
    for _ in range(warmup):
        if run(*args) != 0:
            raise RuntimeError("grouped GEMM failed")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        run(*args)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_s = e0.elapsed_time(e1) / steps / 1e3
    flops = 2.0 * M * N * K
    if dense:
        nbytes = (M + G * N) * K * 2 + M * N * 2
        p = mxg.grouped_bf16_plan(rows, N, K, out)
    else:
        nbytes = (M * mxinputs.row_bytes(fa, K) + G * N * mxinputs.row_bytes(fb, K)
                  + (M + G * N) * (K // 32) + M * N * 2)
        p = mxg.grouped_plan(fa, rows, N, K, out)
    plan_str = "grouped tile %dx%d, %d workgroups" % (p["tile_m"], p["tile_n"], p["workgroups"])
    fname = "bf16" if dense else (mxinputs.fmt_name(fa) if fa == fb else "w4a8")
    workload = "grouped_%s_experts8_4096x4096x2048" % fname
    bound = "mfma" if flops / nbytes >= peak * 1e12 / (PEAK_HBM_GBS * 1e9) else "hbm"
    if bound == "mfma":
        achieved = flops / launch_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
    else:
        achieved = nbytes / launch_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["traffic"] = measured_traffic(workload, GEMM_SOURCES, plan_str)
    hbm_fields(roof)
    roof["algorithmic_bytes"] = nbytes
    roof["launch_us"] = round(launch_s * 1e6, 2)
    tflops = flops * steps / wall / 1e12
    return {"metric": "Grouped GEMM TFLOPS and % of MI355X dense MFMA peak of the format",
            "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": steps, "warmup": warmup, "ms_per_step": round(wall / steps * 1e3, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16" if dense else
                     ("mxfp8_e4m3 x mxfp4_e2m1" if fa != fb else
                      "mxfp8_e4m3" if fa == mxinputs.FMT_E4M3 else "mxfp4_e2m1"),
            "data": "synthetic",
            "config": {"workload": workload, "group_rows": rows, "N": N, "K": K,
                       "format": fname, "out": "bf16",
                       "peak_frac": round(tflops / peak, 4), "plan": plan_str,
                       "kernel_source_sha256": kernel_source_hash(gemm_sources(p))},
            "roofline": roof}


# Other element formats, BF16 out: mixed "W4A8" (A E4M3 activations, B E2M1
# weights) on the fused-QKV shape and the 70B down and gate-up projections
# at batch 8;
# E5M2 for both operands, E4M3 x E5M2, and the two FP6 formats on the
# fused-QKV shape.
MIXED_WORKLOADS = {
    "w4a8_llama8b_qkv": (2048, 6144, 4096, mxinputs.FMT_E4M3, mxinputs.FMT_E2M1),
    "w4a8_llama70b_down_m8": (8, 8192, 28672, mxinputs.FMT_E4M3, mxinputs.FMT_E2M1),
    # the gate and up projections of the same layer (N = 2 x 28672, K = 8192):
    # 1792 column groups of the decode kernel, 7 per workgroup
    "w4a8_llama70b_gateup_m8": (8, 57344, 8192, mxinputs.FMT_E4M3, mxinputs.FMT_E2M1),
    "mxfp8_e5m2_llama8b_qkv": (2048, 6144, 4096, mxinputs.FMT_E5M2, mxinputs.FMT_E5M2),
    "mxfp8_e4m3_x_e5m2_llama8b_qkv": (2048, 6144, 4096, mxinputs.FMT_E4M3, mxinputs.FMT_E5M2),
    "mxfp6_e2m3_llama8b_qkv": (2048, 6144, 4096, mxinputs.FMT_E2M3, mxinputs.FMT_E2M3),
    "mxfp6_e3m2_llama8b_qkv": (2048, 6144, 4096, mxinputs.FMT_E3M2, mxinputs.FMT_E3M2),
}


def bench_mixed(steps, warmup, name):
    """A GEMM in another format pair (mx_gemm_mixed, or one format through
    mx_gemm).  The MFMA peak taken is the MXFP8 one when an operand has 8-bit
    elements (the instruction then runs at the 8-bit rate), else the
    MXFP4/MXFP6 one."""
    import torch
    import microscaled_block_scaled_amd as mxg
    M, N, K, fa, fb = MIXED_WORKLOADS[name]
    out = mxinputs.OUT_BF16
    ca = mxinputs.make_random(fa, M, 1, K, seed=3000)
    cb = mxinputs.make_random(fb, 1, N, K, seed=3001)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    A, As = torch.from_numpy(ca["A"]).to(dev), torch.from_numpy(ca["A_scale"]).to(dev)
    B, Bs = torch.from_numpy(cb["B"]).to(dev), torch.from_numpy(cb["B_scale"]).to(dev)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    args = (fa, M, N, K, A.data_ptr(), As.data_ptr(), B.data_ptr(), Bs.data_ptr(),
            C.data_ptr(), out, stream.cuda_stream, None, 0, fb)
    for _ in range(warmup):
        if mxg.gemm_ptr(*args) != 0:
            raise RuntimeError("mx_gemm_mixed failed")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        mxg.gemm_ptr(*args)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_s = e0.elapsed_time(e1) / steps / 1e3
    flops = 2.0 * M * N * K
    nbytes = (M * mxinputs.row_bytes(fa, K) + N * mxinputs.row_bytes(fb, K)
              + (M + N) * (K // 32) + M * N * 2)
    eight_bit = {mxinputs.FMT_E4M3, mxinputs.FMT_E5M2} & {fa, fb}
    peak = PEAK_TFLOPS[mxinputs.FMT_E4M3 if eight_bit else mxinputs.FMT_E2M1]
    p = mxg.plan(fa, M, N, K, out)
    plan_str = "variant %d tile %dx%d split %d, %d workgroups" % (
        p["variant"], p["tile_m"], p["tile_n"], p["split_k"], p["workgroups"])
    if flops / nbytes >= peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        achieved = flops / launch_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
    else:
        achieved = nbytes / launch_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["traffic"] = measured_traffic(name, gemm_sources(p), plan_str)
    hbm_fields(roof)
    roof["algorithmic_bytes"] = nbytes
    roof["launch_us"] = round(launch_s * 1e6, 2)
    tflops = flops * steps / wall / 1e12
    return {"metric": "MX GEMM TFLOPS (other formats) and % of MI355X dense MX MFMA peak",
            "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": steps, "warmup": warmup, "ms_per_step": round(wall / steps * 1e3, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "%s x %s" % (mxinputs.fmt_name(fa), mxinputs.fmt_name(fb)),
            "data": "synthetic",
            "config": {"workload": name, "M": M, "N": N, "K": K,
                       "format_a": mxinputs.fmt_name(fa), "format_b": mxinputs.fmt_name(fb),
                       "out": "bf16",
                       "peak_frac": round(tflops / peak, 4), "plan": plan_str,
                       "kernel_source_sha256": kernel_source_hash(gemm_sources(p))},
            "roofline": roof}


def copy_calibration(nbytes=256 << 20, reps=3):
    """A plain device copy of known size, for scaling the HBM byte counters
    (FETCH_SIZE, WRITE_SIZE) that rocprofv3 reports for the GEMM kernels."""
    import torch
    dev = torch.device("cuda", 0)
    src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


# Dense BF16 GEMM workloads (mx_gemm_bf16): name -> (M, N, K), BF16 out.
BF16_WORKLOADS = {
    "bf16_llama8b_qkv": (2048, 6144, 4096),
    "bf16_llama70b_down_m2048": (2048, 8192, 28672),
    "bf16_llama70b_down_m8": (8, 8192, 28672),
}
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense BF16 MFMA


def bench_bf16(steps, warmup, name, with_cpu):
    """The dense BF16 NT GEMM on the same tile kernels, from seeded Gaussian
    BF16 operands resident in HBM."""
    import numpy as np
    import torch
    import microscaled_block_scaled_amd as mxg
    M, N, K = BF16_WORKLOADS[name]
    out = mxinputs.OUT_BF16
    ha = mxinputs.make_bf16(M, K, seed=4000, tensor=0)
    hb = mxinputs.make_bf16(N, K, seed=4000, tensor=1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    A = torch.from_numpy(ha.view(np.int16)).to(dev)
    B = torch.from_numpy(hb.view(np.int16)).to(dev)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    args = (M, N, K, A.data_ptr(), B.data_ptr(), C.data_ptr(), out, stream.cuda_stream)
    for _ in range(warmup):
        if mxg.gemm_bf16_ptr(*args) != 0:
            raise RuntimeError("mx_gemm_bf16 failed")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        mxg.gemm_bf16_ptr(*args)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_s = e0.elapsed_time(e1) / steps / 1e3
    flops = 2.0 * M * N * K
    nbytes = (M + N) * K * 2 + M * N * 2
    peak = PEAK_BF16_TFLOPS
    p = mxg.plan_bf16(M, N, K, out)
    plan_str = "variant %d tile %dx%d split %d, %d workgroups" % (
        p["variant"], p["tile_m"], p["tile_n"], p["split_k"], p["workgroups"])
    if flops / nbytes >= peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        achieved = flops / launch_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
    else:
        achieved = nbytes / launch_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["traffic"] = measured_traffic(name, GEMM_SOURCES, plan_str)
    hbm_fields(roof)
    roof["algorithmic_bytes"] = nbytes
    roof["launch_us"] = round(launch_s * 1e6, 2)
    tflops = flops * steps / wall / 1e12
    res = {"metric": "Dense BF16 GEMM TFLOPS and % of MI355X dense BF16 MFMA peak",
           "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": steps, "warmup": warmup, "ms_per_step": round(wall / steps * 1e3, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": name, "M": M, "N": N, "K": K, "format": "bf16",
                      "out": "bf16", "accumulate": "fp32",
                      "peak_frac": round(tflops / peak, 4), "plan": plan_str,
                      "kernel_source_sha256": kernel_source_hash(GEMM_SOURCES)},
           "roofline": roof}
    if with_cpu:
        import oracle
        threads = cpu_threads()
        r0 = min(M, 2)
        t0 = time.perf_counter()
        oracle.gemm_bf16(ha, hb, rows=np.arange(r0), threads=threads)
        t_probe = time.perf_counter() - t0
        nrows = int(max(r0, min(M, r0 * 12.0 / max(t_probe, 1e-6))))
        rows = np.linspace(0, M - 1, nrows).astype(np.int64)
        t0 = time.perf_counter()
        oracle.gemm_bf16(ha, hb, rows=rows, threads=threads)
        t = time.perf_counter() - t0
        res["cpu_baseline"] = {
            "value": round(2.0 * nrows * N * K / t / 1e12, 6), "unit": "TFLOP/s",
            "cores": threads, "kind": "oracle",
            "sample": "%d of %d rows of A (all %d columns, K=%d), %.1f s on %d threads"
                      % (nrows, M, N, K, t, threads)}
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(mxinputs.CONFIGS))
    ap.add_argument("--all", action="store_true",
                    help="one line per workload (no CPU baseline except the default one)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-launches", type=int, default=60,
                    help="launches timed alone for the cold / warm medians (at least 3)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the ceiling measurements (frac_of_measured_ceiling and "
                         "frac_of_measured_hbm null)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 256 MiB device copy (counter calibration)")
    ap.add_argument("--quantize", action="store_true",
                    help="time mx_quantize (both formats, FP32 and BF16 input) instead")
    ap.add_argument("--grouped", action="store_true",
                    help="time the grouped GEMM (eight uneven experts; MXFP8, MXFP4, BF16) instead")
    ap.add_argument("--mixed", action="store_true",
                    help="time the other formats (A E4M3 x B E2M1; E5M2) instead")
    ap.add_argument("--bf16", action="store_true",
                    help="time the dense BF16 GEMM (mx_gemm_bf16) instead")
    ap.add_argument("--ceiling", action="store_true",
                    help="only measure the device's ceilings: HBM streaming read "
                         "(mx_hbm_read_ceiling) and the MFMA rate of both formats "
                         "(mx_mfma_ceiling)")
    a = ap.parse_args()
    if a.gpus != 1:
        sys.stderr.write("bench.py runs on exactly one GPU: the MX GEMM path has no "
                         "multi-GPU component (each GPU would run its own shard "
                         "independently); use --gpus 1.\n")
        sys.exit(2)
    if a.copy_calibration:
        copy_calibration()
        return
    if a.ceiling:
        import microscaled_block_scaled_amd as mxg
        print(json.dumps({"hbm_read_ceiling": "1 GiB buffers", "unit": "GB/s",
                          "value": hbm_ceiling(), "datasheet_peak": PEAK_HBM_GBS,
                          "launch": "%d workgroups x %d threads" % (
                              mxg.HBM_CEILING_WORKGROUPS, mxg.HBM_CEILING_THREADS)}), flush=True)
        for fmt in (mxinputs.FMT_E2M1, mxinputs.FMT_E4M3):
            c = mfma_ceiling(fmt)
            print(json.dumps({"mfma_ceiling": mxinputs.fmt_name(fmt), "unit": "TFLOP/s",
                              "random": c["random"], "constant": c["constant"],
                              "datasheet_peak": PEAK_TFLOPS[fmt],
                              "launch": "%d workgroups x %d threads" % (
                                  mxg.CEILING_WORKGROUPS, mxg.CEILING_THREADS)}), flush=True)
        return
    if a.quantize:
        for fmt in (mxinputs.FMT_E4M3, mxinputs.FMT_E2M1, mxinputs.FMT_E5M2, mxinputs.FMT_E2M3,
                    mxinputs.FMT_E3M2):
            for ind in (1, 2):
                print(json.dumps(bench_quantize(a.steps, a.warmup, fmt, ind)), flush=True)
        return
    if a.mixed:
        for name in MIXED_WORKLOADS:
            print(json.dumps(bench_mixed(a.steps, a.warmup, name)), flush=True)
        return
    if a.bf16:
        for i, name in enumerate(BF16_WORKLOADS):
            with_cpu = (not a.no_cpu_baseline) and i == 0
            print(json.dumps(bench_bf16(a.steps, a.warmup, name, with_cpu)), flush=True)
        return
    if a.grouped:
        for fmt in (mxinputs.FMT_E4M3, mxinputs.FMT_E2M1, (mxinputs.FMT_E4M3, mxinputs.FMT_E2M1),
                    "bf16"):
            print(json.dumps(bench_grouped(a.steps, a.warmup, fmt)), flush=True)
        return
    names = sorted(mxinputs.CONFIGS, key=lambda n: (mxinputs.CONFIGS[n]["index"], n)) \
        if a.all else [a.workload]
    for name in names:
        with_cpu = (not a.no_cpu_baseline) and name == a.workload
        print(json.dumps(bench_one(name, a.steps, a.warmup, with_cpu,
                                   max(3, a.cold_launches), not a.no_ceiling)), flush=True)


if __name__ == "__main__":
    main()
