"""Benchmark of the preshuffle GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME|all]
                    [--configs metric|none] [--act none|relu|silu|gelu]

A step is one GEMM call (A, preshuffled B and scales already resident in
HBM) on the workload's synthetic inputs. The default workload is the FP8
small-batch GEMM M=16, N=7168, K=2048, whose metric is HBM GB/s; the
compute-bound workloads report TFLOP/s. To keep B from being served by the
256 MB last-level cache, each step uses the next of R device-resident copies
of the inputs, with R large enough that the copies together exceed 640 MB,
and one untimed pass over all R copies runs right before the timed region,
so that every timed step finds its inputs last touched R steps earlier.

By default the one JSON line also carries, under `configs`, the same
figures for each of the five workloads of the headline metric (INT8
128x256x512, FP8 16x7168x2048, FP8 512x4096x4096, BF16 8192^3, MXFP4
4096x4096x8192), each timed the same way; --configs none leaves them out.
With --workload all, one line per workload is printed instead.

The line carries the throughput, the roofline of the GEMM
kernel (measured with HIP events on the launch stream over the timed
region; for MFMA-bound shapes also the fraction of the dense peak at the
shader clock sampled from sysfs while the same launches repeat), the B preshuffle pass timed separately (a one-time weight
preparation that the pages keep outside the per-call path), and the CPU
oracle timed on a bounded sample on this host. With --act the GEMM runs with
the fused epilogue (an fp32 bias per column plus the activation) through
gemm_ex; the bytes then include the bias (4 N).
"""
from __future__ import annotations

import argparse
import glob
import json
import math
import os
import re
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402
from oracle import formulas as F  # noqa: E402

METRIC = "GEMM TFLOPS and % of dtype MFMA peak (large M); HBM GB/s and % at M=16"
DEFAULT_WORKLOAD = "fp8_16x7168x2048"
# MI355X published dense peaks (TFLOP/s or TOP/s) and HBM bandwidth (GB/s)
PEAK_TFLOPS = {"int8": 5000.0, "fp8": 5000.0, "bf16": 2500.0, "fp16": 2500.0, "mxfp4": 10100.0,
               "w4a8": 5000.0}   # W4A8 runs on the int8 matrix instructions
PEAK_HBM_GBPS = 8000.0
DTYPE_NAME = {"int8": "i8", "fp8": "f8e4m3", "bf16": "bf16", "fp16": "f16", "mxfp4": "mxfp4_e2m1",
              "w4a8": "i8xi4"}
ROTATE_BYTES = 640 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def workload_numbers(name, act=None):
    dtype, M, N, K, seed, tile = workloads.CONFIGS[name]
    out_bytes = 4 if dtype == "int8" else 2
    flops = F.flops(M, N, K)
    nbytes = F.bytes_moved(dtype, M, N, K, out_bytes=out_bytes) + (4 * N if act else 0)
    ridge = PEAK_TFLOPS[dtype] * 1e12 / (PEAK_HBM_GBPS * 1e9)
    bound = "hbm" if flops / nbytes < ridge else "mfma"
    return dtype, M, N, K, seed, flops, nbytes, bound


def _time_oracle(dtype, host, sel, act, budget_s):
    """Repeat the oracle on rows `sel` for about budget_s seconds; (calls, seconds)."""
    import oracle

    calls, t0 = 0, time.perf_counter()
    while True:
        oracle.gemm(dtype, host, rows=sel, act=act)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s or (calls >= 1 and el * (calls + 1) / calls > 2 * budget_s):
            return calls, el


def cpu_baseline(name, host, budget_s=12.0, act=None, single_thread_s=0.0):
    """Time the oracle (as it is) on a bounded sample of the workload, with
    the BLAS threads it runs with by default (`cores`) and, when
    single_thread_s > 0, also on one thread."""
    dtype, M, N, K, seed, flops, nbytes, bound = workload_numbers(name, act)
    try:
        from threadpoolctl import threadpool_info, threadpool_limits

        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threadpool_limits = None
        cores = os.cpu_count() or 1
    # sample: a block of rows (all columns) sized to about one second per call
    per_row = 2.0 * N * K
    rows = int(min(M, max(16, 2e10 / per_row)))
    sel = np.arange(rows)
    frac = rows / M

    def rate(calls, el):
        per_call_s = el / calls
        return (nbytes * frac / per_call_s / 1e9) if bound == "hbm" else (flops * frac / per_call_s / 1e12)

    calls, el = _time_oracle(dtype, host, sel, act, budget_s)
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):  # pragma: no cover
        affinity = None
    out = {"value": rate(calls, el), "unit": "GB/s" if bound == "hbm" else "TFLOP/s", "cores": int(cores),
           "kind": "oracle",
           "sample": f"{rows} of {M} rows x all {N} columns, K={K}, {calls} call(s) in {el:.1f} s "
                     f"(decode + float64 matmul)",
           "host_cpu": _cpu_model(), "nproc": os.cpu_count(), "affinity_cpus": affinity,
           "seconds_full_problem": el / calls / frac}
    if single_thread_s > 0 and threadpool_limits is not None:
        with threadpool_limits(limits=1):
            c1, e1 = _time_oracle(dtype, host, sel, act, single_thread_s)
        out["single_thread"] = {"value": rate(c1, e1), "seconds_full_problem": e1 / c1 / frac,
                                "sample": f"{rows} rows, {c1} call(s) in {e1:.1f} s"}
    return out


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def bench_one(name, steps, warmup, do_cpu=True, opts=None, use_graph=True, calib_mib=0, act=None, data="randn",
              telemetry_s=0.4, cpu_budget_s=12.0, cpu_single_s=0.0):
    import torch

    import dense_gemm_preshuffle_amd as gp
    from dense_gemm_preshuffle_amd import workload

    dtype, M, N, K, seed, flops, nbytes, bound = workload_numbers(name, act)
    # every GEMM goes through gemm_ex_ws with a workspace allocated (and
    # zeroed) once here, so the planner may split K across workgroups; one
    # workspace serves every launch, since they are ordered on one stream
    plan = gp.gemm_plan_ws(dtype, M, N, K, opts)
    log(f"[bench] {name}: plan {plan}" + (f", fused epilogue bias + {act}" if act else ""))
    host = workloads.make_inputs(dtype, M, N, K, seed, bias=act is not None)
    dev = workload.to_device(dtype, host)
    if data == "zeros":
        # diagnostic only: the same launches on all-zero operands (no bit
        # toggles in the matrix cores) to expose data-dependent clock throttling
        for k in ("a", "b"):
            dev[k].zero_()
    stream = torch.cuda.current_stream()

    # preshuffle pass, timed on its own
    p0 = workload.prepare(dtype, dev)
    p0["workspace"] = gp.workspace(dtype, M, N, K, opts)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record(stream)
    for _ in range(reps):
        gp.gemm_preshuffle_b(dev["b"], dtype, out=p0["b_shuf"])
    e1.record(stream)
    torch.cuda.synchronize()
    pre_us = e0.elapsed_time(e1) * 1e3 / reps
    b_bytes = dev["b"].numel() * dev["b"].element_size()

    # rotation copies so that every step reads its operands from HBM
    set_bytes = nbytes
    R = max(2, min(64, math.ceil(ROTATE_BYTES / set_bytes)))
    sets = [p0]
    for _ in range(R - 1):
        q = {k: (v.clone() if torch.is_tensor(v) and k != "workspace" else v) for k, v in p0.items()}
        sets.append(q)
    outs = [workload.run(dtype, s, opts=opts, act=act) for s in sets]
    torch.cuda.synchronize()
    log(f"[bench] {name}: {R} rotating input sets, {set_bytes / 2**20:.1f} MiB each")

    for i in range(warmup):
        workload.run(dtype, sets[i % R], opts=opts, c=outs[i % R], act=act)
    torch.cuda.synchronize()

    # eager launches (host launch cost included)
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(steps):
        workload.run(dtype, sets[i % R], opts=opts, c=outs[i % R], act=act)
    t_end.record(stream)
    torch.cuda.synchronize()
    eager_ms = t_start.elapsed_time(t_end) / steps

    # context only: the same launches on one input set, whose operands the
    # 256 MB last-level cache then holds across launches (never `value`);
    # timed before the measured region so that a profiler trace still ends
    # with the measured launches
    warm_s = None
    if use_graph and R > 1:
        warm_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(warm_graph):
            for i in range(steps):
                workload.run(dtype, sets[0], opts=opts, c=outs[0], act=act)
        warm_graph.replay()
        torch.cuda.synchronize()
        t_start.record(stream)
        warm_graph.replay()
        t_end.record(stream)
        torch.cuda.synchronize()
        warm_s = t_start.elapsed_time(t_end) / steps / 1e3
        del warm_graph

    # timed region: the same K launches captured once in a HIP graph and
    # replayed, so the GPU sees back-to-back GEMMs without host launch gaps.
    # Launch i uses input set i % R. Right before it, one launch on each of
    # the R sets in the same order (the pre-roll, untimed): every timed launch
    # then finds its inputs last touched exactly R launches (R * set bytes,
    # over 640 MB) earlier, whatever K is, so none of them is served by the
    # 256 MB last-level cache.
    graph = roll = None
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(steps):
                workload.run(dtype, sets[i % R], opts=opts, c=outs[i % R], act=act)
        roll = torch.cuda.CUDAGraph()
        with torch.cuda.graph(roll):
            for i in range(R):
                workload.run(dtype, sets[i], opts=opts, c=outs[i], act=act)
        graph.replay()
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    if roll is not None:
        roll.replay()
    else:
        for i in range(R):
            workload.run(dtype, sets[i], opts=opts, c=outs[i], act=act)
    t_start.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(steps):
            workload.run(dtype, sets[i % R], opts=opts, c=outs[i % R], act=act)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_per_step = t_start.elapsed_time(t_end) / steps
    sec = ms_per_step / 1e3

    tflops = flops / sec / 1e12
    gbps = nbytes / sec / 1e9
    if bound == "hbm":
        value, unit = gbps, "GB/s"
        roof = {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": gbps / PEAK_HBM_GBPS, "traffic": None}
    else:
        value, unit = tflops, "TFLOP/s"
        pk = PEAK_TFLOPS[dtype]
        roof = {"bound": "mfma", "achieved": tflops, "peak": pk, "unit": "TFLOP/s",
                "frac": tflops / pk, "traffic": None}
    line = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": DTYPE_NAME[dtype],
        "data": "synthetic" if data == "randn" else "synthetic, operands zeroed (power diagnostic, not a result)",
        "config": {"workload": name, "M": M, "N": N, "K": K, "kernel": plan["kernel"],
                   "tile": [plan["tile_m"], plan["tile_n"], plan["tile_k"]], "grid": plan["grid"],
                   "epilogue": plan["epilogue"], "fused_epilogue": f"bias+{act}" if act else None,
                   "entry_point": "gemm_ex_ws", "ksplit": plan["ksplit"], "scheduler": plan["scheduler"],
                   "workspace_bytes": plan["workspace_bytes"],
                   "rotating_sets": R, "sets_touched_in_timed_region": min(steps, R),
                   "reuse_distance_mib": round(R * set_bytes / 2**20, 1)},
        "roofline": roof,
        "tflops": tflops, "gbps": gbps, "us_per_gemm": sec * 1e6,
        "preshuffle_b": {"us": pre_us, "GB/s": 2 * b_bytes / (pre_us * 1e-6) / 1e9,
                         "note": "one-time B layout pass, not in the timed step"},
        "timing": "hip graph of the K steps, HIP events on the launch stream" if use_graph
                  else "eager launches, HIP events on the launch stream",
        "eager_us_per_gemm": eager_ms * 1e3,
        "host_wall_s": wall,
    }
    tr = _traffic(name + (f"+{act}" if act else ""), plan)
    if tr is not None:
        roof["traffic"] = tr
        roof["traffic_source"] = ("rocprofv3 FETCH_SIZE + WRITE_SIZE per launch, scaled by a plain copy of known "
                                  "size: bytes between the L2 caches and the memory fabric, an upper bound on "
                                  "HBM bytes (the 256 MB last-level cache may serve part of them)")
    if warm_s is not None:
        line["warm"] = {"us_per_gemm": warm_s * 1e6,
                        "value": (nbytes / warm_s / 1e9) if bound == "hbm" else (flops / warm_s / 1e12),
                        "unit": unit,
                        "note": "one input set for every launch (operands resident in the last-level "
                                "cache), timed before the measured region: context, not the value"}
    if telemetry_s > 0:
        def replay():
            if graph is not None:
                graph.replay()
            else:
                for i in range(steps):
                    workload.run(dtype, sets[i % R], opts=opts, c=outs[i % R], act=act)
        tel = telemetry(replay, telemetry_s)
        line["telemetry"] = tel
        if tel and bound == "mfma":
            # the dense peak scales with the shader clock (2.4 GHz nominal)
            roof["clock_normalised_frac"] = roof["achieved"] / (roof["peak"] * tel["sclk_mhz"] / 2400.0)
    if calib_mib:
        # a plain device-to-device copy of known size, for scaling the HBM
        # byte counters of a profiler run (read calib_mib MiB, write calib_mib MiB)
        src = torch.ones(calib_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
    if do_cpu and data == "randn":
        line["cpu_baseline"] = cpu_baseline(name, host, budget_s=cpu_budget_s, act=act,
                                            single_thread_s=cpu_single_s)
    del sets, outs, graph, roll
    torch.cuda.empty_cache()
    return line


# The five workloads the headline metric is quoted on: INT8 128x256x512 (bit
# exact, launch-bound), FP8 16x7168x2048 (HBM-bound), FP8 512x4096x4096, BF16
# 8192^3 and MXFP4 4096x4096x8192 (MFMA-bound). The one line the bench prints
# carries the default workload's figures at its top level and these five in
# `configs`.
METRIC_CONFIGS = ["int8_128x256x512", "fp8_16x7168x2048", "fp8_512x4096x4096", "bf16_8192x8192x8192",
                  "mxfp4_4096x4096x8192"]
# a 1-thread oracle time is reported for the first three (the small ones)
SINGLE_THREAD_CONFIGS = {"int8_128x256x512", "fp8_16x7168x2048", "fp8_512x4096x4096"}


def config_summary(line):
    """The per-config figures that go into the one JSON line's `configs`."""
    r = line["roofline"]
    out = {"us_per_gemm": line["us_per_gemm"], "value": line["value"], "unit": line["unit"],
           "frac_of_peak": r["frac"], "peak": r["peak"], "bound": r["bound"], "dtype": line["dtype"],
           "tflops": line["tflops"], "gbps": line["gbps"],
           "kernel": line["config"]["kernel"], "tile": line["config"]["tile"], "grid": line["config"]["grid"],
           "rotating_sets": line["config"]["rotating_sets"]}
    for k in ("clock_normalised_frac", "traffic"):
        if r.get(k) is not None:
            out[k] = r[k]
    if "telemetry" in line and line["telemetry"]:
        out["sclk_mhz"] = line["telemetry"]["sclk_mhz"]
        out["power_w"] = line["telemetry"]["power_w"]
    if "warm" in line:
        out["warm_us_per_gemm"] = line["warm"]["us_per_gemm"]
    if "cpu_baseline" in line:
        out["cpu_baseline"] = line["cpu_baseline"]
    return out


def floor_probe(name, steps, warmup, grids=((224, 4), (256, 4), (256, 8), (512, 4), (1024, 4))):
    """The HBM streaming-read floor for the workload's algorithmic bytes: the
    probe kernel (dense_gemm_preshuffle_amd/probe/stream_read.hip) reads that
    many bytes (rounded up to whole 16-byte lanes of its grid) once per
    launch, timed like the GEMM (HIP graph of the K launches over rotating
    buffers, one untimed pass over all of them right before, HIP events)."""
    import ctypes

    import torch

    from dense_gemm_preshuffle_amd import build as _b

    if not os.path.exists(_b.PROBE_LIB):
        raise SystemExit(f"{_b.PROBE_LIB} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(_b.PROBE_LIB)
    lib.gp_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_void_p]
    lib.gp_probe_stream_read.restype = ctypes.c_int
    dtype, M, N, K, seed, flops, nbytes, bound = workload_numbers(name)
    stream = torch.cuda.current_stream()
    out = []
    for wgs, waves in grids:
        unit = 16 * 64 * waves * wgs
        b = -(-nbytes // unit) * unit
        R = max(2, min(64, math.ceil(ROTATE_BYTES / b)))
        bufs = [torch.ones(b, dtype=torch.uint8, device="cuda") for _ in range(R)]
        sink = torch.empty(wgs * waves * 64, dtype=torch.int32, device="cuda")

        def launch(i):
            # the stream current at the call (inside a graph capture, the capturing stream)
            sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            st = lib.gp_probe_stream_read(ctypes.c_void_p(bufs[i % R].data_ptr()), b, wgs, waves,
                                          ctypes.c_void_p(sink.data_ptr()), sp)
            if st != 0:
                raise RuntimeError(f"gp_probe_stream_read: status {st}")

        for i in range(warmup):
            launch(i)
        graph, roll = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(steps):
                launch(i)
        with torch.cuda.graph(roll):
            for i in range(R):
                launch(i)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        roll.replay()
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        out.append({"workgroups": wgs, "waves": waves, "bytes": b, "us_per_read": us, "GB/s": b / (us * 1e-6) / 1e9,
                    "us_for_workload_bytes": us * nbytes / b})
        log(f"[floor] {wgs} x {waves} waves: {us:.3f} us for {b} bytes ({b / (us * 1e-6) / 1e9:.0f} GB/s)")
        del graph, roll, bufs
    torch.cuda.empty_cache()
    return {"workload": name, "algorithmic_bytes": nbytes, "steps": steps, "reads": out,
            "method": "one non-temporal 16-byte-load pass per launch over a fresh buffer (rotating, "
                      f"{ROTATE_BYTES >> 20} MiB and more), HIP graph of the launches, HIP events"}


# (form, instruction, dtype of its dense peak, M x N x K of one instruction)
MFMA_FORMS = [(0, "bf16 16x16x32", "bf16", 16, 16, 32), (1, "f16 16x16x32", "fp16", 16, 16, 32),
              (2, "i8 16x16x64", "int8", 16, 16, 64), (3, "fp8 16x16x128", "fp8", 16, 16, 128),
              (4, "fp4 16x16x128 (scaled)", "mxfp4", 16, 16, 128), (5, "bf16 32x32x16", "bf16", 32, 32, 16),
              (6, "f16 32x32x16", "fp16", 32, 32, 16), (7, "i8 32x32x32", "int8", 32, 32, 32),
              (8, "fp8 32x32x64", "fp8", 32, 32, 64), (9, "fp4 32x32x64 (scaled)", "mxfp4", 32, 32, 64)]


def mfma_rate(iters=4000, grids=(256, 512)):
    """What each MFMA form of the kernels sustains on its own
    (dense_gemm_preshuffle_amd/probe/mfma_rate.hip): 8 independent
    accumulators per wave, operands in registers, `iters` rounds of 8 MFMAs;
    256 workgroups of 4 waves (one wave per SIMD) or 512 (two). Cycles per
    MFMA per wave from the shader clock counter around the loop; FLOP/s from
    HIP events around the launch (launch included)."""
    import ctypes
    import statistics

    import torch

    from dense_gemm_preshuffle_amd import build as _b

    if not os.path.exists(_b.PROBE_LIB):
        raise SystemExit(f"{_b.PROBE_LIB} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(_b.PROBE_LIB)
    f = lib.gp_probe_mfma_rate
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int
    stream = torch.cuda.current_stream()
    rows = []
    for wgs in grids:
        out = torch.zeros(wgs * 256, device="cuda")
        cyc = torch.zeros(wgs * 8, dtype=torch.int64, device="cuda")
        for form, name, dt, m, n, k in MFMA_FORMS:
            flop = 2 * m * n * k
            peak = PEAK_TFLOPS[dt] * 1e12
            nominal = flop / (peak / (1024 * 2.4e9))   # issue cycles at the dense peak
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            for timed in (False, True):
                if timed:
                    e0.record(stream)
                st = f(form, out.data_ptr(), cyc.data_ptr(), iters, wgs, ctypes.c_void_p(stream.cuda_stream))
                if st != 0:
                    raise RuntimeError(f"gp_probe_mfma_rate: status {st}")
                if timed:
                    e1.record(stream)
                torch.cuda.synchronize()
            c = cyc.view(-1, 2).cpu()
            cycles = statistics.median(c[:, 0].tolist())
            ticks = statistics.median(c[:, 1].tolist())
            per = cycles / (iters * 8)
            total = wgs * 4 * iters * 8 * flop
            tf = total / (e0.elapsed_time(e1) * 1e-3) / 1e12
            row = {"workgroups": wgs, "waves_per_simd": wgs // 256, "form": name,
                   "cycles_per_mfma_per_wave": round(per, 2), "nominal_issue_cycles": round(nominal, 1),
                   # one wave per SIMD: the share of the loop's cycles the MFMA pipe is issuing; with
                   # more workgroups than CUs they need not all overlap, so only the FLOP rate is kept
                   "issue_fraction": round(nominal / per, 3) if wgs == 256 else None,
                   "clock_ghz": round(cycles / (ticks / 100e6) / 1e9, 3),
                   "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_TFLOPS[dt], 3)}
            rows.append(row)
            log(f"[mfma] {wgs} wgs {name}: {per:.2f} cycles per MFMA per wave (issue {nominal:.0f}), "
                f"{tf:.0f} TFLOP/s = {tf / PEAK_TFLOPS[dt]:.3f} of peak")
        del out, cyc
    return {"iters": iters, "rows": rows,
            "method": "8 independent accumulators per wave, operands in registers, shader-clock cycles around "
                      "the loop, HIP events around the launch"}


def _gpu_sysfs():
    """sysfs device directory of the GPU when the host has exactly one, else None."""
    cards = [d for d in sorted(glob.glob("/sys/class/drm/card*/device")) if os.path.exists(os.path.join(d, "pp_dpm_sclk"))]
    return cards[0] if len(cards) == 1 else None


def _sclk_mhz(dev):
    """Current shader clock: the pp_dpm_sclk line marked '*'."""
    for line in open(os.path.join(dev, "pp_dpm_sclk")):
        if line.rstrip().endswith("*"):
            return float(re.search(r"(\d+)\s*[Mm][Hh]z", line).group(1))
    return None


def _power_w(dev, name="power1_input"):
    files = glob.glob(os.path.join(dev, "hwmon", "hwmon*", name))
    return int(open(files[0]).read()) / 1e6 if files else None


def telemetry(replay, min_s=0.4):
    """Shader clock and socket power while the timed launches run back to back.

    `replay` runs the timed region once; it is repeated for at least min_s
    seconds (after the timed measurement, so the measurement itself is not
    disturbed) while a host thread reads sysfs every 2 ms. The first fifth
    of the samples (clock ramp) is dropped; medians are reported. None when
    the host exposes no single GPU in sysfs.
    """
    import torch

    dev = _gpu_sysfs()
    if dev is None:
        return None
    samples, stop = [], threading.Event()

    def sample():
        while not stop.is_set():
            try:
                samples.append((_sclk_mhz(dev), _power_w(dev)))
            except (OSError, ValueError, AttributeError):
                pass
            time.sleep(0.002)

    th = threading.Thread(target=sample, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_s:
        replay()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    samples = samples[len(samples) // 5:]
    clk = sorted(c for c, _ in samples if c)
    pw = sorted(w for _, w in samples if w)
    if not clk:
        return None
    try:
        cap = _power_w(dev, "power1_cap")
    except (OSError, ValueError):
        cap = None
    return {"sclk_mhz": clk[len(clk) // 2], "sclk_min_mhz": clk[0], "sclk_max_mhz": clk[-1],
            "power_w": pw[len(pw) // 2] if pw else None, "power_cap_w": cap, "samples": len(samples),
            "source": "sysfs pp_dpm_sclk and hwmon power1_input, sampled while the timed launches repeat"}


def _traffic(name, plan):
    """HBM bytes per launch measured with rocprofv3 counters for this exact
    kernel source (profiles/traffic.json), or None when stale or absent."""
    import dense_gemm_preshuffle_amd as gp

    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(name)
    except ValueError:
        return None
    if not rec or rec.get("source_hash") != gp.source_hash():
        return None
    if rec.get("tile") != [plan["tile_m"], plan["tile_n"], plan["tile_k"]] or rec.get("kernel") != plan["kernel"] \
            or rec.get("ksplit", 1) != plan.get("ksplit", 1):
        return None
    return rec.get("traffic_bytes")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 1000 steps: a timed region of milliseconds even for the microsecond
    # kernels (with 200, the FP8 512x4096x4096 GEMM measured 3% slower: the
    # region was too short for the clocks to settle)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="one of %s, or 'all' (one line per workload)" % ", ".join(sorted(workloads.CONFIGS)))
    ap.add_argument("--configs", default="metric", choices=["metric", "none"],
                    help="metric (default): also time the five workloads of the headline metric and put "
                         "their figures in the line's `configs`; none: the --workload line alone")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a HIP graph")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="after timing, run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--opts", default=None, help="JSON gemm_opts override, e.g. '{\"tile_m\":64,...}'")
    ap.add_argument("--floor", action="store_true",
                    help="instead of the GEMM: time the HBM streaming-read probe over the workload's "
                         "algorithmic bytes (the floor of the memory-bound shapes), one JSON line")
    ap.add_argument("--mfma-rate", action="store_true",
                    help="instead of the GEMM: time each MFMA form the kernels use on its own (registers only), "
                         "one JSON line")
    ap.add_argument("--data", default="randn", choices=["randn", "zeros"],
                    help="zeros: same launches on all-zero A and B (diagnostic of data-dependent clocks)")
    ap.add_argument("--act", default=None, choices=["none", "relu", "silu", "gelu"],
                    help="run with the fused epilogue: a per-column bias, then this activation")
    ap.add_argument("--telemetry-s", type=float, default=0.4, metavar="S",
                    help="after timing, repeat the timed launches for S seconds while sampling the "
                         "shader clock and power (0: skip; profiler runs use 0 so that the trace "
                         "ends with the timed region)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the GEMM here runs on a single MI355X and has no "
              "multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.mfma_rate:
        print(json.dumps({"mfma_rate": mfma_rate()}), flush=True)
        return
    if args.floor:
        print(json.dumps({"floor": floor_probe(args.workload, args.steps, args.warmup)}), flush=True)
        return
    names = sorted(workloads.CONFIGS) if args.workload == "all" else [args.workload]
    opts = json.loads(args.opts) if args.opts else None
    kw = dict(opts=opts, use_graph=not args.eager, act=args.act, data=args.data, telemetry_s=args.telemetry_s)
    for name in names:
        line = bench_one(name, args.steps, args.warmup, do_cpu=not args.no_cpu_baseline,
                         calib_mib=args.calib_copy, cpu_single_s=3.0 if name in SINGLE_THREAD_CONFIGS else 0.0,
                         **kw)
        if args.workload != "all" and args.configs == "metric" and opts is None and args.act is None:
            cfgs = {}
            for other in METRIC_CONFIGS:
                if other == name:
                    cfgs[other] = config_summary(line)
                    continue
                log(f"[bench] metric config {other}")
                o = bench_one(other, args.steps, args.warmup, do_cpu=not args.no_cpu_baseline, cpu_budget_s=8.0,
                              cpu_single_s=3.0 if other in SINGLE_THREAD_CONFIGS else 0.0, **kw)
                cfgs[other] = config_summary(o)
            line["configs"] = cfgs
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
