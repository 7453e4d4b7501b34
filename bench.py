#!/usr/bin/env python3
"""Benchmark of the fp16 TN GEMM on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload lds_4096] [--algo auto]

One step = one D = A B^T GEMM (the whole path: one kernel launch) over the
synthetic 4096^3 workload (A (M,K), B (N,K) fp16 K-contiguous, uniform
[-1,1), C absent, fp32 output), inputs resident in HBM before timing starts.
Prints one JSON line: TFLOP/s over the timed steps (2MNK per step), the
per-launch kernel time from HIP events on the launch stream, the roofline
entry of the GEMM kernel (MFMA bound, dense fp16 peak of the chip), the
shader clock the chip holds under sustained load with the peak scaled to it,
and the float64 CPU oracle timed on a bounded row sample of the same workload.

``--workload chain_b32_2048x2048_k128_n128`` measures the back-to-back GEMM
(D = rne16(A B^T) W^T per batch, one kernel launch per step) the same way,
counting 2 batch M N1 (K + N2) FLOP per step.

``--workload mfma_rate_32x32x16`` / ``mfma_rate_16x16x32`` (``--data
random|zero``) and ``lds_read_b128`` (``--threads``) measure the rates the
GEMM is priced against: the matrix instructions' issue rate with no memory
traffic, and conflict-free LDS reads, each with the shader clock read inside
the kernel.
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

PEAK_FP16_DENSE_TFLOPS = 2516.6   # 256 CU x 4 SIMD x 1024 FLOP/clk x 2.4 GHz
METRIC = "TFLOP/s for fp16 TN GEMM at 4096³ (fp32 acc) and % of dense FP16 MFMA peak"
KERNEL_SOURCES = ["mma_fragment_layouts_tn_amd/csrc/gemm_kernels.hpp",
                  "mma_fragment_layouts_tn_amd/csrc/gemm_tile.hpp",
                  "mma_fragment_layouts_tn_amd/csrc/gemm_launch.hpp"]
CHAIN_SOURCES = ["mma_fragment_layouts_tn_amd/csrc/chain.hpp",
                 "mma_fragment_layouts_tn_amd/csrc/gemm_tile.hpp"]
METRIC_CHAIN = ("TFLOP/s for the back-to-back fp16 GEMM D = rne16(A B^T) W^T "
                "(2 b M N1 (K + N2) FLOP, fp32 acc) and % of dense FP16 MFMA peak")


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, algo: str, sources=None):
    """HBM bytes per launch measured with rocprofv3 counters (committed under
    profiles/), or None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_{algo}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash(sources):
        return None
    return rec.get("bytes_per_launch")


def sustained_clock(step, sync, seconds: float):
    """(shader clock MHz, memory clock MHz, package power W) read with
    rocm-smi, in child processes, while the step runs back to back for
    `seconds`; None for what rocm-smi does not report."""
    import re
    import subprocess
    import threading
    found = {}

    def sample():
        time.sleep(seconds / 2)
        try:
            out = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True,
                                 timeout=20).stdout
        except (OSError, subprocess.SubprocessError):
            return
        m = re.search(r"sclk clock level: \d+: \((\d+)Mhz\)", out)
        if m:
            found["sclk"] = int(m.group(1))
        m = re.search(r"mclk clock level: \d+: \((\d+)Mhz\)", out)
        if m:
            found["mclk"] = int(m.group(1))
        try:
            out = subprocess.run(["rocm-smi", "--showpower"], capture_output=True, text=True,
                                 timeout=20).stdout
        except (OSError, subprocess.SubprocessError):
            return
        m = re.search(r"Power \(W\):\s*([0-9.]+)", out)
        if m:
            found["power"] = float(m.group(1))

    th = threading.Thread(target=sample)
    t0 = time.perf_counter()
    th.start()
    while time.perf_counter() - t0 < seconds or th.is_alive():
        for _ in range(50):
            step()
        sync()
    th.join()
    return found.get("sclk"), found.get("mclk"), found.get("power")


def cpu_baseline(w, x, target_s: float):
    """The float64 oracle, as it stands, on rows [0, r) of the workload: the
    whole GEMM when a calibration run says it fits in target_s, else the
    number of rows that does."""
    from oracle import gemm as G
    cores = G.max_threads()
    rows = min(w.M, 64)
    t0 = time.perf_counter()
    G.gemm_f64(w.M, w.N, w.K, x.A, w.lda_, w.a_order == "m", x.B, w.ldb_, x.C, rows=(0, rows))
    t_cal = time.perf_counter() - t0
    rows = max(rows, min(w.M, int(rows * target_s / max(t_cal, 1e-3))))
    t0 = time.perf_counter()
    G.gemm_f64(w.M, w.N, w.K, x.A, w.lda_, w.a_order == "m", x.B, w.ldb_, x.C, rows=(0, rows))
    t = time.perf_counter() - t0
    flops = 2.0 * rows * w.N * w.K
    what = "the whole" if rows == w.M else f"rows 0..{rows - 1} of the"
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{what} {w.M}x{w.N}x{w.K} GEMM ({flops / 1e9:.1f} GFLOP in {t:.2f} s, "
                      f"float64 loop incl. fp16 decode, {cores} threads)"}


def time_steps(step, stream, args):
    """W untimed steps, then K back-to-back launches on the launch stream,
    bracketed by synchronize and by one pair of HIP events recorded on that
    stream (events between launches would serialise them and distort the
    time); then a short pass with an event pair per launch for the spread.
    Returns (wall ms per step, event ms per launch, per-launch ms array)."""
    import numpy as np
    import torch
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    kern_ms = ev0.elapsed_time(ev1) / args.steps          # average launch duration
    nper = min(20, args.steps)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(nper)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(nper)]
    for i in range(nper):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    per = np.array([st.elapsed_time(en) for st, en in zip(starts, ends)])   # ms
    # cold caches: 512 MiB written between launches (more than the L2s and the
    # 256 MB Infinity Cache hold), so the inputs come from HBM
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=stream.device)
    for i in range(nper):
        with torch.cuda.stream(stream):
            scratch.fill_(i & 0xff)
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    cold = np.array([st.elapsed_time(en) for st, en in zip(starts, ends)])   # ms
    del scratch
    print(f"[bench] avg launch {kern_ms:.4f} ms (events over {args.steps} launches); "
          f"wall/step {ms_per_step:.4f} ms; single-launch median {np.median(per):.4f} "
          f"min {per.min():.4f} p90 {np.percentile(per, 90):.4f}; cold-cache median "
          f"{np.median(cold):.4f} p90 {np.percentile(cold, 90):.4f}", file=sys.stderr, flush=True)
    return ms_per_step, kern_ms, per, cold


def cpu_baseline_chain(w, x, target_s: float):
    """The float64 oracle chain, as it stands, on whole batches of the
    workload: as many as a one-batch calibration says fit in target_s."""
    from oracle import chain as CH
    from oracle import gemm as G
    cores = G.max_threads()

    def run(nb):
        CH.chain_f64(nb, w.M, w.N1, w.N2, w.K, x.A, x.A.shape[2], x.A.shape[1] * x.A.shape[2],
                     x.B, x.B.shape[2], x.B.shape[1] * x.B.shape[2],
                     x.W, x.W.shape[2], x.W.shape[1] * x.W.shape[2])

    t0 = time.perf_counter()
    run(1)
    t_cal = time.perf_counter() - t0
    nb = max(1, min(w.batch, int(target_s / max(t_cal, 1e-3))))
    t0 = time.perf_counter()
    run(nb)
    t = time.perf_counter() - t0
    flops = 2.0 * nb * w.M * w.N1 * (w.K + w.N2)
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{nb} of the {w.batch} batches of the {w.M}x{w.N1}x{w.K} / "
                      f"{w.M}x{w.N2}x{w.N1} chain ({flops / 1e9:.1f} GFLOP in {t:.2f} s, "
                      f"float64 loops incl. fp16 decode and the rounding of S, "
                      f"{cores} threads)"}


def measure_and_report(step, stream, args, flops, metric, config, traffic, source_hash,
                       cpu_leg, extra=None):
    """Time the step (time_steps), read the clocks, print the one JSON line.
    `cpu_leg()` times the oracle unless --no-cpu-baseline; `extra()`, if
    given, returns more keys for the line (measured after the timed steps)."""
    import numpy as np
    import torch
    ms_per_step, kern_ms, per, cold = time_steps(step, stream, args)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kern_ms * 1e-3) / 1e12
    sclk = mclk = power = None
    if args.clock_seconds > 0:
        sclk, mclk, power = sustained_clock(step, torch.cuda.synchronize, args.clock_seconds)
        print(f"[bench] under sustained load: shader clock {sclk} MHz, memory clock {mclk} MHz, "
              f"power {power} W", file=sys.stderr, flush=True)
    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": config,
        "pct_of_peak": round(100.0 * value / PEAK_FP16_DENSE_TFLOPS, 2),
        "kernel_ms": {"avg_back_to_back": round(kern_ms, 5),
                      "single_median": round(float(np.median(per)), 5),
                      "single_min": round(float(per.min()), 5),
                      "single_p90": round(float(np.percentile(per, 90)), 5),
                      "cold_median": round(float(np.median(cold)), 5),
                      "cold_p90": round(float(np.percentile(cold, 90)), 5)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_FP16_DENSE_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_FP16_DENSE_TFLOPS, 4),
                     "traffic": traffic},
        "cpu_baseline": None,
        "kernel_source_hash": source_hash,
    }
    if sclk:
        # the dense peak scales with the shader clock (2400 MHz nominal)
        adj = PEAK_FP16_DENSE_TFLOPS * sclk / 2400.0
        out["clock"] = {"sclk_mhz_sustained": sclk, "peak_at_sclk": round(adj, 1),
                        "pct_of_peak_at_sclk": round(100.0 * value / adj, 2),
                        "mclk_mhz": mclk, "power_w": power,
                        "how": f"rocm-smi during {args.clock_seconds:g} s of back-to-back steps"}
    if args.copy_mib:
        out["config"]["copy_mib_per_step"] = args.copy_mib
    if extra is not None:
        out.update(extra())
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_leg()
    print(json.dumps(out), flush=True)
    return 0


def ramp_report(step, stream, n: int, what: str) -> int:
    """The first n launches of this process, each timed by its own event pair
    and followed by a short full-chip MFMA kernel that reads the shader clock
    (cycle counter against the real-time counter, per workgroup): how launch
    time and clock move from the start of the load.  Prints one JSON line of
    per-bucket means instead of the metric line."""
    import numpy as np
    import torch

    import mma_fragment_layouts_tn_amd as mfl
    dev = stream.device
    nwg, n_ops = 256, 1 << 20
    rng = np.random.default_rng(11)
    ops = torch.from_numpy(rng.uniform(-1.0, 1.0, n_ops).astype(np.float16)).to(dev)
    sink = torch.empty(nwg * 256, dtype=torch.float32, device=dev)
    clk = torch.zeros((n, 4 * nwg), dtype=torch.int64, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
    torch.cuda.synchronize()
    for i in range(n):
        ev[2 * i].record(stream)
        step()
        ev[2 * i + 1].record(stream)
        r = mfl.bench_mfma_raw(1, ops.data_ptr(), n_ops, 4, nwg, sink.data_ptr(),
                               clk[i].data_ptr(), stream.cuda_stream)
        if r != 0:
            raise RuntimeError(mfl.strerror(r))
    torch.cuda.synchronize()
    t = np.array([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n)])
    c = clk.view(n, nwg, 4).cpu().numpy().astype(np.float64)
    mhz = np.median((c[:, :, 2] - c[:, :, 0]) / (c[:, :, 3] - c[:, :, 1]), axis=1) * \
        mfl.wall_clock_khz() / 1e3
    edges = [e for e in (0, 1, 2, 5, 10, 25, 50, 100, 150, 200, 300, 500, 1000, 2000) if e < n] + [n]
    rows = [{"launches": f"{a}-{b - 1}", "ms": round(float(t[a:b].mean()), 4),
             "sclk_mhz": round(float(mhz[a:b].mean()))} for a, b in zip(edges, edges[1:])]
    print(json.dumps({"ramp": what, "launches": n, "buckets": rows,
                      "how": "event pair per launch; shader clock from a 4-iteration "
                             "v_mfma_f32_16x16x32_f16 kernel on 256 workgroups after each "
                             "launch"}), flush=True)
    return 0


MICRO_WORKLOADS = {
    "mfma_rate_32x32x16": ("mfma", 0, "v_mfma_f32_32x32x16_f16"),
    "mfma_rate_16x16x32": ("mfma", 1, "v_mfma_f32_16x16x32_f16"),
    "lds_read_b128": ("lds", None, "ds_read_b128"),
    "lds_dma_b128": ("dma", None, "global_load_lds_dwordx4"),
}


def main_micro(args) -> int:
    """The rates the GEMM kernels are priced against, each from one
    full-chip launch per step with the shader clock read inside the kernel
    (cycle counter against the real-time counter, per workgroup):

      mfma_rate_*: every wave issues independent matrix instructions on
        operand registers filled from random (or zero) fp16 data, 2^20 FLOP
        (32x32x16) or 2^21 FLOP (16x16x32) per wave per iteration, nothing
        else in the loop;
      lds_read_b128: every wave issues conflict-free 16-byte LDS reads,
        --depth of them in flight;
      lds_dma_b128: every wave fetches L2-resident data straight into LDS,
        --depth instructions in flight."""
    import numpy as np
    import torch

    import mma_fragment_layouts_tn_amd as mfl

    kind, op, instr = MICRO_WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    nwg = 256                                   # one workgroup per compute unit
    clocks = torch.zeros(4 * nwg, dtype=torch.int64, device=dev)
    if kind == "mfma":
        n_ops = 1 << 20
        if args.data == "zero":
            ops = torch.zeros(n_ops, dtype=torch.float16, device=dev)
        else:
            rng = np.random.default_rng(11)
            ops = torch.from_numpy(rng.uniform(-1.0, 1.0, n_ops).astype(np.float16)).to(dev)
        sink = torch.empty(nwg * 256, dtype=torch.float32, device=dev)
        iters = args.iters or 16384
        threads = 256
        # per wave per iteration: 2 sets x 16 instructions x 2*32*32*16 FLOP (op 0)
        # or 2 sets x 64 instructions x 2*16*16*32 FLOP (op 1)
        flops = float(nwg * 4 * iters * (1 << 20) * (1 if op == 0 else 2))

        def step():
            r = mfl.bench_mfma_raw(op, ops.data_ptr(), n_ops, iters, nwg, sink.data_ptr(),
                                   clocks.data_ptr(), sptr)
            if r != 0:
                raise RuntimeError(mfl.strerror(r))
    elif kind == "lds":
        threads = args.threads
        depth = args.depth or 8
        iters = args.iters or 32768
        sink = torch.empty(nwg, dtype=torch.int32, device=dev)
        nbytes = float(nwg * (threads // 64) * iters * 16 * 1024)

        def step():
            r = mfl.bench_lds_read_raw(threads, iters, nwg, depth, sink.data_ptr(),
                                       clocks.data_ptr(), sptr)
            if r != 0:
                raise RuntimeError(mfl.strerror(r))
    else:
        threads = args.threads
        depth = args.depth or 12
        iters = args.iters or 98304 // depth
        sink = torch.empty(nwg, dtype=torch.int32, device=dev)
        buf = torch.zeros(nwg * 65536, dtype=torch.uint8, device=dev)
        nbytes = float(nwg * (threads // 64) * iters * depth * 1024)

        def step():
            r = mfl.bench_dma_rate_raw(threads, iters, nwg, depth, buf.data_ptr(),
                                       sink.data_ptr(), clocks.data_ptr(), sptr)
            if r != 0:
                raise RuntimeError(mfl.strerror(r))

    print(f"[bench] {args.workload} ({instr}, data {args.data if kind == 'mfma' else '-'}) "
          f"{nwg} workgroups x {threads} threads, {iters} iterations; warmup={args.warmup} "
          f"steps={args.steps}", file=sys.stderr, flush=True)
    if args.ramp:
        return ramp_report(step, stream, args.ramp, args.workload)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = ev0.elapsed_time(ev1) / args.steps
    c = clocks.view(nwg, 4).cpu().numpy().astype(np.float64)   # last launch
    khz = mfl.wall_clock_khz()
    mhz = (c[:, 2] - c[:, 0]) / (c[:, 3] - c[:, 1]) * khz / 1e3
    loop_ms = float(np.median(c[:, 3] - c[:, 1])) / khz
    sclk = float(np.median(mhz))
    print(f"[bench] avg launch {kern_ms:.4f} ms; loop {loop_ms:.4f} ms (real-time counter at "
          f"{khz} kHz); shader clock in the loop: median {sclk:.0f} MHz, min {mhz.min():.0f}, "
          f"max {mhz.max():.0f}", file=sys.stderr, flush=True)
    config = {"workload": args.workload, "instruction": instr, "workgroups": nwg,
              "threads": threads, "iterations": iters}
    if kind != "mfma":
        config["in_flight_per_wave"] = depth
    clock = {"sclk_mhz_in_kernel_median": round(sclk, 1), "sclk_mhz_min": round(float(mhz.min()), 1),
             "sclk_mhz_max": round(float(mhz.max()), 1),
             "how": "s_memtime cycles / s_memrealtime ticks around the loop, per workgroup, "
                    "last timed launch"}
    if kind == "mfma":
        value = flops / (kern_ms * 1e-3) / 1e12
        adj = PEAK_FP16_DENSE_TFLOPS * sclk / 2400.0
        clock.update(peak_at_sclk=round(adj, 1), pct_of_peak_at_sclk=round(100 * value / adj, 2))
        config["data"] = "zero" if args.data == "zero" else "uniform [-1,1) fp16, seed 11"
        out = {"metric": f"MFMA issue rate ({instr}, {config['data']} operands), TFLOP/s and % "
                         f"of dense FP16 MFMA peak",
               "value": round(value, 2), "unit": "TFLOP/s",
               "roofline": {"bound": "mfma", "achieved": round(value, 2),
                            "peak": PEAK_FP16_DENSE_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(value / PEAK_FP16_DENSE_TFLOPS, 4), "traffic": None},
               "dtype": "f16"}
    else:
        value = nbytes / (kern_ms * 1e-3) / 1e12
        per_clk = nbytes / (loop_ms * 1e-3) / (sclk * 1e6) / nwg
        clock["bytes_per_clk_per_cu"] = round(per_clk, 1)
        what = ("LDS read rate (ds_read_b128, conflict-free)" if kind == "lds" else
                "direct-to-LDS fetch rate (global_load_lds_dwordx4, L2-resident data)")
        out = {"metric": f"{what}, TB/s over 256 CUs and bytes per clock per CU",
               "value": round(value, 2), "unit": "TB/s", "roofline": None, "dtype": "u32"}
    out.update({"n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                "ms_per_step": round(wall * 1e3 / args.steps, 5), "higher_is_better": True,
                "scaling": "weak", "vs_baseline": None, "data": "synthetic", "config": config,
                "kernel_ms": {"avg_back_to_back": round(kern_ms, 5)}, "clock": clock,
                "cpu_baseline": None})
    print(json.dumps(out), flush=True)
    return 0


def main_chain(args) -> int:
    import numpy as np
    import torch

    import mma_fragment_layouts_tn_amd as mfl
    import workloads as W

    w = W.CHAIN_WORKLOADS[args.workload]
    x = W.make_chain_inputs(w)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    A, B, Wt = (torch.from_numpy(np.ascontiguousarray(t)).to(dev) for t in (x.A, x.B, x.W))
    dk = mfl.F16 if w.d == "f16" else mfl.F32
    D = torch.empty((w.batch, w.M, w.N2), dtype=torch.float16 if w.d == "f16" else torch.float32,
                    device=dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    args_c = (w.batch, w.M, w.N1, w.N2, w.K,
              A.data_ptr(), x.A.shape[2], x.A.shape[1] * x.A.shape[2],
              B.data_ptr(), x.B.shape[2], x.B.shape[1] * x.B.shape[2],
              Wt.data_ptr(), x.W.shape[2], x.W.shape[1] * x.W.shape[2],
              D.data_ptr(), w.N2, w.M * w.N2, dk)
    rc = mfl.gemm_chain_validate(*args_c[:14], D.data_ptr(), w.N2, w.M * w.N2, dk)
    if rc != 0:
        print(f"invalid arguments: {mfl.strerror(rc)}", file=sys.stderr)
        return 1
    copy_src = copy_dst = None
    if args.copy_mib:
        copy_src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        copy_dst = torch.empty_like(copy_src)

    def step():
        r = mfl.gemm_chain_raw(*args_c, sptr)
        if r != 0:
            raise RuntimeError(mfl.strerror(r))
        if copy_dst is not None:
            copy_dst.copy_(copy_src)

    print(f"[bench] {w.name} back-to-back GEMM batch={w.batch} M={w.M} N1={w.N1} N2={w.N2} "
          f"K={w.K} warmup={args.warmup} steps={args.steps}", file=sys.stderr, flush=True)
    rc, staging, tile_n = mfl.gemm_chain_plan(*args_c[:14], D.data_ptr(), w.N2, w.M * w.N2, dk)
    config = {"workload": w.name, "batch": w.batch, "M": w.M, "N1": w.N1, "N2": w.N2,
              "K": w.K, "a": "f16 K-contiguous", "b": "f16 K-contiguous",
              "w": "f16 N1-contiguous", "d": w.d, "accumulate": "f32",
              "intermediate": "S rounded once to f16",
              "kernel": f"gemm_chain 256x{tile_n} tile, N1 chunks of {32 if w.K >= 256 else 64}, "
                        f"{staging} staging"}
    def phases():
        """Cycles per iteration of the N1 loop by phase, from the timed
        instance of the kernel (mfl_probe_chain_phases): lane 0 of every wave
        of workgroups 0..7 reads the shader clock at the start of each
        iteration, before the conversion of the next chunk's S, before the
        barrier and after it."""
        stamps = torch.zeros(int(np.prod(mfl.CHAIN_STAMP_SHAPE)), dtype=torch.int32, device=dev)

        def run():
            r = mfl.probe_chain_phases_raw(*args_c, stamps.data_ptr(), sptr)
            if r != 0:
                raise RuntimeError(mfl.strerror(r))
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(args.steps):
            run()
        ev1.record(stream)
        torch.cuda.synchronize()
        timed_ms = ev0.elapsed_time(ev1) / args.steps
        t = stamps.view(*mfl.CHAIN_STAMP_SHAPE).cpu().numpy().astype(np.int64) & 0xFFFFFFFF
        nwg = min(mfl.CHAIN_STAMP_SHAPE[0],
                  w.batch * (-(-w.M // 256)) * (-(-w.N2 // 128)))
        t = t[:nwg]
        nch = (w.N1 + 63) // 64
        cs = np.arange(2, min(nch - 1, 64) - 2)      # steady iterations with a barrier
        d = lambda a, b: (b - a) % (1 << 32)
        s0, s1, s2, s3 = (t[:, :, 4 * cs + k] for k in range(4))
        nxt = t[:, :, 4 * (cs + 1)]
        names = {"K chunks 0..2H-2 of the second product with the next chunk's first product "
                 "and the fetch of slot c+3": d(s0, s1),
                 "wait for this wave's fetch of slot c+1": d(s1, s2),
                 "workgroup barrier": d(s2, s3),
                 "last K chunk with the first reads of slot c+1": d(s3, nxt)}
        total = d(s0, nxt)
        whole = d(t[:, :, 256], t[:, :, 258])
        prologue = d(t[:, :, 256], t[:, :, 0])
        loop = d(t[:, :, 0], t[:, :, 257])
        epilogue = d(t[:, :, 257], t[:, :, 258])
        return {"phases": {
            "how": "shader-clock stamps (s_memtime) of the timed kernel instance, lane 0 of "
                   f"each wave of workgroups 0..{nwg - 1}, iterations {cs[0]}..{cs[-1]}",
            "timed_kernel_ms": round(timed_ms, 5),
            "cycles_per_iteration": round(float(total.mean()), 1),
            "iterations": nch,
            "wave_cycles": {"start to end": round(float(whole.mean()), 1),
                            "prologue (A fragments, first slots, first product of chunk 0)":
                                round(float(prologue.mean()), 1),
                            "N1 loop": round(float(loop.mean()), 1),
                            "epilogue (D stores issued)": round(float(epilogue.mean()), 1)},
            "mfma_cycles_per_iteration": 64 * 32,
            "phase_cycles_mean": {k: round(float(v.mean()), 1) for k, v in names.items()},
            "phase_cycles_by_wave": {k: [round(float(x), 1) for x in v.mean(axis=(0, 2))]
                                     for k, v in names.items()}}}

    return measure_and_report(step, stream, args, float(w.flops), METRIC_CHAIN, config,
                              load_traffic(w.name, "chain", CHAIN_SOURCES),
                              kernel_source_hash(CHAIN_SOURCES),
                              lambda: cpu_baseline_chain(w, x, args.cpu_seconds),
                              phases if args.phases else None)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # A few milliseconds into the load the power controller pulls the shader
    # clock down (launches 10-50 at 4096^3) before it settles (--ramp shows
    # it); the defaults warm up well past that and time steady state.
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default="lds_4096")
    ap.add_argument("--algo", default="auto",
                    help="auto, direct, lds128, lds256, lds256w4, lds128w1, splitk, lds256w4_16, "
                         "lds256_16, lds128_16, splitk_16; '+reg' "
                         "forces register fetch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--clock-seconds", type=float, default=2.0,
                    help="after the timed region, run the step this long and read the shader "
                         "clock under load (0 = skip)")
    ap.add_argument("--cpu-seconds", type=float, default=30.0,
                    help="bound on the CPU oracle sample (the whole workload if it fits)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB per step "
                         "(calibration of the HBM byte counters)")
    ap.add_argument("--data", default="random", choices=["random", "zero"],
                    help="operand data of the MFMA issue-rate workloads")
    ap.add_argument("--threads", type=int, default=512,
                    help="threads per workgroup of the LDS read-rate workload")
    ap.add_argument("--depth", type=int, default=0, choices=[0, 1, 4, 8, 12, 16, 24],
                    help="instructions in flight per wave in the LDS read-rate (1, 4, 8, 16; "
                         "default 8) and direct-to-LDS fetch-rate (4, 12, 24; default 12) "
                         "workloads")
    ap.add_argument("--phases", action="store_true",
                    help="back-to-back GEMM: also report cycles per loop phase from the timed "
                         "kernel instance")
    ap.add_argument("--ramp", type=int, default=0,
                    help="print launch time and shader clock of the first N launches of this "
                         "process (GEMM and MFMA-rate workloads) instead of the metric line")
    ap.add_argument("--iters", type=int, default=0,
                    help="loop iterations of the microbenchmark kernels (0 = default)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); this GEMM build has no multi-GPU path.", file=sys.stderr)
        return 2

    import torch

    import mma_fragment_layouts_tn_amd as mfl
    import workloads as W

    if args.workload in MICRO_WORKLOADS:
        return main_micro(args)
    if args.workload in W.CHAIN_WORKLOADS:
        return main_chain(args)
    w = W.WORKLOADS[args.workload]
    x = W.make_inputs(w)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    A = torch.from_numpy(x.A).to(dev)
    B = torch.from_numpy(x.B).to(dev)
    C = torch.from_numpy(x.C).to(dev) if x.C is not None else None
    D = torch.empty((w.M, w.ldd_), dtype=torch.float16 if w.d == "f16" else torch.float32,
                    device=dev)
    ck = {None: mfl.NONE, "f16": mfl.F16, "f32": mfl.F32}[w.c]
    dk = mfl.F16 if w.d == "f16" else mfl.F32
    a_order = mfl.A_KMAJOR if w.a_order == "k" else mfl.A_MMAJOR
    dt = mfl.dtypes(ck, dk, a_order, mfl.algo_code(args.algo))
    rc, algo, fetch_a, fetch_b = mfl.plan(w.M, w.N, w.K, A.data_ptr(), w.lda_, B.data_ptr(),
                                          w.ldb_, None if C is None else C.data_ptr(), w.ldc_,
                                          D.data_ptr(), w.ldd_, dt)
    if rc != 0:
        print(f"invalid arguments: {mfl.strerror(rc)}", file=sys.stderr)
        return 1
    algo_name = mfl.ALGO_NAMES[algo]
    info = mfl.kernel_info(algo_name, ck, dk, a_order)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    cptr = None if C is None else C.data_ptr()
    copy_src = copy_dst = None
    if args.copy_mib:
        copy_src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        copy_dst = torch.empty_like(copy_src)

    def step():
        r = mfl.gemm_tn_raw(w.M, w.N, w.K, A.data_ptr(), w.lda_, B.data_ptr(), w.ldb_, cptr,
                            w.ldc_, D.data_ptr(), w.ldd_, dt, sptr)
        if r != 0:
            raise RuntimeError(mfl.strerror(r))
        if copy_dst is not None:
            copy_dst.copy_(copy_src)

    print(f"[bench] {w.name} algo={algo_name} fetch A:{mfl.FETCH_NAMES[fetch_a]} "
          f"B:{mfl.FETCH_NAMES[fetch_b]} tile={info['bm']}x{info['bn']}x{info['bk']} "
          f"warmup={args.warmup} steps={args.steps}", file=sys.stderr, flush=True)
    config = {"workload": w.name, "M": w.M, "N": w.N, "K": w.K,
              "a": "f16 K-contiguous" if w.a_order == "k" else f"f16 M-contiguous lda={w.lda_}",
              "b": "f16 K-contiguous", "c": w.c, "d": w.d, "accumulate": "f32",
              "algo": algo_name, "block_tile": f"{info['bm']}x{info['bn']}x{info['bk']}",
              "fetch": f"A:{mfl.FETCH_NAMES[fetch_a]} B:{mfl.FETCH_NAMES[fetch_b]}",
              "threads": info["threads"], "lds_bytes": info["lds_bytes"]}
    traffic = load_traffic(w.name, algo_name + "_" + mfl.FETCH_NAMES[fetch_a] +
                           mfl.FETCH_NAMES[fetch_b])
    metric = METRIC if (w.M, w.N, w.K) == (4096, 4096, 4096) else (
        f"TFLOP/s for fp16 TN GEMM at {w.M}x{w.N}x{w.K} (fp32 acc) and % of dense FP16 MFMA peak")
    if args.ramp:
        return ramp_report(step, stream, args.ramp, f"{w.name} algo={algo_name}")
    return measure_and_report(step, stream, args, float(w.flops), metric, config, traffic,
                              kernel_source_hash(), lambda: cpu_baseline(w, x, args.cpu_seconds))


if __name__ == "__main__":
    sys.exit(main())
