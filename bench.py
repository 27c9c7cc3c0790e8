#!/usr/bin/env python3
"""Benchmark of the RWKV-4 WKV time-mixing hot path on one MI355X.

Workload (one "step" = one call of rwkv4_timemix_fused, i.e. the whole path: token
shift -> r = xr -> WKV recurrence with fp32 state -> sigmoid gate -> y, plus the
final state and x_last): the RWKV-4 14B layer shape B1 T1024 C5120 with fp16
activations, x ~ N(0,1), x_prev ~ N(0,1), mix_* ~ U(0,1), k, v ~ N(0,1), decay and
bonus by the workload recipe, empty prior state.  Inputs are resident in HBM when
the timed region starts; each step uses the next of R rotated buffer sets (>= 1.25
GiB in total), so the 256 MB Infinity Cache cannot serve a step's inputs from an
earlier step.

Prints ONE JSON line: throughput in tokens*channels/s (B*T*C per step over the
wall time of the K timed steps), the roofline of the kernel (algorithmic bytes per
launch over its average duration: a pair of HIP events on the kernel's stream brackets
the K back-to-back launches), and the fp64 CPU oracle timed on the host cores.

    python bench.py [--steps K] [--warmup W] [--chunk-len L] [--algo auto|chunked|sequential]
    python bench.py --copy-kernel      # plain device copy, for counter calibration
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
COUNTERS_FILE = os.path.join(ROOT, "profiles", "timemix_14b_layer_counters.txt")
KERNEL_SRC = os.path.join(ROOT, "rwkv_wkv_linear_amd", "csrc", "wkv_kernels.hip")
WORKLOAD = "rwkv4-14b time-mix fused prefill B1 T1024 C5120 (fp16 I/O)"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--chunk-len", type=int, default=0)
    ap.add_argument("--algo", default="auto", choices=["auto", "chunked", "sequential"])
    ap.add_argument("--rotate-gib", type=float, default=1.25)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-kernel", action="store_true",
                    help="time a plain device-to-device copy instead (counter calibration)")
    ap.add_argument("--copy-mib", type=float, default=256.0)
    return ap.parse_args()


def single_gpu_guard(args):
    ws = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or ws != 1:
        print("bench.py runs on one GPU only: librwkvwkv has no multi-GPU path (every (b, channel) "
              "recurrence is independent, so a multi-GPU job shards batch rows or channels with no "
              "communication). Run with --gpus 1.", file=sys.stderr, flush=True)
        sys.exit(2)


def counters_traffic():
    """HBM bytes per launch from the committed counter run, if the kernel is unchanged since."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    fields = {}
    with open(COUNTERS_FILE) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    with open(KERNEL_SRC, "rb") as f:
        h = hashlib.sha256(f.read()).hexdigest()
    if fields.get("kernel_source_sha256") != h:
        return None
    try:
        return float(fields["traffic_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(case, B, T, C):
    """The fp64 oracle as it stands (token shift + linear-space recurrence + final state)
    on the full workload; median of repeated runs, at least 3, about 3 s in all."""
    import oracle
    times = []
    t_end = time.perf_counter() + 3.0
    while len(times) < 3 or (time.perf_counter() < t_end and len(times) < 10):
        t0 = time.perf_counter()
        oracle.timemix(case)
        times.append(time.perf_counter() - t0)
    med = statistics.median(times)
    return {
        "value": B * T * C / med,
        "unit": "tokens*channels/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"full workload B{B} T{T} C{C}, oracle.timemix (fp64 C, OpenMP over channels: "
                  f"token shift, numerator/denominator recurrence, final state), median of {len(times)} runs",
    }


def copy_kernel(args):
    import torch
    n = int(args.copy_mib * 2**20) // 4
    a = torch.empty(n, dtype=torch.float32, device="cuda:0").normal_()
    b = torch.empty_like(a)
    for _ in range(args.warmup):
        b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(args.steps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / args.steps
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "ms_per_copy": ms,
                      "GBps": 2 * n * 4 / ms / 1e6}), flush=True)


def main():
    args = parse()
    single_gpu_guard(args)
    if args.copy_kernel:
        return copy_kernel(args)

    import numpy as np
    import torch

    import rwkv_wkv_linear_amd as rw
    import wkv_inputs as wi

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = wi.WORKLOADS[2]
    B, T, C = wl.B, wl.T, wl.C
    case = wi.workload_inputs(2)
    E = B * T * C

    # resident inputs, R rotated sets of (x, k, v, y, x_last, state_out)
    h = {n: torch.from_numpy(np.ascontiguousarray(case[n])) for n in ("x", "k", "v")}
    shared = {n: torch.from_numpy(np.ascontiguousarray(case[n])).to(dev)
              for n in ("x_prev", "mix_k", "mix_v", "mix_r", "w", "u")}
    set_bytes = 4 * E * 2 + B * C * 2 + 3 * B * C * 4
    R = max(2, math.ceil(args.rotate_gib * 2**30 / set_bytes))
    sets = []
    for _ in range(R):
        sets.append(dict(x=h["x"].to(dev), k=h["k"].to(dev), v=h["v"].to(dev),
                         y=torch.empty((B, T, C), dtype=torch.float16, device=dev),
                         x_last=torch.empty((B, C), dtype=torch.float16, device=dev),
                         state_out=torch.empty((3, B, C), dtype=torch.float32, device=dev)))
    stream = torch.cuda.current_stream(dev)
    opts = rw.Opts()
    opts.size = ctypes.sizeof(rw.Opts)
    opts.in_dtype = rw.RWKV_F16
    opts.out_dtype = rw.RWKV_F16
    opts.chunk_len = args.chunk_len
    opts.algo = {"auto": 0, "sequential": 1, "chunked": 2}[args.algo]
    vp = ctypes.c_void_p
    hs = vp(stream.cuda_stream)
    fn = rw.lib.rwkv4_timemix_fused
    calls = []
    for s in sets:
        calls.append((B, T, C, vp(s["x"].data_ptr()), vp(shared["x_prev"].data_ptr()), vp(s["x_last"].data_ptr()),
                      vp(shared["mix_k"].data_ptr()), vp(shared["mix_v"].data_ptr()), vp(shared["mix_r"].data_ptr()),
                      vp(s["k"].data_ptr()), vp(s["v"].data_ptr()), vp(shared["w"].data_ptr()),
                      vp(shared["u"].data_ptr()), vp(s["y"].data_ptr()), None, None, None,
                      vp(s["state_out"].data_ptr()), hs, ctypes.byref(opts)))

    def step(i):
        st = fn(*calls[i % R])
        if st != 0:
            raise rw.RwkvError(st, rw.rwkv_last_error())

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # The timed region: K back-to-back launches on `stream`, bracketed by one pair of HIP
    # events on that stream and by device synchronisations.  A timing event between
    # launches is a marker packet with its own cache maintenance that slows the launch it
    # brackets, so per-launch events would not measure the launches as they run in a layer
    # loop; the pair gives their average duration.
    K = args.steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(K):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_avg_ms = ev0.elapsed_time(ev1) / K

    # algorithmic bytes per launch: x, k, v read and y written once (2 B each per element),
    # plus x_prev, x_last (fp16 rows), mix_r/mix_k/mix_v, w, u (fp32 per channel; mix_k/v are
    # read by the kernel even when xk/xv are not requested) and the fp32 state written
    algo_bytes = 8 * E + 2 * 2 * B * C + 5 * 4 * C + 3 * 4 * B * C
    achieved = algo_bytes / (kern_avg_ms * 1e-3) / 1e9
    traffic = counters_traffic()
    chunk = args.chunk_len
    if args.algo != "sequential" and chunk == 0:
        chunk = None
    result = {
        "metric": "WKV tokens*channels/s (and achieved HBM GB/s of the WKV kernel vs MI355X peak), "
                  "RWKV-4 14B layer shape",
        "value": E * K / wall,
        "unit": "tokens*channels/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "B": B, "T": T, "C": C, "io_dtype": "f16",
                   "entry_point": "rwkv4_timemix_fused", "algo": args.algo, "chunk_len": chunk,
                   "rotated_sets": R},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic},
        "kernel_avg_us": kern_avg_ms * 1e3,
        "algorithmic_bytes_per_launch": algo_bytes,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case, B, T, C)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
