#!/usr/bin/env python3
"""Benchmark of the RWKV-4 WKV time-mixing hot path on one MI355X.

Default workload (one "step" = one call of rwkv4_timemix_fused, i.e. the whole path:
token shift -> r = xr -> WKV recurrence with fp32 state -> sigmoid gate -> y, plus the
final state and x_last): the RWKV-4 14B layer shape B1 T1024 C5120 with fp16
activations, x ~ N(0,1), x_prev ~ N(0,1), mix_* ~ U(0,1), k, v ~ N(0,1), decay and
bonus by the workload recipe, empty prior state.  Inputs are resident in HBM when the
timed region starts; each step uses the next of R rotated buffer sets (>= 1.25 GiB in
total), so the 256 MB Infinity Cache cannot serve a step's inputs from an earlier step.

Prints ONE JSON line: throughput in tokens*channels/s (B*T*C per step over the wall
time of the K timed steps), the roofline of the kernel (algorithmic bytes per launch
over its average duration: a pair of HIP events on the kernel's stream brackets the
K back-to-back launches), and the fp64 CPU oracle timed on the host cores (and, for the C
oracle, once on one thread).  Where the buffers rotate, the line also carries a labelled
"warm_same_buffers" figure: the same launches on one buffer set, inputs largely served from
the Infinity Cache; it is context, never the reported value.

--workload selects one of the other shapes the library is tested on (same fields):
  plain169m  rwkv4_wkv_forward  B1 T1024 C768, fp32 in/out, ungated
  gated169m  rwkv4_wkv_forward  B8 T1024 C768, fp16 in/out, gated, prior state
  decode14b  40 x rwkv4_wkv_step  B256 C5120, fp16, gated, state in place (a step = 40 layers)
  long       rwkv4_wkv_forward  B1 T65536 C2048, fp16 in, fp32 out
  lnshift14b rwkv4_shift_mix    B1 T1024 C5120 fp16: LayerNorm + token shift -> xk, xv, xr, x_last
  cmgate14b  rwkv4_channelmix_gate  1024 x 5120 fp16: residual + sigmoid(r) * kv

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--chunk-len L] [--algo A]
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

# name -> (workload index in wkv_inputs.WORKLOADS, description)
WORKLOADS = {
    "timemix14b": (2, "rwkv4-14b time-mix fused prefill B1 T1024 C5120 (fp16 I/O)"),
    "plain169m": (0, "rwkv4-169m wkv forward B1 T1024 C768 (fp32 I/O, ungated)"),
    "gated169m": (1, "rwkv4-169m gated prefill B8 T1024 C768 (fp16 I/O, prior state)"),
    "decode14b": (3, "rwkv4-14b batched decode, 40 layers x B256 C5120 (fp16 I/O, state in place)"),
    "long": (4, "long-sequence forward B1 T65536 C2048 (fp16 in, fp32 out)"),
    "lnshift14b": (5, "rwkv4-14b time-mix prologue: ln1 + token shift -> xk, xv, xr, B1 T1024 C5120 (fp16)"),
    "cmgate14b": (6, "rwkv4-14b channel-mix gate + residual, B1 T1024 C5120 (fp16)"),
}
CPU_BUDGET_S = 10.0  # CPU seconds the oracle leg spends (at least 3 runs)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default by workload)")
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="timemix14b", choices=sorted(WORKLOADS))
    ap.add_argument("--chunk-len", type=int, default=0)
    ap.add_argument("--algo", default="auto", choices=["auto", "chunked", "two_pass", "sequential"])
    ap.add_argument("--publish", default="auto", choices=["auto", "l2_first", "write_through"],
                    help="how the single-pass scan publishes its look-back states (results are identical)")
    ap.add_argument("--rotate-gib", type=float, default=1.25)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--with-xkv", action="store_true",
                    help="timemix14b: also write the xk and xv rows (12 B per element instead of 8)")
    ap.add_argument("--bf16", action="store_true",
                    help="bfloat16 in place of the workload's fp16 activations (inputs rounded from them)")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the same-buffer (cache-warm) figure, e.g. under a profiler")
    ap.add_argument("--graph", action="store_true",
                    help="decode14b: capture the 40 layers' launches into one HIP graph and replay it "
                         "per step")
    ap.add_argument("--ceiling", action="store_true",
                    help="also time the same-pattern bandwidth ceilings (libwkvceiling.so): the workload's "
                         "bytes moved in its kernel's launch shape and memory instructions with no arithmetic, "
                         "and a plain grid-stride stream of the same bytes")
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


def counters_traffic(field="traffic_bytes_per_dispatch"):
    """A figure of the committed counter run (by default the HBM bytes per launch), if the kernel
    is unchanged since."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    fields = {}
    with open(COUNTERS_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    with open(KERNEL_SRC, "rb") as f:
        h = hashlib.sha256(f.read()).hexdigest()
    if fields.get("kernel_source_sha256") != h:
        return None
    try:
        return float(fields[field])
    except (KeyError, ValueError):
        return None


def cpu_baseline(name, case, elements, sample):
    """The fp64 oracle as it stands, on the host cores: median of repeated runs over `case`
    (at least 3, about CPU_BUDGET_S seconds in all), then one run on a single thread.  Returns
    the line's object and the oracle's result of the last run.  Every
    oracle routine is C with OpenMP over independent lanes (channels, or rows and elements for
    the mixers); numpy only marshals the arrays and, for the prologue, runs the token shift's
    elementwise mix."""
    import oracle
    run = {"timemix14b": oracle.timemix, "decode14b": lambda c: [oracle.step(l) for l in c],
           "lnshift14b": oracle.shift_mix,
           "cmgate14b": lambda c: oracle.receptance_gate(c["r"], c["kv"], c["residual"])}.get(
        name, oracle.forward)
    threads = oracle.num_threads()
    times = []
    t_end = time.perf_counter() + CPU_BUDGET_S
    ref = None
    while len(times) < 3 or (time.perf_counter() < t_end and len(times) < 50):
        t0 = time.perf_counter()
        ref = run(case)
        times.append(time.perf_counter() - t0)
    med = statistics.median(times)
    out = {
        "value": elements / med,
        "unit": "tokens\u00b7channels/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{sample}; fp64 C oracle with OpenMP on {threads} threads, median of {len(times)} runs",
    }
    if threads > 1:
        # one run on one thread (the last oracle work of the process)
        one = {"timemix14b": lambda c: oracle.timemix(c, nthreads=1),
               "decode14b": lambda c: [oracle.step(l, nthreads=1) for l in c]}.get(name)
        if one is None and name in ("lnshift14b", "cmgate14b"):
            prev = oracle.num_threads()
            oracle.set_threads(1)
            one = lambda c: run(c)  # noqa: E731
        elif one is None:
            prev = None
            one = lambda c: oracle.forward(c, nthreads=1)  # noqa: E731
        else:
            prev = None
        t0 = time.perf_counter()
        one(case)
        out["value_one_thread"] = elements / (time.perf_counter() - t0)
        if prev is not None:
            oracle.set_threads(prev)
    return out, ref


# Bars of the parity tests for the WKV output (scaled error, by input dtype) and the final state
PARITY_TOL = {"f32": 1e-5, "f16": 2e-3}
STATE_TOL = 1e-5


def parity(su, ref):
    """Error of the timed launches' outputs (those of the first buffer set; every set holds the
    same inputs) against the oracle's result on those inputs, by the parity tests' metrics."""
    from oracle import compare as cmp
    host = lambda t: t.float().cpu().numpy().astype("float64")  # noqa: E731
    y = host(su.check_out["y"])
    err = cmp.scaled_error(y, ref["y"], ref["scale"], cmp.FLOOR[su.out_dtype])
    ea, eb = cmp.state_error(host(su.check_out["state"]), ref["state"], ref["state_abs"])
    tol = PARITY_TOL[su.in_dtype]
    return {"vs": "oracle", "scaled_error": err, "tol": tol, "state_error": max(ea, eb), "state_tol": STATE_TOL,
            "within_tol": bool(err <= tol and max(ea, eb) <= STATE_TOL)}

def copy_kernel(args):
    import torch
    n = int(args.copy_mib * 2**20) // 4
    a = torch.empty(n, dtype=torch.float32, device="cuda:0").normal_()
    b = torch.empty_like(a)
    for _ in range(args.warmup or 2):
        b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    steps = args.steps or 10
    s.record()
    for _ in range(steps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "ms_per_copy": ms,
                      "GBps": 2 * n * 4 / ms / 1e6}), flush=True)


# workload -> (pattern, inputs, input bytes, output bytes, tokens per wave, LDS bytes of the scan kernel)
CEILING_PATTERNS = {
    "timemix14b": ("tile", 3, 2, 2, 32, 3 * 128 * 64 * 2 + 4 * 4 * 64 * 4),
    "gated169m": ("tile", 3, 2, 2, 32, 3 * 128 * 64 * 2 + 4 * 4 * 64 * 4),
    "plain169m": ("tile", 2, 4, 4, 16, 2 * 64 * 64 * 4 + 4 * 4 * 64 * 4),
    "long": ("tile", 2, 2, 4, 32, 2 * 128 * 64 * 2 + 4 * 4 * 64 * 4),
    "decode14b": ("lanes", 3, 2, 2, 0, 0),
}


def ceilings(name, su, args, torch, K, W):
    """Time the same-pattern ceilings of a workload like its kernel: K back-to-back launches
    between one pair of events on the stream, on rotated buffer sets of >= rotate_gib (one set when
    a set alone exceeds 1 GiB).  Returns a dict for the JSON line, or None for the mixers."""
    if name not in CEILING_PATTERNS:
        return None
    from rwkv_wkv_linear_amd.build import CEIL_LIB
    lib = ctypes.CDLL(CEIL_LIB)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.wkvceil_tile.argtypes = [vp, vp, vp, ctypes.c_int, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_int, vp]
    lib.wkvceil_lanes.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, i64, ctypes.c_int, vp]
    lib.wkvceil_stream.argtypes = [vp, vp, vp, ctypes.c_int, vp, i64, ctypes.c_int, vp]
    pattern, n_in, ei, eo, L, lds = CEILING_PATTERNS[name]
    B, T, C = su.B, su.T, su.C
    E = B * T * C
    dev = torch.device("cuda:0")
    hs = vp(su.stream.cuda_stream)
    state_bytes = 24 * B * C if pattern == "lanes" else 0
    set_bytes = (n_in * ei + eo) * E + state_bytes
    R = 1 if set_bytes >= 2**30 else max(2, math.ceil(args.rotate_gib * 2**30 / set_bytes))
    sets = []
    for _ in range(R):
        ins = [torch.empty(E * ei, dtype=torch.uint8, device=dev).random_(0, 60) for _ in range(n_in)]
        out = torch.empty(E * eo, dtype=torch.uint8, device=dev)
        st = torch.empty(3 * B * C, dtype=torch.float32, device=dev).normal_() if pattern == "lanes" else None
        sets.append((ins, out, st))

    def ptrs(ins):
        return [vp(t.data_ptr()) for t in ins] + [None] * (3 - len(ins))

    def launch(i, kind):
        ins, out, st = sets[i % R]
        if kind == "stream":
            # equal-size inputs and output: the output in the inputs' element size
            nbytes = E * ei
            rc = lib.wkvceil_stream(*ptrs(ins), n_in, vp(out.data_ptr()), nbytes, 2048, hs)
        elif pattern == "tile":
            rc = lib.wkvceil_tile(*ptrs(ins), n_in, vp(out.data_ptr()), B, T, C, L, ei, eo, lds, hs)
        else:
            rc = lib.wkvceil_lanes(*ptrs(ins), n_in, vp(out.data_ptr()), vp(st.data_ptr()), E, ei, hs)
        if rc != 0:
            raise RuntimeError(f"ceiling kernel {kind}: status {rc}")

    res = {}
    for kind in ("pattern", "stream"):
        for i in range(W):
            launch(i, kind)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(su.stream)
        for i in range(K):
            launch(W + i, kind)
        ev1.record(su.stream)
        torch.cuda.synchronize()
        us = ev0.elapsed_time(ev1) / K * 1e3
        # state_bytes: the fp32 state read and written once each (12 + 12 bytes per (b, c))
        moved = (n_in * ei + (eo if kind == "pattern" else ei)) * E + (state_bytes if kind == "pattern" else 0)
        res[kind] = {"kernel_avg_us": us, "GBps": moved / (us * 1e-6) / 1e9, "bytes": moved}
    return {"pattern": f"{pattern}: {n_in} x {ei}-byte inputs, {eo}-byte output"
                       + (", fp32 state read and written" if pattern == "lanes" else f", tiles of 4 x {L} tokens"),
            "same_pattern": res["pattern"], "plain_stream": res["stream"]}


class Setup:
    """Device buffers and the raw ctypes calls of one workload."""

    def __init__(self, name, args, torch, rw, wi, np):
        self.name = name
        idx, self.desc = WORKLOADS[name]
        wl = wi.WORKLOADS[idx]
        self.B, self.T, self.C = wl.B, wl.T, wl.C
        B, T, C = self.B, self.T, self.C
        dev = torch.device("cuda:0")
        vp = ctypes.c_void_p
        stream = torch.cuda.current_stream(dev)
        hs = vp(stream.cuda_stream)
        self.stream = stream
        # --bf16: every 2-byte activation (input and output) becomes bfloat16, the inputs rounded
        # from the workload's fp16 values; fp32 tensors and the parameters stay as they are
        act = torch.bfloat16 if args.bf16 else torch.float16
        self.act = act
        self.act_code = rw.RWKV_BF16 if args.bf16 else rw.RWKV_F16
        tdt = {"f16": act, "f32": torch.float32}
        esz = {"f16": 2, "f32": 4}
        ei, eo = esz[wl.in_dtype], esz[wl.out_dtype]
        name16 = "bf16" if args.bf16 else "f16"
        self.io = f"{wl.in_dtype}->{wl.out_dtype}".replace("f16", name16)
        self.in_dtype, self.out_dtype = wl.in_dtype, wl.out_dtype
        # outputs of the first buffer set, checked against the oracle (WKV workloads whose device
        # inputs are the oracle's: not under --bf16, which rounds them again)
        self.check_out = None

        def dev_t(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

        def dev_act(a):
            # a device copy of an activation in the benchmark's 2-byte type (fp32 stays fp32)
            t = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
            return t.to(act) if t.dtype == torch.float16 else t

        opts = rw.Opts()
        opts.size = ctypes.sizeof(rw.Opts)
        opts.in_dtype = self.act_code if wl.in_dtype == "f16" else rw.RWKV_F32
        opts.out_dtype = self.act_code if wl.out_dtype == "f16" else rw.RWKV_F32
        opts.chunk_len = args.chunk_len
        opts.algo = {"auto": 0, "sequential": 1, "chunked": 2, "two_pass": 3}[args.algo]
        opts.publish = {"auto": 0, "l2_first": 1, "write_through": 2}[args.publish]
        self.opts = opts
        self.keep = []
        case = wi.workload_inputs(idx)

        if wl.kind == "step":
            self.entry = "rwkv4_wkv_step"
            self.fn = rw.lib.rwkv4_wkv_step
            self.launches_per_step = len(case)
            self.elements = len(case) * B * C
            # per launch: k, v, r read and y written (2 B each), state read and written
            # (12 B each), w and u (4 B per channel)
            self.launch_bytes = 4 * 2 * B * C + 2 * 12 * B * C + 8 * C
            calls = []
            for layer in case:
                t = {n: dev_act(layer[n]) for n in ("k", "v", "r", "w", "u", "state")}
                y = torch.empty((B, C), dtype=tdt[wl.out_dtype], device=dev)
                self.keep.append((t, y))
                calls.append((B, C, vp(t["w"].data_ptr()), vp(t["u"].data_ptr()), vp(t["k"].data_ptr()),
                              vp(t["v"].data_ptr()), vp(t["r"].data_ptr()), vp(y.data_ptr()),
                              vp(t["state"].data_ptr()), opts.in_dtype, opts.out_dtype, hs))
            self.sets = [calls]  # 40 layers of 42 MB each: no rotation needed beyond the layers
            self.cpu_case = case[:4]
            self.cpu_elements = 4 * B * C
            self.cpu_sample = "4 of the 40 decode layers (B256 C5120, one token each)"
            return

        E = B * T * C
        self.elements = E
        self.launches_per_step = 1
        if wl.kind in ("shift", "gate"):
            self._setup_mix(wl, case, args, torch, rw, np, dev, hs, E)
            return
        if wl.kind == "timemix":
            self.entry = "rwkv4_timemix_fused"
            self.fn = rw.lib.rwkv4_timemix_fused
            # x, k, v read and y written once, x_prev read and x_last written, mix_r/k/v, w, u
            # (fp32 per channel; mix_k/v are read even when xk/xv are not requested), state out
            self.launch_bytes = 3 * ei * E + eo * E + 2 * ei * B * C + 5 * 4 * C + 3 * 4 * B * C
            if args.with_xkv:
                self.launch_bytes += 2 * ei * E  # xk and xv written
            h = {n: dev_act(case[n]).cpu() for n in ("x", "k", "v")}
            sh = {n: dev_act(case[n]) for n in ("x_prev", "mix_k", "mix_v", "mix_r", "w", "u")}
            self.keep.append(sh)
            set_bytes = (3 * ei + eo + (2 * ei if args.with_xkv else 0)) * E
            R = max(2, math.ceil(args.rotate_gib * 2**30 / set_bytes))
            self.sets = []
            for _ in range(R):
                s = dict(x=h["x"].to(dev), k=h["k"].to(dev), v=h["v"].to(dev),
                         y=torch.empty((B, T, C), dtype=tdt[wl.out_dtype], device=dev),
                         x_last=torch.empty((B, C), dtype=tdt[wl.in_dtype], device=dev),
                         state_out=torch.empty((3, B, C), dtype=torch.float32, device=dev))
                if args.with_xkv:
                    s["xk"] = torch.empty((B, T, C), dtype=tdt[wl.in_dtype], device=dev)
                    s["xv"] = torch.empty((B, T, C), dtype=tdt[wl.in_dtype], device=dev)
                self.keep.append(s)
                if self.check_out is None and not args.bf16:
                    self.check_out = {"y": s["y"], "state": s["state_out"]}
                self.sets.append([(B, T, C, vp(s["x"].data_ptr()), vp(sh["x_prev"].data_ptr()),
                                   vp(s["x_last"].data_ptr()), vp(sh["mix_k"].data_ptr()),
                                   vp(sh["mix_v"].data_ptr()), vp(sh["mix_r"].data_ptr()),
                                   vp(s["k"].data_ptr()), vp(s["v"].data_ptr()), vp(sh["w"].data_ptr()),
                                   vp(sh["u"].data_ptr()), vp(s["y"].data_ptr()),
                                   vp(s["xk"].data_ptr()) if args.with_xkv else None,
                                   vp(s["xv"].data_ptr()) if args.with_xkv else None, None,
                                   vp(s["state_out"].data_ptr()), hs, ctypes.byref(opts))])
        else:
            self.entry = "rwkv4_wkv_forward"
            self.fn = rw.lib.rwkv4_wkv_forward
            names = ["k", "v"] + (["r"] if wl.gated else [])
            # k, v (and r) read, y written, w and u, the prior state read (if any), state out
            self.launch_bytes = ((len(names) * ei + eo) * E + 8 * C + (12 * B * C if wl.prior else 0)
                                 + 12 * B * C)
            h = {n: dev_act(case[n]).cpu() for n in names}
            sh = {n: dev_t(case[n]) for n in ("w", "u")}
            if wl.prior:
                sh["state_in"] = dev_t(case["state_in"])
            self.keep.append(sh)
            set_bytes = (len(names) * ei + eo) * E
            # one set of >= 1 GiB (four times the 256 MB Infinity Cache) is not cache-resident by
            # itself and is not rotated (the long workload); smaller ones rotate to rotate_gib
            R = 1 if set_bytes >= 2**30 else max(1, math.ceil(args.rotate_gib * 2**30 / set_bytes))
            self.sets = []
            for _ in range(R):
                s = {n: h[n].to(dev) for n in names}
                s["y"] = torch.empty((B, T, C), dtype=tdt[wl.out_dtype], device=dev)
                s["state_out"] = torch.empty((3, B, C), dtype=torch.float32, device=dev)
                o = rw.Opts()
                ctypes.memmove(ctypes.byref(o), ctypes.byref(opts), ctypes.sizeof(o))
                o.r = s["r"].data_ptr() if wl.gated else None
                s["opts"] = o
                self.keep.append(s)
                if self.check_out is None and not args.bf16:
                    self.check_out = {"y": s["y"], "state": s["state_out"]}
                self.sets.append([(B, T, C, vp(sh["w"].data_ptr()), vp(sh["u"].data_ptr()),
                                   vp(s["k"].data_ptr()), vp(s["v"].data_ptr()), vp(s["y"].data_ptr()),
                                   vp(sh["state_in"].data_ptr()) if wl.prior else None,
                                   vp(s["state_out"].data_ptr()), hs, ctypes.byref(o))])
        self.cpu_case = case
        self.cpu_elements = E
        self.cpu_sample = f"the full workload B{B} T{T} C{C}"

    def _setup_mix(self, wl, case, args, torch, rw, np, dev, hs, E):
        """Buffers of the prologue (LayerNorm + token shift) and gate workloads."""
        B, T, C = self.B, self.T, self.C
        vp = ctypes.c_void_p
        f16 = self.act  # the 2-byte activation type (fp16, or bfloat16 under --bf16)

        def dev_t(a):
            t = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
            return t.to(f16) if t.dtype == torch.float16 else t

        if wl.kind == "shift":
            self.entry = "rwkv4_shift_mix"
            self.fn = rw.lib.rwkv4_shift_mix
            # x read, xk, xv, xr written (2 B each), x_prev read and x_last written, LayerNorm
            # weight and bias and three mixes (fp32 per channel)
            self.launch_bytes = 4 * 2 * E + 2 * 2 * B * C + 5 * 4 * C
            hx = dev_t(case["x"]).cpu()
            sh = {n: dev_t(case[n]) for n in ("x_prev", "ln_weight", "ln_bias", "mix_k", "mix_v", "mix_r")}
            self.keep.append(sh)
            R = max(2, math.ceil(args.rotate_gib * 2**30 / (8 * E)))
            self.sets = []
            for _ in range(R):
                s = dict(x=hx.to(dev), **{n: torch.empty((B, T, C), dtype=f16, device=dev) for n in ("xk", "xv", "xr")},
                         x_last=torch.empty((B, C), dtype=f16, device=dev))
                self.keep.append(s)
                self.sets.append([(B, T, C, vp(s["x"].data_ptr()), vp(sh["x_prev"].data_ptr()),
                                   vp(s["x_last"].data_ptr()), vp(sh["ln_weight"].data_ptr()),
                                   vp(sh["ln_bias"].data_ptr()), ctypes.c_float(case["ln_eps"]),
                                   vp(sh["mix_k"].data_ptr()), vp(sh["mix_v"].data_ptr()),
                                   vp(sh["mix_r"].data_ptr()), vp(s["xk"].data_ptr()), vp(s["xv"].data_ptr()),
                                   vp(s["xr"].data_ptr()), self.act_code, hs)])
        else:
            self.entry = "rwkv4_channelmix_gate"
            self.fn = rw.lib.rwkv4_channelmix_gate
            # r, kv, residual read and y written, 2 B each
            self.launch_bytes = 4 * 2 * E
            h = {n: dev_t(case[n]).cpu() for n in ("r", "kv", "residual")}
            R = max(2, math.ceil(args.rotate_gib * 2**30 / (8 * E)))
            self.sets = []
            for _ in range(R):
                s = {n: h[n].to(dev) for n in h}
                s["y"] = torch.empty(E, dtype=f16, device=dev)
                self.keep.append(s)
                self.sets.append([(E, vp(s["r"].data_ptr()), vp(s["kv"].data_ptr()), vp(s["residual"].data_ptr()),
                                   vp(s["y"].data_ptr()), self.act_code, self.act_code, hs)])
        self.cpu_case = case
        self.cpu_elements = E
        self.cpu_sample = f"the full workload B{B} T{T} C{C}"

    def step(self, i, rw):
        for call in self.sets[i % len(self.sets)]:
            st = self.fn(*call)
            if st != 0:
                raise rw.RwkvError(st, rw.rwkv_last_error())


def main():
    args = parse()
    single_gpu_guard(args)
    if args.copy_kernel:
        return copy_kernel(args)

    import numpy as np
    import torch

    import rwkv_wkv_linear_amd as rw
    import wkv_inputs as wi

    torch.cuda.set_device(torch.device("cuda:0"))
    name = args.workload
    su = Setup(name, args, torch, rw, wi, np)
    default_steps = {"timemix14b": 1000, "plain169m": 1000, "gated169m": 500, "decode14b": 100, "long": 50,
                     "lnshift14b": 1000, "cmgate14b": 1000}
    K = args.steps if args.steps is not None else default_steps[name]
    W = args.warmup if args.warmup is not None else max(5, K // 20)

    for i in range(W):
        su.step(i, rw)
    torch.cuda.synchronize()
    step = su.step
    if args.graph:
        if name != "decode14b":
            print("--graph applies to --workload decode14b", file=sys.stderr, flush=True)
            sys.exit(2)
        # the 40 step launches captured once over the same buffers; a replay is one step
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(su.stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph):
                cap = torch.cuda.current_stream().cuda_stream
                for call in su.sets[0]:
                    st = su.fn(*call[:-1], ctypes.c_void_p(cap))
                    if st != 0:
                        raise rw.RwkvError(st, rw.rwkv_last_error())
        su.stream.wait_stream(side)
        torch.cuda.synchronize()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()

        def step(i, rw_):
            graph.replay()

    # The timed region: K steps launched back to back on the stream, bracketed by one pair
    # of HIP events on that stream and by device synchronisations.  A timing event between
    # launches is a marker packet with its own cache maintenance that slows the launch it
    # brackets, so per-launch events would not measure the launches as they run in a layer
    # loop; the pair gives their average duration.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(su.stream)
    for i in range(K):
        step(W + i, rw)
    ev1.record(su.stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_avg_ms = ev0.elapsed_time(ev1) / (K * su.launches_per_step)

    achieved = su.launch_bytes / (launch_avg_ms * 1e-3) / 1e9
    # the committed counters describe the default headline launch only
    default_launch = (name == "timemix14b" and not args.with_xkv and not args.bf16 and not args.chunk_len
                      and args.algo == "auto" and args.publish == "auto")
    traffic = counters_traffic() if default_launch else None
    chunk = args.chunk_len if args.chunk_len else None
    result = {
        "metric": "WKV tokens\u00b7channels/sec and achieved HBM GB/s (% of MI355X peak), "
                  + ("14B shape" if name == "timemix14b" else su.desc),
        "value": su.elements * K / wall,
        "unit": "tokens\u00b7channels/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": wall * 1e3 / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": su.desc, "B": su.B, "T": su.T, "C": su.C, "io_dtype": su.io,
                   "entry_point": su.entry, "launches_per_step": su.launches_per_step,
                   "algo": args.algo, "chunk_len": chunk, "publish": args.publish, "rotated_sets": len(su.sets),
                   "xk_xv_out": bool(args.with_xkv),
                   "hip_graph": bool(args.graph)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic},
        "kernel_avg_us": launch_avg_ms * 1e3,
        "algorithmic_bytes_per_launch": su.launch_bytes,
    }
    if default_launch:
        # the share of the kernel's time the SIMDs spent issuing VALU instructions, from the same
        # committed counter run (null once the kernel source has changed since)
        result["valu_busy"] = counters_traffic("valu_busy_fraction")
    if len(su.sets) > 1 and not args.graph and not args.no_warm:
        # Context only, not the figure above: the same buffer set every launch, so the inputs
        # are served largely from the 256 MB Infinity Cache (warm).
        Kw = min(K, 200)
        su.step(0, rw)
        torch.cuda.synchronize()
        ev0.record(su.stream)
        for i in range(Kw):
            su.step(0, rw)
        ev1.record(su.stream)
        torch.cuda.synchronize()
        warm_ms = ev0.elapsed_time(ev1) / (Kw * su.launches_per_step)
        result["warm_same_buffers"] = {"kernel_avg_us": warm_ms * 1e3,
                                       "achieved_GBps": su.launch_bytes / (warm_ms * 1e-3) / 1e9,
                                       "launches": Kw}
    if args.ceiling:
        result["ceiling"] = ceilings(name, su, args, torch, min(K, 200), W)
        if result["ceiling"]:
            result["ceiling"]["kernel_over_ceiling"] = (launch_avg_ms * 1e3
                                                        / result["ceiling"]["same_pattern"]["kernel_avg_us"])
    result["cpu_baseline"], ref = (None, None) if args.no_cpu_baseline else \
        cpu_baseline(name, su.cpu_case, su.cpu_elements, su.cpu_sample)
    if ref is not None and su.check_out is not None:
        result["parity"] = parity(su, ref)
    if result["cpu_baseline"]:
        # the GPU's throughput over the oracle's on all host threads (context: the oracle is a
        # plain fp64 reference, never tuned)
        result["gpu_over_cpu_baseline"] = result["value"] / result["cpu_baseline"]["value"]
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
