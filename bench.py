#!/usr/bin/env python3
"""Throughput of the hybrid int4/BF16 partial-sum codec on one MI355X.

One step = one pass of the per-batch hot path over one inference batch:
btq_compress_pack (every shard's sender message) and then
btq_decompress_reduce (the receiver's fused dequantize and fp32 sum over
P shards). Calibration and selection run once before the timed region, as
the method prescribes: they are computed offline on calibration batches.
They are timed separately and reported under "offline".

Metric: bf16-equivalent GB/s = steps * P*T*H*2 bytes / wall time of the
timed steps, launched back to back with nothing between them. Inputs are
resident in HBM before timing starts. R copies of the batch and of every
output rotate, so that each step streams from HBM and not from the 256 MB
last-level cache. The receiver reads the message written two steps earlier.
The same steps captured in a HIP graph (one rotation, replayed) are timed too
and reported under "timing" (graph_ms_per_step); value stays the eager rate.

Roofline: the dominant kernel (compress) is HBM-bound. achieved = its
algorithmic bytes per launch / its mean duration. The durations come from
the same steps run a second time, with HIP events recorded on the launch
stream around every launch (events without the system-scope fence, so
recording them flushes no cache; they still add a few microseconds per
step, which is why the throughput is taken from the first run). traffic =
HBM bytes per launch from rocprofv3 counters (profiles/), reported only
while the kernel source still matches the hash those counters were taken
at.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 7b_prefill]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, published
METRIC = "GB/s (bf16-equiv) of compress+decompress_reduce; % of HBM peak"
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["bit_tensor_activation_amd/csrc/compress.hip",
                  "bit_tensor_activation_amd/csrc/common.hpp"]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(paths) -> str:
    """Hash of the kernel code: comments and blank lines are left out, so
    that only a change to the code itself invalidates a counter summary."""
    import re
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = [line.rstrip() for line in text.splitlines() if line.strip()]
        h.update("\n".join(code).encode())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per compress launch from the committed counter summary."""
    path = os.path.join(PROFILES, f"compress_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            a, b = line.split("=", 1)
            kv[a.strip()] = b.strip()
    if kv.get("source_hash") != source_hash(KERNEL_SOURCES):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class HipEvents:
    """Timing events of the HIP runtime that torch has loaded (one runtime per
    process: libbtq links the same soname).

    They are created with hipEventDisableSystemFence: recording them does
    not write back and invalidate the caches, so a kernel bracketed by two
    of them runs as it would without them. Every elapsed time is read only
    after a device synchronization.
    """
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        self.c = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pool = []

    def new(self):
        e = self.c.c_void_p()
        if self.hip.hipEventCreateWithFlags(self.c.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.pool.append(e)
        return e

    def record(self, e, stream: int) -> None:
        if self.hip.hipEventRecord(e, self.c.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b) -> float:
        t = self.c.c_float()
        if self.hip.hipEventElapsedTime(self.c.byref(t), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return t.value

    def close(self) -> None:
        for e in self.pool:
            self.hip.hipEventDestroy(e)
        self.pool = []


def _csv_rows(d: str, suffix: str):
    import csv
    import glob
    for f in sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)):
        with open(f) as fh:
            yield from csv.DictReader(fh)


def _kernel_class(name: str):
    head = name.split("(")[0].rstrip()
    if "btq::" in name and "decompress_sets" in name:
        return "decompress_reduce_per_shard"
    if "btq::" in name and "compress" in name and "decompress" not in name and \
            head.endswith("true>"):
        return "compress_pack_per_shard"   # the sender's per-shard template flag
    if "btq::" in name and "decompress" in name:
        # the receiver's template flag selects bf16 output
        bf16 = name.split("(")[0].rstrip().endswith("true>")
        return "decompress_reduce_bf16" if bf16 else "decompress_reduce"
    if "btq::" in name and "compress" in name:
        return "compress_pack"
    if "copyBuffer" in name:
        return "copy"
    return None


def summarize_counters(fetch_dir: str, write_dir: str, workload: str, copy_mib: int,
                       note: str) -> str:
    """Traffic summary from two rocprofv3 --pmc runs of this script.

    The runs count FETCH_SIZE and then WRITE_SIZE (KiB per dispatch) over
    `python bench.py ... --copy-probe-mib N`. The last 5 copy dispatches are
    that probe's plain device copies of N MiB: their readings give the scale
    of each counter. The compress and decompress readings are medians over
    the timed dispatches, divided by that scale.
    """
    import statistics
    import workloads as W
    med, copies = {}, {}
    for d, ctr in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        per = {}
        for r in _csv_rows(d, "counter_collection.csv"):
            if r["Counter_Name"] != ctr:
                continue
            c = _kernel_class(r["Kernel_Name"])
            if c:
                per.setdefault(c, []).append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
        for c, v in per.items():
            v.sort()
            if c == "copy":
                copies[ctr] = [x for _, x in v[-5:]]
            else:
                med[(c, ctr)] = statistics.median(x for _, x in v)
    kib = copy_mib * 1024.0
    fscale = statistics.median(copies["FETCH_SIZE"]) / kib
    wscale = statistics.median(copies["WRITE_SIZE"]) / kib
    w = W.WORKLOADS[workload]
    comp_alg, deco_alg = algorithmic_bytes(w.P, w.T[0], w.H, w.k)
    deco16_alg = algorithmic_bytes(w.P, w.T[0], w.H, w.k, y_bytes=2)[1]
    comp_ps_alg, deco_ps_alg = algorithmic_bytes_per_shard(w.P, w.T[0], w.H, w.k)
    lines = [f"# HBM traffic per launch, workload {workload} (P={w.P}, T={w.T[0]}, H={w.H}, k={w.k})",
             "# " + note.replace("\n", "\n# "),
             f"source_hash={source_hash(KERNEL_SOURCES)}",
             f"workload={workload}",
             f"copy_probe_bytes={copy_mib * 2 ** 20}",
             f"copy_fetch_kib={statistics.median(copies['FETCH_SIZE']):.1f}",
             f"copy_write_kib={statistics.median(copies['WRITE_SIZE']):.1f}",
             f"fetch_scale={fscale:.4f}",
             f"write_scale={wscale:.4f}"]
    for name, alg in (("compress_pack", comp_alg), ("decompress_reduce", deco_alg),
                      ("decompress_reduce_bf16", deco16_alg),
                      ("compress_pack_per_shard", comp_ps_alg),
                      ("decompress_reduce_per_shard", deco_ps_alg)):
        if (name, "FETCH_SIZE") not in med or (name, "WRITE_SIZE") not in med:
            continue
        f_kib, w_kib = med[(name, "FETCH_SIZE")], med[(name, "WRITE_SIZE")]
        traffic = f_kib / fscale * 1024 + w_kib / wscale * 1024
        tag = "" if name == "compress_pack" else name + "_"
        lines += [f"{name}_fetch_kib_median={f_kib:.1f}",
                  f"{name}_write_kib_median={w_kib:.1f}",
                  f"{tag}traffic_bytes_per_launch={traffic:.0f}",
                  f"{name}_algorithmic_bytes={alg}",
                  f"{name}_traffic_over_algorithmic={traffic / alg:.4f}"]
    return "\n".join(lines) + "\n"


SQ_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY",
               "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM", "SQ_INSTS_VALU")


def summarize_sq(sq_dir: str, note: str, n_simd: int = 1024, mhz: float = 2400.0) -> str:
    """Where the waves of each libbtq kernel spend their time, from one
    rocprofv3 --pmc run with the SQ_COUNTERS (medians over dispatches).

    SQ_WAVE_CYCLES and the SQ_ACTIVE_INST_* / SQ_WAIT_* counters count in
    units of 4 cycles, summed over waves; one VALU instruction of a wave64
    occupies its SIMD for 4 cycles. valu_us_per_simd = SQ_INSTS_VALU * 4
    cycles / SIMDs / clock: the time each SIMD spends issuing VALU work.
    """
    import statistics
    per = {}
    for r in _csv_rows(sq_dir, "counter_collection.csv"):
        name = r["Kernel_Name"].split("(")[0].replace("void ", "").strip()
        if "btq::" not in name:
            continue
        per.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    lines = ["# " + note.replace("\n", "\n# "),
             "# kernel | wait_inst_any | wait_any | valu_active | lds_active | vmem_active "
             "(fractions of wave time) | VALU instructions | valu_us_per_simd"]
    for name, cs in per.items():
        med = {c: statistics.median(v) for c, v in cs.items()}
        wc = med.get("SQ_WAVE_CYCLES", 0.0) or 1.0
        valu_us = med.get("SQ_INSTS_VALU", 0.0) * 4.0 / n_simd / mhz
        lines.append(f"{name} | {med.get('SQ_WAIT_INST_ANY', 0) / wc:.2f} | "
                     f"{med.get('SQ_WAIT_ANY', 0) / wc:.2f} | "
                     f"{med.get('SQ_ACTIVE_INST_VALU', 0) / wc:.2f} | "
                     f"{med.get('SQ_ACTIVE_INST_LDS', 0) / wc:.2f} | "
                     f"{med.get('SQ_ACTIVE_INST_VMEM', 0) / wc:.2f} | "
                     f"{med.get('SQ_INSTS_VALU', 0):.3g} | {valu_us:.1f}")
    return "\n".join(lines) + "\n"


def summarize_trace(trace_dir: str, note: str) -> str:
    """The libbtq rows of a rocprofv3 --kernel-trace --stats run."""
    lines = ["# " + note.replace("\n", "\n# "),
             "# kernel | calls | average ns | min ns | max ns | share of GPU time %"]
    for r in _csv_rows(trace_dir, "kernel_stats.csv"):
        if "btq::" in r["Name"]:
            name = r["Name"].split("(")[0].replace("void ", "")
            lines.append(f"{name} | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | "
                         f"{r['MaxNs']} | {float(r['Percentage']):.2f}")
    return "\n".join(lines) + "\n"


def algorithmic_bytes(P, T, H, k, y_bytes=4):
    """Bytes the method must move per launch (inputs once, outputs once);
    y_bytes is 4 for the fp32 receiver, 2 for the bf16 one."""
    Bq = (H - k + 1) // 2
    Hq = H - k
    maps = 4 * H                             # cmap and outlier_idx
    message = P * T * (Bq + 2 * k)
    compress = P * T * H * 2 + message + P * Hq * 8 + maps           # + (rscale, zero point) table
    decompress = message + T * H * y_bytes + (P + 1) * Hq * 4 + maps  # + scale rows, constant row
    return compress, decompress


def algorithmic_bytes_per_shard(P, T, H, k):
    """The same for per-shard BF16 sets: per-shard maps; the receiver reads
    scale, zero point and fmap by feature (9 bytes per (p,h))."""
    Bq = (H - k + 1) // 2
    message = P * T * (Bq + 2 * k)
    compress = P * T * H * 2 + message + P * (H - k) * 8 + 4 * P * H
    decompress = message + T * H * 4 + 9 * P * H
    return compress, decompress


def cpu_baseline(w, T_sample: int, min_seconds: float):
    """The oracle, as it is, on a bounded sample of the same workload."""
    import numpy as np
    import workloads as W
    from oracle import oracle as O
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(1)
    except Exception:   # numpy's elementwise ops are single-threaded anyway
        limiter = None
    x = W.to_u16(W.batch(w, W.PHASE_INFER, 0, T=T_sample, device="cpu"))
    mn, mx = O.batch_min_max(x)
    sel = O.select_outliers(mn, mx, w.k)
    reps, t0 = 0, time.perf_counter()
    while True:
        pk, ol = O.compress_pack(x, sel["rscale"], sel["zero_point"], sel["idx"], sel["cmap"])
        O.decompress_reduce(pk, ol, sel["scale"], sel["zero_point"], sel["fmap"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    if limiter is not None:
        limiter.unregister()
    gbps = reps * x.nbytes / el / 1e9
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": (f"{w.name}: P={w.P} x T={T_sample} of {w.T[0]} tokens x H={w.H}, k={w.k}; "
                       f"numpy oracle compress_pack + decompress_reduce, {reps} reps in "
                       f"{el:.1f} s, one thread; parameters from the sample's own min/max")}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="7b_prefill")
    ap.add_argument("--T", type=int, default=None, help="token count (decode sweep)")
    ap.add_argument("--k", type=int, default=None, help="BF16 feature count (stress sweep)")
    ap.add_argument("--rotate-mib", type=int, default=1024,
                    help="minimum MiB streamed between reuses of one buffer set")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-sample-T", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=256,
                    help="size of the plain device copy timed for the copy roofline (and the "
                         "counter scale); 0 skips it")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the traffic summary of two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="print the libbtq rows of a rocprofv3 --stats run and exit")
    ap.add_argument("--summarize-sq", metavar="SQ_DIR",
                    help="print the wave-time breakdown of a rocprofv3 --pmc run of the SQ "
                         "counters and exit")
    ap.add_argument("--note", default="", help="header text for the summaries")
    args = ap.parse_args()
    if args.summarize_counters:
        print(summarize_counters(*args.summarize_counters, args.workload, args.copy_probe_mib,
                                 args.note), end="")
        return 0
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.note), end="")
        return 0
    if args.summarize_sq:
        print(summarize_sq(args.summarize_sq, args.note), end="")
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the P shards of one tensor-parallel group share one GPU's HBM). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import bit_tensor_activation_amd as B
    from bit_tensor_activation_amd import _lib
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    w = W.WORKLOADS[args.workload]
    T = args.T if args.T is not None else w.T[0]
    k = args.k if args.k is not None else w.k
    P, H = w.P, w.H
    lib = _lib.load()
    stream = torch.cuda.current_stream(dev)
    sh = int(stream.cuda_stream)
    hev = HipEvents()

    # ---- offline: calibration over the calibration set, then selection ----
    log(f"workload {w.name}: P={P} T={T} H={H} k={k}; calibrating on {w.calib_batches} batches")
    rmin = torch.empty((P, H), dtype=torch.float32, device=dev)
    rmax = torch.empty_like(rmin)
    ws = torch.empty(max(B.btq_calib_workspace_bytes(P, w.calib_T, H), 1), dtype=torch.uint8,
                     device=dev)
    calib_ms = 0.0
    for b in range(w.calib_batches):
        xb = W.batch(w, W.PHASE_CALIB, b, device=dev)
        e0, e1 = hev.new(), hev.new()
        hev.record(e0, sh)
        B.btq_calib_update(xb, rmin, rmax, w.momentum, b == 0, workspace=ws)
        hev.record(e1, sh)
        torch.cuda.synchronize()
        calib_ms += hev.ms(e0, e1)
        del xb
    e0, e1 = hev.new(), hev.new()
    B.btq_select_outliers(rmin, rmax, k)     # warm
    hev.record(e0, sh)
    sel = B.btq_select_outliers(rmin, rmax, k)
    hev.record(e1, sh)
    torch.cuda.synchronize()
    select_ms = hev.ms(e0, e1)

    # ---- resident inputs and rotated buffer sets ----
    x0 = W.batch(w, W.PHASE_INFER, 0, T=T, device=dev)
    pitch = B.btq_packed_pitch(H, k)
    set_bytes = P * T * H * 2 + P * T * (pitch + 2 * k) + T * H * 4
    R = max(3, -(-args.rotate_mib * 2 ** 20 // set_bytes) + 1)
    xs = [x0.clone() for _ in range(R)]
    pks = [torch.empty((P, T, pitch), dtype=torch.uint8, device=dev) for _ in range(R)]
    ols = [torch.empty((P, T, k), dtype=torch.int16, device=dev) for _ in range(R)]
    ys = [torch.empty((T, H), dtype=torch.float32, device=dev) for _ in range(R)]
    del x0
    p = lambda t: t.data_ptr() if t.numel() else None
    enc, dec, oi, cm = p(sel["enc"]), p(sel["dec"]), p(sel["outlier_idx"]), p(sel["cmap"])
    comp_args = [(p(xs[r]), P, T, H, k, enc, oi, cm, p(pks[r]), pitch, p(ols[r]), sh)
                 for r in range(R)]
    deco_args = [(p(pks[(r - 2) % R]), pitch, p(ols[(r - 2) % R]), P, T, H, k, dec, oi, cm,
                  p(ys[r]), sh) for r in range(R)]
    compress, decompress = lib.btq_compress_pack, lib.btq_decompress_reduce
    # first fill every message buffer once, so the receiver always reads a real message
    for r in range(R):
        _lib.check(compress(*comp_args[r]), "btq_compress_pack")
    torch.cuda.synchronize()
    log(f"{R} rotating buffer sets of {set_bytes / 2**20:.1f} MiB; warmup {args.warmup}, "
        f"steps {args.steps}")

    def step(i, ev=None):
        r = i % R
        if ev is not None:
            hev.record(ev[0], sh)
        st = compress(*comp_args[r])
        if ev is not None:
            hev.record(ev[1], sh)
        st |= decompress(*deco_args[r])
        if ev is not None:
            hev.record(ev[2], sh)
        return st

    st = 0
    for i in range(args.warmup):
        st |= step(i)
    torch.cuda.synchronize()
    _lib.check(st, "warmup")
    # Timed region 1: the steps as a caller runs them, with no instrumentation
    # between the launches (value, ms_per_step).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        st |= step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    _lib.check(st, "timed steps")
    # Timed region 2: the same steps again with a HIP event around every
    # launch, on the launch stream (each kernel's duration). The events cost
    # a few microseconds per step, so region 1 alone gives the throughput.
    evs = [[hev.new() for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(args.steps):
        st |= step(i, evs[i])
    torch.cuda.synchronize()
    wall_ev = time.perf_counter() - t1
    _lib.check(st, "instrumented steps")
    comp_ms = [hev.ms(e[0], e[1]) for e in evs]
    deco_ms = [hev.ms(e[1], e[2]) for e in evs]
    comp_mean = sum(comp_ms) / len(comp_ms)
    deco_mean = sum(deco_ms) / len(deco_ms)
    med = lambda v: sorted(v)[len(v) // 2]

    # Timed region 3 (reported beside value, not value): G steps of the
    # rotation (all R, at most 512, which still spans well past the last-level
    # cache) captured in a HIP graph on a side stream (default priority) and
    # replayed, as a caller that captures its steps would run them. The
    # kernels clear nothing with memset, so the graph holds kernel nodes only.
    G = min(R, 512)
    gs = torch.cuda.Stream(device=dev)
    g_comp = [a[:-1] + (gs.cuda_stream,) for a in comp_args[:G]]
    g_deco = [a[:-1] + (gs.cuda_stream,) for a in deco_args[:G]]
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=gs):
        for r in range(G):
            st |= compress(*g_comp[r])
            st |= decompress(*g_deco[r])
    _lib.check(st, "graph capture")
    graph.replay()
    torch.cuda.synchronize()
    n_rep = max(1, args.steps // G)
    t2 = time.perf_counter()
    for _ in range(n_rep):
        graph.replay()
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t2) / (n_rep * G) * 1e3
    del graph

    # The bf16-output receiver, timed on its own after the steps (it is not
    # part of a step: the step's receiver writes fp32).
    y16 = [torch.empty((T, H), dtype=torch.int16, device=dev) for _ in range(2)]
    d16_args = [(a[0], a[1], a[2], P, T, H, k, dec, oi, cm, p(y16[r % 2]), sh)
                for r, a in enumerate(deco_args)]
    n16 = max(20, min(args.steps, 200))
    for i in range(5):
        st |= lib.btq_decompress_reduce_bf16(*d16_args[i % R])
    e16 = [(hev.new(), hev.new()) for _ in range(n16)]
    torch.cuda.synchronize()
    for i in range(n16):
        hev.record(e16[i][0], sh)
        st |= lib.btq_decompress_reduce_bf16(*d16_args[i % R])
        hev.record(e16[i][1], sh)
    torch.cuda.synchronize()
    _lib.check(st, "bf16-output receiver")
    d16_mean = sum(hev.ms(a, b) for a, b in e16) / n16
    d16_bytes = algorithmic_bytes(P, T, H, k, y_bytes=2)[1]
    del y16

    # Per-shard BF16 sets (every shard keeps its own k features), timed on
    # their own in the same rotation: another selection reading, not part of
    # a step.
    def time_calls(fn, args_list, n, what):
        for i in range(5):
            _lib.check(fn(*args_list[i % len(args_list)]), what)
        ev = [(hev.new(), hev.new()) for _ in range(n)]
        torch.cuda.synchronize()
        s_ = 0
        for i in range(n):
            hev.record(ev[i][0], sh)
            s_ |= fn(*args_list[i % len(args_list)])
            hev.record(ev[i][1], sh)
        torch.cuda.synchronize()
        _lib.check(s_, what)
        return sum(hev.ms(a, b) for a, b in ev) / n

    sps = B.btq_select_outliers_per_shard(rmin, rmax, k)
    cps_args = [(p(xs[r]), P, T, H, k, p(sps["enc"]), p(sps["outlier_idx"]), p(sps["cmap"]),
                 p(pks[r]), pitch, p(ols[r]), sh) for r in range(R)]
    dps_args = [(p(pks[(r - 2) % R]), pitch, p(ols[(r - 2) % R]), P, T, H, k, p(sps["scale"]),
                 p(sps["zero_point"]), p(sps["fmap"]), p(ys[r]), sh) for r in range(R)]
    for r in range(R):
        _lib.check(lib.btq_compress_pack_per_shard(*cps_args[r]), "per-shard sender")
    cps_mean = time_calls(lib.btq_compress_pack_per_shard, cps_args, n16, "per-shard sender")
    dps_mean = time_calls(lib.btq_decompress_reduce_per_shard, dps_args, n16,
                          "per-shard receiver")
    cps_bytes, dps_bytes = algorithmic_bytes_per_shard(P, T, H, k)

    copy_probe = None
    if args.copy_probe_mib:
        n = args.copy_probe_mib * 2 ** 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)   # warm-up
        torch.cuda.synchronize()
        c0, c1 = hev.new(), hev.new()
        hev.record(c0, sh)
        for _ in range(5):
            dst.copy_(src)
        hev.record(c1, sh)
        torch.cuda.synchronize()
        copy_probe = {"bytes_per_copy": 2 * n, "GBps": round(5 * 2 * n / (hev.ms(c0, c1) * 1e-3) / 1e9, 1)}
        del src, dst

    bf16_bytes = P * T * H * 2
    comp_bytes, deco_bytes = algorithmic_bytes(P, T, H, k)
    value = args.steps * bf16_bytes / wall / 1e9
    achieved = comp_bytes / (comp_mean * 1e-3) / 1e9
    traffic = read_traffic(w.name) if (T == w.T[0] and k == w.k) else None
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "P": P, "T": T, "H": H, "k": k,
                   "input": "bf16 partial sums", "message": "int4 packed + bf16 outlier block",
                   "output": "fp32", "rotating_sets": R},
        "roofline": {"bound": "hbm", "kernel": "compress_pack", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes": comp_bytes},
        "kernels": {
            "compress_pack": {"mean_us": round(comp_mean * 1e3, 2), "median_us": round(med(comp_ms) * 1e3, 2),
                              "algorithmic_bytes": comp_bytes,
                              "hbm_GBps": round(comp_bytes / (comp_mean * 1e-3) / 1e9, 1),
                              "bf16_equiv_GBps": round(bf16_bytes / (comp_mean * 1e-3) / 1e9, 1)},
            "decompress_reduce": {"mean_us": round(deco_mean * 1e3, 2), "median_us": round(med(deco_ms) * 1e3, 2),
                                  "algorithmic_bytes": deco_bytes,
                                  "hbm_GBps": round(deco_bytes / (deco_mean * 1e-3) / 1e9, 1),
                                  "frac": round(deco_bytes / (deco_mean * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                                  "bf16_equiv_GBps": round(bf16_bytes / (deco_mean * 1e-3) / 1e9, 1)},
            "kernel_sum_bf16_equiv_GBps": round(bf16_bytes / ((comp_mean + deco_mean) * 1e-3) / 1e9, 1),
            "decompress_reduce_bf16": {"mean_us": round(d16_mean * 1e3, 2), "algorithmic_bytes": d16_bytes,
                                       "hbm_GBps": round(d16_bytes / (d16_mean * 1e-3) / 1e9, 1),
                                       "frac": round(d16_bytes / (d16_mean * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                                       "note": "bf16 output (one rounding of the fp32 sum); "
                                               "timed separately, not part of value"},
            "compress_pack_per_shard": {
                "mean_us": round(cps_mean * 1e3, 2), "algorithmic_bytes": cps_bytes,
                "hbm_GBps": round(cps_bytes / (cps_mean * 1e-3) / 1e9, 1),
                "frac": round(cps_bytes / (cps_mean * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "note": "one BF16 set per shard; timed separately, not part of value"},
            "decompress_reduce_per_shard": {
                "mean_us": round(dps_mean * 1e3, 2), "algorithmic_bytes": dps_bytes,
                "hbm_GBps": round(dps_bytes / (dps_mean * 1e-3) / 1e9, 1),
                "frac": round(dps_bytes / (dps_mean * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "note": "one BF16 set per shard; timed separately, not part of value"},
        },
        "timing": {"value": f"{args.steps} steps with no instrumentation between launches",
                   "kernels": f"the same {args.steps} steps again with HIP events around every "
                              "launch on the launch stream (fence-free events)",
                   "ms_per_step_instrumented": round(wall_ev / args.steps * 1e3, 5),
                   "graph": f"{min(R, 512)} steps of the rotation captured in a HIP graph, "
                            f"replayed {max(1, args.steps // min(R, 512))} times",
                   "graph_ms_per_step": round(graph_ms, 5),
                   "graph_GBps": round(bf16_bytes / (graph_ms * 1e-3) / 1e9, 2)},
        "offline": {"calib_batches": w.calib_batches, "calib_ms_total": round(calib_ms, 3),
                    "calib_GBps": round(w.calib_batches * P * w.calib_T * H * 2 / (calib_ms * 1e-3) / 1e9, 1),
                    "select_us": round(select_ms * 1e3, 2)},
    }
    if copy_probe:
        out["copy_probe"] = copy_probe
        # the same kernel against what a plain device copy (read + write)
        # reaches on this GPU
        out["roofline"]["copy_GBps"] = copy_probe["GBps"]
        out["roofline"]["frac_of_copy"] = round(achieved / copy_probe["GBps"], 4)
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle for >= {args.cpu_seconds:.0f} s")
        out["cpu_baseline"] = cpu_baseline(w, min(args.cpu_sample_T, T), args.cpu_seconds)
    hev.close()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
