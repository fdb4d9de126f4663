#!/usr/bin/env python3
"""Throughput of the hybrid int4/BF16 partial-sum codec on one MI355X.

One step = one pass of the per-batch hot path over one inference batch: the
sender (every shard's message) and then the receiver (the fused dequantize
and fp32 sum over P shards). Calibration and selection run once before the
timed region, as the method prescribes: they are computed offline on
calibration batches. They are timed separately and reported under "offline".

Two message layouts are timed, each as a caller runs it:
  * padded: btq_compress_pack_ex / btq_decompress_reduce_ex with rows at
    btq_packed_pitch (the code bytes rounded up to 128, so every row starts
    on a cache line) -- this gives `value`;
  * dense: the path's own calls btq_compress_pack / btq_decompress_reduce,
    rows of exactly the code bytes.

Metric: bf16-equivalent GB/s = steps * P*T*H*2 bytes / wall time of the
timed steps, launched back to back with nothing between them. Inputs are
resident in HBM before timing starts. R copies of the batch and of every
output rotate, so that each step streams from HBM and not from the 256 MB
last-level cache. The receiver reads the message written two steps earlier.
The same steps captured in a HIP graph (one rotation, replayed) are timed too
and reported under "timing" (graph_ms_per_step); value stays the eager rate.

Roofline: the dominant kernel (the sender) is HBM-bound. achieved = its
algorithmic bytes per launch / its mean duration. The algorithmic bytes are
what the method must move: the bf16 input, the message, and the per-feature
parameters and maps (5 bytes per (shard, feature) and 4 per feature). The
durations come from the same steps run a second time, with HIP events
recorded on the launch stream around every launch (events without the
system-scope fence, so recording them flushes no cache; they still add a few
microseconds per step, which is why the throughput is taken from the first
run). traffic = HBM bytes per launch from rocprofv3 counters (profiles/),
reported only while the kernel source still matches the hash those counters
were taken at.

CPU baseline: the oracle as it stands, on a bounded sample of the same
workload, on one core and on a pool of worker processes (one row chunk of
every shard per task), each with its core count. It runs before the GPU is
touched, so the pool's workers fork from a process with no GPU state.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload stress] [--k 32]
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


def traffic_path(workload: str, k: int) -> str:
    return os.path.join(PROFILES, f"compress_{workload}_k{k}_traffic.txt")


def read_traffic(workload: str, k: int):
    """HBM bytes per sender launch (padded layout) from the committed counter
    summary, while the kernel code still matches the hash it was taken at."""
    path = traffic_path(workload, k)
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


def _template_args(name: str):
    head = name.split("(")[0]
    return [t.strip() for t in head[head.index("<") + 1:head.rindex(">")].split(",")] \
        if "<" in head else []


def _kernel_class(name: str):
    """The benchmark's name for a kernel of a rocprofv3 record, or None."""
    if "btq::" in name and "dq_window_kernel" in name:
        # template <NP, kOR, kR, kPs, kBf>
        t = _template_args(name)
        per, bf = t[3] == "true", t[4] == "true"
        return ("decompress_reduce_per_shard" if per else
                "decompress_reduce_bf16" if bf else "decompress_reduce")
    if "btq::" in name and "compress" in name and "decompress" not in name:
        # the sender's last template flag: one set per shard
        per = _template_args(name)[-1:] == ["true"]
        return "compress_pack_per_shard" if per else "compress_pack"
    if "copyBuffer" in name:
        return "copy"
    return None


def summarize_counters(fetch_dir: str, write_dir: str, workload: str, k, copy_mib: int,
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
    k = w.k if k is None else k
    comp_alg, deco_alg = algorithmic_bytes(w.P, w.T[0], w.H, k)
    deco16_alg = algorithmic_bytes(w.P, w.T[0], w.H, k, y_bytes=2)[1]
    comp_ps_alg, deco_ps_alg = algorithmic_bytes_per_shard(w.P, w.T[0], w.H, k)
    lines = [f"# HBM traffic per launch, workload {workload} (P={w.P}, T={w.T[0]}, H={w.H}, k={k})",
             "# " + note.replace("\n", "\n# "),
             f"source_hash={source_hash(KERNEL_SOURCES)}",
             f"workload={workload}",
             f"k={k}",
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


def _quantile(sorted_x, q):
    """Linear-interpolation quantile of an ascending list."""
    if not sorted_x:
        return float("nan")
    pos = q * (len(sorted_x) - 1)
    lo = int(pos)
    hi = min(lo + 1, len(sorted_x) - 1)
    return sorted_x[lo] + (sorted_x[hi] - sorted_x[lo]) * (pos - lo)


def trace_durations(trace_dir: str) -> dict:
    """{kernel: [durations in ns]} of the libbtq dispatches in a rocprofv3
    --kernel-trace run (End_Timestamp - Start_Timestamp per dispatch)."""
    out = {}
    for r in _csv_rows(trace_dir, "kernel_trace.csv"):
        name = r.get("Kernel_Name", "")
        if "btq::" in name and r.get("Start_Timestamp") and r.get("End_Timestamp"):
            key = name.split("(")[0].replace("void ", "")
            out.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return out


def summarize_trace(trace_dir: str, note: str) -> str:
    """The libbtq rows of a rocprofv3 --kernel-trace --stats run: the stats
    file's calls, average, min and max, and the median, p10 and p90 of the
    per-dispatch durations in the trace file."""
    durs = trace_durations(trace_dir)
    lines = ["# " + note.replace("\n", "\n# "),
             "# kernel | calls | average ns | median ns | p10 ns | p90 ns | min ns | max ns | "
             "share of GPU time %"]
    for r in _csv_rows(trace_dir, "kernel_stats.csv"):
        if "btq::" in r["Name"]:
            name = r["Name"].split("(")[0].replace("void ", "")
            d = sorted(durs.get(name, []))
            qs = " | ".join(f"{_quantile(d, q):.0f}" if d else "-" for q in (0.5, 0.1, 0.9))
            lines.append(f"{name} | {r['Calls']} | {float(r['AverageNs']):.0f} | {qs} | "
                         f"{r['MinNs']} | {r['MaxNs']} | {float(r['Percentage']):.2f}")
    return "\n".join(lines) + "\n"


# Steps shorter than this (wall time, no instrumentation) are timed behind a
# head start (gpu_head_start).
SHORT_STEP_S = 60e-6


def gpu_head_start(torch, n_ops: int) -> None:
    """Queues a bounded spin kernel (torch's) on the current stream, long
    enough for the host to enqueue about n_ops launches and event records
    (about 25 us each at 2.4 GHz, at most 2000 of them) before the GPU reaches
    them. Events around each launch then time the GPU's work: without it a
    kernel shorter than the host's enqueue time waits for its own launch
    after its start event has been stamped."""
    torch.cuda._sleep(int(min(n_ops, 2000) * 60000))


def algorithmic_bytes(P, T, H, k, y_bytes=4):
    """Bytes the method must move per launch, inputs once and outputs once:
    sender  P*T*H*2 (bf16 input) + P*T*(Bq + 2k) (message) + 5*P*H (rscale
            and zero point per (shard, feature)) + 4*H (cmap and outlier_idx);
    receiver P*T*(Bq + 2k) + T*H*y_bytes (4: fp32 y, 2: bf16 y) + 5*P*H
            (scale and zero point) + 4*H (fmap).
    The padded layout's zero bytes past each row's codes are not counted."""
    Bq = (H - k + 1) // 2
    message = P * T * (Bq + 2 * k)
    params = 5 * P * H + 4 * H
    return P * T * H * 2 + message + params, message + T * H * y_bytes + params


def algorithmic_bytes_per_shard(P, T, H, k):
    """The same for one BF16 set per shard: the maps are per shard
    (4*P*H bytes in place of 4*H)."""
    Bq = (H - k + 1) // 2
    message = P * T * (Bq + 2 * k)
    params = 5 * P * H + 4 * P * H
    return P * T * H * 2 + message + params, message + T * H * 4 + params


def cpu_cores() -> int:
    """Host cores for the oracle pool: this process's CPUs, at most 16 (the
    host share of one GPU)."""
    return max(1, min(len(os.sched_getaffinity(0)), 16))


# The pool's task state: set in the parent before the workers fork.
_POOL_STATE = {}


def _oracle_rows(span):
    """Sender then receiver of the oracle on token rows [a, b) of every shard
    (rows are independent)."""
    from oracle import oracle as O
    x, sel = _POOL_STATE["x"], _POOL_STATE["sel"]
    a, b = span
    pk, ol = O.compress_pack(x[:, a:b], sel["rscale"], sel["zero_point"], sel["idx"], sel["cmap"])
    y = O.decompress_reduce(pk, ol, sel["scale"], sel["zero_point"], sel["fmap"])
    return int(pk.nbytes + y.nbytes)


def _limit_threads():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:   # numpy's elementwise ops are single-threaded anyway
        pass


def cpu_baseline(w, k: int, T: int, T_sample: int, min_seconds: float):
    """The oracle, as it is, on a bounded sample of the same workload: one
    core, then a pool of worker processes over row chunks of every shard."""
    import multiprocessing as mp
    import workloads as W
    from oracle import oracle as O
    _limit_threads()
    cores = cpu_cores()
    rows_pool = min(T, T_sample * cores)
    x = W.to_u16(W.batch(w, W.PHASE_INFER, 0, T=rows_pool, device="cpu"))
    mn, mx = O.batch_min_max(x)
    sel = O.select_outliers(mn, mx, k)
    _POOL_STATE.update(x=x, sel=sel)
    bytes_per_row = w.P * w.H * 2
    # one core: T_sample rows per call, repeated for >= min_seconds
    reps, t0 = 0, time.perf_counter()
    while True:
        _oracle_rows((0, min(T_sample, rows_pool)))
        reps += 1
        el1 = time.perf_counter() - t0
        if el1 >= min_seconds:
            break
    one = reps * min(T_sample, rows_pool) * bytes_per_row / el1 / 1e9
    # a pool: every task is a chunk of 32 rows of all shards
    chunk = 32
    spans = [(a, min(rows_pool, a + chunk)) for a in range(0, rows_pool, chunk)]
    ctx = mp.get_context("fork")
    with ctx.Pool(cores, initializer=_limit_threads) as pool:
        pool.map(_oracle_rows, spans[:cores])   # workers up
        passes, t0 = 0, time.perf_counter()
        while True:
            pool.map(_oracle_rows, spans, chunksize=1)
            passes += 1
            elp = time.perf_counter() - t0
            if elp >= min_seconds:
                break
    pooled = passes * rows_pool * bytes_per_row / elp / 1e9
    _POOL_STATE.clear()
    return {"value": round(pooled, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "value_1core": round(one, 4), "cores_1core": 1,
            "sample": (f"{w.name}: P={w.P} x H={w.H}, k={k}, bf16-equiv rate of the numpy oracle's "
                       f"compress_pack + decompress_reduce; one core: {reps} calls on "
                       f"{min(T_sample, rows_pool)} of {T} tokens in {el1:.1f} s; "
                       f"{cores} worker processes: {passes} passes over {rows_pool} tokens in "
                       f"{len(spans)} tasks of {chunk} rows of every shard, {elp:.1f} s; "
                       "parameters from the sample's own min/max")}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="stress")
    ap.add_argument("--T", type=int, default=None, help="token count (decode sweep)")
    ap.add_argument("--k", type=int, default=None,
                    help="BF16 feature count (default: the workload's first, 32 for stress)")
    ap.add_argument("--layouts", default="padded,dense",
                    help="message layouts to time, the first gives value: padded (rows at "
                         "btq_packed_pitch, the *_ex calls) and/or dense (rows of the code "
                         "bytes, the path's own calls)")
    ap.add_argument("--rotate-mib", type=int, default=1024,
                    help="minimum MiB streamed between reuses of one buffer set")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--cpu-sample-T", type=int, default=128,
                    help="token rows of the one-core sample (the pool takes this many per core)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the steps (no bf16 receiver, per-shard sets or graph)")
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
        print(summarize_counters(*args.summarize_counters, args.workload, args.k,
                                 args.copy_probe_mib, args.note), end="")
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
    layouts = [l.strip() for l in args.layouts.split(",") if l.strip()]
    if not layouts or any(l not in ("padded", "dense") for l in layouts):
        print("--layouts takes padded and/or dense", file=sys.stderr)
        return 2

    import workloads as W
    w = W.WORKLOADS[args.workload]
    T = args.T if args.T is not None else w.T[0]
    k = args.k if args.k is not None else w.k
    P, H = w.P, w.H

    # ---- the CPU baseline first: its worker processes fork before any GPU use
    cpu = None
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle for >= {args.cpu_seconds:.0f} s on one core and on a pool")
        cpu = cpu_baseline(w, k, T, min(args.cpu_sample_T, T), args.cpu_seconds)

    import torch
    import bit_tensor_activation_amd as B
    from bit_tensor_activation_amd import _lib

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
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
    Bq = B.btq_packed_row_bytes(H, k)
    pitches = {"padded": B.btq_packed_pitch(H, k), "dense": Bq}
    wmax = max(pitches[l] for l in layouts)
    set_bytes = P * T * H * 2 + P * T * (wmax + 2 * k) + T * H * 4
    R = max(3, -(-args.rotate_mib * 2 ** 20 // set_bytes) + 1)
    xs = [x0.clone() for _ in range(R)]
    msg = [torch.empty(P * T * wmax, dtype=torch.uint8, device=dev) for _ in range(R)]
    ols = [torch.empty((P, T, k), dtype=torch.int16, device=dev) for _ in range(R)]
    ys = [torch.empty((T, H), dtype=torch.float32, device=dev) for _ in range(R)]
    del x0
    p = lambda t: t.data_ptr() if t.numel() else None
    rs, sc, zp = p(sel["rscale"]), p(sel["scale"]), p(sel["zero_point"])
    oi, cm, fm = p(sel["outlier_idx"]), p(sel["cmap"]), p(sel["fmap"])
    SHARED, F32 = _lib.BTQ_SETS_SHARED, _lib.BTQ_Y_F32

    def calls(layout):
        """(sender, receiver, their argument tuples per buffer set)."""
        pitch = pitches[layout]
        if layout == "padded":
            comp = [(p(xs[r]), P, T, H, k, rs, zp, oi, cm, SHARED, p(msg[r]), pitch, p(ols[r]), sh)
                    for r in range(R)]
            deco = [(p(msg[(r - 2) % R]), pitch, p(ols[(r - 2) % R]), P, T, H, k, sc, zp, fm,
                     SHARED, p(ys[r]), F32, sh) for r in range(R)]
            return lib.btq_compress_pack_ex, lib.btq_decompress_reduce_ex, comp, deco
        comp = [(p(xs[r]), P, T, H, k, rs, zp, oi, cm, p(msg[r]), p(ols[r]), sh) for r in range(R)]
        deco = [(p(msg[(r - 2) % R]), p(ols[(r - 2) % R]), P, T, H, k, sc, zp, fm, p(ys[r]), sh)
                for r in range(R)]
        return lib.btq_compress_pack, lib.btq_decompress_reduce, comp, deco

    log(f"{R} rotating buffer sets of {set_bytes / 2**20:.1f} MiB; layouts {layouts}; "
        f"warmup {args.warmup}, steps {args.steps}")
    bf16_bytes = P * T * H * 2
    comp_bytes, deco_bytes = algorithmic_bytes(P, T, H, k)
    med = lambda v: sorted(v)[len(v) // 2]
    results = {}
    for layout in layouts:
        compress, decompress, comp_args, deco_args = calls(layout)
        # first fill every message buffer once, so the receiver always reads a real message
        for r in range(R):
            _lib.check(compress(*comp_args[r]), "sender")
        torch.cuda.synchronize()

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
        # Steps shorter than the host's enqueue time (decode) give the GPU a
        # head start, so that the events time its work and not the rate at
        # which the host enqueues launches. Longer steps keep the host ahead
        # by themselves, and there the spin's idle time measurably slows the
        # kernels that follow it (2-4% at large prefill and stress).
        short_steps = wall / args.steps < SHORT_STEP_S
        evs = [[hev.new() for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        if short_steps:
            gpu_head_start(torch, 5 * args.steps)
        for i in range(args.steps):
            st |= step(i, evs[i])
        torch.cuda.synchronize()
        wall_ev = hev.ms(evs[0][0], evs[-1][2]) * 1e-3
        _lib.check(st, "instrumented steps")
        comp_ms = [hev.ms(e[0], e[1]) for e in evs]
        deco_ms = [hev.ms(e[1], e[2]) for e in evs]
        results[layout] = dict(wall=wall, wall_ev=wall_ev, comp_ms=comp_ms, deco_ms=deco_ms,
                               short_steps=short_steps,
                               calls=(compress, decompress, comp_args, deco_args))
        log(f"{layout}: {wall / args.steps * 1e6:.1f} us per step, sender "
            f"{sum(comp_ms) / len(comp_ms) * 1e3:.1f} us, receiver "
            f"{sum(deco_ms) / len(deco_ms) * 1e3:.1f} us")

    def kernel_entry(ms_list, nbytes):
        mean = sum(ms_list) / len(ms_list)
        srt = sorted(ms_list)
        return {"mean_us": round(mean * 1e3, 2), "median_us": round(med(ms_list) * 1e3, 2),
                "p10_us": round(_quantile(srt, 0.1) * 1e3, 2),
                "p90_us": round(_quantile(srt, 0.9) * 1e3, 2),
                "algorithmic_bytes": nbytes, "hbm_GBps": round(nbytes / (mean * 1e-3) / 1e9, 1),
                "frac": round(nbytes / (mean * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "bf16_equiv_GBps": round(bf16_bytes / (mean * 1e-3) / 1e9, 1)}

    head = results[layouts[0]]
    comp_mean = sum(head["comp_ms"]) / len(head["comp_ms"])
    value = args.steps * bf16_bytes / head["wall"] / 1e9
    achieved = comp_bytes / (comp_mean * 1e-3) / 1e9
    kernels = {}
    for layout in layouts:
        r = results[layout]
        tag = "" if layout == layouts[0] else f"_{layout}"
        kernels["compress_pack" + tag] = kernel_entry(r["comp_ms"], comp_bytes)
        kernels["decompress_reduce" + tag] = kernel_entry(r["deco_ms"], deco_bytes)
        kernels["compress_pack" + tag]["layout"] = layout
        kernels["decompress_reduce" + tag]["layout"] = layout
    layout_rates = {l: {"ms_per_step": round(results[l]["wall"] / args.steps * 1e3, 5),
                        "GBps": round(args.steps * bf16_bytes / results[l]["wall"] / 1e9, 2),
                        "pitch": pitches[l]} for l in layouts}

    def time_calls(fn, args_list, n, what):
        for i in range(5):
            _lib.check(fn(*args_list[i % len(args_list)]), what)
        ev = [(hev.new(), hev.new()) for _ in range(n)]
        torch.cuda.synchronize()
        if head["short_steps"]:
            gpu_head_start(torch, 3 * n)
        s_ = 0
        for i in range(n):
            hev.record(ev[i][0], sh)
            s_ |= fn(*args_list[i % len(args_list)])
            hev.record(ev[i][1], sh)
        torch.cuda.synchronize()
        _lib.check(s_, what)
        return [hev.ms(a, b) for a, b in ev]

    graph_ms = None
    if not args.no_extras:
        compress, decompress, comp_args, deco_args = head["calls"]
        # Timed region 3 (reported beside value, not value): G steps of the
        # rotation captured in a HIP graph on a side stream (default priority)
        # and replayed. The kernels clear nothing with memset, so the graph holds
        # kernel nodes only.
        G = min(R, 512)
        gs = torch.cuda.Stream(device=dev)
        g_comp = [a[:-1] + (gs.cuda_stream,) for a in comp_args[:G]]
        g_deco = [a[:-1] + (gs.cuda_stream,) for a in deco_args[:G]]
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        st = 0
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

        n16 = max(20, min(args.steps, 200))
        pitch = pitches[layouts[0]]
        msg_of = lambda r: p(msg[(r - 2) % R])
        # The bf16-output receiver (not part of a step: the step's receiver
        # writes fp32), on the headline layout.
        y16 = [torch.empty((T, H), dtype=torch.int16, device=dev) for _ in range(2)]
        d16_args = [(msg_of(r), pitch, p(ols[(r - 2) % R]), P, T, H, k, sc, zp, fm, SHARED,
                     p(y16[r % 2]), _lib.BTQ_Y_BF16, sh) for r in range(R)]
        d16 = time_calls(lib.btq_decompress_reduce_ex, d16_args, n16, "bf16-output receiver")
        kernels["decompress_reduce_bf16"] = kernel_entry(
            d16, algorithmic_bytes(P, T, H, k, y_bytes=2)[1])
        kernels["decompress_reduce_bf16"]["note"] = ("bf16 output (one rounding of the fp32 sum); "
                                                     "timed separately, not part of value")
        del y16
        # Per-shard BF16 sets (every shard keeps its own k features), in the
        # same rotation: another selection reading, not part of a step.
        sps = B.btq_select_outliers_per_shard(rmin, rmax, k)
        PER = _lib.BTQ_SETS_PER_SHARD
        cps_args = [(p(xs[r]), P, T, H, k, p(sps["rscale"]), p(sps["zero_point"]),
                     p(sps["outlier_idx"]), p(sps["cmap"]), PER, p(msg[r]), pitch, p(ols[r]), sh)
                    for r in range(R)]
        dps_args = [(msg_of(r), pitch, p(ols[(r - 2) % R]), P, T, H, k, p(sps["scale"]),
                     p(sps["zero_point"]), p(sps["fmap"]), PER, p(ys[r]), F32, sh)
                    for r in range(R)]
        for r in range(R):
            _lib.check(lib.btq_compress_pack_ex(*cps_args[r]), "per-shard sender")
        cps_bytes, dps_bytes = algorithmic_bytes_per_shard(P, T, H, k)
        kernels["compress_pack_per_shard"] = kernel_entry(
            time_calls(lib.btq_compress_pack_ex, cps_args, n16, "per-shard sender"), cps_bytes)
        kernels["decompress_reduce_per_shard"] = kernel_entry(
            time_calls(lib.btq_decompress_reduce_ex, dps_args, n16, "per-shard receiver"),
            dps_bytes)
        for key in ("compress_pack_per_shard", "decompress_reduce_per_shard"):
            kernels[key]["note"] = "one BF16 set per shard; timed separately, not part of value"

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
        copy_probe = {"bytes_per_copy": 2 * n,
                      "GBps": round(5 * 2 * n / (hev.ms(c0, c1) * 1e-3) / 1e9, 1)}
        del src, dst

    traffic = read_traffic(w.name, k) if (T == w.T[0] and layouts[0] == "padded") else None
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["wall"] / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "P": P, "T": T, "H": H, "k": k,
                   "input": "bf16 partial sums", "message": "int4 packed + bf16 outlier block",
                   "layout": layouts[0], "packed_pitch": pitches[layouts[0]],
                   "output": "fp32", "rotating_sets": R},
        "roofline": {"bound": "hbm", "kernel": "compress_pack", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes": comp_bytes},
        "layouts": layout_rates,
        "kernels": kernels,
        "timing": {"value": f"{args.steps} steps with no instrumentation between launches",
                   "kernels": f"the same {args.steps} steps again with HIP events around every "
                              "launch on the launch stream (fence-free events); steps shorter "
                              "than 60 us are queued behind a spin kernel, so that the events "
                              "time the GPU and not the host's enqueue rate",
                   "ms_per_step_instrumented": round(head["wall_ev"] / args.steps * 1e3, 5)},
        "offline": {"calib_batches": w.calib_batches, "calib_ms_total": round(calib_ms, 3),
                    "calib_GBps": round(w.calib_batches * P * w.calib_T * H * 2 / (calib_ms * 1e-3) / 1e9, 1),
                    "select_us": round(select_ms * 1e3, 2)},
    }
    if graph_ms is not None:
        out["timing"]["graph"] = (f"{min(R, 512)} steps of the rotation captured in a HIP graph, "
                                  f"replayed {max(1, args.steps // min(R, 512))} times")
        out["timing"]["graph_ms_per_step"] = round(graph_ms, 5)
        out["timing"]["graph_GBps"] = round(bf16_bytes / (graph_ms * 1e-3) / 1e9, 2)
    if copy_probe:
        out["copy_probe"] = copy_probe
        # the same kernel against what a plain device copy (read + write)
        # reaches on this GPU
        out["roofline"]["copy_GBps"] = copy_probe["GBps"]
        out["roofline"]["frac_of_copy"] = round(achieved / copy_probe["GBps"], 4)
    if cpu is not None:
        out["cpu_baseline"] = cpu
    hev.close()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
