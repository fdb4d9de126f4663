"""Shared helpers for the GPU-vs-oracle parity tests.

Both sides always see one tensor: the inputs are drawn on the GPU by
`workloads`, the HIP path reads them in place, and the oracle reads a host
copy. No oracle input or expected value comes from the HIP path.
"""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from oracle import oracle as O
import workloads as W

# Reduced-output tolerance: |y_gpu - y_oracle| <= 1e-3*|y_oracle| + 1e-2*max_p scale[p,h]
TOL_REL = 1e-3
TOL_ABS_SCALE = 1e-2

POOL = ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def u16(t: torch.Tensor) -> np.ndarray:
    return W.to_u16(t)


def oracle_calib(x: np.ndarray, mn, mx, momentum: float, first: bool):
    """Oracle calibration step, one shard per thread (shards are independent)."""
    P = x.shape[0]

    def one(p):
        return O.calib_update(x[p:p + 1], None if first else mn[p:p + 1],
                              None if first else mx[p:p + 1], momentum, first)

    res = list(POOL.map(one, range(P)))
    return (np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res]))


def oracle_compress_rows(x: np.ndarray, sel: dict, rows=None, pitch=None):
    """Oracle message for token rows `rows` (all if None), shard-parallel."""
    if rows is not None:
        x = x[:, rows, :]
    P = x.shape[0]

    per_shard = np.asarray(sel["cmap"]).ndim == 2

    def one(p):
        idx = sel["idx"][p:p + 1] if per_shard else sel["idx"]
        cmap = sel["cmap"][p:p + 1] if per_shard else sel["cmap"]
        return O.compress_pack(x[p:p + 1], sel["rscale"][p:p + 1], sel["zero_point"][p:p + 1],
                               idx, cmap, pitch=pitch)

    res = list(POOL.map(one, range(P)))
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])


def oracle_path(x: np.ndarray, sel: dict, pitch=None, rows_per_chunk: int = 512):
    """Oracle message (packed, outliers) and fp32 y for every token row.

    The oracle's rows are independent, so the work is split into (shard,
    row-chunk) tiles for the sender and row chunks for the receiver, run in
    the thread pool; each tile is one call of the oracle's own functions.
    """
    P, T, H = x.shape
    per_shard = np.asarray(sel["cmap"]).ndim == 2
    k = np.asarray(sel["idx"]).shape[-1]
    width = (H - k + 1) // 2 if pitch is None else pitch
    packed = np.empty((P, T, width), np.uint8)
    outl = np.empty((P, T, k), np.uint16)
    spans = [(a, min(T, a + rows_per_chunk)) for a in range(0, T, rows_per_chunk)]

    def send(job):
        p, (a, b) = job
        idx = sel["idx"][p:p + 1] if per_shard else sel["idx"]
        cmap = sel["cmap"][p:p + 1] if per_shard else sel["cmap"]
        pk, ol = O.compress_pack(x[p:p + 1, a:b], sel["rscale"][p:p + 1],
                                 sel["zero_point"][p:p + 1], idx, cmap, pitch=pitch)
        packed[p, a:b] = pk[0]
        outl[p, a:b] = ol[0]

    list(POOL.map(send, [(p, s) for p in range(P) for s in spans]))
    y = np.empty((T, H), np.float32)

    def receive(span):
        a, b = span
        y[a:b] = O.decompress_reduce(packed[:, a:b], outl[:, a:b], sel["scale"],
                                     sel["zero_point"], sel["fmap"])

    list(POOL.map(receive, spans))
    return packed, outl, y


def assert_stats_equal(gpu: torch.Tensor, orc: np.ndarray, name: str) -> None:
    g = gpu.cpu().numpy()
    bad = g != orc          # by value: -0 == +0
    assert not bad.any(), f"{name}: {int(bad.sum())} of {bad.size} differ, first at {np.argwhere(bad)[0]}"


def assert_bits_equal(gpu: torch.Tensor, orc: np.ndarray, name: str) -> None:
    g = gpu.cpu().contiguous().numpy()
    o = np.ascontiguousarray(orc)
    assert g.shape == o.shape, f"{name}: shape {g.shape} vs {o.shape}"
    gb = g.view(np.uint8).reshape(-1)
    ob = o.view(np.uint8).reshape(-1)
    if gb.size != ob.size or not np.array_equal(gb, ob):
        first = np.argmax(gb != ob) if gb.size == ob.size else -1
        raise AssertionError(f"{name}: bytes differ (first differing byte {first})")


def assert_selection_equal(sel_gpu: dict, sel_orc: dict) -> None:
    assert_bits_equal(sel_gpu["scale"], sel_orc["scale"], "scale")
    assert_bits_equal(sel_gpu["rscale"], sel_orc["rscale"], "rscale")
    assert_bits_equal(sel_gpu["zero_point"], sel_orc["zero_point"], "zero_point")
    assert_bits_equal(sel_gpu["outlier_idx"], sel_orc["idx"].astype(np.int32), "outlier_idx")
    assert_bits_equal(sel_gpu["fmap"], sel_orc["fmap"].astype(np.int32), "fmap")
    assert_bits_equal(sel_gpu["cmap"], sel_orc["cmap"].astype(np.int32), "cmap")


def assert_y_close_rows(y_gpu: torch.Tensor, y_orc: np.ndarray, scale: np.ndarray, idx,
                        bf16: bool = False, rows_per_chunk: int = 2048) -> None:
    """assert_y_close (or assert_y_bf16_close) over every row of a large y,
    one row chunk at a time so the float64 temporaries stay small."""
    T = y_orc.shape[0]
    for a in range(0, T, rows_per_chunk):
        b = min(T, a + rows_per_chunk)
        g = y_gpu[a:b].cpu().numpy()
        if bf16:
            assert_y_bf16_close(g, y_orc[a:b], scale, idx)
        else:
            assert_y_close(g, y_orc[a:b], scale, idx)


def assert_y_bf16_close(y_gpu_bits: np.ndarray, y_orc: np.ndarray, scale: np.ndarray, idx) -> None:
    """bf16 output: within the fp32 tolerance plus half a bf16 ulp (<= 2^-8 |y|)
    of the oracle's fp32 sum; BF16 columns equal the oracle's rounding exactly."""
    g = (np.asarray(y_gpu_bits).view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    tol = TOL_REL * np.abs(y_orc) + TOL_ABS_SCALE * scale.max(0)[None, :] + \
        np.abs(y_orc.astype(np.float64)) * 2.0 ** -8
    err = np.abs(g.astype(np.float64) - y_orc.astype(np.float64))
    bad = ~(err <= tol)
    assert not bad.any(), (f"y bf16: {int(bad.sum())} outside tolerance; worst excess "
                           f"{float(np.max(err - tol))} at {np.argwhere(bad)[0]}")
    idx = np.asarray(idx, np.int64)
    if idx.size:
        want = O.f32_to_bf16(y_orc[:, idx])
        assert np.array_equal(np.asarray(y_gpu_bits).view(np.uint16)[:, idx], want), \
            "y bf16: BF16 feature columns differ from the oracle's rounding"


def assert_y_close(y_gpu: np.ndarray, y_orc: np.ndarray, scale: np.ndarray, idx) -> None:
    tol = TOL_REL * np.abs(y_orc) + TOL_ABS_SCALE * scale.max(0)[None, :]
    err = np.abs(y_gpu.astype(np.float64) - y_orc.astype(np.float64))
    bad = ~(err <= tol)
    assert not bad.any(), (f"y: {int(bad.sum())} outside tolerance; worst excess "
                           f"{float(np.max(err - tol))} at {np.argwhere(bad)[0]}")
    idx = np.asarray(idx, np.int64)
    if idx.size:   # BF16 features are summed in the oracle's order: exact
        assert np.array_equal(y_gpu[:, idx].view(np.uint32), y_orc[:, idx].view(np.uint32)), \
            "y: BF16 feature columns not bit-exact"
