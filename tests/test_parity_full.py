"""GPU parity at the workloads' full sizes, through the same calls and
launch configuration that the benchmark times (default stream, default
packed pitch).

Every workload runs at its real [P,T,H] and k. Its calibration uses the
workload's batch shape, but fewer batches than the full recipe, so that the
oracle's exact statistics over all of H stay cheap. The kernels' launch
shape depends on (P,T,H) only, not on the number of batches.

Checked on every case:
  * running min/max over all (p,h): equal by value;
  * parameters, outlier set, maps and codec tables: bitwise;
  * packed rows and BF16 blocks of sampled token rows: bitwise against the
    oracle's message for those rows (the rows include both ends, the
    benchmark's row-block boundaries and random rows);
  * y on the same rows: within 1e-3*|y| + 1e-2*max_p scale, BF16 columns
    bit-exact; the bf16-output receiver within that plus half a bf16 ulp,
    its BF16 columns equal to the oracle's rounding, and over the whole
    tensor bit-identical to rounding the fp32 receiver's output;
  * properties over the whole tensors: every padding byte of the packed
    rows is zero and y is finite.
"""
import numpy as np
import pytest
import torch

import bit_tensor_activation_amd as B
from oracle import oracle as O
import workloads as W
from helpers import (assert_bits_equal, assert_selection_equal, assert_stats_equal, assert_y_close,
                     assert_y_bf16_close, oracle_calib, oracle_compress_rows, say, u16)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

# (workload, inference T, k, calibration batches used here)
CASES = [
    ("7b_prefill", 2048, 64, 4),
    # 32768 row-tiles: the bf16-output receiver takes about 2048 waves here
    ("7b_prefill", 4096, 64, 4),
    ("large_prefill", 2048, 128, 3),
    ("decode", 1, 64, 3),
    ("decode", 8, 64, 3),
    ("decode", 32, 64, 3),
    ("decode", 64, 64, 3),
    ("large_prefill", 8192, 128, 3),
    ("stress", 16384, 0, 2),
    ("stress", 16384, 32, 2),
    ("stress", 16384, 256, 2),
]

_calib_cache = {}


def calibrated(name: str, nb: int):
    """GPU and oracle running stats after `nb` calibration batches (cached)."""
    key = (name, nb)
    if key not in _calib_cache:
        _calib_cache.clear()
        w = W.WORKLOADS[name]
        rmin = torch.empty((w.P, w.H), dtype=torch.float32, device=DEV)
        rmax = torch.empty_like(rmin)
        mn = mx = None
        for b in range(nb):
            xb = W.batch(w, W.PHASE_CALIB, b, device=DEV)
            B.btq_calib_update(xb, rmin, rmax, w.momentum, first_batch=(b == 0))
            mn, mx = oracle_calib(u16(xb), mn, mx, w.momentum, first=(b == 0))
            del xb
        torch.cuda.synchronize()
        _calib_cache[key] = (rmin, rmax, mn, mx)
    return _calib_cache[key]


def sample_rows(T: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 7, 8, 15, 16, 31, 32, 63, 64, T // 2, T - 2, T - 1]
    rows = set(r for r in fixed if 0 <= r < T)
    rows |= set(rng.integers(0, T, size=min(T, 24)).tolist())
    return np.array(sorted(rows), np.int64)


@pytest.mark.parametrize("name,T,k,nb", CASES, ids=[f"{c[0]}-T{c[1]}-k{c[2]}" for c in CASES])
def test_full_size(name, T, k, nb):
    w = W.WORKLOADS[name]
    P, H = w.P, w.H
    say(f"case: {name} P={P} T={T} H={H} k={k} ({nb} calibration batches)")
    rmin, rmax, mn, mx = calibrated(name, nb)
    assert_stats_equal(rmin, mn, "run_min")
    assert_stats_equal(rmax, mx, "run_max")

    sel_g = B.btq_select_outliers(rmin, rmax, k)
    sel_o = O.select_outliers(mn, mx, k)
    torch.cuda.synchronize()
    assert_selection_equal(sel_g, sel_o)

    b = w.T.index(T) if T in w.T else 0
    x = W.batch(w, W.PHASE_INFER, b, T=T, device=DEV)
    pk, ol = B.btq_compress_pack(x, k, sel_g["enc"], sel_g["outlier_idx"], sel_g["cmap"])
    y = B.btq_decompress_reduce(pk, ol, H, sel_g["dec"], sel_g["outlier_idx"], sel_g["cmap"])
    y16 = B.btq_decompress_reduce_bf16(pk, ol, H, sel_g["dec"], sel_g["outlier_idx"],
                                       sel_g["cmap"])
    torch.cuda.synchronize()
    assert torch.equal(y16, y.to(torch.bfloat16).view(torch.int16)), "bf16 y is not RNE(fp32 y)"
    pitch = pk.shape[2]
    assert pitch == B.btq_packed_pitch(H, k)
    Bq = B.btq_packed_row_bytes(H, k)

    # whole-tensor properties
    assert not bool(pk[:, :, Bq:].any()), "packed padding bytes must be zero"
    assert bool(torch.isfinite(y).all()), "y must be finite"

    rows = sample_rows(T, seed=T * 131 + k)
    xs = u16(x[:, torch.as_tensor(rows, device=DEV), :])
    pk_o, ol_o = oracle_compress_rows(xs, sel_o, pitch=pitch)
    ridx = torch.as_tensor(rows, device=DEV)
    assert_bits_equal(pk[:, ridx, :], pk_o, "packed (sampled rows)")
    assert_bits_equal(ol[:, ridx, :].view(torch.int16), ol_o.view(np.int16),
                      "outliers (sampled rows)")
    y_o = O.decompress_reduce(pk_o, ol_o, sel_o["scale"], sel_o["zero_point"], sel_o["fmap"])
    assert_y_close(y[ridx].cpu().numpy(), y_o, sel_o["scale"], sel_o["idx"])
    assert_y_bf16_close(y16[ridx].cpu().numpy(), y_o, sel_o["scale"], sel_o["idx"])
    del x, pk, ol, y, y16
    torch.cuda.empty_cache()


def test_message_beyond_2_gib():
    """A batch whose packed message passes 2^31 bytes (P=8, T=65552, H=8192,
    k=64: 2.15 GB of codes). The receivers take their general kernels there
    (the fast ones address a whole message with one 32-bit descriptor), and
    every offset is 64-bit. Checked on sampled rows, both ends included, for
    the shared path (fp32 and bf16 output) and for per-shard sets."""
    from test_parity_per_shard import assert_per_shard_selection_equal
    P, H, k, T = 8, 8192, 64, 65552
    pitch = B.btq_packed_pitch(H, k)
    assert P * T * pitch >= 2 ** 31
    say(f"case: message beyond 2 GiB, P={P} T={T} H={H} k={k} pitch={pitch}")
    cols = list(range(17, H, 199))
    calib = [W.draw(P, 256, H, 8000 + b, sigma=0.5, cols=cols, outlier_factor=50.0, device=DEV)
             for b in range(2)]
    rmin = torch.empty((P, H), dtype=torch.float32, device=DEV)
    rmax = torch.empty_like(rmin)
    mn = mx = None
    for b, xb in enumerate(calib):
        B.btq_calib_update(xb, rmin, rmax, 0.9, first_batch=(b == 0))
        mn, mx = oracle_calib(u16(xb), mn, mx, 0.9, first=(b == 0))
    del calib
    sel_g = B.btq_select_outliers(rmin, rmax, k)
    sel_o = O.select_outliers(mn, mx, k)
    ps_g = B.btq_select_outliers_per_shard(rmin, rmax, k)
    ps_o = O.select_outliers_per_shard(mn, mx, k)
    torch.cuda.synchronize()
    assert_selection_equal(sel_g, sel_o)
    assert_per_shard_selection_equal(ps_g, ps_o)

    x = W.draw(P, T, H, 8100, sigma=0.5, cols=cols, outlier_factor=50.0, device=DEV)
    rows = np.array(sorted({0, 1, 63, 64, 32767, 32768, T // 2, T - 17, T - 2, T - 1} |
                           set(np.random.default_rng(5).integers(0, T, 16).tolist())))
    ridx = torch.as_tensor(rows, device=DEV)
    xs = u16(x[:, ridx, :])
    for name, sel_gpu, sel_orc, comp, deco in (
            ("shared", sel_g, sel_o, B.btq_compress_pack, None),
            ("per-shard", ps_g, ps_o, B.btq_compress_pack_per_shard, None)):
        say(f"  {name} sets")
        pk, ol = comp(x, k, sel_gpu["enc"], sel_gpu["outlier_idx"], sel_gpu["cmap"])
        if name == "shared":
            y = B.btq_decompress_reduce(pk, ol, H, sel_gpu["dec"], sel_gpu["outlier_idx"],
                                        sel_gpu["cmap"])
            y16 = B.btq_decompress_reduce_bf16(pk, ol, H, sel_gpu["dec"],
                                               sel_gpu["outlier_idx"], sel_gpu["cmap"])
        else:
            y = B.btq_decompress_reduce_per_shard(pk, ol, H, sel_gpu["scale"],
                                                  sel_gpu["zero_point"], sel_gpu["fmap"])
            y16 = None
        torch.cuda.synchronize()
        pk_o, ol_o = oracle_compress_rows(xs, sel_orc, pitch=pitch)
        assert_bits_equal(pk[:, ridx, :], pk_o, f"packed ({name}, sampled rows)")
        assert_bits_equal(ol[:, ridx, :].view(torch.int16), ol_o.view(np.int16),
                          f"outliers ({name}, sampled rows)")
        y_o = O.decompress_reduce(pk_o, ol_o, sel_orc["scale"], sel_orc["zero_point"],
                                  sel_orc["fmap"])
        if name == "shared":
            assert_y_close(y[ridx].cpu().numpy(), y_o, sel_orc["scale"], sel_orc["idx"])
            assert_y_bf16_close(y16[ridx].cpu().numpy(), y_o, sel_orc["scale"], sel_orc["idx"])
            assert torch.equal(y16[ridx], y[ridx].to(torch.bfloat16).view(torch.int16))
        else:
            assert_bits_equal(y[ridx], y_o, "y (per-shard, sampled rows)")
        del pk, ol, y, y16
        torch.cuda.empty_cache()
    del x
    torch.cuda.empty_cache()
