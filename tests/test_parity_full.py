"""GPU parity at the workloads' full sizes, every element compared.

Every workload runs at its real [P,T,H] and k, through the path's four calls
(rows of Bq code bytes, no gap) and through the padded launch that the
benchmark also times (btq_compress_pack_ex / btq_decompress_reduce_ex with
btq_packed_pitch, default stream). Its calibration runs the workload's full
recipe (32 batches of its batch shape; 64 for large prefill), so the moving
average's whole chain at full size is compared with the oracle's.

Checked on every case, over whole tensors:
  * running min/max over all (p,h): equal by value;
  * parameters, outlier set and maps: bitwise;
  * packed rows and BF16 blocks of every token row: bitwise against the
    oracle's message; the padded message: the same codes, zero padding;
  * y of every row: within 1e-3*|y| + 1e-2*max_p scale, BF16 columns
    bit-exact; the bf16-output receiver within that plus half a bf16 ulp,
    its BF16 columns equal to the oracle's rounding, and bit-identical to
    rounding the fp32 receiver's output; the padded message's y to the
    same bar.
The oracle runs over (shard, row-chunk) tiles in a thread pool.
"""
import numpy as np
import pytest
import torch

import bit_tensor_activation_amd as B
from oracle import oracle as O
import workloads as W
from helpers import (assert_bits_equal, assert_selection_equal, assert_stats_equal, assert_y_close,
                     assert_y_bf16_close, assert_y_close_rows, oracle_calib,
                     oracle_compress_rows, oracle_path, say, u16)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

# (workload, inference T, k, calibration batches used here)
CASES = [
    ("7b_prefill", 2048, 64, 32),
    # 32768 row-tiles: two waves per SIMD
    ("7b_prefill", 4096, 64, 32),
    ("decode", 1, 64, 32),
    ("decode", 8, 64, 32),
    ("decode", 32, 64, 32),
    ("decode", 64, 64, 32),
    ("large_prefill", 2048, 128, 64),
    ("large_prefill", 8192, 128, 64),
    ("stress", 16384, 0, 32),
    ("stress", 16384, 32, 32),
    ("stress", 16384, 256, 32),
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
            if b % 16 == 0:
                say(f"  calibration batch {b} of {nb}")
            xb = W.batch(w, W.PHASE_CALIB, b, device=DEV)
            B.btq_calib_update(xb, rmin, rmax, w.momentum, first_batch=(b == 0))
            mn, mx = oracle_calib(u16(xb), mn, mx, w.momentum, first=(b == 0))
            del xb
        torch.cuda.synchronize()
        _calib_cache[key] = (rmin, rmax, mn, mx)
    return _calib_cache[key]


def compare_all(x, pk, ol, y, y16, pkp, olp, yp, sel_o):
    """Every element of both messages and all outputs against the oracle."""
    H = x.shape[2]
    pk_o, ol_o, y_o = oracle_path(u16(x), sel_o)
    Bq = pk_o.shape[2]
    assert_bits_equal(pk, pk_o, "packed")
    assert_bits_equal(ol.view(torch.int16), ol_o.view(np.int16), "outliers")
    assert_bits_equal(pkp[:, :, :Bq], pk_o, "packed (padded rows)")
    assert not bool(pkp[:, :, Bq:].any()), "padding bytes must be zero"
    assert torch.equal(olp, ol)
    assert torch.equal(y16, y.to(torch.bfloat16).view(torch.int16)), "bf16 y is not RNE(fp32 y)"
    assert_y_close_rows(y, y_o, sel_o["scale"], sel_o["idx"])
    assert_y_close_rows(y16, y_o, sel_o["scale"], sel_o["idx"], bf16=True)
    assert_y_close_rows(yp, y_o, sel_o["scale"], sel_o["idx"])
    assert y.shape == (x.shape[1], H)


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
    enc = (sel_g["rscale"], sel_g["zero_point"], sel_g["outlier_idx"], sel_g["cmap"])
    dec = (sel_g["scale"], sel_g["zero_point"], sel_g["fmap"])
    pk, ol = B.btq_compress_pack(x, k, *enc)
    y = B.btq_decompress_reduce(pk, ol, H, *dec)
    y16 = B.btq_decompress_reduce_bf16(pk, ol, H, *dec)
    pkp, olp = B.btq_compress_pack_ex(x, k, *enc, pitch=B.btq_packed_pitch(H, k))
    yp = B.btq_decompress_reduce_ex(pkp, olp, H, *dec)
    torch.cuda.synchronize()
    compare_all(x, pk, ol, y, y16, pkp, olp, yp, sel_o)
    del x, pk, ol, y, y16, pkp, olp, yp
    torch.cuda.empty_cache()


def test_message_beyond_2_gib():
    """A batch whose packed message passes 2^31 bytes (P=8, T=65552, H=8192,
    k=64: 2.15 GB of codes, padded rows). The senders address it through
    per-wave descriptors. The fp32 receiver with one set runs its window
    kernel on groups of 7 and 1 shards (a group's message stays under 2^31
    bytes, the second adding to y); the bf16 output and per-shard sets take
    the general kernel, where every offset is 64-bit. Checked on sampled rows,
    both ends included."""
    from test_parity_per_shard import assert_per_shard_selection_equal, bf16_everywhere
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
    for name, sel_gpu, sel_orc, per in (("shared", sel_g, sel_o, False),
                                        ("per-shard", ps_g, ps_o, True)):
        say(f"  {name} sets")
        pk, ol = B.btq_compress_pack_ex(x, k, sel_gpu["rscale"], sel_gpu["zero_point"],
                                        sel_gpu["outlier_idx"], sel_gpu["cmap"], per_shard=per,
                                        pitch=pitch)
        dec = (sel_gpu["scale"], sel_gpu["zero_point"], sel_gpu["fmap"])
        y = B.btq_decompress_reduce_ex(pk, ol, H, *dec, per_shard=per)
        y16 = None if per else B.btq_decompress_reduce_ex(pk, ol, H, *dec, bf16=True)
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
            # the general kernel's sum is the oracle's: its bf16 output is the
            # rounding of the oracle's y, bit for bit
            ref = torch.from_numpy(np.ascontiguousarray(y_o)).to(torch.bfloat16).view(torch.int16)
            assert torch.equal(y16[ridx].cpu(), ref)
        else:
            assert_y_close(y[ridx].cpu().numpy(), y_o, sel_orc["scale"],
                           bf16_everywhere(sel_orc))
        del pk, ol, y, y16
        torch.cuda.empty_cache()
    del x
    torch.cuda.empty_cache()
