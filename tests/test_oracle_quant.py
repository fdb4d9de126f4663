"""Pins for the oracle's parameters, 4-bit codes, packing and dequantization.

Page: "Revolutionizing LLM Inference: The Power of Efficient Low-Bit
Communication", section "The Hybrid Quantization Algorithm": Calibration
bullet (per-feature parameters) and Inference bullet (non-selected features
quantized to 4 bits).
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hex32(s):
    return np.uint32(int(s, 16))


def test_qparams_worked_examples():
    g = json.load(open(os.path.join(GOLDEN, "qparams_worked.json")))
    for c in g["cases"]:
        mn = np.array([[float(c["run_min"])]], np.float32)
        mx = np.array([[float(c["run_max"])]], np.float32)
        s, r, z, _ = O.quant_params(mn, mx)
        assert s.view(np.uint32)[0, 0] == _hex32(c["scale"]), c
        assert r.view(np.uint32)[0, 0] == _hex32(c["rscale"]), c
        assert z[0, 0] == c["zero_point"], c


def test_codes_worked_examples():
    g = json.load(open(os.path.join(GOLDEN, "codes_worked.json")))
    for c in g["cases"]:
        x = np.array(c["x"], np.float32)
        q = O.quantize(x, np.float32(c["rscale"]), np.uint8(c["zero_point"]))
        assert q.tolist() == c["q"], c


def _random_ranges(n, seed):
    rng = np.random.default_rng(seed)
    lo = -np.exp(rng.uniform(-12, 12, n)).astype(np.float32) * (rng.random(n) < 0.95)
    hi = np.exp(rng.uniform(-12, 12, n)).astype(np.float32) * (rng.random(n) < 0.95)
    return lo.astype(np.float32), hi.astype(np.float32)


def test_codes_brute_force_all_bf16_against_exact_product():
    # Every finite bf16 x against 1,000 random ranges. A bf16 (8-bit significand)
    # times an fp32 (24-bit) is exact in float64, so rint64(x*r) is the exact
    # round-half-even of the exact product. The fp32 path differs only where
    # its single rounding of x*r moves the value across a half-integer.
    u = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = O.bf16_to_f32(u)
    f = f[np.isfinite(f)]
    lo, hi = _random_ranges(1000, 11)
    s, r, z, _ = O.quant_params(lo[:, None], hi[:, None])
    diffs = 0
    for i in range(0, 1000, 50):
        rr, zz = r[i:i + 50], z[i:i + 50]
        q = O.quantize(f[None, :], rr, zz)
        v = f[None, :].astype(np.float64) * rr.astype(np.float64)
        qe = np.clip(np.rint(v) + zz.astype(np.float64), 0, 15).astype(np.uint8)
        bad = q != qe
        if bad.any():
            frac = np.abs(v[bad] - np.floor(v[bad]) - 0.5)
            mag = np.maximum(np.abs(v[bad]), 1.0)
            assert np.all(frac <= mag * 2.0 ** -23), "mismatch away from a half-integer"
            diffs += int(bad.sum())
    assert diffs < 1e-5 * f.size * 1000


def test_codes_error_bound_in_range():
    # In the calibrated range [lo,hi], |x - (q-z)*s| <= s/2 (plus fp32 slack).
    lo, hi = _random_ranges(300, 12)
    s, r, z, _ = O.quant_params(lo[:, None], hi[:, None])
    rng = np.random.default_rng(3)
    for i in range(300):
        l, h = float(min(lo[i], 0)), float(max(hi[i], 0))
        x = rng.uniform(l, h, 4000).astype(np.float32)
        q = O.quantize(x, r[i, 0], z[i, 0])
        d = O.dequantize(q, s[i, 0], z[i, 0]).astype(np.float64)
        err = np.abs(x.astype(np.float64) - d)
        assert np.all(err <= 0.5 * float(s[i, 0]) * (1 + 1e-5)), i


def test_codes_outside_range_clamp_to_grid_ends():
    lo, hi = np.float32(-2.0), np.float32(6.0)
    s, r, z, _ = O.quant_params(np.array([[lo]]), np.array([[hi]]))
    x = np.array([-1e30, -5.0, -2.6, 6.6, 9.0, 3e38], np.float32)
    q = O.quantize(x, r[0, 0], z[0, 0])
    assert q.tolist() == [0, 0, 0, 15, 15, 15]


def test_dequant_matches_torch_fake_quantize_per_channel():
    # Library routine: torch.fake_quantize_per_channel_affine computes
    # (clamp(rint(x * (1/s)) + z, 0, 15) - z) * s per channel.
    x = W.to_u16(W.draw(1, 512, 96, 9, base="laplace", cols=[3, 50], outlier_factor=40.0))[0]
    f = O.bf16_to_f32(x)
    mn = f.min(0) * np.float32(0.6)
    mx = f.max(0) * np.float32(0.6)        # 0.6: force some clipping
    s, r, z, _ = O.quant_params(mn[None], mx[None])
    q = O.quantize(f, r[0], z[0])
    ours = O.dequantize(q, s[0], z[0])
    ref = torch.fake_quantize_per_channel_affine(
        torch.from_numpy(f), torch.from_numpy(s[0]), torch.from_numpy(z[0].astype(np.int32)),
        1, 0, 15).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    assert ((q == 0) | (q == 15)).mean() > 0.01


def test_pack_worked_and_round_trip():
    g = json.load(open(os.path.join(GOLDEN, "message_worked.json")))
    for c in g["pack"]:
        b = O.pack_nibbles(np.array(c["q"], np.uint8))
        assert b.tolist() == c["bytes"]
        assert O.unpack_nibbles(b, len(c["q"])).tolist() == c["q"]
    rng = np.random.default_rng(4)
    for n in (1, 2, 7, 8, 31, 64, 255):
        q = rng.integers(0, 16, (3, 5, n)).astype(np.uint8)
        b = O.pack_nibbles(q)
        assert b.shape == (3, 5, (n + 1) // 2)
        assert np.array_equal(O.unpack_nibbles(b, n), q)
        if n % 2:
            assert np.all(b[..., -1] >> 4 == 0)


def test_compress_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "message_worked.json")))["compress"]
    x = np.array([[[int(v, 16) for v in row] for row in sh] for sh in g["x"]], np.uint16)
    packed, outl = O.compress_pack(x, np.array(g["rscale"], np.float32),
                                   np.array(g["zero_point"], np.uint8),
                                   np.array(g["idx"]), np.array(g["cmap"]))
    assert packed.tolist() == g["packed"]
    assert outl.tolist() == [[[int(v, 16) for v in row] for row in sh] for sh in g["outliers"]]


def test_compress_outlier_block_is_column_copy():
    x = W.to_u16(W.draw(3, 4, 20, 8))
    idx = np.array([2, 5, 19])
    cmap = np.setdiff1d(np.arange(20), idx)
    r = np.ones((3, 20), np.float32)
    z = np.full((3, 20), 8, np.uint8)
    _, outl = O.compress_pack(x, r, z, idx, cmap)
    for p in range(3):
        for t in range(4):
            for i, h in enumerate(idx):
                assert outl[p, t, i] == x[p, t, h]


def test_pitch_pads_rows_with_zeros_and_receiver_ignores_them():
    # The row pitch is layout only: the code bytes are unchanged, the extra
    # bytes are zero, and the reduced output is the same for any pitch.
    x = W.to_u16(W.draw(2, 3, 24, 11))
    idx = np.array([4, 17])
    cmap = np.setdiff1d(np.arange(24), idx)
    rng = np.random.default_rng(12)
    r = (rng.random((2, 24)) + 0.5).astype(np.float32)
    z = rng.integers(0, 16, (2, 24)).astype(np.uint8)
    s = (np.float32(1) / r).astype(np.float32)
    fmap = np.empty(24, np.int64)
    fmap[cmap] = np.arange(cmap.size)
    fmap[idx] = -1 - np.arange(idx.size)
    base, outl = O.compress_pack(x, r, z, idx, cmap)
    assert base.shape == (2, 3, 11)
    y0 = O.decompress_reduce(base, outl, s, z, fmap)
    for pitch in (11, 12, 16, 128):
        pk, ol = O.compress_pack(x, r, z, idx, cmap, pitch=pitch)
        assert pk.shape == (2, 3, pitch)
        assert np.array_equal(pk[..., :11], base) and not pk[..., 11:].any()
        assert np.array_equal(ol, outl)
        y = O.decompress_reduce(pk, ol, s, z, fmap)
        assert np.array_equal(y.view(np.uint32), y0.view(np.uint32))
    with pytest.raises(ValueError):
        O.compress_pack(x, r, z, idx, cmap, pitch=10)
