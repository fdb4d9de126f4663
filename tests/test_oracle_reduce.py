"""Pins for the oracle's receiver side: convert back and sum over shards.

Page: "Revolutionizing LLM Inference: The Power of Efficient Low-Bit
Communication": section "The Hybrid Quantization Algorithm", Inference bullet
(after communication everything is converted back and summed across
devices), and section "Combating Quantization Errors with Tensor
Parallelism" (partial sums are quantized before the sum, so the summed error
is Irwin-Hall-like and clusters around 0).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pipeline(x, k, mn=None, mx=None):
    if mn is None:
        mn, mx = O.batch_min_max(x)
    sel = O.select_outliers(mn, mx, k)
    packed, outl = O.compress_pack(x, sel["rscale"], sel["zero_point"], sel["idx"], sel["cmap"])
    y = O.decompress_reduce(packed, outl, sel["scale"], sel["zero_point"], sel["fmap"])
    return sel, packed, outl, y


def test_decompress_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "message_worked.json")))["decompress"]
    outl = np.array([[[int(v, 16) for v in row] for row in sh] for sh in g["outliers"]], np.uint16)
    y = O.decompress_reduce(np.array(g["packed"], np.uint8), outl,
                            np.array(g["scale"], np.float32),
                            np.array(g["zero_point"], np.uint8), np.array(g["fmap"]))
    assert y.tolist() == g["y"]


def test_all_bf16_sum_of_integers_is_exact():
    # k = H: nothing is quantized. With integer-valued inputs every partial sum
    # is exact in fp32, so y equals the exact integer sum over shards.
    rng = np.random.default_rng(8)
    v = rng.integers(-120, 121, (8, 6, 40)).astype(np.float32)
    x = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    _, _, _, y = _pipeline(x, 40)
    assert np.array_equal(y, v.astype(np.int64).sum(0).astype(np.float32))


def test_bf16_columns_two_shards_round_once():
    x = W.to_u16(W.draw(2, 50, 30, 21, cols=[1, 7], outlier_factor=1000.0))
    sel, _, _, y = _pipeline(x, 30)
    f = O.bf16_to_f32(x).astype(np.float64)
    assert np.array_equal(y, (f[0] + f[1]).astype(np.float32))


def test_bf16_columns_many_shards_error_bound():
    x = W.to_u16(W.draw(8, 40, 24, 22, base="laplace"))
    _, _, _, y = _pipeline(x, 24)
    f = O.bf16_to_f32(x).astype(np.float64)
    exact = np.array([[math.fsum(f[:, t, h]) for h in range(24)] for t in range(40)])
    bound = 7 * 2.0 ** -24 * np.abs(f).sum(0)
    assert np.all(np.abs(y - exact) <= bound)


def test_single_shard_is_fake_quantize():
    # P = 1: y is the dequantized int4 value (torch's fake-quantize, a library
    # routine) on int4 features, and the exact bf16 value on BF16 features.
    x = W.to_u16(W.draw(1, 64, 50, 23, cols=[4, 9, 33], outlier_factor=60.0))
    mn, mx = O.batch_min_max(x)
    mn, mx = mn * np.float32(0.8), mx * np.float32(0.8)
    sel, _, _, y = _pipeline(x, 3, mn, mx)
    f = O.bf16_to_f32(x)[0]
    ref = torch.fake_quantize_per_channel_affine(
        torch.from_numpy(f), torch.from_numpy(sel["scale"][0]),
        torch.from_numpy(sel["zero_point"][0].astype(np.int32)), 1, 0, 15).numpy()
    c, i = sel["cmap"], sel["idx"]
    assert sorted(i.tolist()) == [4, 9, 33]
    assert np.array_equal(y[:, c].view(np.uint32), ref[:, c].view(np.uint32))
    assert np.array_equal(y[:, i], f[:, i])


def test_int4_columns_error_at_most_half_scale_per_shard():
    x = W.to_u16(W.draw(4, 300, 64, 24))
    sel, _, _, y = _pipeline(x, 5)
    f = O.bf16_to_f32(x).astype(np.float64)
    exact = f.sum(0)
    c = sel["cmap"]
    half = 0.5 * sel["scale"].astype(np.float64).sum(0)            # sum_p s_p / 2
    slack = 4 * 2.0 ** -24 * (np.abs(f).sum(0) + 16 * sel["scale"].sum(0))
    err = np.abs(y.astype(np.float64) - exact)
    assert np.all(err[:, c] <= half[None, c] * (1 + 1e-5) + slack[:, c])


def test_summed_error_is_irwin_hall_like():
    # Per-shard rounding errors are ~uniform on [-s/2, s/2]; their sum over P
    # shards has mean 0 and variance sum_p s_p^2 / 12, with excess kurtosis
    # -1.2/P for equal scales (Irwin-Hall shape, tending to Gaussian).
    P = 8
    x = W.to_u16(W.draw(P, 512, 256, 25, sigma=0.5))
    sel, _, _, y = _pipeline(x, 0)
    f = O.bf16_to_f32(x).astype(np.float64)
    e = (y.astype(np.float64) - f.sum(0))
    s = sel["scale"].astype(np.float64)
    var_pred = (s ** 2).sum(0) / 12.0
    z = e / np.sqrt(var_pred)[None, :]          # standardised error
    n = z.size
    assert abs(z.mean()) < 4.0 / math.sqrt(n)
    assert abs(z.var() - 1.0) < 0.05
    kurt = (z ** 4).mean() / z.var() ** 2 - 3.0
    assert abs(kurt - (-1.2 / P)) < 0.1


def test_range_ranked_beats_random_selection():
    # "Key Observations and Future Directions": picking BF16 features at random
    # helps little over pure int4; picking by range is what matters.
    w = W.WORKLOADS["tiny"]
    mn = mx = None
    for b in range(w.calib_batches):
        xb = W.to_u16(W.batch(w, W.PHASE_CALIB, b))
        mn, mx = O.calib_update(xb, mn, mx, w.momentum, first=(b == 0))
    x = W.to_u16(W.batch(w, W.PHASE_INFER, 0))
    exact = O.bf16_to_f32(x).astype(np.float64).sum(0)

    def mse_for(idx):
        s, r, z, _ = O.quant_params(mn, mx)
        idx = np.sort(np.asarray(idx, np.int64))
        cmap = np.setdiff1d(np.arange(w.H), idx)
        fmap = np.empty(w.H, np.int64)
        fmap[cmap] = np.arange(cmap.size)
        fmap[idx] = -1 - np.arange(idx.size)
        pk, ol = O.compress_pack(x, r, z, idx, cmap)
        y = O.decompress_reduce(pk, ol, s, z, fmap)
        return float(((y - exact) ** 2).mean())

    ranked = mse_for(O.select_outliers(mn, mx, w.k)["idx"])
    none = mse_for([])
    rnd = np.mean([mse_for(np.random.default_rng(i).choice(w.H, w.k, replace=False))
                   for i in range(8)])
    assert ranked < 0.1 * rnd
    assert rnd > 0.5 * none


def test_f32_to_bf16_matches_torch_round_to_nearest_even():
    # Library routine: torch's fp32 -> bf16 conversion rounds to nearest even.
    rng = np.random.default_rng(21)
    u = rng.integers(0, 2 ** 32, 1 << 20, dtype=np.uint64).astype(np.uint32)
    u = u[(u & 0x7F800000) != 0x7F800000]                      # finite only
    ties = (rng.integers(0, 2 ** 16, 4096).astype(np.uint32) << 16) | 0x8000   # exact halves
    ties = ties[(ties & 0x7F800000) != 0x7F800000]
    special = np.array([0, 0x80000000, 0x00000001, 0x7F7FFFFF, 0x3F808000, 0x3F818000,
                        0x3F7FFFFF, 0xBF808000], np.uint32)
    f = np.concatenate([u, ties, special]).view(np.float32)
    ours = O.f32_to_bf16(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # ties go to the even neighbour: 1 + 2^-8 exactly halfway between 1 and 1 + 2^-7
    assert O.f32_to_bf16(np.array([1.0 + 2.0 ** -8], np.float32))[0] == 0x3F80
    assert O.f32_to_bf16(np.array([1.0 + 3 * 2.0 ** -8], np.float32))[0] == 0x3F82


def test_bf16_output_is_one_rounding_of_the_fp32_sum():
    rng = np.random.default_rng(22)
    x = W.to_u16(W.draw(4, 16, 96, 31, cols=[5, 50], outlier_factor=30.0))
    sel, packed, outl, y32 = _pipeline(x, 6)
    y16 = O.decompress_reduce_bf16(packed, outl, sel["scale"], sel["zero_point"], sel["fmap"])
    assert y16.dtype == np.uint16 and y16.shape == y32.shape
    back = (y16.astype(np.uint32) << 16).view(np.float32)
    # half a bf16 ulp (8 significant bits) is at most 2^-8 |y|
    assert np.all(np.abs(back.astype(np.float64) - y32) <= np.abs(y32.astype(np.float64)) * 2.0 ** -8)
    assert np.array_equal(y16, O.f32_to_bf16(y32))


@pytest.mark.parametrize("P,T,H,k", [(3, 4, 9, 2), (2, 3, 8, 0), (4, 2, 6, 6), (2, 5, 11, 4)])
def test_per_shard_sets_brute_force(P, T, H, k):
    # Element by element: shard p sends feature h as its bf16 value when h is
    # in its own set, else as a 4-bit code with its own parameters; the
    # receiver adds the P fp32 terms in shard order from 0.
    rng = np.random.default_rng(P * 1000 + T * 100 + H + k)
    x = W.to_u16(W.draw(P, T, H, P + H, cols=[1], outlier_factor=20.0))
    mn, mx = O.batch_min_max(x)
    mx = mx.copy()
    mx[rng.integers(0, P), rng.integers(0, H)] += 30.0     # a shard-local wide range
    sel = O.select_outliers_per_shard(mn, mx, k)
    pk, ol = O.compress_pack(x, sel["rscale"], sel["zero_point"], sel["idx"], sel["cmap"],
                             pitch=(H - k + 1) // 2 + 3)
    y = O.decompress_reduce(pk, ol, sel["scale"], sel["zero_point"], sel["fmap"])
    f = O.bf16_to_f32(x)
    for t in range(T):
        for h in range(H):
            acc = np.float32(0)
            for p in range(P):
                if h in set(sel["idx"][p].tolist()):
                    term = f[p, t, h]
                else:
                    r, z, s = sel["rscale"][p, h], sel["zero_point"][p, h], sel["scale"][p, h]
                    q = O.quantize(np.float32(f[p, t, h]), r, z)
                    term = O.dequantize(q, s, z)
                acc = np.float32(acc + np.float32(term))
            assert y[t, h].view(np.uint32) == acc.view(np.uint32), (t, h)
    # the message itself: shard p's outlier block is its own columns
    for p in range(P):
        assert np.array_equal(ol[p], x[p][:, sel["idx"][p]])
