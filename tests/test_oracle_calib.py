"""Pins for the oracle's bf16 decode and calibration steps (CPU only).

Page: "Revolutionizing LLM Inference: The Power of Efficient Low-Bit
Communication", section "The Hybrid Quantization Algorithm", Calibration
bullet: per-feature parameters from moving averages of the min and max
observed on each device.
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


def test_bf16_decode_all_patterns_match_torch():
    # library routine: torch's own bf16 -> fp32 widening, for all 65,536 patterns
    u = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = O.bf16_to_f32(u)
    ref = torch.from_numpy(u.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_batch_min_max_brute_force():
    x = W.to_u16(W.draw(3, 7, 11, 123, base="laplace"))
    bmin, bmax = O.batch_min_max(x)
    for p in range(3):
        for h in range(11):
            vals = [float(O.bf16_to_f32(x[p, t, h])) for t in range(7)]
            assert bmin[p, h] == min(vals)
            assert bmax[p, h] == max(vals)


def test_batch_min_max_ignores_token_order():
    x = W.to_u16(W.draw(2, 33, 40, 5))
    perm = np.random.default_rng(1).permutation(33)
    a = O.batch_min_max(x)
    b = O.batch_min_max(x[:, perm, :])
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_ema_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "ema_worked.json")))
    m = g["momentum"]
    assert (np.float32(1) - np.float32(m)).view(np.uint32) == int(g["c_bits"], 16)
    run = None
    for i, obs in enumerate(g["observed"]):
        run = O.ema(run, np.array([obs], np.float32), m, first=(i == 0))
        assert run.view(np.uint32)[0] == int(g["running"][i], 16)


@pytest.mark.parametrize("m", [0.9, 0.95, 0.5])
def test_ema_matches_closed_form(m):
    # Closed form of the recursion: a^(n-1) b_1 + sum_{i>=2} (1-a) a^(n-i) b_i,
    # evaluated in float64 with a, 1-a taken as the fp32 values.
    rng = np.random.default_rng(7)
    n = 40
    obs = (rng.standard_normal((n, 64)) * 3).astype(np.float32)
    run = None
    for i in range(n):
        run = O.ema(run, obs[i], m, first=(i == 0))
    a = float(np.float32(m))
    c = float(np.float32(1) - np.float32(m))
    ref = a ** (n - 1) * obs[0].astype(np.float64)
    for i in range(1, n):
        ref = ref + c * a ** (n - 1 - i) * obs[i].astype(np.float64)
    bound = 3 * n * 2.0 ** -24 * np.abs(obs).max()
    assert np.max(np.abs(run - ref)) <= bound


def test_ema_zero_momentum_is_last_batch():
    obs = np.random.default_rng(2).standard_normal((5, 17)).astype(np.float32)
    run = None
    for i in range(5):
        run = O.ema(run, obs[i], 0.0, first=(i == 0))
    assert np.array_equal(run, obs[-1])


def test_ema_first_batch_copies():
    obs = np.array([-3.5, 0.0, 2.25], np.float32)
    prev = np.array([100.0, 100.0, 100.0], np.float32)
    assert np.array_equal(O.ema(prev, obs, 0.9, first=True), obs)


def test_calibration_resume_is_bitwise():
    # Saving the running state and resuming gives the uninterrupted result.
    xs = [W.to_u16(W.draw(2, 9, 30, 100 + i)) for i in range(6)]
    mn = mx = None
    for i, x in enumerate(xs):
        mn, mx = O.calib_update(x, mn, mx, 0.9, first=(i == 0))
    a_mn = a_mx = None
    for i, x in enumerate(xs[:4]):
        a_mn, a_mx = O.calib_update(x, a_mn, a_mx, 0.9, first=(i == 0))
    saved = (a_mn.copy(), a_mx.copy())
    b_mn, b_mx = saved
    for x in xs[4:]:
        b_mn, b_mx = O.calib_update(x, b_mn, b_mx, 0.9, first=False)
    assert np.array_equal(b_mn.view(np.uint32), mn.view(np.uint32))
    assert np.array_equal(b_mx.view(np.uint32), mx.view(np.uint32))


def test_tiny_workload_calibration_brackets_data():
    w = W.WORKLOADS["tiny"]
    mn = mx = None
    lo = hi = None
    for b in range(w.calib_batches):
        x = W.to_u16(W.batch(w, W.PHASE_CALIB, b))
        mn, mx = O.calib_update(x, mn, mx, w.momentum, first=(b == 0))
        f = O.bf16_to_f32(x)
        lo = f.min(1) if lo is None else np.minimum(lo, f.min(1))
        hi = f.max(1) if hi is None else np.maximum(hi, f.max(1))
    # a convex combination of batch extremes stays inside the overall extremes
    assert np.all(mn >= lo) and np.all(mx <= hi)
    assert np.all(mn < 0) and np.all(mx > 0)   # every feature spans 0 on this data
