"""GPU parity on seeded random shapes: shard counts 1-16 (past 8 the fp32
receiver runs in shard groups), feature counts with and without 4- and
8-alignment, token counts from 1 to 40, any k from 0 to H, and default,
tight (code bytes, multiple of 4) or padded pitches. Each shape runs the
shared-set path and the per-shard path against the oracle, to the bars of
the two parity suites they reuse, so whichever kernel each shape selects is
checked. BTQ_RANDOM_SHAPES sets how many seeds run (24 by default) and
BTQ_RANDOM_T_MAX the largest token count (40 by default)."""
import os
import numpy as np
import pytest
import torch

import workloads as W
from helpers import say
import test_parity as shared
import test_parity_per_shard as per_shard

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


T_MAX = int(os.environ.get("BTQ_RANDOM_T_MAX", "40"))


def shape(seed):
    g = np.random.default_rng([20260, seed])
    P = int(g.integers(1, 17))
    H = int(g.choice([8, 4, 1])) * int(g.integers(2, 700))
    T = int(g.integers(1, T_MAX + 1))
    k = int(g.integers(0, H + 1)) if g.random() < 0.3 else int(g.integers(0, min(H, 80) + 1))
    code_bytes = (H - k + 1) // 2
    pick = g.random()
    if pick < 0.5 or code_bytes == 0:
        pitch = None
    elif pick < 0.75:
        pitch = max(code_bytes + (-code_bytes) % 4, 4)   # tight, a multiple of 4
    else:
        pitch = code_bytes + int(g.integers(1, 40))       # padded, any alignment
    return P, T, H, k, pitch


SEEDS = list(range(int(os.environ.get("BTQ_RANDOM_SHAPES", "24"))))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_shape(seed):
    P, T, H, k, pitch = shape(seed)
    say(f"case: random shape seed={seed} P={P} T={T} H={H} k={k} pitch={pitch}")
    cols = sorted({(37 * seed + 5) % H, (101 * seed + 17) % H, H - 1})
    calib = [W.draw(P, 8, H, 5000 + 10 * seed + b, cols=cols, outlier_factor=30.0, device=DEV)
             for b in range(2)]
    x = W.draw(P, T, H, 5500 + seed, cols=cols, outlier_factor=30.0, device=DEV)
    shared.run_both(calib, x, k, 0.9, pitch=pitch)
    per_shard.run_both(calib, x, k, 0.9, pitch=pitch)
