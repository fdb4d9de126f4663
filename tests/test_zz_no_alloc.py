"""btq_calib_update_noalloc against btq_calib_update, through the C ABI.

The no-alloc call keeps its partial extremes in the library's static device
scratch instead of a workspace. The running extremes do not depend on how
the token axis is split into chunks, so both calls must give the same bits.
Calls run back to back, each later one with a smaller input than the one
before, so every call after the first runs over what the previous call
left in the scratch.
"""
import pytest
import torch

import bit_tensor_activation_amd as B
from bit_tensor_activation_amd import _lib
import workloads as W
from helpers import say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def state(P, H, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    lo = torch.randn((P, H), generator=g, device=DEV) - 3.0
    return lo, lo + 6.0 * torch.rand((P, H), generator=g, device=DEV)


def both(P, T, H, seed, momentum, first):
    """One batch through both calls from the same running state."""
    say(f"case: no-alloc calibration P={P} T={T} H={H} first={first}")
    x = W.draw(P, T, H, seed, base="laplace", cols=[0, H // 2], outlier_factor=30.0, device=DEV)
    mn, mx = state(P, H, seed + 1)
    a_min, a_max = mn.clone(), mx.clone()
    b_min, b_max = mn.clone(), mx.clone()
    B.btq_calib_update(x, a_min, a_max, momentum, first)
    B.btq_calib_update_noalloc(x, b_min, b_max, momentum, first)
    torch.cuda.synchronize()
    assert torch.equal(a_min.view(torch.int32), b_min.view(torch.int32)), "run_min differs"
    assert torch.equal(a_max.view(torch.int32), b_max.view(torch.int32)), "run_max differs"


def test_noalloc_matches_the_allocating_call():
    # 1. the scratch filled (the usual plan's partials take all 8 MiB)
    both(8, 4096, 8192, 101, 0.9, True)
    # 2. smaller, a later batch: P=3 asks for more chunks than fit, so the
    #    call uses fewer, longer chunks
    both(3, 4000, 8192, 102, 0.9, False)
    # 3. smaller again, ragged sizes and a momentum of 0
    both(2, 37, 1000, 103, 0.0, False)


def test_noalloc_largest_and_oversized():
    P, H = 8, (1 << 20) // 8      # 2*P*H*4 bytes = the scratch exactly: one chunk
    both(P, 40, H, 201, 0.5, False)
    # one feature more does not fit: an error, and nothing enqueued
    H += 1
    x = torch.zeros((P, 4, H), dtype=torch.int16, device=DEV)
    mn = torch.full((P, H), 7.0, device=DEV)
    mx = torch.full((P, H), 9.0, device=DEV)
    with pytest.raises(RuntimeError, match="no-alloc scratch"):
        B.btq_calib_update_noalloc(x, mn, mx, 0.9, False)
    torch.cuda.synchronize()
    assert bool((mn == 7.0).all()) and bool((mx == 9.0).all())
    assert _lib.BTQ_NOALLOC_SCRATCH_BYTES == 8 << 20
