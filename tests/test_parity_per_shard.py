"""GPU parity of per-shard BF16 sets (every shard keeps its own k widest
features): selection, sender and receiver against the oracle.

Bar: parameters, per-shard sets and maps bitwise; packed rows (with
padding) and BF16 blocks bitwise; y within the receiver tolerance, with the
features that are BF16 on every shard bit-exact. The window receiver (H a
multiple of 4, a pitch of at least 8 bytes and a multiple of 4; past 8
shards in groups of up to 6, each later group adding to y) seeds
each feature with -sum z*s over its int4 shards and adds one fma per int4
term, then the shard-ordered sum of its BF16 values: within fp32 rounding of
the oracle. The general receiver evaluates every term as fl(q - z) * s and
adds the terms in shard order from +0, the oracle's arithmetic step for
step, so its output is checked bit for bit. Every receiver output is also
checked to repeat bitwise on a second call. Past 8 shards the bf16 output
takes the general kernel and is checked against the rounding of the
oracle's sum, bit for bit.
"""
import numpy as np
import pytest
import torch

import bit_tensor_activation_amd as B
from oracle import oracle as O
import workloads as W
from helpers import (assert_bits_equal, assert_stats_equal, assert_y_close, assert_y_close_rows,
                     oracle_calib, oracle_compress_rows, oracle_path, say, u16)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def assert_per_shard_selection_equal(g: dict, o: dict) -> None:
    for key, okey in (("scale", "scale"), ("rscale", "rscale"), ("zero_point", "zero_point"),
                      ("outlier_idx", "idx"), ("fmap", "fmap"), ("cmap", "cmap")):
        assert_bits_equal(g[key], np.asarray(o[okey]), key)


def bf16_everywhere(sel_o: dict) -> np.ndarray:
    sets = [set(r.tolist()) for r in sel_o["idx"]]
    return np.array(sorted(set.intersection(*sets)) if sets else [], np.int64)


def run_both(calib_xs, x, k, momentum, *, pitch=None):
    P, T, H = x.shape
    rmin = torch.empty((P, H), dtype=torch.float32, device=DEV)
    rmax = torch.empty_like(rmin)
    mn = mx = None
    for b, xb in enumerate(calib_xs):
        B.btq_calib_update(xb, rmin, rmax, momentum, first_batch=(b == 0))
        mn, mx = oracle_calib(u16(xb), mn, mx, momentum, first=(b == 0))
    torch.cuda.synchronize()
    assert_stats_equal(rmin, mn, "run_min")
    assert_stats_equal(rmax, mx, "run_max")
    sel_g = B.btq_select_outliers_per_shard(rmin, rmax, k)
    sel_o = O.select_outliers_per_shard(mn, mx, k)
    torch.cuda.synchronize()
    assert_per_shard_selection_equal(sel_g, sel_o)
    if pitch is None:
        pitch = B.btq_packed_pitch(H, k)
    args = (sel_g["rscale"], sel_g["zero_point"], sel_g["outlier_idx"], sel_g["cmap"])
    if pitch == B.btq_packed_row_bytes(H, k):   # the per-shard call: rows with no gap
        pk, ol = B.btq_compress_pack_per_shard(x, k, *args)
    else:
        pk, ol = B.btq_compress_pack_ex(x, k, *args, per_shard=True, pitch=pitch)
    pk_o, ol_o = oracle_compress_rows(u16(x), sel_o, pitch=pitch)
    torch.cuda.synchronize()
    assert_bits_equal(pk, pk_o, "packed")
    assert_bits_equal(ol.view(torch.int16), ol_o.view(np.int16), "outliers")
    par = (sel_g["scale"], sel_g["zero_point"], sel_g["fmap"])
    if pitch == B.btq_packed_row_bytes(H, k):
        y = B.btq_decompress_reduce_per_shard(pk, ol, H, *par)
    else:
        y = B.btq_decompress_reduce_ex(pk, ol, H, *par, per_shard=True)
    y2 = B.btq_decompress_reduce_ex(pk, ol, H, *par, per_shard=True)
    y16 = B.btq_decompress_reduce_ex(pk, ol, H, *par, per_shard=True, bf16=True)
    y_o = O.decompress_reduce(pk_o, ol_o, sel_o["scale"], sel_o["zero_point"], sel_o["fmap"])
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32)), "y does not repeat"
    if P <= 8:
        assert torch.equal(y16, y.to(torch.bfloat16).view(torch.int16)), "bf16 y is not RNE(fp32 y)"
    else:   # the bf16 output takes the general kernel: the rounding of the oracle's sum
        ref = torch.from_numpy(np.ascontiguousarray(y_o)).to(torch.bfloat16).view(torch.int16)
        assert torch.equal(y16.cpu(), ref), "bf16 y is not RNE(oracle y)"
    assert_y_close(y.cpu().numpy(), y_o, sel_o["scale"], bf16_everywhere(sel_o))
    if not window_receiver(P, H, pk.shape[2]):
        assert_bits_equal(y, y_o, "y")
    return sel_g, sel_o


def window_receiver(P, H, pitch):
    """Whether the receiver may take its window kernel, in one launch or (past
    8 shards) in shard groups (torch's allocations meet its alignment and
    size conditions here)."""
    return H % 4 == 0 and pitch % 4 == 0 and pitch >= 8


def shard_local(P, T, H, seed, factor=30.0):
    """Normal data, two columns wide everywhere, two more wide on each shard."""
    x = W.draw(P, T, H, seed, cols=[H // 5, H // 2], outlier_factor=8.0, device=DEV)
    xb = x.view(torch.bfloat16).clone()
    for p in range(P):
        xb[p][:, [(37 * p + 11) % H, (53 * p + 101) % H]] *= factor
    return xb.view(torch.int16)


# (P, T, H, k, pitch extra (None: default pitch), note)
CASES = [
    (4, 12, 1024, 8, None, "shard-local outliers"),
    (8, 70, 2048, 64, None, "fast paths, ragged T"),
    (3, 5, 250, 7, None, "H not a multiple of 4: general kernels"),
    (2, 9, 256, 0, None, "k=0"),
    (2, 9, 256, 256, None, "k=H"),
    (5, 33, 1032, 13, None, "H-k odd"),
    (8, 3, 4104, 64, None, "T=3, partial last tile"),
    (4, 6, 2048, 24, 0, "pitch = code bytes (multiple of 4)"),
    (4, 6, 2048, 23, 0, "pitch = code bytes (odd): general receiver"),
    (4, 6, 2048, 24, 4, "pitch = code bytes + 4"),
    (1, 16, 512, 16, None, "one shard"),
    (4, 6, 2048, 100, None, "k in (64, 128]: two entry registers"),
    (8, 5, 4096, 300, None, "k > 128: four entry registers, post-loop recompute"),
    (9, 7, 1024, 16, None, "P=9: shard groups of 6 and 3"),
    (9, 7, 1020, 16, None, "P=9, H not a multiple of 8: general kernel"),
    (16, 40, 2048, 64, None, "P=16: shard groups of 6, 6 and 4"),
    (3, 40, 1028, 9, None, "H a multiple of 4 but not 8: window kernel"),
    (2, 5, 24, 8, 0, "pitch = 8 bytes: the code window moves back one dword"),
    (2, 5, 12, 4, 0, "pitch = 4 bytes: general kernel"),
    (8, 33, 4096, 64, 0, "7B-like rows, pitch = code bytes"),
    (3, 5, 16, 14, None, "k=H-2: two int4 slots"),
    (2, 4, 4, 1, None, "H=4"),
    (16, 3, 64, 2, None, "P=16, tiny H: shard groups"),
    (8, 1, 8192, 64, None, "T=1 (decode): 2-row ring"),
    (4, 2, 1024, 16, None, "T=2"),
]


@pytest.mark.parametrize("P,T,H,k,extra,note", CASES, ids=[c[-1] for c in CASES])
def test_per_shard_sets(P, T, H, k, extra, note):
    say(f"case: per-shard sets P={P} T={T} H={H} k={k} pitch+{extra} ({note})")
    calib = [shard_local(P, 8, H, 4000 + b) for b in range(2)]
    x = shard_local(P, T, H, 4100)
    pitch = None if extra is None else (H - k + 1) // 2 + extra
    sel_g, sel_o = run_both(calib, x, k, 0.9, pitch=pitch)
    if 2 <= k < H:   # each shard keeps its own two wide columns
        for p in range(P):
            own = {(37 * p + 11) % H, (53 * p + 101) % H}
            assert own <= set(sel_o["idx"][p].tolist())


def shard_blocks(P, T, H, seed, width=16, factor=40.0):
    """Normal data; shard p has `width` consecutive wide columns of its own,
    starting at 520 + 8*p (so neighbouring shards' blocks overlap by half)."""
    x = W.draw(P, T, H, seed, device=DEV)
    xb = x.view(torch.bfloat16).clone()
    for p in range(P):
        a = 520 + 8 * p
        xb[p][:, a:a + width] *= factor
    return xb.view(torch.int16)


@pytest.mark.parametrize("P,T,H,k", [(4, 6, 2048, 16), (8, 9, 2048, 24), (12, 9, 2048, 24),
                                     (16, 5, 2048, 16)],
                         ids=["P4-k16", "P8-k24", "P12-k24-groups", "P16-k16-groups"])
def test_per_shard_clustered_blocks(P, T, H, k):
    """Every lane of a block has all 8 of its features BF16 on some shard and
    int4 on others: the owners' loop over several BF16 features, the inverse
    map's longest runs, and features whose BF16 and int4 terms mix across
    shards, in the window kernel. Past 8 shards the same in shard groups:
    features BF16 on every shard of one group and int4 in another."""
    say(f"case: per-shard clustered blocks P={P} T={T} H={H} k={k}")
    calib = [shard_blocks(P, 8, H, 4300 + b) for b in range(2)]
    x = shard_blocks(P, T, H, 4400)
    assert window_receiver(P, H, B.btq_packed_pitch(H, k))
    sel_g, sel_o = run_both(calib, x, k, 0.9)
    for p in range(P):   # each shard's block is its BF16 set
        a = 520 + 8 * p
        assert set(range(a, a + 16)) <= set(sel_o["idx"][p].tolist())


def test_signed_zero_ranges_rank_by_feature():
    # A width of -0 (run_max = -0, run_min = +0) ranks equal to +0: with all
    # ranges zero the sets are the lowest k features, for every rule.
    say("case: signed-zero ranges")
    P, H, k = 3, 64, 5
    rmin = torch.zeros((P, H), dtype=torch.float32, device=DEV)
    rmax = torch.zeros((P, H), dtype=torch.float32, device=DEV)
    rmax[:, 40:50] = -0.0
    per = B.btq_select_outliers_per_shard(rmin, rmax, k)
    mx = B.btq_select_outliers_rule(rmin, rmax, k, "max")
    sm = B.btq_select_outliers(rmin, rmax, k)
    torch.cuda.synchronize()
    assert per["outlier_idx"].cpu().tolist() == [list(range(k))] * P
    assert mx["outlier_idx"].cpu().tolist() == list(range(k))
    assert sm["outlier_idx"].cpu().tolist() == list(range(k))
    o = O.select_outliers_per_shard(rmin.cpu().numpy(), rmax.cpu().numpy(), k)
    assert o["idx"].tolist() == [list(range(k))] * P


@pytest.mark.parametrize("name,k,T,nb", [("7b_prefill", 64, 2048, 4), ("stress", 256, 16384, 2),
                                         ("large_prefill", 128, 8192, 2)])
def test_full_size(name, k, T, nb):
    """A workload's full shape with nb of its calibration batches, through the
    per-shard calls; every element against the oracle. At stress size the
    tiles hold up to P*k/16 BF16 values per row on average, so the receiver
    runs with four entry registers, and tiles beyond four registers take the
    post-loop recompute."""
    w = W.WORKLOADS[name]
    P, H = w.P, w.H
    say(f"case: per-shard sets at full size {name} P={P} T={T} H={H} k={k}")
    rmin = torch.empty((P, H), dtype=torch.float32, device=DEV)
    rmax = torch.empty_like(rmin)
    mn = mx = None
    for b in range(nb):
        xb = W.batch(w, W.PHASE_CALIB, b, device=DEV)
        B.btq_calib_update(xb, rmin, rmax, w.momentum, first_batch=(b == 0))
        mn, mx = oracle_calib(u16(xb), mn, mx, w.momentum, first=(b == 0))
    sel_g = B.btq_select_outliers_per_shard(rmin, rmax, k)
    sel_o = O.select_outliers_per_shard(mn, mx, k)
    torch.cuda.synchronize()
    assert_per_shard_selection_equal(sel_g, sel_o)
    x = W.batch(w, W.PHASE_INFER, 0, T=T, device=DEV)
    pk, ol = B.btq_compress_pack_per_shard(x, k, sel_g["rscale"], sel_g["zero_point"],
                                           sel_g["outlier_idx"], sel_g["cmap"])
    y = B.btq_decompress_reduce_per_shard(pk, ol, H, sel_g["scale"], sel_g["zero_point"],
                                          sel_g["fmap"])
    torch.cuda.synchronize()
    pk_o, ol_o, y_o = oracle_path(u16(x), sel_o)
    assert_bits_equal(pk, pk_o, "packed")
    assert_bits_equal(ol.view(torch.int16), ol_o.view(np.int16), "outliers")
    assert_y_close_rows(y, y_o, sel_o["scale"], bf16_everywhere(sel_o))
    assert window_receiver(P, H, pk.shape[2])


def test_sets_concentrated_in_one_tile():
    """Every shard keeps the same wide block of features, inside the first one
    or two 256-feature tiles: such a tile holds more BF16 values per row than
    the receiver's registers, so it adds the rest after its row loop."""
    for P, T, H, k in ((8, 21, 1024, 200), (4, 9, 2048, 300)):
        say(f"case: per-shard sets concentrated P={P} T={T} H={H} k={k}")
        def draw(T_, seed):
            x = W.draw(P, T_, H, seed, cols=[], outlier_factor=1.0, device=DEV)
            xb = x.view(torch.bfloat16).clone()
            xb[:, :, 40:40 + k] *= 30.0
            return xb.view(torch.int16)
        calib = [draw(8, 4200 + b) for b in range(2)]
        sel_g, sel_o = run_both(calib, draw(T, 4300), k, 0.9)
        assert sel_o["idx"].tolist() == [list(range(40, 40 + k))] * P
