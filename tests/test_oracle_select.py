"""Pins for the oracle's selection of BF16 features (CPU only).

Page: "Revolutionizing LLM Inference: The Power of Efficient Low-Bit
Communication", section "The Hybrid Quantization Algorithm", Selection
bullet (rank features by quantization range, keep a number of them in BF16),
and section "Leveraging Outliers for Efficient Communication" (a handful of
features have very wide ranges).
"""
import json
import os

import numpy as np
import pytest

from oracle import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_selection_worked_examples():
    g = json.load(open(os.path.join(GOLDEN, "selection_worked.json")))
    for c in g["cases"]:
        sel = O.select_outliers(np.array(c["run_min"], np.float32),
                                np.array(c["run_max"], np.float32), c["k"])
        assert sel["score"].tolist() == c["score"]
        assert sel["idx"].tolist() == c["idx"]
        assert sel["fmap"].tolist() == c["fmap"]
        assert sel["cmap"].tolist() == c["cmap"]


def _check_maps(idx, fmap, cmap, H, k):
    assert idx.shape == (k,) and cmap.shape == (H - k,) and fmap.shape == (H,)
    assert np.all(np.diff(idx) > 0) and np.all(np.diff(cmap) > 0)
    assert sorted(idx.tolist() + cmap.tolist()) == list(range(H))
    for i, h in enumerate(idx):
        assert fmap[h] == -1 - i
    for j, h in enumerate(cmap):
        assert fmap[h] == j


@pytest.mark.parametrize("H,k", [(1, 0), (1, 1), (9, 3), (64, 0), (64, 64), (300, 17)])
def test_top_k_brute_force(H, k):
    rng = np.random.default_rng(H * 31 + k)
    score = rng.integers(0, 6, H).astype(np.float32)      # many ties
    idx, fmap, cmap = O.top_k_features(score, k)
    want = sorted(sorted(range(H), key=lambda h: (-float(score[h]), h))[:k])
    assert idx.tolist() == want
    _check_maps(idx, fmap, cmap, H, k)


def test_score_two_shards_is_exact_sum():
    # For P=2 the fp32 sum equals the exact sum rounded once to fp32.
    rng = np.random.default_rng(5)
    w = np.abs(rng.standard_normal((2, 1000))).astype(np.float32) * 7
    s = O.range_score(w)
    exact = (w[0].astype(np.float64) + w[1].astype(np.float64)).astype(np.float32)
    assert np.array_equal(s, exact)


def test_score_many_shards_error_bound():
    rng = np.random.default_rng(6)
    w = np.abs(rng.standard_normal((8, 500))).astype(np.float32)
    s = O.range_score(w).astype(np.float64)
    exact = w.astype(np.float64).sum(0)
    assert np.all(np.abs(s - exact) <= 8 * 2.0 ** -24 * exact)


def test_tiny_workload_selects_planted_outliers():
    w = W.WORKLOADS["tiny"]
    mn = mx = None
    for b in range(w.calib_batches):
        x = W.to_u16(W.batch(w, W.PHASE_CALIB, b))
        mn, mx = O.calib_update(x, mn, mx, w.momentum, first=(b == 0))
    sel = O.select_outliers(mn, mx, w.k)
    planted = set(W.outlier_columns(w).tolist())
    assert planted <= set(sel["idx"].tolist())
    _check_maps(sel["idx"], sel["fmap"], sel["cmap"], w.H, w.k)
    # the planted columns are ranked first, with a wide margin
    order = np.argsort(-sel["score"], kind="stable")
    assert set(order[:len(planted)].tolist()) == planted
    assert sel["score"][order[len(planted) - 1]] > 10 * sel["score"][order[len(planted)]]


def test_zero_inclusion_holds_on_tiny_workload():
    # lo <= 0 <= hi already holds for calibrated features of the workloads, so
    # widening the range to include 0 changes nothing there.
    w = W.WORKLOADS["tiny"]
    mn = mx = None
    for b in range(w.calib_batches):
        x = W.to_u16(W.batch(w, W.PHASE_CALIB, b))
        mn, mx = O.calib_update(x, mn, mx, w.momentum, first=(b == 0))
    assert np.all(mn < 0) and np.all(mx > 0)


@pytest.mark.parametrize("H,k,seed", [(1, 0, 0), (1, 1, 1), (40, 7, 2), (300, 0, 3), (300, 300, 4),
                                      (517, 64, 5)])
def test_maps_for_a_given_set_brute_force(H, k, seed):
    rng = np.random.default_rng(seed)
    want = np.sort(rng.choice(H, k, replace=False))
    idx, fmap, cmap = O.maps_for_set(want, H)
    assert idx.tolist() == want.tolist()
    _check_maps(idx, fmap, cmap, H, k)


def test_maps_for_a_given_set_rejects_bad_sets():
    for bad in ([3, 2], [1, 1], [-1, 2], [0, 10]):
        with pytest.raises(ValueError):
            O.maps_for_set(np.array(bad), 10)


def test_given_set_selection_matches_ranked_selection_on_its_set():
    rng = np.random.default_rng(13)
    mn = -np.abs(rng.standard_normal((4, 70))).astype(np.float32) * 2
    mx = np.abs(rng.standard_normal((4, 70))).astype(np.float32) * 2
    ranked = O.select_outliers(mn, mx, 9)
    given = O.select_features(mn, mx, ranked["idx"])
    for key in ("scale", "rscale", "zero_point", "score", "idx", "fmap", "cmap"):
        assert np.array_equal(np.ascontiguousarray(given[key]).view(np.uint8),
                              np.ascontiguousarray(ranked[key]).view(np.uint8)), key
    # a random set: the maps follow the set, the parameters do not change
    other = np.sort(rng.choice(70, 9, replace=False))
    g2 = O.select_features(mn, mx, other)
    assert g2["idx"].tolist() == other.tolist()
    assert np.array_equal(g2["scale"], ranked["scale"])
    _check_maps(g2["idx"], g2["fmap"], g2["cmap"], 70, 9)


def test_score_rules_worked_example():
    # widths [P=4, H=3]: feature 1 is wide on one shard only, feature 2 on
    # every shard a little. Sum: [4, 7, 5] -> feature 1 first; max: [1, 4, 5]
    # -> feature 2 first.
    w = np.array([[1, 1, 5], [1, 1, 0], [1, 1, 0], [1, 4, 0]], np.float32)
    assert O.range_score(w, "sum").tolist() == [4.0, 7.0, 5.0]
    assert O.range_score(w, "max").tolist() == [1.0, 4.0, 5.0]
    assert O.top_k_features(O.range_score(w, "sum"), 1)[0].tolist() == [1]
    assert O.top_k_features(O.range_score(w, "max"), 1)[0].tolist() == [2]
    with pytest.raises(ValueError):
        O.range_score(w, "mean")


def test_max_score_is_an_attained_upper_bound():
    rng = np.random.default_rng(8)
    w = np.abs(rng.standard_normal((7, 400))).astype(np.float32) * 3
    s = O.range_score(w, "max")
    assert np.all(s[None, :] >= w)
    assert np.all((w == s[None, :]).any(axis=0))
    # one shard: both rules give the shard's own ranges
    assert np.array_equal(O.range_score(w[:1], "max"), w[0])
    assert np.array_equal(O.range_score(w[:1], "sum"), w[0])


def test_select_outliers_rule_changes_only_score_and_set():
    rng = np.random.default_rng(14)
    mn = -np.abs(rng.standard_normal((4, 90))).astype(np.float32)
    mx = np.abs(rng.standard_normal((4, 90))).astype(np.float32)
    mx[2, 10] = 50.0                      # wide on one shard only
    mx[:, 20] += 20.0                     # moderately wide on every shard
    a = O.select_outliers(mn, mx, 1, "sum")
    b = O.select_outliers(mn, mx, 1, "max")
    assert a["idx"].tolist() == [20] and b["idx"].tolist() == [10]
    for key in ("scale", "rscale", "zero_point"):
        assert np.array_equal(a[key], b[key])
    c = O.select_features(mn, mx, b["idx"])
    for key in ("fmap", "cmap"):
        assert np.array_equal(b[key], c[key])


def test_per_shard_selection_worked_example():
    # widths shard 0 = [1, 5, 2, 3], shard 1 = [4, 1, 1, 1] (run_min 0, so
    # width = run_max exactly); k = 1: shard 0 keeps feature 1, shard 1
    # feature 0.
    mx = np.array([[1, 5, 2, 3], [4, 1, 1, 1]], np.float32)
    sel = O.select_outliers_per_shard(np.zeros_like(mx), mx, 1)
    assert sel["idx"].tolist() == [[1], [0]]
    assert sel["fmap"].tolist() == [[0, -1, 1, 2], [-1, 0, 1, 2]]
    assert sel["cmap"].tolist() == [[0, 2, 3], [1, 2, 3]]
    # the parameters stay per (shard, feature): scale = w/15, zero point 0
    assert np.array_equal(sel["scale"], mx / np.float32(15))
    assert not sel["zero_point"].any()


def test_per_shard_selection_of_equal_shards_is_the_shared_one():
    # Two equal shards: the summed score is exactly twice each shard's width,
    # so every shard's own ranking equals the shared ranking.
    rng = np.random.default_rng(31)
    mn = -np.abs(rng.standard_normal((1, 300))).astype(np.float32)
    mx = np.abs(rng.standard_normal((1, 300))).astype(np.float32)
    mn2, mx2 = np.repeat(mn, 2, 0), np.repeat(mx, 2, 0)
    shared = O.select_outliers(mn2, mx2, 17)
    per = O.select_outliers_per_shard(mn2, mx2, 17)
    for p in range(2):
        assert per["idx"][p].tolist() == shared["idx"].tolist()
        assert per["cmap"][p].tolist() == shared["cmap"].tolist()
        assert per["fmap"][p].tolist() == shared["fmap"].tolist()


@pytest.mark.parametrize("P,H,k", [(3, 50, 0), (3, 50, 7), (4, 64, 64), (5, 33, 32)])
def test_per_shard_selection_invariants(P, H, k):
    rng = np.random.default_rng(P * 100 + H + k)
    mn = -np.abs(rng.standard_normal((P, H))).astype(np.float32)
    mx = np.abs(rng.standard_normal((P, H))).astype(np.float32)
    sel = O.select_outliers_per_shard(mn, mx, k)
    for p in range(P):
        _check_maps(sel["idx"][p], sel["fmap"][p], sel["cmap"][p], H, k)
        chosen = sel["width"][p, sel["idx"][p]]
        rest = sel["width"][p, sel["cmap"][p]]
        if k and k < H:
            assert chosen.min() >= rest.max()
