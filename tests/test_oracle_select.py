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


def test_codec_tables_are_the_parameters_in_message_order():
    # Brute force: walk the slots and read the per-feature arrays directly.
    rng = np.random.default_rng(9)
    P, H, k = 3, 40, 6
    mn = -np.abs(rng.standard_normal((P, H))).astype(np.float32) * 3
    mx = np.abs(rng.standard_normal((P, H))).astype(np.float32) * 3
    sel = O.select_outliers(mn, mx, k)
    enc, dec = sel["enc"], sel["dec"]
    assert enc.shape == (P, H - k, 2) and dec.shape == (2 * P + 1, H - k)
    for j, h in enumerate(sel["cmap"]):
        exact = 0.0
        for p in range(P):
            assert enc[p, j, 0] == sel["rscale"][p, h]
            assert enc[p, j, 1] == float(sel["zero_point"][p, h])
            assert dec[p, j] == sel["scale"][p, h]
            assert dec[P + p, j] == float(sel["zero_point"][p, h])
            exact -= float(sel["zero_point"][p, h]) * float(sel["scale"][p, h])
        # the fp32 bias is the exact sum up to P roundings
        assert abs(dec[2 * P, j] - exact) <= 2 * P * 2.0 ** -24 * (abs(exact) + 15 * P * sel["scale"][:, h].max())


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
    for key in ("scale", "rscale", "zero_point", "score", "idx", "fmap", "cmap", "enc", "dec"):
        assert np.array_equal(np.ascontiguousarray(given[key]).view(np.uint8),
                              np.ascontiguousarray(ranked[key]).view(np.uint8)), key
    # a random set: maps and tables follow the set, parameters do not change
    other = np.sort(rng.choice(70, 9, replace=False))
    g2 = O.select_features(mn, mx, other)
    assert g2["idx"].tolist() == other.tolist()
    assert np.array_equal(g2["scale"], ranked["scale"])
    _check_maps(g2["idx"], g2["fmap"], g2["cmap"], 70, 9)
