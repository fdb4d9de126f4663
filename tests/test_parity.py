"""GPU parity: every HIP step against the CPU oracle, element by element.

Bar: calibration statistics equal by value; parameters, outlier set, maps,
packed codes and BF16 blocks bitwise; reduced output within
1e-3*|y| + 1e-2*max_p scale (BF16 feature columns bit-exact). The bf16-output
receiver: within that bound plus half a bf16 ulp, BF16 columns equal to the
oracle's rounding, and bit-identical to rounding the fp32 receiver's output.

Every case runs the four calls of the path with rows of Bq code bytes and no
gap (btq_compress_pack, btq_decompress_reduce), and again through the *_ex
calls with a packed row pitch (by default Bq rounded up to 128): the padded
message must be the oracle's rows padded with zeros, and its receivers must
meet the same bar.
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


def _shifted(t: torch.Tensor, off: int) -> torch.Tensor:
    """Same values in storage that starts `off` elements past an allocation."""
    big = torch.empty(t.numel() + off, dtype=t.dtype, device=t.device)
    big[off:] = t.reshape(-1)
    return big[off:].view(t.shape)


def run_both(calib_xs, x, k, momentum, *, x_offset=0, param_offset=0, pitch=None,
             features=None, rule=None):
    """Calibrate, select, compress and decompress on both sides; compare all.

    features: a BF16 set given to both sides in place of the range ranking.
    rule: the rank score ("sum" or "max") through btq_select_outliers_rule.
    param_offset: the per-feature arrays and fmap moved off 16-byte alignment.
    pitch: the packed row pitch of the *_ex pass (default btq_packed_pitch)."""
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

    if features is None and rule is None:
        sel_g = B.btq_select_outliers(rmin, rmax, k)
        sel_o = O.select_outliers(mn, mx, k)
    elif features is None:
        sel_g = B.btq_select_outliers_rule(rmin, rmax, k, rule)
        sel_o = O.select_outliers(mn, mx, k, rule)
    else:
        sel_g = B.btq_select_features(rmin, rmax, features)
        sel_o = O.select_features(mn, mx, features)
    torch.cuda.synchronize()
    assert_selection_equal(sel_g, sel_o)

    if x_offset:   # misaligned base pointer: same values, shifted storage
        x = _shifted(x, x_offset)
    par = {key: sel_g[key] for key in ("scale", "rscale", "zero_point", "fmap")}
    if param_offset:   # aligned to the element type but not to 16 bytes
        par = {key: _shifted(v, param_offset) for key, v in par.items()}
    idx, cmap = sel_g["outlier_idx"], sel_g["cmap"]

    # the path's four calls: rows of Bq bytes, no gap
    pk, ol = B.btq_compress_pack(x, k, par["rscale"], par["zero_point"], idx, cmap)
    pk_o, ol_o = oracle_compress_rows(u16(x), sel_o)
    torch.cuda.synchronize()
    assert pk.shape == (P, T, B.btq_packed_row_bytes(H, k))
    assert_bits_equal(pk, pk_o, "packed")
    assert_bits_equal(ol.view(torch.int16), ol_o.view(np.int16), "outliers")
    y = B.btq_decompress_reduce(pk, ol, H, par["scale"], par["zero_point"], par["fmap"])
    y16 = B.btq_decompress_reduce_bf16(pk, ol, H, par["scale"], par["zero_point"], par["fmap"])
    y_o = O.decompress_reduce(pk_o, ol_o, sel_o["scale"], sel_o["zero_point"], sel_o["fmap"])
    torch.cuda.synchronize()
    assert_y_close(y.cpu().numpy(), y_o, sel_o["scale"], sel_o["idx"])
    assert_y_bf16_close(y16.cpu().numpy(), y_o, sel_o["scale"], sel_o["idx"])
    assert_bf16_is_rne(y16, y, y_o, P)

    # the same through the *_ex calls with a row pitch
    if pitch is None:
        pitch = B.btq_packed_pitch(H, k)
    pkp, olp = B.btq_compress_pack_ex(x, k, par["rscale"], par["zero_point"], idx, cmap,
                                      pitch=pitch)
    torch.cuda.synchronize()
    assert_bits_equal(pkp, O.pad_rows(pk_o, pitch), "packed (pitched)")
    assert torch.equal(olp, ol)
    yp = B.btq_decompress_reduce_ex(pkp, olp, H, par["scale"], par["zero_point"], par["fmap"])
    yp16 = B.btq_decompress_reduce_ex(pkp, olp, H, par["scale"], par["zero_point"], par["fmap"],
                                      bf16=True)
    torch.cuda.synchronize()
    assert_y_close(yp.cpu().numpy(), y_o, sel_o["scale"], sel_o["idx"])
    assert_bf16_is_rne(yp16, yp, y_o, P)
    return sel_g, pk, ol, y


def assert_bf16_is_rne(y16, y, y_o, P):
    """Up to 8 shards the bf16 output is one round-to-nearest-even of the
    fp32 output. With more, the fp32 output runs the window kernel once per
    group of 8 shards and the bf16 output takes the general kernel, whose sum
    is the oracle's: it is then the rounding of the oracle's y, bit for bit."""
    if P <= 8:
        assert torch.equal(y16, y.to(torch.bfloat16).view(torch.int16))
    else:
        ref = torch.from_numpy(np.ascontiguousarray(y_o)).to(torch.bfloat16).view(torch.int16)
        assert torch.equal(y16.cpu(), ref), "bf16 y is not RNE(oracle y)"


def test_tiny_workload_end_to_end():
    w = W.WORKLOADS["tiny"]
    say("case: tiny workload")
    calib = [W.batch(w, W.PHASE_CALIB, b, device=DEV) for b in range(w.calib_batches)]
    x = W.batch(w, W.PHASE_INFER, 0, device=DEV)
    sel, *_ = run_both(calib, x, w.k, w.momentum)
    planted = set(W.outlier_columns(w).tolist())
    assert planted <= set(sel["outlier_idx"].cpu().tolist())


# (P, T, H, k, base, outlier columns, note)
CASES = [
    (2, 16, 256, 8, "normal", [3, 77, 128, 200], "tiny shape"),
    (8, 70, 2048, 64, "normal", list(range(5, 2048, 41)), "fast path, 4 tiles, ragged T"),
    (4, 3, 4104, 8, "laplace", [0, 1, 2, 4103], "H=4104, outliers at both ends"),
    (3, 33, 1032, 8, "normal", [10, 500, 1031], "P=3"),
    (5, 9, 1024, 16, "laplace", [7, 8, 9, 10], "P=5"),
    (6, 12, 520, 8, "normal", [519], "P=6, partial last tile"),
    (7, 5, 1040, 0, "normal", [], "P=7, k=0"),
    (1, 40, 512, 0, "normal", [], "P=1, k=0, one full tile"),
    (2, 9, 256, 256, "normal", [1, 2], "k=H: all BF16"),
    (9, 17, 512, 16, "laplace", [100, 101], "P=9: groups of 8 and 1 shards"),
    (16, 40, 2048, 64, "normal", list(range(5, 2048, 37)), "P=16: two groups of 8 shards"),
    (12, 10, 2048, 64, "normal", list(range(700, 745)),
     "P=12, 45 clustered BF16: post-loop pass in both groups"),
    (3, 5, 250, 7, "normal", [0, 249, 100], "H not a multiple of 4: general receiver"),
    (3, 40, 1028, 9, "normal", [5, 600, 1027], "H=1028: a partial last tile of 4-feature lanes"),
    (5, 33, 1032, 13, "normal", [1, 2, 3], "H-k odd: pad nibble, general sender"),
    (2, 8, 1024, 200, "normal", list(range(100, 300)), "200 clustered BF16 features in one tile"),
    (4, 6, 2048, 600, "laplace", list(range(0, 2048, 3))[:600], "k=600: wide LDS span"),
    (1, 1, 8, 3, "normal", [1], "smallest: P=1, T=1, H=8"),
    (3, 5, 16, 15, "normal", [2], "k=H-1: a single int4 slot"),
    (2, 4, 1, 0, "normal", [0], "H=1, k=0"),
    (2, 4, 1, 1, "normal", [0], "H=1, k=1"),
    (5, 7, 2, 1, "laplace", [1], "H=2"),
    (64, 3, 64, 2, "normal", [5, 40], "P=64: many shards"),
    (8, 1, 8192, 64, "normal", list(range(3, 8192, 200)), "decode-like T=1"),
    (8, 24, 2048, 96, "normal", list(range(600, 624)), "P=8, 24 clustered BF16: 3-4 registers"),
    (8, 20, 2048, 64, "normal", list(range(700, 745)), "P=8, 45 clustered BF16: post-loop sums"),
    (8, 40, 4096, 64, "laplace", list(range(5, 4096, 64)), "P=8, T=40: 2-row ring"),
]


@pytest.mark.parametrize("P,T,H,k,base,cols,note", CASES, ids=[c[-1] for c in CASES])
def test_shapes(P, T, H, k, base, cols, note):
    say(f"case: P={P} T={T} H={H} k={k} ({note})")
    calib = [W.draw(P, max(T, 4), H, 1000 + b, base=base, cols=cols, outlier_factor=40.0,
                    device=DEV) for b in range(3)]
    x = W.draw(P, T, H, 2000, base=base, cols=cols, outlier_factor=40.0, device=DEV)
    run_both(calib, x, k, 0.9)


# Batches long enough for many token rows per receiver wave (the window
# kernel's 4-row ring and ragged last row blocks): a partial last tile, 1-8
# shards, an odd code count (dense rows then take the general receiver,
# padded rows the window kernel), clustered BF16 features (four entry
# registers; tiles beyond them take the post-loop pass) and k = 256 of 8192.
# (P, T, H, k, base, outlier columns, note)
LONG_BATCH_CASES = [
    (8, 2050, 4096, 64, "normal", list(range(5, 4096, 97)), "7B-like, ragged last row block"),
    (4, 2600, 4104, 8, "laplace", [0, 1, 2, 4103], "partial last tile"),
    (3, 3000, 2056, 24, "normal", [10, 500, 2055], "P=3"),
    (1, 9000, 1024, 0, "normal", [], "P=1, k=0"),
    (8, 2048, 2048, 200, "normal", list(range(300, 500)), "200 clustered BF16 features"),
    (8, 1024, 8192, 256, "laplace", list(range(3, 8192, 61)), "k=256 of 8192"),
    (5, 4000, 2048, 13, "normal", [1, 2, 3], "odd code count"),
    (8, 2048, 4096, 0, "laplace", [], "P=8, k=0"),
]


@pytest.mark.parametrize("P,T,H,k,base,cols,note", LONG_BATCH_CASES,
                         ids=[c[-1] for c in LONG_BATCH_CASES])
def test_long_batches(P, T, H, k, base, cols, note):
    say(f"case: long batch P={P} T={T} H={H} k={k} ({note})")
    calib = [W.draw(P, 64, H, 1500 + b, base=base, cols=cols, outlier_factor=40.0, device=DEV)
             for b in range(2)]
    x = W.draw(P, T, H, 2500, base=base, cols=cols, outlier_factor=40.0, device=DEV)
    run_both(calib, x, k, 0.9)


# (P, T, H, k, note): a seeded random BF16 set of size k
SET_CASES = [
    (2, 16, 256, 8, "tiny shape"),
    (8, 70, 2048, 64, "fast path, 4 tiles"),
    (4, 9, 4104, 5, "partial last tile"),
    (3, 5, 250, 0, "empty set"),
    (2, 4, 256, 256, "every feature"),
    (9, 17, 512, 16, "P=9: groups of 8 and 1 shards"),
    (5, 3, 3000, 1500, "half the features"),
]


@pytest.mark.parametrize("P,T,H,k,note", SET_CASES, ids=[c[-1] for c in SET_CASES])
def test_given_feature_set(P, T, H, k, note):
    say(f"case: given set P={P} T={T} H={H} k={k} ({note})")
    cols = [H // 3, H - 1]
    calib = [W.draw(P, 8, H, 3000 + b, cols=cols, outlier_factor=40.0, device=DEV)
             for b in range(2)]
    x = W.draw(P, T, H, 3100, cols=cols, outlier_factor=40.0, device=DEV)
    feats = np.sort(np.random.default_rng(H * 7 + k).choice(H, k, replace=False))
    sel, *_ = run_both(calib, x, k, 0.9, features=feats)
    assert sel["outlier_idx"].cpu().numpy().tolist() == feats.tolist()


# A contiguous block of BF16 features puts one sender tile's span far beyond
# its 512 slots (the staged sender kernel), and gives the receiver's tiles
# more BF16 entries than its registers hold (its post-loop recompute).
WIDE_SPAN_CASES = [
    (4, 37, 4096, (600, 3200), "tile spanning ~3100 features"),
    (8, 20, 2048, (512, 1400), "tile spanning ~1400 features"),
    (2, 9, 6000, (100, 5000), "tile spanning ~5400 features"),
]


@pytest.mark.parametrize("P,T,H,block,note", WIDE_SPAN_CASES, ids=[c[-1] for c in WIDE_SPAN_CASES])
def test_wide_tile_span(P, T, H, block, note):
    say(f"case: wide span P={P} T={T} H={H} block={block} ({note})")
    cols = [block[0] + 5, H - 1]
    calib = [W.draw(P, 8, H, 3300 + b, cols=cols, outlier_factor=40.0, device=DEV)
             for b in range(2)]
    x = W.draw(P, T, H, 3400, cols=cols, outlier_factor=40.0, device=DEV)
    feats = np.arange(block[0], block[1])
    sel, *_ = run_both(calib, x, len(feats), 0.9, features=feats)
    assert sel["outlier_idx"].cpu().numpy().tolist() == feats.tolist()


def test_given_set_reproduces_the_ranked_selection():
    say("case: select_features(top-k set) == select_outliers")
    P, H, k = 8, 4104, 64
    x = W.draw(P, 16, H, 3200, cols=list(range(7, H, 67)), outlier_factor=40.0, device=DEV)
    rmin = torch.empty((P, H), dtype=torch.float32, device=DEV)
    rmax = torch.empty_like(rmin)
    B.btq_calib_update(x, rmin, rmax, 0.9, first_batch=True)
    ranked = B.btq_select_outliers(rmin, rmax, k)
    given = B.btq_select_features(rmin, rmax, ranked["outlier_idx"].cpu())
    torch.cuda.synchronize()
    for key in ranked:
        assert torch.equal(given[key], ranked[key]), key


def _shard_local(x: torch.Tensor, cols_by_shard: dict, factor: float) -> torch.Tensor:
    """x with the listed columns widened on one shard each."""
    xb = x.view(torch.bfloat16).clone()
    for p, cols in cols_by_shard.items():
        xb[p][:, cols] *= factor
    return xb.view(torch.int16)


# (P, T, H, k, rule, note)
RULE_CASES = [
    (4, 12, 1024, 8, "max", "max rule, shard-local outliers"),
    (8, 70, 2048, 64, "max", "max rule, fast path"),
    (3, 5, 250, 7, "max", "max rule, general paths"),
    (4, 12, 1024, 8, "sum", "sum rule through the rule entry"),
]


@pytest.mark.parametrize("P,T,H,k,rule,note", RULE_CASES, ids=[c[-1] for c in RULE_CASES])
def test_score_rule(P, T, H, k, rule, note):
    say(f"case: rule={rule} P={P} T={T} H={H} k={k} ({note})")
    everywhere = [H // 5, H // 2]
    local = {p: [(37 * p + 11) % H, (53 * p + 101) % H] for p in range(P)}

    def make(T_, seed):
        x = W.draw(P, T_, H, seed, cols=everywhere, outlier_factor=8.0, device=DEV)
        return _shard_local(x, local, 30.0)
    calib = [make(8, 3300 + b) for b in range(2)]
    sel, *_ = run_both(calib, make(T, 3400), k, 0.9, rule=rule)
    got = set(sel["outlier_idx"].cpu().tolist())
    if rule == "max" and k >= 2 * P:   # every shard-local column outranks the shared ones
        assert {c for cs in local.values() for c in cs} <= got


def test_given_set_rejects_bad_sets():
    rmin = torch.zeros((2, 16), dtype=torch.float32, device=DEV)
    for bad in ([3, 2], [1, 1], [-1, 4], [0, 16]):
        with pytest.raises(RuntimeError):
            B.btq_select_features(rmin, rmin, bad)


def test_misaligned_input_pointer():
    say("case: x base pointer offset by one element")
    P, T, H, k = 4, 10, 1024, 16
    calib = [W.draw(P, T, H, 3000 + b, device=DEV) for b in range(2)]
    x = W.draw(P, T, H, 3100, device=DEV)
    run_both(calib, x, k, 0.95, x_offset=1)


@pytest.mark.parametrize("pitch_extra", [0, 4, 130, 1])
def test_packed_pitch(pitch_extra):
    # pitch = code bytes (densest), a few bytes more, more than one line, and
    # an odd pitch (general kernels)
    P, T, H, k = 3, 20, 2048, 64
    say(f"case: packed pitch = code bytes + {pitch_extra}")
    calib = [W.draw(P, T, H, 3400 + b, device=DEV) for b in range(2)]
    x = W.draw(P, T, H, 3500, device=DEV)
    run_both(calib, x, k, 0.9, pitch=B.btq_packed_row_bytes(H, k) + pitch_extra)


def test_misaligned_parameter_arrays():
    say("case: scale, rscale, zero points and fmap offset by one element")
    P, T, H, k = 3, 12, 1024, 8
    calib = [W.draw(P, T, H, 3200 + b, device=DEV) for b in range(2)]
    x = W.draw(P, T, H, 3300, device=DEV)
    run_both(calib, x, k, 0.9, param_offset=1)


def test_bf16_sum_overflow_stays_in_its_feature():
    """BF16 features whose shard sums overflow fp32: their outputs are +inf on
    both sides (fp32 and bf16 receivers), and every other feature, the int4
    ones that share their lane included, stays finite and within tolerance."""
    P, T, H = 4, 6, 1024
    feats = np.array([100, 101, 102, 600])   # 100-102 share a receiver lane with 96-103
    say("case: BF16 sums that overflow to inf")
    xb = W.draw(P, T, H, 5200, device=DEV).view(torch.bfloat16).clone()
    ramp = torch.linspace(1.0e38, 3.0e38, P * T, device=DEV).reshape(P, T, 1)
    xb[:, :, feats.tolist()] = ramp.to(torch.bfloat16)
    x = xb.view(torch.int16)
    rmin = torch.empty((P, H), dtype=torch.float32, device=DEV)
    rmax = torch.empty_like(rmin)
    B.btq_calib_update(x, rmin, rmax, 0.9, first_batch=True)
    mn, mx = oracle_calib(u16(x), None, None, 0.9, first=True)
    sel_g = B.btq_select_features(rmin, rmax, feats)
    sel_o = O.select_features(mn, mx, feats)
    torch.cuda.synchronize()
    assert_selection_equal(sel_g, sel_o)
    pk, ol = B.btq_compress_pack(x, len(feats), sel_g["rscale"], sel_g["zero_point"],
                                 sel_g["outlier_idx"], sel_g["cmap"])
    par = (sel_g["scale"], sel_g["zero_point"], sel_g["fmap"])
    y = B.btq_decompress_reduce(pk, ol, H, *par)
    y16 = B.btq_decompress_reduce_bf16(pk, ol, H, *par)
    pk_o, ol_o = oracle_compress_rows(u16(x), sel_o)
    y_o = O.decompress_reduce(pk_o, ol_o, sel_o["scale"], sel_o["zero_point"], sel_o["fmap"])
    torch.cuda.synchronize()
    assert np.isposinf(y_o[:, feats]).all()
    yg = y.cpu().numpy()
    assert np.array_equal(yg[:, feats].view(np.uint32), y_o[:, feats].view(np.uint32))
    rest = np.setdiff1d(np.arange(H), feats)
    assert np.isfinite(yg[:, rest]).all()
    assert_y_close(yg[:, rest], y_o[:, rest], sel_o["scale"][:, rest], [])
    assert torch.equal(y16, y.to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("P", [8, 12])
def test_scales_past_2_to_104(P):
    """int4 features whose scale is 2^104 or more (values near 1e33): the
    receiver's fast arithmetic holds scales times 2^24, which would overflow,
    so such waves recompute their outputs term by term. Every output, those
    features' and their tiles' others, stays within the tolerance (P=12 also
    runs a later group of shards that adds to y)."""
    T, H = 40, 2048
    feats = np.array([5, 300, 301, 1030, 2047])
    huge = [700, 701, 1500]
    say(f"case: scales past 2^104, P={P}")

    def drawn(seed):
        xb = W.draw(P, T, H, seed, device=DEV).view(torch.bfloat16).clone()
        xb[:, :, huge] = xb[:, :, huge] * 1.0e33
        return xb.view(torch.int16)

    calib = [drawn(5400 + b) for b in range(2)]
    sel, *_ = run_both(calib, drawn(5500), len(feats), 0.9, features=feats)
    assert (sel["scale"][:, huge] >= 2.0 ** 104).all()


def test_momentum_range():
    say("case: momentum 0 and the largest fp32 below 1; 1 is rejected")
    P, T, H = 2, 8, 64
    xs = [W.draw(P, T, H, 4000 + b, device=DEV) for b in range(3)]
    for m in (0.0, float(np.nextafter(np.float32(1), np.float32(0)))):
        run_both(xs, xs[-1], 4, m)
    rmin = torch.empty((P, H), dtype=torch.float32, device=DEV)
    with pytest.raises(RuntimeError):
        B.btq_calib_update(xs[0], rmin, rmin.clone(), 1.0, first_batch=False)


def test_empty_batch_leaves_outputs_untouched():
    say("case: T=0")
    P, H, k = 3, 256, 8
    xs = [W.draw(P, 4, H, 5000, device=DEV)]
    rmin = torch.empty((P, H), dtype=torch.float32, device=DEV)
    rmax = torch.empty_like(rmin)
    B.btq_calib_update(xs[0], rmin, rmax, 0.9, True)
    sel = B.btq_select_outliers(rmin, rmax, k)
    x0 = torch.empty((P, 0, H), dtype=torch.int16, device=DEV)
    pk, ol = B.btq_compress_pack(x0, k, sel["rscale"], sel["zero_point"], sel["outlier_idx"],
                                 sel["cmap"])
    assert pk.shape == (P, 0, B.btq_packed_row_bytes(H, k)) and ol.shape == (P, 0, k)
    y = B.btq_decompress_reduce(pk, ol, H, sel["scale"], sel["zero_point"], sel["fmap"])
    torch.cuda.synchronize()
    assert y.shape == (0, H)


def test_repeatable_bitwise():
    say("case: repeat runs give identical bytes")
    w = W.WORKLOADS["tiny"]
    P, T, H, k = 8, 64, 4096, 64
    cols = W.outlier_columns(W.WORKLOADS["7b_prefill"])
    calib = [W.draw(P, T, H, 6000 + b, sigma=0.5, cols=cols, outlier_factor=100.0, device=DEV)
             for b in range(2)]
    x = W.draw(P, T, H, 6100, sigma=0.5, cols=cols, outlier_factor=100.0, device=DEV)
    outs = []
    for _ in range(2):
        rmin = torch.empty((P, H), dtype=torch.float32, device=DEV)
        rmax = torch.empty_like(rmin)
        for b, xb in enumerate(calib):
            B.btq_calib_update(xb, rmin, rmax, 0.9, b == 0)
        sel = B.btq_select_outliers(rmin, rmax, k)
        pk, ol = B.btq_compress_pack(x, k, sel["rscale"], sel["zero_point"], sel["outlier_idx"],
                                     sel["cmap"])
        y = B.btq_decompress_reduce(pk, ol, H, sel["scale"], sel["zero_point"], sel["fmap"])
        torch.cuda.synchronize()
        outs.append([t.cpu().clone() for t in (rmin, rmax, sel["scale"], sel["cmap"], pk, ol, y)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                           b.view(torch.uint8) if b.dtype != torch.uint8 else b)


def test_calibration_resume_is_bitwise():
    # The calibration state is the caller's running extremes: saving them to
    # host memory after some batches and continuing from a restored copy
    # gives the uninterrupted run's bytes (and the oracle's values).
    say("case: calibration checkpoint and resume")
    P, T, H = 4, 96, 2056
    xs = [W.draw(P, T, H, 9000 + b, sigma=0.5, cols=[3, 700, 2055], outlier_factor=30.0,
                 device=DEV) for b in range(4)]
    straight = [torch.empty((P, H), dtype=torch.float32, device=DEV) for _ in range(2)]
    for b, xb in enumerate(xs):
        B.btq_calib_update(xb, *straight, 0.9, first_batch=(b == 0))
    part = [torch.empty((P, H), dtype=torch.float32, device=DEV) for _ in range(2)]
    for b, xb in enumerate(xs[:2]):
        B.btq_calib_update(xb, *part, 0.9, first_batch=(b == 0))
    saved = [t.cpu().clone() for t in part]          # the checkpoint
    del part
    resumed = [t.to(DEV) for t in saved]
    for xb in xs[2:]:
        B.btq_calib_update(xb, *resumed, 0.9, first_batch=False)
    torch.cuda.synchronize()
    for a, b in zip(straight, resumed):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    mn = mx = None
    for b, xb in enumerate(xs):
        mn, mx = oracle_calib(u16(xb), mn, mx, 0.9, first=(b == 0))
    assert_stats_equal(resumed[0], mn, "run_min")
    assert_stats_equal(resumed[1], mx, "run_max")
