"""The receiver's int4 arithmetic, bit for bit (GPU).

The parity tests hold y to a tolerance of the oracle's sequential sum. The
receiver documents how it evaluates an int4 feature (include/btq.h, the
receiver): it starts from the constant b = -sum_p z_p*s_p, built by fp32
fmas in shard order from +0, and adds one fma(q_p, s_p, acc) per shard in
shard order, each rounded once. Its kernels compute those fmas with a mixed
f16/f32 instruction on codes held as f16 denormals and scales times 2^24;
this test checks, over whole outputs, that the result is exactly that
sequence of correctly rounded fp32 fmas (past 8 shards, per group of 8,
each later group starting from y plus its own constant, one fp32 add). The fmas are evaluated here with
Python integers (exact products and sums, then one round-to-nearest-even to
fp32), from the oracle's codes and parameters; only the receiver's output
comes from the GPU.
"""
import numpy as np
import pytest
import torch

import bit_tensor_activation_amd as B
from oracle import oracle as O
import workloads as W
from helpers import assert_bits_equal, oracle_calib, oracle_compress_rows, say, u16

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _parts(x: np.float32):
    """(m, e) with x = m * 2**e exactly (finite fp32)."""
    b = int(np.float32(x).view(np.uint32))
    sign, ex, m = b >> 31, (b >> 23) & 0xFF, b & 0x7FFFFF
    mant, exp = (m, -149) if ex == 0 else (m | 0x800000, ex - 150)
    return (-mant if sign else mant), exp


def _round_f32(n: int, e: int) -> float:
    """The fp32 nearest n * 2**e, ties to even (no overflow on these inputs)."""
    if n == 0:
        return 0.0
    neg, n = n < 0, abs(n)
    top = e + n.bit_length() - 1          # 2**top <= value < 2**(top + 1)
    lsb = max(top - 23, -149)             # weight of the last kept bit
    sh = lsb - e
    if sh > 0:
        q, r = divmod(n, 1 << sh)
        half = 1 << (sh - 1)
        if r > half or (r == half and q & 1):
            q += 1
    else:
        q = n << -sh
    v = float(np.float32(np.ldexp(float(q), lsb)))
    return -v if neg else v


def fma32(a: int, s: float, c: float) -> float:
    """fl(a*s + c) for a small integer a and fp32 s, c: exact, then rounded."""
    ms, es = _parts(s)
    mc, ec = _parts(c)
    e0 = min(es, ec)
    n = a * ms * (1 << (es - e0)) + mc * (1 << (ec - e0))
    return _round_f32(n, e0)


def add32(a: float, b: float) -> float:
    ma, ea = _parts(a)
    mb, eb = _parts(b)
    e0 = min(ea, eb)
    return _round_f32(ma * (1 << (ea - e0)) + mb * (1 << (eb - e0)), e0)


def expected_int4(pk, scale, zp, fmap, cols, group=8):
    """y[t, h] for the int4 features h in cols, evaluated as the receiver does:
    per group of `group` shards in shard order, a constant from +0 and one
    fma per shard; a later group starts from the earlier groups' y plus its
    own constant."""
    P, T, _ = pk.shape
    out = np.zeros((T, len(cols)), np.float32)
    groups = [range(g, min(g + group, P)) for g in range(0, P, group)]
    for ci, h in enumerate(cols):
        j = int(fmap[h])
        byte, hi = j >> 1, j & 1
        s = [float(scale[p, h]) for p in range(P)]
        consts = []
        for g in groups:
            b = 0.0
            for p in g:
                b = fma32(-int(zp[p, h]), s[p], b)
            consts.append(b)
        codes = pk[:, :, byte]
        codes = (codes >> 4) if hi else (codes & 0xF)
        for t in range(T):
            acc = None
            for g, b in zip(groups, consts):
                acc = b if acc is None else add32(acc, b)
                for p in g:
                    acc = fma32(int(codes[p, t]), s[p], acc)
            out[t, ci] = acc
    return out


def _shards_scaled(x16: torch.Tensor, factors) -> torch.Tensor:
    xb = x16.view(torch.bfloat16).clone()
    for p, f in enumerate(factors):
        xb[p] *= f
    return xb.view(torch.int16)


CASES = [
    # P, T, H, k, shard scale factors (None: 1), note
    (8, 12, 2048, 64, None, "8 shards, 4 tiles"),
    (3, 9, 1024, 8, None, "3 shards"),
    (8, 6, 1024, 16, [1e-30, 1.0, 1e20, 3.0, 1e-10, 1e10, 0.5, 1e30], "scales 2^-100 to 2^100 apart"),
    (12, 5, 1024, 16, None, "12 shards: groups of 8 and 4, the second adding to y"),
]


@pytest.mark.parametrize("P,T,H,k,factors,note", CASES, ids=[c[-1] for c in CASES])
def test_int4_features_are_the_documented_fma_sequence(P, T, H, k, factors, note):
    say(f"case: receiver fma order, P={P} T={T} H={H} k={k} ({note})")
    draw = lambda seed, t: W.draw(P, t, H, seed, base="laplace", cols=[7, 600], outlier_factor=30.0,
                                  device=DEV)
    calib = [draw(6100 + b, 8) for b in range(2)]
    x = draw(6200, T)
    if factors is not None:
        calib = [_shards_scaled(c, factors) for c in calib]
        x = _shards_scaled(x, factors)
    rmin = torch.empty((P, H), dtype=torch.float32, device=DEV)
    rmax = torch.empty_like(rmin)
    mn = mx = None
    for b, xb in enumerate(calib):
        B.btq_calib_update(xb, rmin, rmax, 0.9, first_batch=(b == 0))
        mn, mx = oracle_calib(u16(xb), mn, mx, 0.9, first=(b == 0))
    sel_g = B.btq_select_outliers(rmin, rmax, k)
    sel_o = O.select_outliers(mn, mx, k)
    pk, ol = B.btq_compress_pack(x, k, sel_g["rscale"], sel_g["zero_point"], sel_g["outlier_idx"],
                                 sel_g["cmap"])
    pkp, olp = B.btq_compress_pack_ex(x, k, sel_g["rscale"], sel_g["zero_point"],
                                      sel_g["outlier_idx"], sel_g["cmap"],
                                      pitch=B.btq_packed_pitch(H, k))
    par = (sel_g["scale"], sel_g["zero_point"], sel_g["fmap"])
    y = B.btq_decompress_reduce(pk, ol, H, *par)
    yp = B.btq_decompress_reduce_ex(pkp, olp, H, *par)
    pk_o, _ = oracle_compress_rows(u16(x), sel_o)
    torch.cuda.synchronize()
    assert_bits_equal(pk, pk_o, "packed")
    cols = [h for h in range(H) if sel_o["fmap"][h] >= 0]
    want = expected_int4(pk_o, sel_o["scale"], sel_o["zero_point"], sel_o["fmap"], cols)
    for name, yy in (("dense rows", y), ("padded rows", yp)):
        got = yy.cpu().numpy()[:, cols]
        same = (got == want)   # +0 and -0 count as equal
        assert same.all(), (name, int((~same).sum()), "of", same.size)
