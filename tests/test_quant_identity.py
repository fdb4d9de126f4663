"""The sender's float-domain quantizer, checked on the CPU.

The sender finds the 4-bit code clamp(rint(fl(x*r)) + z, 0, 15) without a
float-to-integer conversion: it clamps fl(fl(x*r) + M), M = 1.5 * 2^23, to
[M - z, M + 15 - z] and takes the clamped float's bit pattern, which is
0x4B400000 + (q - z). The packed dword is then the sum of the patterns
shifted to their nibbles plus the constant -sum_e (0x4B400000 - z_e) << 4e,
mod 2^32. The widest-span kernel uses a form with fewer registers: it adds
z as a second float add and clamps fl(fl(v + M) + z) to [M, M + 15]. This test restates both forms in float32 numpy and compares them
over every finite bf16 pattern with a spread of scales and every zero
point, plus random products near rounding ties. The GPU parity tests check
the kernel itself.
"""
import numpy as np

F32 = np.float32
M = F32(12582912.0)


def direct(v, z):
    return np.clip(np.rint(v) + z, F32(0), F32(15)).astype(np.uint32)


def magic_bits(v, z):
    s = (v + M).astype(F32)
    c = np.minimum(np.maximum(s, M - z), M + (F32(15) - z)).astype(F32)
    return c.view(np.uint32)


def lean_bits(v, z):
    """The form with fewer registers: fl(fl(v + M) + z) clamped to [M, M + 15]."""
    s = ((v + M).astype(F32) + z).astype(F32)
    c = np.minimum(np.maximum(s, M), M + F32(15)).astype(F32)
    return c.view(np.uint32)


def test_every_bf16_pattern():
    b = np.arange(65536, dtype=np.uint32)
    b = b[((b >> 7) & 0xFF) != 0xFF]   # finite patterns
    x = (b << 16).view(F32)
    for r in (1.0, 0.5, 2.0, 1 / 3, 7.5, 1e-3, 1e3, 1e30, 1e-30, 15 / 7):
        v = (x * F32(r)).astype(F32)
        for z in range(16):
            zf = F32(z)
            q = direct(v, zf)
            bits = magic_bits(v, zf)
            # one feature in nibble 0: the pattern minus (0x4B400000 - z)
            got = (bits - (np.uint32(0x4B400000) - np.uint32(z))).astype(np.uint32)
            assert np.array_equal(got, q), (r, z)
            lean = (lean_bits(v, zf) - np.uint32(0x4B400000)).astype(np.uint32)
            assert np.array_equal(lean, q), (r, z, "lean")


def test_packed_sum_and_ties():
    rng = np.random.default_rng(7)
    n = 200000
    # products near half-integers and across the clamp range
    v = (rng.integers(-40, 40, size=(n, 8)) / 2).astype(F32)
    v = np.where(rng.random((n, 8)) < 0.5, np.nextafter(v, F32(np.inf)), v).astype(F32)
    v = np.where(rng.random((n, 8)) < 0.1, (rng.standard_normal((n, 8)) * 1e7).astype(F32), v)
    z = rng.integers(0, 16, size=(n, 8)).astype(F32)
    q = direct(v, z)
    want = np.zeros(n, dtype=np.uint64)
    for e in range(8):
        want |= q[:, e].astype(np.uint64) << np.uint64(4 * e)
    k = np.zeros(n, dtype=np.uint64)
    w = np.zeros(n, dtype=np.uint64)
    for e in range(8):
        k -= (np.uint64(0x4B400000) - z[:, e].astype(np.uint64)) << np.uint64(4 * e)
        w += magic_bits(v[:, e], z[:, e]).astype(np.uint64) << np.uint64(4 * e)
    got = (w + k) & np.uint64(0xFFFFFFFF)
    assert np.array_equal(got, want)
    kl = np.uint64(0)
    wl = np.zeros(n, dtype=np.uint64)
    for e in range(8):
        kl -= np.uint64(0x4B400000) << np.uint64(4 * e)
        wl += lean_bits(v[:, e], z[:, e]).astype(np.uint64) << np.uint64(4 * e)
    assert np.array_equal((wl + kl) & np.uint64(0xFFFFFFFF), want)
