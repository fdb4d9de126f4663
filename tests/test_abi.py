"""C ABI checks that need no GPU: the library loads, exports every function
that include/btq.h declares, and rejects bad arguments before any HIP call.
"""
import ctypes
import os
import re

import pytest

from bit_tensor_activation_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "btq.h")

OK, ARG, SHAPE, ALIGN, WS = (_lib.BTQ_OK, _lib.BTQ_ERR_ARG, _lib.BTQ_ERR_SHAPE,
                             _lib.BTQ_ERR_ALIGN, _lib.BTQ_ERR_WORKSPACE)
SHARED, PER = _lib.BTQ_SETS_SHARED, _lib.BTQ_SETS_PER_SHARD
F32, BF16 = _lib.BTQ_Y_F32, _lib.BTQ_Y_BF16
# Fake, never dereferenced "device" addresses: every call below returns from
# host-side validation before it touches the HIP runtime.
A = 0x10000          # 64 KiB aligned
BIG = 1 << 40


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(btq_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(_lib.SIGNATURES), set(names) ^ set(_lib.SIGNATURES)
    for n in names:
        assert hasattr(lib, n), n


def test_the_four_calls_of_the_path_have_their_arguments():
    # calib_update, select_outliers, compress_pack, decompress_reduce with the
    # arguments their header comments document (pointer, int64, float, size_t)
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)

    def args(name):
        m = re.search(name + r"\s*\(([^)]*)\)", text)
        return [a.split()[-1].lstrip("*") for a in m.group(1).split(",")]
    assert args("btq_compress_pack") == ["x", "P", "T", "H", "k", "rscale", "zero_point",
                                         "outlier_idx", "cmap", "packed", "outliers", "stream"]
    assert args("btq_decompress_reduce") == ["packed", "outliers", "P", "T", "H", "k", "scale",
                                             "zero_point", "fmap", "y", "stream"]
    assert args("btq_select_outliers") == ["run_min", "run_max", "P", "H", "k", "scale",
                                           "rscale", "zero_point", "outlier_idx", "fmap", "cmap",
                                           "workspace", "workspace_bytes", "stream"]
    assert args("btq_calib_update") == ["x", "P", "T", "H", "momentum", "first_batch",
                                        "run_min", "run_max", "workspace", "workspace_bytes",
                                        "stream"]
    assert args("btq_select_workspace_bytes") == ["P", "H", "k"]


def test_status_strings_and_version(lib):
    for s in (OK, ARG, SHAPE, ALIGN, WS, _lib.BTQ_ERR_HIP, 17):
        assert lib.btq_status_str(s)
    assert re.fullmatch(rb"\d+\.\d+\.\d+", lib.btq_version())


def test_size_helpers(lib):
    assert lib.btq_packed_row_bytes(4096, 64) == 2016
    assert lib.btq_packed_row_bytes(5, 2) == 2
    assert lib.btq_packed_row_bytes(8, 8) == 0
    assert lib.btq_packed_row_bytes(8, 9) == -1
    assert lib.btq_packed_row_bytes(0, 0) == -1
    assert lib.btq_packed_pitch(4096, 64) == 2048
    assert lib.btq_packed_pitch(8192, 256) == 3968
    assert lib.btq_packed_pitch(5, 2) == 128
    assert lib.btq_packed_pitch(8, 8) == 0
    assert lib.btq_packed_pitch(8, 9) == -1
    assert lib.btq_select_workspace_bytes(8, 4096, 64) == 8 * 4096 * 4
    assert lib.btq_select_workspace_bytes(0, 4096, 64) == 0
    assert lib.btq_select_workspace_bytes(8, 4096, 4097) == 0
    n = lib.btq_calib_workspace_bytes(8, 2048, 4096)
    assert n > 0 and n % (2 * 8 * 4096 * 4) == 0
    assert lib.btq_calib_workspace_bytes(8, 0, 4096) == 0


def calib(lib, x=A, P=2, T=4, H=16, m=0.9, rmin=A, rmax=A, ws=A, wsb=BIG):
    return lib.btq_calib_update(x, P, T, H, m, 0, rmin, rmax, ws, wsb, None)


def test_calib_validation(lib):
    assert calib(lib, P=0) == SHAPE
    assert calib(lib, T=0) == SHAPE
    assert calib(lib, H=0) == SHAPE
    assert calib(lib, P=70000) == SHAPE
    assert calib(lib, H=(1 << 30) + 1) == SHAPE
    assert calib(lib, P=65535, T=1 << 40, H=1 << 20) == SHAPE     # P*T*H overflow
    assert calib(lib, x=None) == ARG
    assert calib(lib, rmin=None) == ARG
    assert calib(lib, m=-0.1) == ARG
    assert calib(lib, m=1.0) == ARG          # momentum must lie in [0, 1)
    assert calib(lib, m=1.5) == ARG
    assert calib(lib, m=float("nan")) == ARG
    assert calib(lib, x=A + 1) == ALIGN
    assert calib(lib, rmax=A + 2) == ALIGN
    assert calib(lib, ws=None) == ARG
    assert calib(lib, wsb=8) == WS
    assert calib(lib, ws=A + 2) == ALIGN


def select(lib, rmin=A, rmax=A, P=2, H=16, k=4, sc=A, rs=A, zp=A, idx=A, fmap=A, cmap=A, ws=A,
           wsb=BIG):
    return lib.btq_select_outliers(rmin, rmax, P, H, k, sc, rs, zp, idx, fmap, cmap, ws, wsb, None)


def test_select_validation(lib):
    assert select(lib, k=-1) == SHAPE
    assert select(lib, k=17) == SHAPE
    assert select(lib, P=0) == SHAPE
    assert select(lib, sc=None) == ARG
    assert select(lib, rs=None) == ARG
    assert select(lib, zp=None) == ARG
    assert select(lib, fmap=None) == ARG
    assert select(lib, idx=None) == ARG
    assert select(lib, cmap=None) == ARG
    assert select(lib, ws=None) == ARG
    assert select(lib, wsb=2 * 16 * 4 - 1) == WS
    assert select(lib, sc=A + 1) == ALIGN
    assert select(lib, cmap=A + 2) == ALIGN
    assert select(lib, ws=A + 2) == ALIGN
    # zero-length outputs may be NULL; these pass validation, so they are not
    # called here (they would launch).


def test_select_rule_validation(lib):
    def call(rule, k=4):
        return lib.btq_select_outliers_rule(A, A, 2, 16, k, rule, A, A, A, A, A, A, A, BIG, None)
    assert call(2) == ARG
    assert call(-1) == ARG
    assert call(_lib.BTQ_SCORE_MAX, k=17) == SHAPE


def test_per_shard_validation(lib):
    def sel(P=2, H=16, k=4, idx=A, cmap=A, ws=A, wsb=BIG, fmap=A):
        return lib.btq_select_outliers_per_shard(A, A, P, H, k, A, A, A, idx, fmap, cmap, ws, wsb,
                                                 None)
    assert sel(k=17) == SHAPE
    assert sel(P=0) == SHAPE
    assert sel(idx=None) == ARG
    assert sel(cmap=None) == ARG
    assert sel(fmap=None) == ARG
    assert sel(ws=None) == ARG
    assert sel(wsb=2 * 16 * 4 - 1) == WS
    assert sel(fmap=A + 2) == ALIGN

    def comp(x=A, k=4, idx=A, rs=A):
        return lib.btq_compress_pack_per_shard(x, 2, 4, 16, k, rs, A, idx, A, A, A, None)
    assert comp(k=17) == SHAPE
    assert comp(idx=None) == ARG
    assert comp(rs=None) == ARG
    assert comp(x=A + 1) == ALIGN

    def dec(y=A, k=4, fmap=A, zp=A, T=4):
        return lib.btq_decompress_reduce_per_shard(A, A, 2, T, 16, k, A, zp, fmap, y, None)
    assert dec(k=-1) == SHAPE
    assert dec(fmap=None) == ARG
    assert dec(zp=None) == ARG
    assert dec(y=None) == ARG
    assert dec(y=A + 2) == ALIGN
    assert dec(T=0, y=None) == OK      # empty batch: nothing to do, nothing enqueued


def host_set(*h):
    arr = (ctypes.c_int32 * max(len(h), 1))(*h)
    return arr, ctypes.addressof(arr)


GOOD_SET = host_set(1, 5, 9, 15)


def select_set(lib, rmin=A, rmax=A, P=2, H=16, k=4, feat=GOOD_SET[1], sc=A, rs=A, zp=A, idx=A,
               fmap=A, cmap=A):
    return lib.btq_select_features(rmin, rmax, P, H, k, feat, sc, rs, zp, idx, fmap, cmap, None)


def test_select_features_validation(lib):
    assert select_set(lib, k=-1) == SHAPE
    assert select_set(lib, k=17) == SHAPE
    assert select_set(lib, H=0) == SHAPE
    assert select_set(lib, feat=None) == ARG
    assert select_set(lib, idx=None) == ARG
    assert select_set(lib, cmap=None) == ARG
    assert select_set(lib, zp=None) == ARG
    assert select_set(lib, feat=GOOD_SET[1] + 2) == ALIGN
    assert select_set(lib, fmap=A + 1) == ALIGN
    # sets that are not k distinct ascending features of [0, H): rejected on
    # the host before anything is enqueued
    for bad in ((1, 5, 5, 9), (5, 1, 9, 15), (-1, 5, 9, 15), (1, 5, 9, 16), (0, 1, 2, 99)):
        arr, ptr = host_set(*bad)
        assert select_set(lib, feat=ptr) == ARG, bad


def compress(lib, x=A, P=2, T=4, H=16, k=4, rs=A, zp=A, idx=A, cmap=A, pk=A, ol=A):
    return lib.btq_compress_pack(x, P, T, H, k, rs, zp, idx, cmap, pk, ol, None)


def test_compress_validation(lib):
    assert compress(lib, k=17) == SHAPE
    assert compress(lib, k=-1) == SHAPE
    assert compress(lib, T=-1) == SHAPE
    assert compress(lib, P=0) == SHAPE
    assert compress(lib, H=0) == SHAPE
    assert compress(lib, rs=None) == ARG
    assert compress(lib, zp=None) == ARG
    assert compress(lib, idx=None) == ARG
    assert compress(lib, cmap=None) == ARG
    assert compress(lib, x=None) == ARG
    assert compress(lib, pk=None) == ARG
    assert compress(lib, ol=None) == ARG
    assert compress(lib, x=A + 1) == ALIGN
    assert compress(lib, rs=A + 2) == ALIGN
    assert compress(lib, ol=A + 1) == ALIGN
    # T == 0 is an empty batch: valid, nothing enqueued
    assert compress(lib, T=0, x=None, pk=None, ol=None) == OK
    # zero-length maps may be NULL
    assert compress(lib, T=0, k=0, idx=None) == OK
    assert compress(lib, T=0, k=16, cmap=None) == OK


def compress_ex(lib, x=A, P=2, T=4, H=16, k=4, sets=SHARED, pk=A, pitch=128, ol=A):
    return lib.btq_compress_pack_ex(x, P, T, H, k, A, A, A, A, sets, pk, pitch, ol, None)


def test_compress_ex_validation(lib):
    assert compress_ex(lib, pitch=5) == SHAPE       # below the 6 code bytes of a row
    assert compress_ex(lib, pitch=-1) == SHAPE
    assert compress_ex(lib, T=1 << 40, P=1, H=16, pitch=1 << 30) == SHAPE   # P*T*pitch overflow
    assert compress_ex(lib, sets=2) == ARG
    assert compress_ex(lib, sets=-1) == ARG
    assert compress_ex(lib, pk=None) == ARG
    assert compress_ex(lib, T=0, pitch=6, x=None, pk=None, ol=None) == OK
    assert compress_ex(lib, T=0, pitch=6, sets=PER) == OK


def decompress(lib, pk=A, ol=A, P=2, T=4, H=16, k=4, sc=A, zp=A, fmap=A, y=A):
    return lib.btq_decompress_reduce(pk, ol, P, T, H, k, sc, zp, fmap, y, None)


def test_decompress_validation(lib):
    assert decompress(lib, k=17) == SHAPE
    assert decompress(lib, P=0) == SHAPE
    assert decompress(lib, H=0) == SHAPE
    assert decompress(lib, sc=None) == ARG
    assert decompress(lib, zp=None) == ARG
    assert decompress(lib, fmap=None) == ARG
    assert decompress(lib, y=None) == ARG
    assert decompress(lib, pk=None) == ARG
    assert decompress(lib, ol=None) == ARG
    assert decompress(lib, y=A + 2) == ALIGN
    assert decompress(lib, sc=A + 1) == ALIGN
    assert decompress(lib, fmap=A + 2) == ALIGN
    assert decompress(lib, T=0, y=None, pk=None, ol=None) == OK
    assert decompress(lib, T=0, k=16, pk=None) == OK


def decompress_ex(lib, pitch=128, T=4, k=4, sets=SHARED, y=A, ytype=F32):
    return lib.btq_decompress_reduce_ex(A, pitch, A, 2, T, 16, k, A, A, A, sets, y, ytype, None)


def test_decompress_ex_validation(lib):
    assert decompress_ex(lib, pitch=5) == SHAPE
    assert decompress_ex(lib, sets=3) == ARG
    assert decompress_ex(lib, ytype=2) == ARG
    assert decompress_ex(lib, y=A + 2) == ALIGN              # fp32 y: 4-byte alignment
    assert decompress_ex(lib, y=A + 1, ytype=BF16) == ALIGN  # bf16 y: 2-byte alignment
    assert decompress_ex(lib, T=0, ytype=BF16, sets=PER) == OK


def decompress_bf16(lib, pk=A, ol=A, P=2, T=4, H=16, k=4, sc=A, zp=A, fmap=A, y=A):
    return lib.btq_decompress_reduce_bf16(pk, ol, P, T, H, k, sc, zp, fmap, y, None)


def test_decompress_bf16_validation(lib):
    assert decompress_bf16(lib, k=17) == SHAPE
    assert decompress_bf16(lib, sc=None) == ARG
    assert decompress_bf16(lib, y=None) == ARG
    assert decompress_bf16(lib, y=A + 1) == ALIGN      # bf16 y: 2-byte alignment
    assert decompress_bf16(lib, sc=A + 2) == ALIGN
    assert decompress_bf16(lib, T=0, y=None, pk=None, ol=None) == OK
