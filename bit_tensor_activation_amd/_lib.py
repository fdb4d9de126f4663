"""ctypes loader for libbtq.so: the C ABI declared in include/btq.h.

The loader fails loudly when the library is missing. There is no fallback
implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbtq.so")

# Every function that include/btq.h declares: (name, restype, argtypes).
_c = ctypes
_P, _I64, _I, _F, _SZ = _c.c_void_p, _c.c_int64, _c.c_int, _c.c_float, _c.c_size_t
SIGNATURES = {
    "btq_calib_update": (_I, [_P, _I64, _I64, _I64, _F, _I, _P, _P, _P, _SZ, _P]),
    "btq_calib_update_noalloc": (_I, [_P, _I64, _I64, _I64, _F, _I, _P, _P, _P]),
    "btq_calib_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "btq_select_outliers": (_I, [_P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "btq_select_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "btq_compress_pack": (_I, [_P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "btq_decompress_reduce": (_I, [_P, _P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "btq_packed_row_bytes": (_I64, [_I64, _I64]),
    "btq_decompress_reduce_bf16": (_I, [_P, _P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "btq_select_outliers_rule": (_I, [_P, _P, _I64, _I64, _I64, _I, _P, _P, _P, _P, _P, _P, _P,
                                      _SZ, _P]),
    "btq_select_features": (_I, [_P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P]),
    "btq_select_outliers_per_shard": (_I, [_P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P,
                                           _SZ, _P]),
    "btq_compress_pack_per_shard": (_I, [_P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "btq_decompress_reduce_per_shard": (_I, [_P, _P, _I64, _I64, _I64, _I64, _P, _P, _P, _P,
                                             _P]),
    "btq_compress_pack_ex": (_I, [_P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _I, _P, _I64, _P,
                                  _P]),
    "btq_decompress_reduce_ex": (_I, [_P, _I64, _P, _I64, _I64, _I64, _I64, _P, _P, _P, _I, _P,
                                      _I, _P]),
    "btq_packed_pitch": (_I64, [_I64, _I64]),
    "btq_status_str": (_c.c_char_p, [_I]),
    "btq_version": (_c.c_char_p, []),
}

BTQ_OK = 0
BTQ_ERR_ARG = -1
BTQ_ERR_SHAPE = -2
BTQ_ERR_ALIGN = -3
BTQ_ERR_WORKSPACE = -4
BTQ_ERR_HIP = -5
BTQ_ERR_SCRATCH = -6
BTQ_NOALLOC_SCRATCH_BYTES = 8 << 20

BTQ_SCORE_SUM = 0
BTQ_SCORE_MAX = 1

BTQ_SETS_SHARED = 0
BTQ_SETS_PER_SHARD = 1

BTQ_Y_F32 = 0
BTQ_Y_BF16 = 1

_lock = threading.Lock()
_lib = None


def load() -> ctypes.CDLL:
    """The loaded libbtq (once per process)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build the HIP library first "
                    "(python -m bit_tensor_activation_amd.build)")
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def check(status: int, what: str) -> None:
    if status != BTQ_OK:
        msg = load().btq_status_str(status).decode()
        raise RuntimeError(f"{what}: {msg} (status {status})")
