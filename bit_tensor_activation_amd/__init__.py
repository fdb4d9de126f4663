"""MI355X-native hybrid int4/BF16 codec for tensor-parallel partial sums.

The codec runs in HIP kernels for gfx950 behind the C ABI of libbtq.so
(include/btq.h). This package holds the kernels' sources (csrc/), the build
script, and a thin torch binding whose functions carry the C names.
"""
from .api import (  # noqa: F401
    btq_calib_update,
    btq_calib_update_noalloc,
    btq_calib_workspace_bytes,
    btq_compress_pack,
    btq_compress_pack_ex,
    btq_compress_pack_per_shard,
    btq_decompress_reduce,
    btq_decompress_reduce_bf16,
    btq_decompress_reduce_ex,
    btq_decompress_reduce_per_shard,
    btq_packed_pitch,
    btq_packed_row_bytes,
    btq_select_features,
    btq_select_outliers,
    btq_select_outliers_per_shard,
    btq_select_outliers_rule,
    btq_select_workspace_bytes,
    btq_status_str,
    btq_version,
)
from ._lib import LIB_PATH  # noqa: F401
