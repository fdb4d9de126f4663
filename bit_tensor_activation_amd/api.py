"""Python binding of libbtq: one function per C entry point, same names.

The functions only marshal arguments. They check tensor dtypes, shapes and
devices, allocate outputs and workspaces with torch when the caller passes
none, and hand raw device pointers and a HIP stream to the C ABI. Every step
of the codec runs in the library's HIP kernels; nothing here computes on
tensor values.

Streams: every function takes `stream=None` (torch's current stream) or a
torch stream or a raw hipStream_t handle. Outputs and workspaces that a
function allocates are allocated with that stream current, so torch's
caching allocator orders their reuse after the launched kernels.

Layouts (contiguous, row-major, last index fastest):
  x             int16 [P,T,H]  bf16 bit patterns (torch.bfloat16 is also accepted)
  run_min/max   float32 [P,H]
  scale, rscale float32 [P,H];  zero_point uint8 [P,H]
  outlier_idx   int32 [k];  fmap int32 [H];  cmap int32 [H-k]
                (per-shard sets: [P,k], [P,H], [P,H-k])
  packed        uint8 [P,T,Bq], Bq = ceil((H-k)/2); the *_ex calls take
                [P,T,pitch] with pitch >= Bq (btq_packed_pitch(H,k) rounds
                Bq up to 128)
  outliers      int16 [P,T,k]
  y             float32 [T,H]  (bf16 bits, int16 [T,H], for bf16 output)
"""
from __future__ import annotations

import contextlib
from typing import Optional

import torch

from . import _lib


def _device(x: torch.Tensor) -> torch.device:
    if x.device.type != "cuda":
        raise ValueError("libbtq runs on the GPU: pass device tensors")
    return x.device


def _launch(dev: torch.device, stream):
    """(hipStream_t handle, context that makes that stream current)."""
    if stream is None:
        return int(torch.cuda.current_stream(dev).cuda_stream), contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream), device=dev)
    return int(stream.cuda_stream), torch.cuda.stream(stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None or t.numel() == 0 else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtypes, shape, dev) -> None:
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device != dev:
        raise ValueError(f"{name}: on {t.device}, expected {dev}")


_BF16 = (torch.int16, torch.bfloat16)


def _bits(x: torch.Tensor) -> torch.Tensor:
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x


def btq_packed_row_bytes(H: int, k: int) -> int:
    n = _lib.load().btq_packed_row_bytes(H, k)
    if n < 0:
        raise ValueError(f"invalid H={H}, k={k}")
    return int(n)


def btq_packed_pitch(H: int, k: int) -> int:
    n = _lib.load().btq_packed_pitch(H, k)
    if n < 0:
        raise ValueError(f"invalid H={H}, k={k}")
    return int(n)


def btq_calib_workspace_bytes(P: int, T: int, H: int) -> int:
    return int(_lib.load().btq_calib_workspace_bytes(P, T, H))


def btq_select_workspace_bytes(P: int, H: int, k: int) -> int:
    return int(_lib.load().btq_select_workspace_bytes(P, H, k))


def btq_calib_update(x: torch.Tensor, run_min: torch.Tensor, run_max: torch.Tensor,
                     momentum: float, first_batch: bool,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Fold one calibration batch x [P,T,H] into run_min/run_max [P,H] in place."""
    dev = _device(x)
    P, T, H = x.shape
    _need(x, "x", _BF16, (P, T, H), dev)
    _need(run_min, "run_min", (torch.float32,), (P, H), dev)
    _need(run_max, "run_max", (torch.float32,), (P, H), dev)
    sh, ctx = _launch(dev, stream)
    with ctx:
        need = btq_calib_workspace_bytes(P, T, H)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        st = _lib.load().btq_calib_update(_ptr(_bits(x)), P, T, H, float(momentum),
                                          int(bool(first_batch)), _ptr(run_min), _ptr(run_max),
                                          _ptr(workspace),
                                          workspace.numel() * workspace.element_size(), sh)
    _lib.check(st, "btq_calib_update")


def btq_calib_update_noalloc(x: torch.Tensor, run_min: torch.Tensor, run_max: torch.Tensor,
                             momentum: float, first_batch: bool, stream=None) -> None:
    """btq_calib_update with the library's static scratch: nothing is
    allocated, here or in the library (P*H at most 2^20)."""
    dev = _device(x)
    P, T, H = x.shape
    _need(x, "x", _BF16, (P, T, H), dev)
    _need(run_min, "run_min", (torch.float32,), (P, H), dev)
    _need(run_max, "run_max", (torch.float32,), (P, H), dev)
    sh, ctx = _launch(dev, stream)
    with ctx:
        st = _lib.load().btq_calib_update_noalloc(_ptr(_bits(x)), P, T, H, float(momentum),
                                                  int(bool(first_batch)), _ptr(run_min),
                                                  _ptr(run_max), sh)
    _lib.check(st, "btq_calib_update_noalloc")


def _select_outputs(run_min, run_max, k, out, per_shard=False) -> dict:
    dev = _device(run_min)
    P, H = run_min.shape
    _need(run_min, "run_min", (torch.float32,), (P, H), dev)
    _need(run_max, "run_max", (torch.float32,), (P, H), dev)
    if not 0 <= k <= H:
        raise ValueError(f"k={k} outside [0, H={H}]")
    lead = (P,) if per_shard else ()
    shapes = (("scale", torch.float32, (P, H)), ("rscale", torch.float32, (P, H)),
              ("zero_point", torch.uint8, (P, H)), ("outlier_idx", torch.int32, lead + (k,)),
              ("fmap", torch.int32, lead + (H,)), ("cmap", torch.int32, lead + (H - k,)))
    o = dict(out or {})
    for name, dt, shp in shapes:
        o.setdefault(name, torch.empty(shp, dtype=dt, device=dev))
        _need(o[name], name, (dt,), shp, dev)
    return o


def _select(name, run_min, run_max, k, extra, out, workspace, stream, per_shard=False) -> dict:
    dev = _device(run_min)
    P, H = run_min.shape
    sh, ctx = _launch(dev, stream)
    with ctx:
        o = _select_outputs(run_min, run_max, k, out, per_shard)
        if workspace is None:
            workspace = torch.empty(btq_select_workspace_bytes(P, H, k), dtype=torch.uint8,
                                    device=dev)
        st = getattr(_lib.load(), name)(
            _ptr(run_min), _ptr(run_max), P, H, k, *extra, _ptr(o["scale"]), _ptr(o["rscale"]),
            _ptr(o["zero_point"]), _ptr(o["outlier_idx"]), _ptr(o["fmap"]), _ptr(o["cmap"]),
            _ptr(workspace), workspace.numel() * workspace.element_size(), sh)
    _lib.check(st, name)
    return o


def btq_select_outliers(run_min: torch.Tensor, run_max: torch.Tensor, k: int, out: dict = None,
                        workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Parameters and the BF16 feature set from the running extremes.

    Returns a dict with scale, rscale, zero_point, outlier_idx, fmap and cmap.
    """
    return _select("btq_select_outliers", run_min, run_max, k, (), out, workspace, stream)


_RULES = {"sum": _lib.BTQ_SCORE_SUM, "max": _lib.BTQ_SCORE_MAX}


def btq_select_outliers_rule(run_min: torch.Tensor, run_max: torch.Tensor, k: int, rule: str,
                             out: dict = None, workspace: Optional[torch.Tensor] = None,
                             stream=None) -> dict:
    """btq_select_outliers with the rank score chosen by `rule`: "sum" (the
    per-shard ranges added) or "max" (the widest shard's range)."""
    if rule not in _RULES:
        raise ValueError(f"rule must be one of {sorted(_RULES)}")
    return _select("btq_select_outliers_rule", run_min, run_max, k, (_RULES[rule],), out,
                   workspace, stream)


def btq_select_outliers_per_shard(run_min: torch.Tensor, run_max: torch.Tensor, k: int,
                                  out: dict = None, workspace: Optional[torch.Tensor] = None,
                                  stream=None) -> dict:
    """One BF16 set per shard, ranked by the shard's own ranges. Returns
    scale, rscale, zero_point [P,H], outlier_idx [P,k], fmap [P,H] and
    cmap [P,H-k]."""
    return _select("btq_select_outliers_per_shard", run_min, run_max, k, (), out, workspace,
                   stream, per_shard=True)


def btq_select_features(run_min: torch.Tensor, run_max: torch.Tensor, features, out: dict = None,
                        stream=None) -> dict:
    """Parameters and maps for a BF16 set chosen by the caller.

    features: the k BF16 features (any int sequence, array or tensor), distinct
    and ascending. Returns the same dict as btq_select_outliers. The call
    waits for its stream, because the set travels from host memory.
    """
    dev = _device(run_min)
    P, H = run_min.shape
    feat = torch.as_tensor(features).to(device="cpu", dtype=torch.int32).contiguous().reshape(-1)
    k = feat.numel()
    sh, ctx = _launch(dev, stream)
    with ctx:
        o = _select_outputs(run_min, run_max, k, out)
        st = _lib.load().btq_select_features(
            _ptr(run_min), _ptr(run_max), P, H, k, _ptr(feat), _ptr(o["scale"]), _ptr(o["rscale"]),
            _ptr(o["zero_point"]), _ptr(o["outlier_idx"]), _ptr(o["fmap"]), _ptr(o["cmap"]), sh)
        _lib.check(st, "btq_select_features")
        torch.cuda.current_stream(dev).synchronize()
    return o


def btq_compress_pack_ex(x: torch.Tensor, k: int, rscale: torch.Tensor, zero_point: torch.Tensor,
                         outlier_idx: torch.Tensor, cmap: torch.Tensor, per_shard: bool = False,
                         packed: Optional[torch.Tensor] = None,
                         outliers: Optional[torch.Tensor] = None, pitch: Optional[int] = None,
                         stream=None):
    """Sender message of every shard: (packed uint8 [P,T,pitch], outliers int16 [P,T,k]).

    The row pitch is packed.shape[2] when `packed` is given, else `pitch`,
    else Bq (rows with no gap). per_shard: outlier_idx [P,k] and cmap
    [P,H-k] hold one set per shard.
    """
    dev = _device(x)
    P, T, H = x.shape
    _need(x, "x", _BF16, (P, T, H), dev)
    if packed is not None:
        pitch = packed.shape[2] if packed.dim() == 3 else -1
    elif pitch is None:
        pitch = btq_packed_row_bytes(H, k)
    _need(rscale, "rscale", (torch.float32,), (P, H), dev)
    _need(zero_point, "zero_point", (torch.uint8,), (P, H), dev)
    lead = (P,) if per_shard else ()
    _need(outlier_idx, "outlier_idx", (torch.int32,), lead + (k,), dev)
    _need(cmap, "cmap", (torch.int32,), lead + (H - k,), dev)
    sh, ctx = _launch(dev, stream)
    with ctx:
        if packed is None:
            packed = torch.empty((P, T, pitch), dtype=torch.uint8, device=dev)
        if outliers is None:
            outliers = torch.empty((P, T, k), dtype=torch.int16, device=dev)
        _need(packed, "packed", (torch.uint8,), (P, T, pitch), dev)
        _need(outliers, "outliers", _BF16, (P, T, k), dev)
        sets = _lib.BTQ_SETS_PER_SHARD if per_shard else _lib.BTQ_SETS_SHARED
        st = _lib.load().btq_compress_pack_ex(
            _ptr(_bits(x)), P, T, H, k, _ptr(rscale), _ptr(zero_point), _ptr(outlier_idx),
            _ptr(cmap), sets, _ptr(packed), pitch, _ptr(_bits(outliers)), sh)
    _lib.check(st, "btq_compress_pack_ex")
    return packed, outliers


def btq_compress_pack(x: torch.Tensor, k: int, rscale: torch.Tensor, zero_point: torch.Tensor,
                      outlier_idx: torch.Tensor, cmap: torch.Tensor,
                      packed: Optional[torch.Tensor] = None,
                      outliers: Optional[torch.Tensor] = None, stream=None):
    """Sender message of every shard, rows of Bq bytes with no gap:
    (packed uint8 [P,T,Bq], outliers int16 [P,T,k])."""
    _dense(packed, x.shape[2], k)
    return btq_compress_pack_ex(x, k, rscale, zero_point, outlier_idx, cmap, False, packed,
                                outliers, None, stream)


def btq_compress_pack_per_shard(x: torch.Tensor, k: int, rscale: torch.Tensor,
                                zero_point: torch.Tensor, outlier_idx: torch.Tensor,
                                cmap: torch.Tensor, packed: Optional[torch.Tensor] = None,
                                outliers: Optional[torch.Tensor] = None, stream=None):
    """btq_compress_pack with one BF16 set per shard: outlier_idx [P,k] and
    cmap [P,H-k] from btq_select_outliers_per_shard."""
    _dense(packed, x.shape[2], k)
    return btq_compress_pack_ex(x, k, rscale, zero_point, outlier_idx, cmap, True, packed,
                                outliers, None, stream)


def _dense(packed, H, k):
    if packed is not None and packed.dim() == 3 and packed.shape[2] != btq_packed_row_bytes(H, k):
        raise ValueError("packed rows must be btq_packed_row_bytes(H, k) bytes here "
                         "(the *_ex calls take a pitch)")


def btq_decompress_reduce_ex(packed: torch.Tensor, outliers: torch.Tensor, H: int,
                             scale: torch.Tensor, zero_point: torch.Tensor, fmap: torch.Tensor,
                             per_shard: bool = False, y: Optional[torch.Tensor] = None,
                             bf16: bool = False, stream=None) -> torch.Tensor:
    """Receiver: y [T,H] = sum over shards of the dequantized messages.

    packed is uint8 [P,T,pitch]: its rows' first btq_packed_row_bytes(H,k)
    bytes are read. y is float32, or bf16 bits (int16) when bf16. per_shard:
    fmap [P,H] holds one map per shard.
    """
    dev = _device(packed)
    P, T, pitch = packed.shape
    k = outliers.shape[2]
    if pitch < btq_packed_row_bytes(H, k):
        raise ValueError(f"packed rows of {pitch} bytes are shorter than H={H}, k={k} needs")
    _need(packed, "packed", (torch.uint8,), (P, T, pitch), dev)
    _need(outliers, "outliers", _BF16, (P, T, k), dev)
    _need(scale, "scale", (torch.float32,), (P, H), dev)
    _need(zero_point, "zero_point", (torch.uint8,), (P, H), dev)
    _need(fmap, "fmap", (torch.int32,), ((P, H) if per_shard else (H,)), dev)
    sh, ctx = _launch(dev, stream)
    with ctx:
        if y is None:
            y = torch.empty((T, H), dtype=torch.int16 if bf16 else torch.float32, device=dev)
        _need(y, "y", _BF16 if bf16 else (torch.float32,), (T, H), dev)
        sets = _lib.BTQ_SETS_PER_SHARD if per_shard else _lib.BTQ_SETS_SHARED
        st = _lib.load().btq_decompress_reduce_ex(
            _ptr(packed), pitch, _ptr(_bits(outliers)), P, T, H, k, _ptr(scale), _ptr(zero_point),
            _ptr(fmap), sets, _ptr(_bits(y)), _lib.BTQ_Y_BF16 if bf16 else _lib.BTQ_Y_F32, sh)
    _lib.check(st, "btq_decompress_reduce_ex")
    return y


def _need_dense(packed, outliers, H):
    k = outliers.shape[2]
    if packed.dim() != 3 or packed.shape[2] != btq_packed_row_bytes(H, k):
        raise ValueError("packed rows must be btq_packed_row_bytes(H, k) bytes here "
                         "(btq_decompress_reduce_ex takes a pitch)")


def btq_decompress_reduce(packed: torch.Tensor, outliers: torch.Tensor, H: int,
                          scale: torch.Tensor, zero_point: torch.Tensor, fmap: torch.Tensor,
                          y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Receiver: y float32 [T,H] from packed [P,T,Bq] and outliers [P,T,k]."""
    _need_dense(packed, outliers, H)
    return btq_decompress_reduce_ex(packed, outliers, H, scale, zero_point, fmap, False, y, False,
                                    stream)


def btq_decompress_reduce_bf16(packed: torch.Tensor, outliers: torch.Tensor, H: int,
                               scale: torch.Tensor, zero_point: torch.Tensor, fmap: torch.Tensor,
                               y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Receiver with bf16 output: the fp32 sum rounded once to bf16.

    Returns int16 [T,H] bf16 bits (torch.bfloat16 is also accepted for y).
    """
    _need_dense(packed, outliers, H)
    return btq_decompress_reduce_ex(packed, outliers, H, scale, zero_point, fmap, False, y, True,
                                    stream)


def btq_decompress_reduce_per_shard(packed: torch.Tensor, outliers: torch.Tensor, H: int,
                                    scale: torch.Tensor, zero_point: torch.Tensor,
                                    fmap: torch.Tensor, y: Optional[torch.Tensor] = None,
                                    stream=None) -> torch.Tensor:
    """Reduced fp32 y [T,H] from per-shard-set messages: fmap [P,H] from
    btq_select_outliers_per_shard."""
    _need_dense(packed, outliers, H)
    return btq_decompress_reduce_ex(packed, outliers, H, scale, zero_point, fmap, True, y, False,
                                    stream)


def btq_status_str(status: int) -> str:
    return _lib.load().btq_status_str(status).decode()


def btq_version() -> str:
    return _lib.load().btq_version().decode()
