"""Python binding of libbtq: one function per C entry point, same names.

The functions only marshal arguments. They check tensor dtypes, shapes and
devices, allocate outputs and workspaces with torch when the caller passes
none, and hand raw device pointers and torch's current HIP stream to the C
ABI. Every step of the codec runs in the library's HIP kernels; nothing
here computes on tensor values.

Layouts (contiguous, row-major, last index fastest):
  x           int16 [P,T,H]  bf16 bit patterns (torch.bfloat16 is also accepted)
  run_min/max float32 [P,H]
  scale, rscale float32 [P,H];  zero_point uint8 [P,H]
  outlier_idx int32 [k];  fmap int32 [H];  cmap int32 [H-k]
  enc_table   float32 [P,H-k,2]  (rscale, zero point) per int4 slot
  dec_table   float32 [2P+1,H-k] scale rows, zero-point rows, constant row
  packed      uint8 [P,T,pitch]: ceil((H-k)/2) code bytes per row, then zeros;
              pitch defaults to btq_packed_pitch(H,k) (a multiple of 128)
  outliers    int16 [P,T,k]
  y           float32 [T,H]  (bf16 [T,H] from btq_decompress_reduce_bf16)
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib


def _stream(dev: torch.device, stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


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


def _device(x: torch.Tensor) -> torch.device:
    if x.device.type != "cuda":
        raise ValueError("libbtq runs on the GPU: pass device tensors")
    return x.device


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


def btq_select_workspace_bytes(P: int, H: int) -> int:
    return int(_lib.load().btq_select_workspace_bytes(P, H))


def btq_enc_table_floats(P: int, H: int, k: int) -> int:
    return int(_lib.load().btq_enc_table_floats(P, H, k))


def btq_dec_table_floats(P: int, H: int, k: int) -> int:
    return int(_lib.load().btq_dec_table_floats(P, H, k))


def btq_calib_update(x: torch.Tensor, run_min: torch.Tensor, run_max: torch.Tensor,
                     momentum: float, first_batch: bool,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Fold one calibration batch x [P,T,H] into run_min/run_max [P,H] in place."""
    dev = _device(x)
    P, T, H = x.shape
    _need(x, "x", _BF16, (P, T, H), dev)
    _need(run_min, "run_min", (torch.float32,), (P, H), dev)
    _need(run_max, "run_max", (torch.float32,), (P, H), dev)
    need = btq_calib_workspace_bytes(P, T, H)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    lib = _lib.load()
    st = lib.btq_calib_update(_ptr(_bits(x)), P, T, H, float(momentum), int(bool(first_batch)),
                              _ptr(run_min), _ptr(run_max), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(dev, stream))
    _lib.check(st, "btq_calib_update")


def btq_select_outliers(run_min: torch.Tensor, run_max: torch.Tensor, k: int, out: dict = None,
                        workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Parameters and the BF16 feature set from the running extremes.

    Returns a dict with scale, rscale, zero_point, outlier_idx, fmap, cmap,
    enc (the encoder table) and dec (the decoder table).
    """
    return _select_ranked("btq_select_outliers", run_min, run_max, k, None, out, workspace,
                          stream)


_RULES = {"sum": _lib.BTQ_SCORE_SUM, "max": _lib.BTQ_SCORE_MAX}


def btq_select_outliers_rule(run_min: torch.Tensor, run_max: torch.Tensor, k: int, rule: str,
                             out: dict = None, workspace: Optional[torch.Tensor] = None,
                             stream=None) -> dict:
    """btq_select_outliers with the rank score chosen by `rule`: "sum" (the
    per-shard ranges added) or "max" (the widest shard's range)."""
    if rule not in _RULES:
        raise ValueError(f"rule must be one of {sorted(_RULES)}")
    return _select_ranked("btq_select_outliers_rule", run_min, run_max, k, _RULES[rule], out,
                          workspace, stream)


def _select_ranked(name, run_min, run_max, k, rule, out, workspace, stream) -> dict:
    dev = _device(run_min)
    P, H = run_min.shape
    o = _select_outputs(run_min, run_max, k, out)
    need = btq_select_workspace_bytes(P, H)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    lib = _lib.load()
    head = [_ptr(run_min), _ptr(run_max), P, H, k] + ([] if rule is None else [rule])
    st = getattr(lib, name)(*head, _ptr(o["scale"]), _ptr(o["rscale"]), _ptr(o["zero_point"]),
                            _ptr(o["outlier_idx"]), _ptr(o["fmap"]), _ptr(o["cmap"]),
                            _ptr(o["enc"]), _ptr(o["dec"]), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(dev, stream))
    _lib.check(st, name)
    return o


def btq_select_features(run_min: torch.Tensor, run_max: torch.Tensor, features, out: dict = None,
                        stream=None) -> dict:
    """Parameters, maps and tables for a BF16 set chosen by the caller.

    features: the k BF16 features (any int sequence, array or tensor), distinct
    and ascending. Returns the same dict as btq_select_outliers. The call
    waits for its stream, because the set travels from host memory.
    """
    dev = _device(run_min)
    P, H = run_min.shape
    feat = torch.as_tensor(features).to(device="cpu", dtype=torch.int32).contiguous().reshape(-1)
    k = feat.numel()
    o = _select_outputs(run_min, run_max, k, out)
    lib = _lib.load()
    st = lib.btq_select_features(_ptr(run_min), _ptr(run_max), P, H, k, _ptr(feat),
                                 _ptr(o["scale"]), _ptr(o["rscale"]), _ptr(o["zero_point"]),
                                 _ptr(o["outlier_idx"]), _ptr(o["fmap"]), _ptr(o["cmap"]),
                                 _ptr(o["enc"]), _ptr(o["dec"]), _stream(dev, stream))
    _lib.check(st, "btq_select_features")
    if stream is None:
        torch.cuda.current_stream(dev).synchronize()
    elif hasattr(stream, "synchronize"):
        stream.synchronize()
    else:
        torch.cuda.ExternalStream(int(stream), device=dev).synchronize()
    return o


def _select_outputs(run_min: torch.Tensor, run_max: torch.Tensor, k: int, out) -> dict:
    dev = _device(run_min)
    P, H = run_min.shape
    _need(run_min, "run_min", (torch.float32,), (P, H), dev)
    _need(run_max, "run_max", (torch.float32,), (P, H), dev)
    if not 0 <= k <= H:
        raise ValueError(f"k={k} outside [0, H={H}]")
    o = dict(out or {})
    o.setdefault("scale", torch.empty((P, H), dtype=torch.float32, device=dev))
    o.setdefault("rscale", torch.empty((P, H), dtype=torch.float32, device=dev))
    o.setdefault("zero_point", torch.empty((P, H), dtype=torch.uint8, device=dev))
    o.setdefault("outlier_idx", torch.empty((k,), dtype=torch.int32, device=dev))
    o.setdefault("fmap", torch.empty((H,), dtype=torch.int32, device=dev))
    o.setdefault("cmap", torch.empty((H - k,), dtype=torch.int32, device=dev))
    o.setdefault("enc", torch.empty((P, H - k, 2), dtype=torch.float32, device=dev))
    o.setdefault("dec", torch.empty((2 * P + 1, H - k), dtype=torch.float32, device=dev))
    for name, dt, shp in (("scale", torch.float32, (P, H)), ("rscale", torch.float32, (P, H)),
                          ("zero_point", torch.uint8, (P, H)), ("outlier_idx", torch.int32, (k,)),
                          ("fmap", torch.int32, (H,)), ("cmap", torch.int32, (H - k,)),
                          ("enc", torch.float32, (P, H - k, 2)),
                          ("dec", torch.float32, (2 * P + 1, H - k))):
        _need(o[name], name, (dt,), shp, dev)
    return o


def btq_compress_pack(x: torch.Tensor, k: int, enc_table: torch.Tensor,
                      outlier_idx: torch.Tensor, cmap: torch.Tensor,
                      packed: Optional[torch.Tensor] = None,
                      outliers: Optional[torch.Tensor] = None, pitch: Optional[int] = None,
                      stream=None):
    """Sender message of every shard: (packed uint8 [P,T,pitch], outliers int16 [P,T,k]).

    The row pitch is packed.shape[2] when `packed` is given, else `pitch`,
    else btq_packed_pitch(H, k).
    """
    return _compress("btq_compress_pack", x, k, enc_table, outlier_idx, cmap, packed, outliers,
                     pitch, stream)


def btq_compress_pack_per_shard(x: torch.Tensor, k: int, enc_table: torch.Tensor,
                                outlier_idx: torch.Tensor, cmap: torch.Tensor,
                                packed: Optional[torch.Tensor] = None,
                                outliers: Optional[torch.Tensor] = None,
                                pitch: Optional[int] = None, stream=None):
    """btq_compress_pack with one BF16 set per shard: outlier_idx [P,k] and
    cmap [P,H-k] from btq_select_outliers_per_shard."""
    return _compress("btq_compress_pack_per_shard", x, k, enc_table, outlier_idx, cmap, packed,
                     outliers, pitch, stream)


def _compress(entry, x, k, enc_table, outlier_idx, cmap, packed, outliers, pitch, stream):
    dev = _device(x)
    P, T, H = x.shape
    _need(x, "x", _BF16, (P, T, H), dev)
    if packed is not None:
        pitch = packed.shape[2] if packed.dim() == 3 else -1
    elif pitch is None:
        pitch = btq_packed_pitch(H, k)
    _need(enc_table, "enc_table", (torch.float32,), (P, H - k, 2), dev)
    per = entry.endswith("_per_shard")
    _need(outlier_idx, "outlier_idx", (torch.int32,), (P, k) if per else (k,), dev)
    _need(cmap, "cmap", (torch.int32,), (P, H - k) if per else (H - k,), dev)
    if packed is None:
        packed = torch.empty((P, T, pitch), dtype=torch.uint8, device=dev)
    if outliers is None:
        outliers = torch.empty((P, T, k), dtype=torch.int16, device=dev)
    _need(packed, "packed", (torch.uint8,), (P, T, pitch), dev)
    _need(outliers, "outliers", _BF16, (P, T, k), dev)
    lib = _lib.load()
    st = getattr(lib, entry)(_ptr(_bits(x)), P, T, H, k, _ptr(enc_table), _ptr(outlier_idx),
                             _ptr(cmap), _ptr(packed), pitch, _ptr(_bits(outliers)),
                             _stream(dev, stream))
    _lib.check(st, entry)
    return packed, outliers


def btq_decompress_reduce_per_shard(packed: torch.Tensor, outliers: torch.Tensor, H: int,
                                    scale: torch.Tensor, zero_point: torch.Tensor,
                                    fmap: torch.Tensor, y: Optional[torch.Tensor] = None,
                                    stream=None) -> torch.Tensor:
    """Reduced fp32 y [T,H] from per-shard-set messages: scale [P,H],
    zero_point [P,H] and fmap [P,H] from btq_select_outliers_per_shard."""
    dev = _device(packed)
    P, T, pitch = packed.shape
    k = outliers.shape[2]
    if pitch < btq_packed_row_bytes(H, k):
        raise ValueError(f"packed rows of {pitch} bytes are shorter than H={H}, k={k} needs")
    _need(packed, "packed", (torch.uint8,), (P, T, pitch), dev)
    _need(outliers, "outliers", _BF16, (P, T, k), dev)
    _need(scale, "scale", (torch.float32,), (P, H), dev)
    _need(zero_point, "zero_point", (torch.uint8,), (P, H), dev)
    _need(fmap, "fmap", (torch.int32,), (P, H), dev)
    if y is None:
        y = torch.empty((T, H), dtype=torch.float32, device=dev)
    _need(y, "y", (torch.float32,), (T, H), dev)
    lib = _lib.load()
    st = lib.btq_decompress_reduce_per_shard(_ptr(packed), pitch, _ptr(_bits(outliers)), P, T, H,
                                             k, _ptr(scale), _ptr(zero_point), _ptr(fmap),
                                             _ptr(y), _stream(dev, stream))
    _lib.check(st, "btq_decompress_reduce_per_shard")
    return y


def btq_select_outliers_per_shard(run_min: torch.Tensor, run_max: torch.Tensor, k: int,
                                  out: dict = None, workspace: Optional[torch.Tensor] = None,
                                  stream=None) -> dict:
    """One BF16 set per shard, ranked by the shard's own ranges. Returns
    scale, rscale, zero_point [P,H], outlier_idx [P,k], fmap [P,H],
    cmap [P,H-k] and enc [P,H-k,2]."""
    dev = _device(run_min)
    P, H = run_min.shape
    _need(run_min, "run_min", (torch.float32,), (P, H), dev)
    _need(run_max, "run_max", (torch.float32,), (P, H), dev)
    if not 0 <= k <= H:
        raise ValueError(f"k={k} outside [0, H={H}]")
    o = dict(out or {})
    shapes = (("scale", torch.float32, (P, H)), ("rscale", torch.float32, (P, H)),
              ("zero_point", torch.uint8, (P, H)), ("outlier_idx", torch.int32, (P, k)),
              ("fmap", torch.int32, (P, H)), ("cmap", torch.int32, (P, H - k)),
              ("enc", torch.float32, (P, H - k, 2)))
    for name, dt, shp in shapes:
        o.setdefault(name, torch.empty(shp, dtype=dt, device=dev))
        _need(o[name], name, (dt,), shp, dev)
    if workspace is None:
        workspace = torch.empty(btq_select_workspace_bytes(P, H), dtype=torch.uint8, device=dev)
    lib = _lib.load()
    st = lib.btq_select_outliers_per_shard(_ptr(run_min), _ptr(run_max), P, H, k,
                                           _ptr(o["scale"]), _ptr(o["rscale"]),
                                           _ptr(o["zero_point"]), _ptr(o["outlier_idx"]),
                                           _ptr(o["fmap"]), _ptr(o["cmap"]), _ptr(o["enc"]),
                                           _ptr(workspace),
                                           workspace.numel() * workspace.element_size(),
                                           _stream(dev, stream))
    _lib.check(st, "btq_select_outliers_per_shard")
    return o


def _decompress(entry: str, packed: torch.Tensor, outliers: torch.Tensor, H: int,
                dec_table: torch.Tensor, outlier_idx: torch.Tensor, cmap: torch.Tensor,
                y: Optional[torch.Tensor], ydtypes, ynew, stream) -> torch.Tensor:
    dev = _device(packed)
    P, T, pitch = packed.shape
    k = outliers.shape[2]
    if pitch < btq_packed_row_bytes(H, k):
        raise ValueError(f"packed rows of {pitch} bytes are shorter than H={H}, k={k} needs")
    _need(packed, "packed", (torch.uint8,), (P, T, pitch), dev)
    _need(outliers, "outliers", _BF16, (P, T, k), dev)
    _need(dec_table, "dec_table", (torch.float32,), (2 * P + 1, H - k), dev)
    _need(outlier_idx, "outlier_idx", (torch.int32,), (k,), dev)
    _need(cmap, "cmap", (torch.int32,), (H - k,), dev)
    if y is None:
        y = torch.empty((T, H), dtype=ynew, device=dev)
    _need(y, "y", ydtypes, (T, H), dev)
    lib = _lib.load()
    st = getattr(lib, entry)(_ptr(packed), pitch, _ptr(_bits(outliers)), P, T, H, k,
                             _ptr(dec_table), _ptr(outlier_idx), _ptr(cmap), _ptr(_bits(y)),
                             _stream(dev, stream))
    _lib.check(st, entry)
    return y


def btq_decompress_reduce(packed: torch.Tensor, outliers: torch.Tensor, H: int,
                          dec_table: torch.Tensor, outlier_idx: torch.Tensor, cmap: torch.Tensor,
                          y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Receiver: y float32 [T,H] = sum over shards of the dequantized messages.

    packed is uint8 [P,T,pitch]; its rows' first btq_packed_row_bytes(H,k)
    bytes are read.
    """
    return _decompress("btq_decompress_reduce", packed, outliers, H, dec_table, outlier_idx, cmap,
                       y, (torch.float32,), torch.float32, stream)


def btq_decompress_reduce_bf16(packed: torch.Tensor, outliers: torch.Tensor, H: int,
                               dec_table: torch.Tensor, outlier_idx: torch.Tensor,
                               cmap: torch.Tensor, y: Optional[torch.Tensor] = None,
                               stream=None) -> torch.Tensor:
    """Receiver with bf16 output: the fp32 sum rounded once to bf16.

    Returns int16 [T,H] bf16 bits (torch.bfloat16 is also accepted for y).
    """
    return _decompress("btq_decompress_reduce_bf16", packed, outliers, H, dec_table, outlier_idx,
                       cmap, y, _BF16, torch.int16, stream)


def btq_status_str(status: int) -> str:
    return _lib.load().btq_status_str(status).decode()


def btq_version() -> str:
    return _lib.load().btq_version().decode()
