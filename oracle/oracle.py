"""CPU oracle for the hybrid int4/BF16 partial-sum codec.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import or run this module. The
library under ``bit_tensor_activation_amd/`` never calls it, and it shares no
code, tables or helpers with that library.

What it follows. One page describes the method: "Revolutionizing LLM
Inference: The Power of Efficient Low-Bit Communication" (aiexpert.world),
a summary of the paper "Towards Efficient Low-Bit Communication for Tensor
Parallel LLM Inference". Its section "The Hybrid Quantization Algorithm"
lists three steps, cited below as [Calibration], [Selection] and
[Inference]. Its section "Combating Quantization Errors with Tensor
Parallelism" says that each device quantizes its partial sum before the
sum across devices, cited as [TP errors]. The page gives no formulas, so
every formula here is the plainest reading that the rest supports, and
each reading is stated where it is used.

Arithmetic: numpy float32 arrays with every constant an explicit
``np.float32``. Each operation is one IEEE round-to-nearest-even step, with
no fused multiply-add. bf16 values are carried as uint16 bit patterns.
The step order below is the page's order: calibrate, select, quantize
(sender), convert back and sum (receiver).

Every function here has a pin in ``tests/test_oracle_*.py`` that fixes it by
something other than itself. The pins are brute force, exact rational or
float64 arithmetic, closed forms, hand-worked examples under
``tests/golden/``, and a library routine
(``torch.fake_quantize_per_channel_affine``).
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
FLT_MIN = np.finfo(np.float32).tiny     # smallest normal fp32, 2**-126
QMAX = 15                               # 4-bit codes 0..15


# ---------------------------------------------------------------- bf16 ----
def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    """Exact bf16 -> fp32: the 16 bf16 bits are the high half of the fp32."""
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(F32)


# --------------------------------------------------------- calibration ----
def batch_min_max(x: np.ndarray):
    """Per-shard, per-feature min and max over the tokens of one batch.

    [Calibration]: parameters come from the observed minimum and maximum
    on each device. The page does not say over what the extremes are
    taken. The reading here is: over all tokens of the batch, separately
    for each device p and feature h. x: uint16 [P,T,H]. Returns two
    float32 arrays [P,H]. Both are exact; -0 and +0 compare equal.
    """
    f = bf16_to_f32(x)
    return f.min(axis=1), f.max(axis=1)


def ema(run: np.ndarray, obs: np.ndarray, momentum: float, first: bool) -> np.ndarray:
    """One moving-average step of a running extreme.

    [Calibration] says "moving averages" and gives no formula. The reading
    here: the first batch copies the observed value. Each later batch
    gives new = m*old + (1-m)*obs, with m the momentum weighting the old
    value. The steps are fp32: a = fl(m), c = fl(1 - a), then two rounded
    products and one rounded sum.
    """
    obs = np.asarray(obs, dtype=F32)
    if first:
        return obs.copy()
    a = F32(momentum)
    c = F32(1) - a
    return (a * np.asarray(run, dtype=F32)) + (c * obs)


def calib_update(x, run_min, run_max, momentum: float, first: bool):
    """One calibration batch: batch extremes, then the moving average."""
    bmin, bmax = batch_min_max(x)
    return ema(run_min, bmin, momentum, first), ema(run_max, bmax, momentum, first)


# ----------------------------------------------------------- selection ----
def quant_params(run_min: np.ndarray, run_max: np.ndarray):
    """Asymmetric 4-bit parameters per shard and feature.

    [Calibration] fixes parameters per feature and per device from the
    running extremes. The page gives no formula. The reading here is
    standard asymmetric uniform quantization onto the codes 0..15:
      lo = min(run_min, 0), hi = max(run_max, 0)  (the grid holds 0 exactly)
      width = hi - lo
      scale = width / 15, or 1 if that is below the smallest normal fp32
      rscale = 1 / scale
      zero_point = clamp(round_half_even(-lo / scale), 0, 15)
    Every division is one IEEE fp32 division.
    Returns (scale f32, rscale f32, zero_point u8, width f32), each [P,H].
    """
    lo = np.minimum(np.asarray(run_min, F32), F32(0))
    hi = np.maximum(np.asarray(run_max, F32), F32(0))
    width = hi - lo
    scale = width / F32(QMAX)
    scale = np.where(scale < F32(FLT_MIN), F32(1), scale).astype(F32)
    rscale = F32(1) / scale
    zp = np.clip(np.rint(-lo / scale), F32(0), F32(QMAX)).astype(np.uint8)
    return scale, rscale, zp, width


SCORE_RULES = ("sum", "max")


def range_score(width: np.ndarray, rule: str = "sum") -> np.ndarray:
    """Rank score of each feature from its per-shard quantization ranges.

    [Selection] ranks features by their quantization ranges, and ranges
    are per device ([Calibration]). The receiver has to know which
    features every sender kept in BF16, so one set serves all shards, and
    the P ranges of a feature must become one score. The page does not say
    how. The main reading ("sum") adds them in fp32, folding p = 0, 1, ...
    from 0: that sum over 30 bounds the rounding error of the summed
    output. The alternative reading ("max") takes the widest shard's range,
    which is exact.
    """
    width = np.asarray(width, F32)
    if rule not in SCORE_RULES:
        raise ValueError(f"unknown score rule {rule!r}")
    score = np.zeros(width.shape[1], F32)
    for p in range(width.shape[0]):
        score = score + width[p] if rule == "sum" else np.maximum(score, width[p])
    return score


def top_k_features(score: np.ndarray, k: int):
    """The k highest-scoring features, and the maps between the feature
    index h and the message slots.

    Ties go to the lower h. Returns:
      idx  int32 [k]    BF16 features, in ascending h
      fmap int32 [H]    fmap[h] = j, its int4 slot; or -1-i if h = idx[i]
      cmap int32 [H-k]  cmap[j] = the j-th int4 feature in ascending h
    """
    score = np.asarray(score, F32)
    H = score.shape[0]
    if not 0 <= k <= H:
        raise ValueError("k must lie in [0, H]")
    h = np.arange(H)
    order = np.lexsort((h, -score))           # score descending, then h ascending
    return maps_for_set(np.sort(order[:k]), H)


def maps_for_set(idx, H: int):
    """Maps for a BF16 set given as k distinct features in ascending h.

    Returns (idx, fmap, cmap) as top_k_features does: the int4 slots are the
    other features in ascending h.
    """
    idx = np.asarray(idx, np.int64)
    k = idx.shape[0]
    if k and (np.any(np.diff(idx) <= 0) or idx[0] < 0 or idx[-1] >= H):
        raise ValueError("the BF16 set must be distinct features in [0, H), ascending")
    keep = np.ones(H, bool)
    keep[idx] = False
    cmap = np.nonzero(keep)[0].astype(np.int32)
    fmap = np.empty(H, np.int32)
    fmap[cmap] = np.arange(H - k, dtype=np.int32)
    fmap[idx] = -1 - np.arange(k, dtype=np.int32)
    return idx.astype(np.int32), fmap, cmap


def select_outliers(run_min, run_max, k: int, rule: str = "sum") -> dict:
    """[Selection] after [Calibration]: the per-(shard, feature) parameters,
    the rank scores, the BF16 set and the maps between features and message
    slots. rule: see range_score."""
    scale, rscale, zp, width = quant_params(run_min, run_max)
    score = range_score(width, rule)
    idx, fmap, cmap = top_k_features(score, k)
    return dict(scale=scale, rscale=rscale, zero_point=zp, width=width,
                score=score, idx=idx, fmap=fmap, cmap=cmap)


def select_features(run_min, run_max, idx) -> dict:
    """[Calibration] parameters with a BF16 set chosen by the caller instead
    of the range ranking of [Selection] (for instance random features, the
    baseline that [Future] compares against). Same outputs as
    select_outliers."""
    scale, rscale, zp, width = quant_params(run_min, run_max)
    score = range_score(width)
    idx, fmap, cmap = maps_for_set(idx, scale.shape[1])
    return dict(scale=scale, rscale=rscale, zero_point=zp, width=width,
                score=score, idx=idx, fmap=fmap, cmap=cmap)


def select_outliers_per_shard(run_min, run_max, k: int) -> dict:
    """A second reading of [Selection]: every shard keeps its own k widest
    features in BF16, ranked by that shard's own quantization range (ties:
    lower h first).

    The message stays k BF16 values and H-k codes per row, but its layout
    now differs between shards, so the receiver needs every shard's map.
    Returns scale, rscale, zero_point, width, and per shard idx [P,k],
    fmap [P,H] and cmap [P,H-k].
    """
    scale, rscale, zp, width = quant_params(run_min, run_max)
    P, H = width.shape
    if not 0 <= k <= H:
        raise ValueError("k must lie in [0, H]")
    idx = np.empty((P, k), np.int32)
    fmap = np.empty((P, H), np.int32)
    cmap = np.empty((P, H - k), np.int32)
    for p in range(P):
        idx[p], fmap[p], cmap[p] = top_k_features(width[p], k)
    return dict(scale=scale, rscale=rscale, zero_point=zp, width=width, idx=idx, fmap=fmap,
                cmap=cmap)


# ------------------------------------------------- inference, sender ----
def quantize(f: np.ndarray, rscale: np.ndarray, zero_point: np.ndarray) -> np.ndarray:
    """Codes q = clamp(round_half_even(f * rscale) + zero_point, 0, 15).

    The product is rounded to fp32 first, then rounded to an integer, and
    only then is the zero point added. Order matters at ties when the zero
    point is odd. Values outside the calibrated range clamp to the grid
    ends. f is float32; rscale and zero_point broadcast against it.
    """
    v = np.asarray(f, F32) * np.asarray(rscale, F32)
    q = np.rint(v) + np.asarray(zero_point).astype(F32)
    return np.clip(q, F32(0), F32(QMAX)).astype(np.uint8)


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte along the last axis.

    Code 2b goes in the low nibble of byte b and code 2b+1 in the high
    nibble. An odd count leaves the last high nibble 0. Length ceil(n/2).
    """
    q = np.asarray(q, np.uint8)
    n = q.shape[-1]
    nb = (n + 1) // 2
    qq = np.zeros(q.shape[:-1] + (2 * nb,), np.uint8)
    qq[..., :n] = q
    return (qq[..., 0::2] | (qq[..., 1::2] << np.uint8(4))).astype(np.uint8)


def unpack_nibbles(b: np.ndarray, n: int) -> np.ndarray:
    """Inverse of pack_nibbles: the first n codes along the last axis."""
    b = np.asarray(b, np.uint8)
    q = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.uint8)
    q[..., 0::2] = b & np.uint8(0x0F)
    q[..., 1::2] = b >> np.uint8(4)
    return q[..., :n]


def pad_rows(b: np.ndarray, pitch: int) -> np.ndarray:
    """Rows of bytes widened to `pitch` bytes with zeros (layout only).

    The packed message may carry its rows at a pitch larger than the code
    bytes; the extra bytes of a row are zero and carry nothing.
    """
    b = np.asarray(b, np.uint8)
    n = b.shape[-1]
    if pitch < n:
        raise ValueError(f"pitch {pitch} below the row's {n} bytes")
    out = np.zeros(b.shape[:-1] + (pitch,), np.uint8)
    out[..., :n] = b
    return out


def compress_pack(x, rscale, zero_point, idx, cmap, pitch=None):
    """Sender side of [Inference]: the message each device sends.

    The BF16 features stay BF16. Every other feature is quantized to 4
    bits with its own shard's parameters (quantized before the sum, [TP
    errors]). The message holds only the int4 features, in ascending h,
    packed two per byte, plus the BF16 features as a separate block.
    x: uint16 [P,T,H]. rscale, zero_point: [P,H]. idx [k], cmap [H-k]
    shared by all shards, or idx [P,k], cmap [P,H-k] with one set per shard
    (select_outliers_per_shard).
    Returns packed uint8 [P,T,pitch] (pitch defaults to the ceil((H-k)/2)
    code bytes; extra bytes are zero) and outliers uint16 [P,T,k].
    """
    x = np.asarray(x, np.uint16)
    P = x.shape[0]
    cmap = np.asarray(cmap, np.int64)
    idx = np.asarray(idx, np.int64)
    if cmap.ndim == 1:
        cmap = np.broadcast_to(cmap, (P,) + cmap.shape)
        idx = np.broadcast_to(idx, (P,) + idx.shape)
    rscale = np.asarray(rscale, F32)
    zero_point = np.asarray(zero_point, np.uint8)
    packed, outl = [], []
    for p in range(P):
        f = bf16_to_f32(x[p][:, cmap[p]])
        q = quantize(f, rscale[p, cmap[p]][None, :], zero_point[p, cmap[p]][None, :])
        packed.append(pack_nibbles(q))
        outl.append(x[p][:, idx[p]])
    packed = np.stack(packed)
    if pitch is not None:
        packed = pad_rows(packed, pitch)
    return packed, np.stack(outl).astype(np.uint16)


# ----------------------------------------------- inference, receiver ----
def dequantize(q: np.ndarray, scale: np.ndarray, zero_point: np.ndarray) -> np.ndarray:
    """fp32 value of a code: fl32(q - zero_point) * scale.

    The difference is a small integer, exact in fp32, so only the product
    rounds.
    """
    d = np.asarray(q).astype(F32) - np.asarray(zero_point).astype(F32)
    return d * np.asarray(scale, F32)


def maps_from_fmap(fmap: np.ndarray):
    """(idx, cmap) recovered from fmap: both list h in ascending order."""
    fmap = np.asarray(fmap, np.int64)
    h = np.arange(fmap.shape[0])
    ints = fmap >= 0
    cmap = np.empty(int(ints.sum()), np.int64)
    cmap[fmap[ints]] = h[ints]
    idx = np.empty(int((~ints).sum()), np.int64)
    idx[-1 - fmap[~ints]] = h[~ints]
    return idx, cmap


def decompress_reduce(packed, outliers, scale, zero_point, fmap) -> np.ndarray:
    """Receiver side of [Inference]: convert every shard's message back and
    sum over shards.

    The page says the tensors are converted back and summed across
    devices. The reading here: each term is an fp32 value (dequantized
    int4, or the exact BF16 value), and the sum runs in fp32 over
    p = 0, 1, ..., P-1, starting from 0. The output is fp32 [T,H].
    A packed row may be wider than its code bytes (a pitch); only the first
    ceil((H-k)/2) bytes are read. fmap [H] is shared by all shards; fmap
    [P,H] gives every shard its own map (select_outliers_per_shard).
    """
    packed = np.asarray(packed, np.uint8)
    outliers = np.asarray(outliers, np.uint16)
    P, T = packed.shape[:2]
    fmap = np.asarray(fmap)
    if fmap.ndim == 1:
        fmap = np.broadcast_to(fmap, (P,) + fmap.shape)
    H = fmap.shape[1]
    y = np.zeros((T, H), F32)
    for p in range(P):
        idx, cmap = maps_from_fmap(fmap[p])
        q = unpack_nibbles(packed[p], cmap.shape[0])
        term = np.empty((T, H), F32)
        term[:, cmap] = dequantize(q, np.asarray(scale, F32)[p, cmap],
                                   np.asarray(zero_point, np.uint8)[p, cmap])
        term[:, idx] = bf16_to_f32(outliers[p])
        y = y + term
    return y


def f32_to_bf16(y: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even (finite inputs).

    The bf16-output receiver of [Inference] (every tensor converts back to
    BF16) rounds its fp32 sum once with this.
    """
    u = np.asarray(y, F32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def decompress_reduce_bf16(packed, outliers, scale, zero_point, fmap) -> np.ndarray:
    """The receiver with bf16 output: the fp32 sum of decompress_reduce,
    rounded once to bf16 (round to nearest even). Returns uint16 bits [T,H].

    Page section "The Hybrid Quantization Algorithm", Inference bullet: after
    communication the tensors are converted back to BF16. Here the terms are
    summed in fp32 first and the sum is converted once, so the BF16 output
    carries a single rounding.
    """
    return f32_to_bf16(decompress_reduce(packed, outliers, scale, zero_point, fmap))
