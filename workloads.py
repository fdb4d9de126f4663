"""Seeded synthetic inputs for the hybrid int4/BF16 partial-sum codec.

This module only draws numbers. It holds none of the codec's arithmetic:
no statistics, no quantization, no packing and no sums. The oracle and the
HIP path receive the identical bf16 tensor that it returns.

The inputs stand in for the per-device partial sums of a tensor-parallel
row-parallel layer. The pages name no dataset. They do describe the data's
structure: a handful of features have very wide ranges, and they are the same
features on every device and for every batch ("Revolutionizing LLM Inference:
The Power of Efficient Low-Bit Communication", section "Leveraging Outliers
for Efficient Communication"). So every workload plants a fixed set of
outlier columns shared by all shards.

Draws use torch's counter-based generator on the device that will consume
the data, so a full-size batch never crosses PCIe. The CPU and GPU generators
give different streams for one seed. Each comparison therefore runs both
sides on one tensor: the oracle reads a host copy of the device tensor.
bf16 values are carried as int16 bit patterns (``torch.int16``), the format
the C ABI takes.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch

# phase tags mixed into every seed
PHASE_COLUMNS = 0   # choice of the outlier columns
PHASE_CALIB = 1     # calibration batches
PHASE_INFER = 2     # inference batches


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, value distribution, outlier plan."""
    name: str
    wid: int                 # mixed into every seed
    P: int                   # shards (tensor-parallel devices)
    T: tuple                 # token counts of the inference batches
    H: int                   # hidden features
    ks: tuple                # BF16 feature counts to run (the first is the default)
    base: str                # "normal" or "laplace"
    sigma: float             # std of the normal base (ignored for laplace)
    n_outliers: int          # planted outlier columns
    outlier_mode: str        # "scale": multiply; "student_t": replace
    outlier_factor: float
    calib_batches: int
    calib_T: int
    momentum: float
    drift: int = 0           # outlier columns swapped between calibration and inference

    @property
    def k(self) -> int:
        return self.ks[0]


WORKLOADS = {
    w.name: w for w in (
        Workload("tiny", 0, P=2, T=(16,), H=256, ks=(8,), base="normal", sigma=1.0,
                 n_outliers=4, outlier_mode="scale", outlier_factor=50.0,
                 calib_batches=4, calib_T=16, momentum=0.9),
        Workload("7b_prefill", 1, P=8, T=(2048,), H=4096, ks=(64,), base="normal",
                 sigma=0.5, n_outliers=41, outlier_mode="scale", outlier_factor=100.0,
                 calib_batches=32, calib_T=2048, momentum=0.9),
        Workload("decode", 2, P=8, T=(1, 8, 32, 64), H=8192, ks=(64,), base="normal",
                 sigma=0.5, n_outliers=41, outlier_mode="student_t", outlier_factor=30.0,
                 calib_batches=32, calib_T=2048, momentum=0.9),
        Workload("large_prefill", 3, P=4, T=(8192,), H=8192, ks=(128,), base="normal",
                 sigma=1.0, n_outliers=164, outlier_mode="scale", outlier_factor=200.0,
                 calib_batches=64, calib_T=8192, momentum=0.95),
        Workload("stress", 4, P=8, T=(16384,), H=8192, ks=(32, 0, 256), base="laplace",
                 sigma=1.0, n_outliers=164, outlier_mode="scale", outlier_factor=100.0,
                 calib_batches=32, calib_T=16384, momentum=0.9, drift=16),
    )
}


def seed_of(wid: int, phase: int, b: int) -> int:
    """64-bit seed for (workload, phase, batch index)."""
    return ((wid & 0xFFFF) << 40) | ((phase & 0xFF) << 32) | (b & 0xFFFFFFFF)


def outlier_columns(w: Workload, phase: int = PHASE_CALIB) -> np.ndarray:
    """Sorted planted outlier columns for `phase`.

    Calibration and inference share one set, except that a drifting workload
    swaps `w.drift` of its columns for as many ordinary ones at inference.
    """
    rng = np.random.default_rng([w.wid, PHASE_COLUMNS, 0, 0])
    cols = np.sort(rng.choice(w.H, size=w.n_outliers, replace=False))
    if phase == PHASE_INFER and w.drift:
        gone = rng.choice(cols, size=w.drift, replace=False)
        rest = np.setdiff1d(np.arange(w.H), cols)
        new = rng.choice(rest, size=w.drift, replace=False)
        cols = np.sort(np.concatenate([np.setdiff1d(cols, gone), new]))
    return cols.astype(np.int64)


def draw(P: int, T: int, H: int, seed: int, *, base: str = "normal", sigma: float = 1.0,
         cols: Optional[Sequence[int]] = None, outlier_mode: str = "scale",
         outlier_factor: float = 1.0, device="cpu") -> torch.Tensor:
    """Draw a [P,T,H] partial-sum tensor and return its bf16 bits as int16.

    Shards are drawn one after another from one generator, so the result for
    a seed does not depend on how much memory is free.
    """
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    out = torch.empty((P, T, H), dtype=torch.bfloat16, device=dev)
    colt = None
    if cols is not None and len(cols):
        colt = torch.as_tensor(np.asarray(cols, dtype=np.int64), device=dev)
    for p in range(P):
        if base == "normal":
            x = torch.randn((T, H), generator=g, device=dev, dtype=torch.float32)
            if sigma != 1.0:
                x.mul_(sigma)
        elif base == "laplace":
            x = torch.empty((T, H), device=dev, dtype=torch.float32).exponential_(generator=g)
            neg = torch.rand((T, H), generator=g, device=dev) < 0.5
            x = torch.where(neg, -x, x)
        else:
            raise ValueError(f"unknown base distribution {base!r}")
        if colt is not None:
            if outlier_mode == "scale":
                x[:, colt] *= outlier_factor
            elif outlier_mode == "student_t":
                # Student-t with 2 degrees of freedom: Z / sqrt(E), E ~ Exp(1)
                z = torch.randn((T, colt.numel()), generator=g, device=dev)
                e = torch.empty((T, colt.numel()), device=dev).exponential_(generator=g)
                x[:, colt] = z / torch.sqrt(e) * outlier_factor
            else:
                raise ValueError(f"unknown outlier mode {outlier_mode!r}")
        out[p] = x.to(torch.bfloat16)
        del x
    return out.view(torch.int16)


def batch(w: Workload, phase: int, b: int, T: Optional[int] = None, device="cpu") -> torch.Tensor:
    """Batch `b` of `phase` for workload `w` as int16 bf16 bits, shape [P,T,H]."""
    if T is None:
        T = w.calib_T if phase == PHASE_CALIB else w.T[0]
    return draw(w.P, T, w.H, seed_of(w.wid, phase, b), base=w.base, sigma=w.sigma,
                cols=outlier_columns(w, phase), outlier_mode=w.outlier_mode,
                outlier_factor=w.outlier_factor, device=device)


def to_u16(t: torch.Tensor) -> np.ndarray:
    """Host numpy uint16 copy of an int16 bf16-bits tensor."""
    return t.detach().to("cpu").contiguous().numpy().view(np.uint16)
