"""Quality of the hybrid int4/BF16 codec on the synthetic workloads (GPU).

Every codec step runs in the library's HIP kernels (calibration, selection,
compress, decompress). This script only draws inputs and measures the reduced
output y against the exact sum of the unquantized bf16 partial sums,
sum_p x[p] in float64. It reports:

  * error vs k: how the error falls as range-ranked BF16 features are added;
  * selection rules at a workload's k: range-ranked (shard ranges summed,
    the widest shard, or one set per shard), random sets, and pure int4
    (k = 0), also on a case with shard-local outliers. The page's section
    "Key Observations and Future Directions" reports that random BF16
    features help little over pure int4 and that ranking by range is what
    matters;
  * the summed int4 error vs the shard count P. The page's section
    "Combating Quantization Errors with Tensor Parallelism" says the errors
    of quantized partial sums cluster around zero, Irwin-Hall-like, nearing a
    Gaussian as devices are added. For independent per-shard rounding errors,
    uniform on [-s_p/2, s_p/2], the sum has variance sum_p s_p^2/12 and
    excess kurtosis -1.2 sum_p s_p^4 / (sum_p s_p^2)^2 (-1.2/P for equal
    scales);
  * drift: outlier columns that move after calibration (the stress workload)
    are quantized with ranges that do not hold them;
  * output precision: the fp32 and the bf16-output receivers against the
    same exact sum.

Error measures over y [T,H]: nmse = sum (y - exact)^2 / sum exact^2, its
SNR in dB, and the largest absolute error.

    python quality.py                      # every report, default sizes
    python quality.py --only irwin_hall    # one report
    python quality.py --out report.txt     # also write the text tables

Each record is printed as one JSON line, and a text table follows at the end.
"""
from __future__ import annotations

import argparse
import json
import math
import sys
import time

import numpy as np
import torch

import bit_tensor_activation_amd as B
import workloads as W

DEV = torch.device("cuda:0")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------ measures ----
def exact_sum(x: torch.Tensor) -> torch.Tensor:
    """sum_p x[p] in float64, [T,H]."""
    xb = x.view(torch.bfloat16)
    ex = torch.zeros(xb.shape[1:], dtype=torch.float64, device=x.device)
    for p in range(xb.shape[0]):
        ex += xb[p].double()
    return ex


def error_stats(y: torch.Tensor, ex: torch.Tensor) -> dict:
    d = y.double() - ex
    num = float((d * d).sum())
    den = float((ex * ex).sum())
    nmse = num / den if den > 0 else float("nan")
    return dict(nmse=nmse, snr_db=(-10.0 * math.log10(nmse)) if nmse > 0 else float("inf"),
                max_abs_err=float(d.abs().max()))


def calibrate(P, H, batches, momentum):
    """Running (min, max) [P,H] after the given calibration batches."""
    rmin = torch.empty((P, H), dtype=torch.float32, device=DEV)
    rmax = torch.empty_like(rmin)
    for b, xb in enumerate(batches):
        B.btq_calib_update(xb() if callable(xb) else xb, rmin, rmax, momentum,
                           first_batch=(b == 0))
    return rmin, rmax


def run_codec(x: torch.Tensor, sel: dict) -> torch.Tensor:
    """y = decompress_reduce(compress_pack(x)) with the selection's parameters
    and maps (the per-shard calls when the selection holds one set per
    shard)."""
    H = x.shape[2]
    enc = (sel["rscale"], sel["zero_point"], sel["outlier_idx"], sel["cmap"])
    dec = (sel["scale"], sel["zero_point"], sel["fmap"])
    if sel["outlier_idx"].dim() == 2:
        k = sel["outlier_idx"].shape[1]
        pk, ol = B.btq_compress_pack_per_shard(x, k, *enc)
        return B.btq_decompress_reduce_per_shard(pk, ol, H, *dec)
    k = sel["outlier_idx"].numel()
    pk, ol = B.btq_compress_pack(x, k, *enc)
    return B.btq_decompress_reduce(pk, ol, H, *dec)


def workload_state(name: str, calib_batches=None, T=None):
    """Calibrated stats and inference batch 0 (T tokens: the workload's
    largest inference batch by default) of a workload."""
    w = W.WORKLOADS[name]
    nb = w.calib_batches if calib_batches is None else calib_batches
    rmin, rmax = calibrate(w.P, w.H, [lambda b=b: W.batch(w, W.PHASE_CALIB, b, device=DEV)
                                      for b in range(nb)], w.momentum)
    x = W.batch(w, W.PHASE_INFER, 0, T=max(w.T) if T is None else T, device=DEV)
    return w, rmin, rmax, x


# ------------------------------------------------------------- reports ----
def error_vs_k(name: str, ks, calib_batches=None) -> list:
    """Range-ranked selection (shard ranges summed) at each k."""
    w, rmin, rmax, x = workload_state(name, calib_batches)
    ex = exact_sum(x)
    planted = set(W.outlier_columns(w, W.PHASE_INFER).tolist())
    out = []
    for k in ks:
        if not 0 <= k <= w.H:
            continue
        sel = B.btq_select_outliers(rmin, rmax, k)
        st = error_stats(run_codec(x, sel), ex)
        got = set(sel["outlier_idx"].cpu().tolist())
        out.append(dict(report="error_vs_k", workload=name, P=w.P, T=x.shape[1], H=w.H, k=k,
                        planted_kept=len(planted & got), planted=len(planted), **st))
    return out


def shard_local_state(P=8, T=2048, H=4096, n_shared=24, n_local=8, calib_batches=4, seed=57):
    """Calibrated stats and an inference batch of normal data (sigma 0.5)
    with n_shared outlier columns wide on every shard (x40) and n_local more
    per shard, each wide on its own shard only (x80)."""
    rng = np.random.default_rng(seed)
    cols = rng.choice(H, n_shared + P * n_local, replace=False)
    shared, local = cols[:n_shared], cols[n_shared:].reshape(P, n_local)

    def draw(s):
        x = W.draw(P, T, H, s, sigma=0.5, cols=shared.tolist(), outlier_factor=40.0,
                   device=DEV).view(torch.bfloat16)
        for p in range(P):
            x[p][:, torch.as_tensor(local[p], device=DEV)] *= 80.0
        return x.view(torch.int16)
    rmin, rmax = calibrate(P, H, [lambda b=b: draw(seed * 100 + b) for b in range(calib_batches)],
                           0.9)
    return rmin, rmax, draw(seed * 100 + 99)


def selection_rules(name: str, k: int, n_random: int = 4, calib_batches=None) -> list:
    """Range-ranked (sum, max, per-shard sets), random sets and pure int4 at
    one k. name "shard_local" is the synthetic case of shard_local_state."""
    if name == "shard_local":
        rmin, rmax, x = shard_local_state()
        P, H = rmin.shape
        wid = 99
    else:
        w, rmin, rmax, x = workload_state(name, calib_batches)
        P, H, wid = w.P, w.H, w.wid
    ex = exact_sum(x)
    base = dict(report="selection", workload=name, P=P, T=x.shape[1], H=H)
    out = []
    for rule in ("sum", "max"):
        sel = B.btq_select_outliers_rule(rmin, rmax, k, rule)
        out.append(dict(base, rule=f"range_{rule}", k=k, **error_stats(run_codec(x, sel), ex)))
    sel = B.btq_select_outliers_per_shard(rmin, rmax, k)
    out.append(dict(base, rule="range_per_shard", k=k, **error_stats(run_codec(x, sel), ex)))
    rnd = []
    for s in range(n_random):
        feats = np.sort(np.random.default_rng([wid, 77, s]).choice(H, k, replace=False))
        sel = B.btq_select_features(rmin, rmax, feats)
        rnd.append(error_stats(run_codec(x, sel), ex))
    out.append(dict(base, rule="random", k=k, sets=n_random,
                    nmse=float(np.mean([r["nmse"] for r in rnd])),
                    nmse_min=min(r["nmse"] for r in rnd), nmse_max=max(r["nmse"] for r in rnd),
                    snr_db=float(np.mean([r["snr_db"] for r in rnd])),
                    max_abs_err=max(r["max_abs_err"] for r in rnd)))
    sel = B.btq_select_outliers(rmin, rmax, 0)
    out.append(dict(base, rule="int4_only", k=0, **error_stats(run_codec(x, sel), ex)))
    return out


def output_precision(name: str, calib_batches=None) -> list:
    """Error of the fp32 and the bf16-output receivers at the workload's k:
    the bf16 output adds one rounding (at most half a bf16 ulp of y) to the
    int4 error."""
    w, rmin, rmax, x = workload_state(name, calib_batches)
    ex = exact_sum(x)
    sel = B.btq_select_outliers(rmin, rmax, w.k)
    pk, ol = B.btq_compress_pack(x, w.k, sel["rscale"], sel["zero_point"], sel["outlier_idx"],
                                 sel["cmap"])
    args = (pk, ol, w.H, sel["scale"], sel["zero_point"], sel["fmap"])
    y32 = B.btq_decompress_reduce(*args)
    y16 = B.btq_decompress_reduce_bf16(*args).view(torch.bfloat16).float()
    base = dict(report="output", workload=name, P=w.P, T=x.shape[1], H=w.H, k=w.k)
    return [dict(base, output="fp32", **error_stats(y32, ex)),
            dict(base, output="bf16", **error_stats(y16, ex))]


def irwin_hall(Ps, T=2048, H=4096, sigma=0.5, calib_batches=4, seed=91) -> list:
    """Statistics of the summed int4 error (k = 0) vs the shard count P.

    Normal partial sums with no outliers. Only elements whose P shard values
    all lie inside their calibrated ranges are counted (clipped values carry
    larger errors that the rounding model does not describe). The error is
    standardized per feature by sqrt(sum_p s_p^2 / 12).
    """
    out = []
    for P in Ps:
        calib = [lambda b=b: W.draw(P, T, H, seed * 1000 + 10 * P + b, sigma=sigma, device=DEV)
                 for b in range(calib_batches)]
        rmin, rmax = calibrate(P, H, calib, 0.9)
        x = W.draw(P, T, H, seed * 1000 + 10 * P + 9, sigma=sigma, device=DEV)
        sel = B.btq_select_outliers(rmin, rmax, 0)
        y = run_codec(x, sel)
        e = y.double() - exact_sum(x)
        lo = torch.clamp(rmin, max=0.0)
        hi = torch.clamp(rmax, min=0.0)
        xb = x.view(torch.bfloat16).float()
        inside = ((xb >= lo[:, None, :]) & (xb <= hi[:, None, :])).all(dim=0)
        s = sel["scale"].double()
        s2 = (s * s).sum(0)
        z = (e / torch.sqrt(s2 / 12.0)[None, :])[inside]
        n = z.numel()
        m = float(z.mean())
        v = float(((z - m) ** 2).mean())
        kurt = float(((z - m) ** 4).mean()) / (v * v) - 3.0
        pred = (-1.2 * (s ** 4).sum(0) / (s2 * s2))          # per feature
        counts = inside.sum(0).double()
        pred_kurt = float((pred * counts).sum() / counts.sum())
        out.append(dict(report="irwin_hall", P=P, T=T, H=H, n=n,
                        frac_in_range=n / float(inside.numel()), mean_z=m,
                        mean_z_tolerance=4.0 / math.sqrt(n), var_z=v, excess_kurtosis=kurt,
                        predicted_excess_kurtosis=pred_kurt, equal_scale_value=-1.2 / P))
        del x, y, e, xb, inside, z
    return out


def drift(name: str, ks, calib_batches=None) -> list:
    """Error with the inference batch's outlier columns moved after
    calibration (the workload's own inference batch) against the same draw
    with the calibration columns."""
    w, rmin, rmax, x = workload_state(name, calib_batches)
    x_still = W.draw(w.P, x.shape[1], w.H, W.seed_of(w.wid, W.PHASE_INFER, 0), base=w.base,
                     sigma=w.sigma, cols=W.outlier_columns(w, W.PHASE_CALIB),
                     outlier_mode=w.outlier_mode, outlier_factor=w.outlier_factor, device=DEV)
    calib_cols = set(W.outlier_columns(w, W.PHASE_CALIB).tolist())
    moved_in = sorted(set(W.outlier_columns(w, W.PHASE_INFER).tolist()) - calib_cols)
    mi = torch.as_tensor(moved_in, device=DEV)
    lo = torch.clamp(rmin, max=0.0)
    hi = torch.clamp(rmax, min=0.0)
    out = []
    for label, xi in (("drifted", x), ("no_drift", x_still)):
        ex = exact_sum(xi)
        xb = xi.view(torch.bfloat16).float()
        clipped = float(((xb < lo[:, None, :]) | (xb > hi[:, None, :])).double().mean())
        del xb
        for k in ks:
            sel = B.btq_select_outliers(rmin, rmax, k)
            y = run_codec(xi, sel)
            st = error_stats(y, ex)
            st_moved = error_stats(y[:, mi], ex[:, mi]) if len(moved_in) else {}
            out.append(dict(report="drift", workload=name, inference=label, k=k,
                            moved_columns=len(moved_in), clipped_fraction=clipped, **st,
                            nmse_moved_columns=st_moved.get("nmse")))
            del y
    return out


# -------------------------------------------------------------- output ----
def table(records: list) -> str:
    lines = []
    by = {}
    for r in records:
        by.setdefault(r["report"], []).append(r)
    if "error_vs_k" in by:
        lines += ["error vs k (range-ranked, shard ranges summed)",
                  "workload | k | planted kept | nmse | SNR dB | max |err|"]
        lines += [f"{r['workload']} | {r['k']} | {r['planted_kept']}/{r['planted']} | "
                  f"{r['nmse']:.3e} | {r['snr_db']:.1f} | {r['max_abs_err']:.3g}"
                  for r in by["error_vs_k"]]
        lines.append("")
    if "selection" in by:
        lines += ["selection rules at the workload's k",
                  "workload | rule | k | nmse | SNR dB | max |err|"]
        for r in by["selection"]:
            extra = (f" (min {r['nmse_min']:.3e}, max {r['nmse_max']:.3e}, {r['sets']} sets)"
                     if r["rule"] == "random" else "")
            lines.append(f"{r['workload']} | {r['rule']} | {r['k']} | {r['nmse']:.3e}{extra} | "
                         f"{r['snr_db']:.1f} | {r['max_abs_err']:.3g}")
        lines.append("")
    if "output" in by:
        lines += ["output precision at the workload's k (fp32 vs bf16 receiver)",
                  "workload | k | output | nmse | SNR dB | max |err|"]
        lines += [f"{r['workload']} | {r['k']} | {r['output']} | {r['nmse']:.3e} | "
                  f"{r['snr_db']:.1f} | {r['max_abs_err']:.3g}" for r in by["output"]]
        lines.append("")
    if "irwin_hall" in by:
        lines += ["summed int4 error vs P (k=0, normal data, in-range elements, z = e/sd)",
                  "P | elements | in range | mean z (tol) | var z | excess kurtosis | predicted "
                  "| -1.2/P"]
        lines += [f"{r['P']} | {r['n']} | {r['frac_in_range']:.4f} | {r['mean_z']:+.2e} "
                  f"({r['mean_z_tolerance']:.1e}) | {r['var_z']:.4f} | {r['excess_kurtosis']:+.4f}"
                  f" | {r['predicted_excess_kurtosis']:+.4f} | {r['equal_scale_value']:+.4f}"
                  for r in by["irwin_hall"]]
        lines.append("")
    if "drift" in by:
        lines += ["drift (outlier columns moved after calibration)",
                  "workload | inference | k | clipped | nmse | SNR dB | nmse on moved columns"]
        lines += [f"{r['workload']} | {r['inference']} | {r['k']} | {r['clipped_fraction']:.2e} | "
                  f"{r['nmse']:.3e} | {r['snr_db']:.1f} | "
                  + (f"{r['nmse_moved_columns']:.3e}" if r["nmse_moved_columns"] is not None
                     else "-") for r in by["drift"]]
        lines.append("")
    return "\n".join(lines)


REPORTS = ("error_vs_k", "selection", "output", "irwin_hall", "drift")


def run(only=None) -> list:
    recs = []
    todo = REPORTS if only is None else (only,)
    for rep in todo:
        t0 = time.time()
        if rep == "error_vs_k":
            recs += error_vs_k("7b_prefill", [0, 8, 16, 32, 41, 48, 64, 128, 256])
            recs += error_vs_k("large_prefill", [0, 32, 64, 128, 164, 256])
        elif rep == "selection":
            recs += selection_rules("7b_prefill", 64)
            recs += selection_rules("large_prefill", 128)
            recs += selection_rules("decode", 64)
            recs += selection_rules("shard_local", 32)
            recs += selection_rules("shard_local", 64)
        elif rep == "output":
            recs += output_precision("7b_prefill")
            recs += output_precision("large_prefill")
        elif rep == "irwin_hall":
            recs += irwin_hall([1, 2, 4, 8, 16])
        elif rep == "drift":
            recs += drift("stress", [0, 32, 256])
        torch.cuda.synchronize()
        log(f"[quality] {rep} done in {time.time() - t0:.1f} s")
    return recs


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--only", choices=REPORTS)
    ap.add_argument("--out", help="also write the text tables here")
    a = ap.parse_args()
    if not torch.cuda.is_available():
        print("quality.py needs a GPU (the codec runs in HIP kernels)", file=sys.stderr)
        return 2
    recs = run(a.only)
    for r in recs:
        print(json.dumps(r))
    txt = table(recs)
    print(txt)
    if a.out:
        with open(a.out, "w") as f:
            f.write(txt + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
