"""The oracle's pins catch plausible mistakes.

Each mutant below is the oracle's own source with one plausible mistake
planted in it: a dropped term, a wrong sign, index or axis, swapped
operands, another rounding or tie rule, a transposed layout. The planted
copy runs on the CPU only, as a separate module. The pins of
tests/test_oracle_*.py then run against it, and at least one of them must
fail. The unmodified source, loaded the same way, must pass every pin, so
a failure is the mistake's and not the loading's. (Edits that cannot change
a result are not listed: the zero point's clamp, for one, never binds,
since lo <= 0 <= hi puts -lo/scale in [0, 15(1+eps)].)

Page: "Revolutionizing LLM Inference: The Power of Efficient Low-Bit
Communication", section "The Hybrid Quantization Algorithm" (Calibration,
Selection and Inference bullets): the steps each mutant breaks.
"""
import importlib
import inspect
import types
import warnings

import pytest

from oracle import oracle as O

PIN_MODULES = ("test_oracle_calib", "test_oracle_quant", "test_oracle_select", "test_oracle_reduce")

# (name, [(text in the oracle's source, its planted replacement), ...])
MUTANTS = [
    ("bf16 decode shifts by 15", [("<< np.uint32(16)).view(F32)", "<< np.uint32(15)).view(F32)")]),
    ("batch min and max swapped", [("return f.min(axis=1), f.max(axis=1)",
                                    "return f.max(axis=1), f.min(axis=1)")]),
    ("batch extremes over features, not tokens",
     [("return f.min(axis=1), f.max(axis=1)",
       "return np.broadcast_to(f.min(axis=(1, 2))[:, None], f.shape[::2]), f.max(axis=1)")]),
    ("moving-average weights swapped", [("return (a * np.asarray(run, dtype=F32)) + (c * obs)",
                                         "return (c * np.asarray(run, dtype=F32)) + (a * obs)")]),
    ("first batch averaged with the old value", [("    if first:\n        return obs.copy()\n",
                                                  "")]),
    ("moving average in fp64", [("return (a * np.asarray(run, dtype=F32)) + (c * obs)",
                                 "return ((np.float64(a) * np.asarray(run, np.float64))"
                                 " + (np.float64(c) * obs)).astype(F32)")]),
    ("range does not hold zero", [("lo = np.minimum(np.asarray(run_min, F32), F32(0))",
                                   "lo = np.asarray(run_min, F32)")]),
    ("16 steps instead of 15", [("scale = width / F32(QMAX)", "scale = width / F32(QMAX + 1)")]),
    ("zero point sign", [("np.rint(-lo / scale)", "np.rint(lo / scale)")]),
    ("zero point floored", [("np.rint(-lo / scale)", "np.floor(-lo / scale)")]),
    ("degenerate range not guarded", [("scale = np.where(scale < F32(FLT_MIN), F32(1), scale)",
                                       "scale = np.where(scale < F32(0), F32(1), scale)")]),
    ("score skips the last shard", [("for p in range(width.shape[0]):\n        score = score + width[p]",
                                     "for p in range(width.shape[0] - 1):\n        score = score + width[p]")]),
    ("score takes the first shard's range only",
     [("score = score + width[p] if rule == \"sum\"",
       "score = width[0] if rule == \"sum\"")]),
    ("max rule takes the minimum", [("else np.maximum(score, width[p])",
                                     "else np.minimum(score, width[p])")]),
    ("given set replaced by the ranked one",
     [("idx, fmap, cmap = maps_for_set(idx, scale.shape[1])",
       "idx, fmap, cmap = top_k_features(score, len(idx))")]),
    ("fmap inverted without the -1 offset", [("idx[-1 - fmap[~ints]] = h[~ints]",
                                              "idx[np.abs(fmap[~ints]) % len(idx)] = h[~ints]")]),
    ("ties go to the higher feature", [("np.lexsort((h, -score))", "np.lexsort((-h, -score))")]),
    ("the narrowest features kept", [("np.lexsort((h, -score))", "np.lexsort((h, score))")]),
    ("BF16 set listed in rank order", [("return maps_for_set(np.sort(order[:k]), H)",
                                        "return maps_for_set(order[:k], H)")]),
    ("BF16 slot code off by one", [("fmap[idx] = -1 - np.arange(k, dtype=np.int32)",
                                    "fmap[idx] = -np.arange(k, dtype=np.int32)")]),
    ("zero point added before rounding",
     [("q = np.rint(v) + np.asarray(zero_point).astype(F32)",
       "q = np.rint(v + np.asarray(zero_point).astype(F32))")]),
    ("ties round away from zero", [("q = np.rint(v) + np.asarray",
                                    "q = np.sign(v) * np.floor(np.abs(v) + F32(0.5)) + np.asarray")]),
    ("codes truncated", [("q = np.rint(v) + np.asarray", "q = np.trunc(v) + np.asarray")]),
    ("division instead of the stored reciprocal",
     [("v = np.asarray(f, F32) * np.asarray(rscale, F32)",
       "v = np.asarray(f, F32) / (F32(1) / np.asarray(rscale, F32))")]),
    ("codes not clamped at 15", [("return np.clip(q, F32(0), F32(QMAX)).astype(np.uint8)",
                                  "return np.clip(q, F32(0), F32(255)).astype(np.uint8)")]),
    ("nibbles swapped in both directions",
     [("(qq[..., 0::2] | (qq[..., 1::2] << np.uint8(4)))",
       "(qq[..., 1::2] | (qq[..., 0::2] << np.uint8(4)))"),
      ("q[..., 0::2] = b & np.uint8(0x0F)\n    q[..., 1::2] = b >> np.uint8(4)",
       "q[..., 1::2] = b & np.uint8(0x0F)\n    q[..., 0::2] = b >> np.uint8(4)")]),
    ("row padding not zero", [("out = np.zeros(b.shape[:-1] + (pitch,), np.uint8)",
                               "out = np.full(b.shape[:-1] + (pitch,), 0x11, np.uint8)")]),
    ("shard 0's parameters for every shard",
     [("q = quantize(f, rscale[p, cmap[p]][None, :], zero_point[p, cmap[p]][None, :])",
       "q = quantize(f, rscale[0, cmap[p]][None, :], zero_point[0, cmap[p]][None, :])")]),
    ("BF16 block in descending feature order", [("outl.append(x[p][:, idx[p]])",
                                                 "outl.append(x[p][:, idx[p][::-1]])")]),
    ("zero point dropped in dequantization",
     [("d = np.asarray(q).astype(F32) - np.asarray(zero_point).astype(F32)",
       "d = np.asarray(q).astype(F32)")]),
    ("dequantization divides by the scale", [("return d * np.asarray(scale, F32)",
                                              "return d / np.asarray(scale, F32)")]),
    ("the last shard dropped from the sum", [("        y = y + term\n",
                                              "        y = y + term if p < P - 1 else y\n")]),
    ("shard 0's BF16 block for every shard", [("term[:, idx] = bf16_to_f32(outliers[p])",
                                               "term[:, idx] = bf16_to_f32(outliers[0])")]),
    ("shard 0's map for every shard", [("idx, cmap = maps_from_fmap(fmap[p])",
                                        "idx, cmap = maps_from_fmap(fmap[0])")]),
    ("sum in fp64", [("y = np.zeros((T, H), F32)", "y = np.zeros((T, H), np.float64)")]),
    ("bf16 output truncated", [("((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16))",
                                "(u >> np.uint64(16))")]),
    ("bf16 output ties round up", [("((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16))",
                                    "((u + np.uint64(0x8000)) >> np.uint64(16))")]),
    ("per-shard sets ranked by the shared score",
     [("idx[p], fmap[p], cmap[p] = top_k_features(width[p], k)",
       "idx[p], fmap[p], cmap[p] = top_k_features(range_score(width), k)")]),
]


def _load(source: str) -> types.ModuleType:
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = O.__file__
    exec(compile(source, O.__file__, "exec"), mod.__dict__)
    return mod


def _cases(fn):
    """Argument sets of a test function from its parametrize marks."""
    combos = [{}]
    for m in getattr(fn, "pytestmark", []):
        if m.name != "parametrize":
            continue
        names = m.args[0]
        names = [n.strip() for n in names.split(",")] if isinstance(names, str) else list(names)
        out = []
        for c in combos:
            for v in m.args[1]:
                vals = v.values if hasattr(v, "values") else ((v,) if len(names) == 1 else tuple(v))
                out.append({**c, **dict(zip(names, vals))})
        combos = out
    return combos


def _pins():
    pins = []
    for name in PIN_MODULES:
        mod = importlib.import_module(name)
        for attr, fn in sorted(vars(mod).items()):
            if attr.startswith("test_") and inspect.isfunction(fn):
                for kw in _cases(fn):
                    pins.append((mod, f"{name}::{attr}{sorted(kw.items()) if kw else ''}", fn, kw))
    return pins


def _first_failure(oracle_module, monkeypatch):
    """The first pin that fails against oracle_module, or None."""
    pins = _pins()
    for mod in {p[0] for p in pins}:
        monkeypatch.setattr(mod, "O", oracle_module)
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        for _, pid, fn, kw in pins:
            try:
                fn(**kw)
            except pytest.skip.Exception:
                continue
            except Exception as e:   # an assertion, or a crash the mistake causes
                return f"{pid}: {type(e).__name__}"
    return None


def test_every_pin_runs_and_the_unmodified_source_passes(monkeypatch):
    assert len(_pins()) >= 60
    assert _first_failure(_load(inspect.getsource(O)), monkeypatch) is None


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_a_pin_catches_the_mistake(name, edits, monkeypatch):
    src = inspect.getsource(O)
    for old, new in edits:
        assert src.count(old) == 1, f"the mutant's text no longer matches the oracle once: {old!r}"
        src = src.replace(old, new)
    caught = _first_failure(_load(src), monkeypatch)
    assert caught is not None, f"no pin fails when the oracle has: {name}"
