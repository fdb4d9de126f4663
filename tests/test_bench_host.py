"""Host logic of bench.py (CPU): kernel classification, the rocprofv3
summaries, the algorithmic byte counts and the traffic hash check.

The rocprofv3 CSV files here are small hand-made stand-ins with the columns
the summaries read; the numbers are chosen so that every figure can be
checked by hand.
"""
import csv
import os

import pytest

import bench

W7 = dict(P=8, T=2048, H=4096, k=64)


@pytest.mark.parametrize("name,cls", [
    ("void btq::compress_ring_kernel<1, 8, false>(unsigned short const*, long)", "compress_pack"),
    ("btq::compress_kernel<2, false>(x)", "compress_pack"),
    ("btq::compress_general_kernel<false>(x)", "compress_pack"),
    ("btq::compress_ring_kernel<1, 8, true>(x)", "compress_pack_per_shard"),
    ("btq::compress_general_kernel<true>(x)", "compress_pack_per_shard"),
    ("void btq::dq_window_kernel<8, 2, 4, false, false>(unsigned char const*, int)",
     "decompress_reduce"),
    ("btq::dq_window_kernel<8, 4, 2, false, true>(x)", "decompress_reduce_bf16"),
    ("btq::dq_window_kernel<8, 2, 4, true, false>(x)", "decompress_reduce_per_shard"),
    ("btq::dq_general_kernel<false, false>(x)", None),
    ("void at::native::copyBuffer<...>(...)", "copy"),
    ("btq::calib_partial_kernel<true>(x)", None),
])
def test_kernel_classes(name, cls):
    assert bench._kernel_class(name) == cls


def test_algorithmic_bytes_by_hand():
    # 5 bytes of parameters per (shard, feature) and 4 of maps per feature
    P, T, H, k = W7["P"], W7["T"], W7["H"], W7["k"]
    Bq = (H - k) // 2                              # 2016
    message = P * T * (Bq + 2 * k)
    comp, deco = bench.algorithmic_bytes(P, T, H, k)
    assert comp == P * T * H * 2 + message + 5 * P * H + 4 * H == 169_525_248
    assert deco == message + T * H * 4 + 5 * P * H + 4 * H == 68_861_952
    assert bench.algorithmic_bytes(P, T, H, k, y_bytes=2)[1] == deco - T * H * 2
    comp_ps, deco_ps = bench.algorithmic_bytes_per_shard(P, T, H, k)
    assert comp_ps == P * T * H * 2 + message + 9 * P * H
    assert deco_ps == message + T * H * 4 + 9 * P * H
    # the stress workload (P=8, T=16384, H=8192) at k = 0, 32, 256, in MB, worked by hand
    for kk, c_mb, d_mb in ((0, 2684.72, 1074.10), (32, 2691.01, 1080.39), (256, 2735.05, 1124.43)):
        c, d = bench.algorithmic_bytes(8, 16384, 8192, kk)
        assert round(c / 1e6, 2) == c_mb and round(d / 1e6, 2) == d_mb


def write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_counter_summary(tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    mib = 256
    copy_kib = mib * 1024
    rows_f, rows_w = [], []
    d = 0
    for _ in range(3):   # three compress dispatches (median is the middle one)
        for v_f, v_w in ((100.0, 50.0), (300.0, 70.0), (200.0, 60.0)):
            d += 1
            rows_f.append([d, "btq::compress_ring_kernel<1, 8, false>(x)", "FETCH_SIZE", v_f])
            rows_w.append([d, "btq::compress_ring_kernel<1, 8, false>(x)", "WRITE_SIZE", v_w])
    d += 1
    rows_f.append([d, "btq::dq_window_kernel<8, 2, 4, false, false>(x)", "FETCH_SIZE", 40.0])
    rows_w.append([d, "btq::dq_window_kernel<8, 2, 4, false, false>(x)", "WRITE_SIZE", 80.0])
    for _ in range(5):   # the copy probe: FETCH reads half the bytes, WRITE all of them
        d += 1
        rows_f.append([d, "void at::native::copyBuffer<x>(x)", "FETCH_SIZE", copy_kib / 2])
        rows_w.append([d, "void at::native::copyBuffer<x>(x)", "WRITE_SIZE", copy_kib])
    write_csv(str(tmp_path / "f" / "run_counter_collection.csv"), hdr, rows_f)
    write_csv(str(tmp_path / "w" / "run_counter_collection.csv"), hdr, rows_w)
    out = bench.summarize_counters(str(tmp_path / "f"), str(tmp_path / "w"), "7b_prefill", 64,
                                   mib, "note")
    kv = dict(l.split("=", 1) for l in out.splitlines() if "=" in l and not l.startswith("#"))
    assert float(kv["fetch_scale"]) == 0.5 and float(kv["write_scale"]) == 1.0
    assert float(kv["compress_pack_fetch_kib_median"]) == 200.0
    assert float(kv["compress_pack_write_kib_median"]) == 60.0
    # (200 / 0.5 + 60 / 1.0) KiB
    assert float(kv["traffic_bytes_per_launch"]) == (400 + 60) * 1024
    assert float(kv["decompress_reduce_traffic_bytes_per_launch"]) == (80 + 80) * 1024
    assert "decompress_reduce_bf16_fetch_kib_median" not in kv   # no such dispatches
    assert kv["source_hash"] == bench.source_hash(bench.KERNEL_SOURCES)


def test_trace_and_sq_summaries(tmp_path):
    write_csv(str(tmp_path / "t" / "run_kernel_stats.csv"),
              ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
              [["void btq::dq_window_kernel<8, 2, 4, false, false>(x)", 10, 19000.4, 18000, 22000,
                12.5],
               ["void at::native::elementwise(x)", 3, 5.0, 4, 6, 1.0]])
    out = bench.summarize_trace(str(tmp_path / "t"), "note")
    rows = [l for l in out.splitlines() if not l.startswith("#")]
    # no per-dispatch trace file: no quantiles
    assert rows == ["btq::dq_window_kernel<8, 2, 4, false, false> | 10 | 19000 | - | - | - | "
                    "18000 | 22000 | 12.50"]
    # durations 18000, 18100, ..., 18900 ns (ten dispatches, in shuffled order)
    durs = [18000 + 100 * i for i in (3, 7, 0, 9, 1, 5, 2, 8, 4, 6)]
    write_csv(str(tmp_path / "t" / "run_kernel_trace.csv"),
              ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp"],
              [["KERNEL_DISPATCH", "void btq::dq_window_kernel<8, 2, 4, false, false>(x)",
                1000 * i, 1000 * i + d] for i, d in enumerate(durs)] +
              [["KERNEL_DISPATCH", "void at::native::elementwise(x)", 5, 9]])
    rows = [l for l in bench.summarize_trace(str(tmp_path / "t"), "note").splitlines()
            if not l.startswith("#")]
    # median 18450, p10 18090, p90 18810 (linear interpolation)
    assert rows == ["btq::dq_window_kernel<8, 2, 4, false, false> | 10 | 19000 | 18450 | 18090 | "
                    "18810 | 18000 | 22000 | 12.50"]
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    vals = {"SQ_WAVE_CYCLES": 1000.0, "SQ_WAIT_INST_ANY": 590.0, "SQ_WAIT_ANY": 130.0,
            "SQ_ACTIVE_INST_VALU": 150.0, "SQ_ACTIVE_INST_LDS": 50.0,
            "SQ_ACTIVE_INST_VMEM": 20.0, "SQ_INSTS_VALU": 2.4e6}
    write_csv(str(tmp_path / "s" / "run_counter_collection.csv"), hdr,
              [[1, "btq::compress_ring_kernel<1, 8, false>(x)", c, v] for c, v in vals.items()])
    out = bench.summarize_sq(str(tmp_path / "s"), "note", n_simd=1000, mhz=2400.0)
    row = [l for l in out.splitlines() if not l.startswith("#")][0].split(" | ")
    assert row[0] == "btq::compress_ring_kernel<1, 8, false>"
    assert row[1:6] == ["0.59", "0.13", "0.15", "0.05", "0.02"]
    assert float(row[7]) == 4.0    # 2.4e6 instructions * 4 cycles / 1000 SIMDs / 2400 MHz


def test_traffic_is_dropped_when_the_sources_change(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    good = bench.source_hash(bench.KERNEL_SOURCES)
    (prof / "compress_x_k32_traffic.txt").write_text(
        f"# note\nsource_hash={good}\ntraffic_bytes_per_launch=1234\n")
    (prof / "compress_y_k32_traffic.txt").write_text(
        "source_hash=0000000000000000\ntraffic_bytes_per_launch=1234\n")
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    assert bench.read_traffic("x", 32) == 1234.0
    assert bench.read_traffic("x", 0) is None    # another k
    assert bench.read_traffic("y", 32) is None   # taken on other kernel sources
    assert bench.read_traffic("z", 32) is None   # no summary at all


def test_oracle_pool_task_is_the_oracle_on_its_rows():
    # one pool task = the oracle's sender and receiver on a row chunk of every
    # shard; the bytes it reports are its outputs' sizes
    import numpy as np
    from oracle import oracle as O
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((2, 40, 64)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    mn, mx = O.batch_min_max(x)
    sel = O.select_outliers(mn, mx, 4)
    bench._POOL_STATE.update(x=x, sel=sel)
    try:
        n = bench._oracle_rows((8, 40))
    finally:
        bench._POOL_STATE.clear()
    assert n == 2 * 32 * 30 + 32 * 64 * 4
    assert 1 <= bench.cpu_cores() <= 16


def test_more_than_one_gpu_is_refused(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    assert bench.main() == 2
    assert "one GPU" in capsys.readouterr().err


def test_source_hash_follows_code_not_comments(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    src.write_text("// header\nint f(int a) {  // note\n  return a + 1;\n}\n")
    h0 = bench.source_hash(["k.hip"])
    src.write_text("/* a longer\n   header */\n\nint f(int a) {\n  return a + 1;   // other note\n}\n")
    assert bench.source_hash(["k.hip"]) == h0
    src.write_text("int f(int a) {\n  return a + 2;\n}\n")
    assert bench.source_hash(["k.hip"]) != h0
