"""CPU tests of the benchmark's measurement tooling: the algorithmic byte count
of a step, the rocprofv3 csv summaries (kernel trace percentiles, counter
means, copy-calibrated traffic), the tie between a traffic summary and the
kernel sources, and the one-GPU guard. No GPU is touched."""
import csv
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import bit_unstructured_sparse_amd as bsp  # noqa: E402


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_step_bytes_counts_each_array_once():
    # a small encoded matrix: the step's bytes are the arrays the kernel
    # reads, counted from their own sizes, plus X and Y
    rng = np.random.default_rng(5)
    M, K, N = 40, 200, 3
    W = (rng.integers(-8, 8, size=(M, K)) * (rng.random((M, K)) < 0.4)).astype(np.int8)
    enc = bsp.encode(W)
    dm = enc.to_device("cpu")   # the byte count needs only the arrays' sizes
    T = (K + 63) // 64
    assert enc.bitmaps.size == M * T and enc.offsets.size == M * T + 1
    payload = (enc.nnz + 1) // 2
    block_offsets = 4 * ((M + 15) // 16 + 1)
    assert bench.step_bytes(dm, N, "mfma", False) == 8 * M * T + payload + block_offsets + N * (K // 2) + 4 * M * N
    # the row-wave kernel reads every tile offset instead of the block starts
    assert bench.step_bytes(dm, N, "rowwave", False) == 8 * M * T + 4 * (M * T + 1) + payload + N * (K // 2) + 4 * M * N
    W16 = (rng.normal(size=(M, K)) * (rng.random((M, K)) < 0.4)).astype(np.float16)
    e16 = bsp.encode(W16)
    assert bench.step_bytes(e16.to_device("cpu"), N, "mfma", True) == 8 * M * T + 2 * e16.nnz + block_offsets + 2 * N * K + 2 * M * N


def test_trace_summary_percentiles(tmp_path):
    d = str(tmp_path / "trace")
    durs = [float(x) for x in range(1, 11)]   # 1..10 us
    _write_csv(os.path.join(d, "run", "t_kernel_trace.csv"),
               [{"Kernel_Name": "k_demo(int)", "Start_Timestamp": 1000 * i, "End_Timestamp": 1000 * i + int(u * 1000)}
                for i, u in enumerate(durs)])
    _write_csv(os.path.join(d, "run", "t_kernel_stats.csv"),
               [{"Name": "k_demo(int)", "Calls": 10, "TotalDurationNs": 55000, "AverageNs": 5500, "MinNs": 1000,
                 "MaxNs": 10000, "Percentage": 100.0}])
    out = str(tmp_path / "trace.txt")
    bench.summarize_trace(d, out, ["demo"])
    line = [l for l in open(out) if l.startswith("k_demo")][0].split()
    calls, avg, mn, p10, p50, p90, mx = line[1:8]
    assert int(calls) == 10 and float(avg) == 5.5 and float(mn) == 1.0 and float(mx) == 10.0
    # nearest-rank on the sorted durations: index round(q * 9)
    assert (float(p10), float(p50), float(p90)) == (2.0, 6.0, 9.0)


def _counter_rows(kernel, counter, values):
    return [{"Kernel_Name": kernel, "Dispatch_Id": i, "Counter_Name": counter, "Counter_Value": v}
            for i, v in enumerate(values)]


def test_counter_summary_and_traffic_calibration(tmp_path):
    k = "void k_bt64s_w4a4<1, 3>(unsigned int const*)"
    cp = "at::native::bitwise_not_kernel_cuda"
    base = str(tmp_path)
    # the copy reads and writes COPY_BYTES; its counters read 1/2 and 1/1 of that in KiB
    copy_kib = bench.COPY_BYTES / 1024.0
    _write_csv(os.path.join(base, "cf", "x_counter_collection.csv"), _counter_rows(cp, "FETCH_SIZE", [copy_kib / 2] * 3))
    _write_csv(os.path.join(base, "cw", "x_counter_collection.csv"), _counter_rows(cp, "WRITE_SIZE", [copy_kib] * 3))
    _write_csv(os.path.join(base, "f", "x_counter_collection.csv"),
               _counter_rows(k, "FETCH_SIZE", [100.0, 110.0]) + _counter_rows("other", "FETCH_SIZE", [5.0]))
    _write_csv(os.path.join(base, "w", "x_counter_collection.csv"), _counter_rows(k, "WRITE_SIZE", [8.0, 8.0]))
    out = os.path.join(base, "traffic.txt")
    bench.summarize_traffic(out, os.path.join(base, "f"), os.path.join(base, "w"), os.path.join(base, "cf"),
                            os.path.join(base, "cw"), "w4a4", ["demo"])
    kv = dict(l.split(":", 1) for l in open(out) if ":" in l and not l.startswith("#"))
    assert float(kv["fetch_factor"]) == pytest.approx(2.0) and float(kv["write_factor"]) == pytest.approx(1.0)
    # mean fetch 105 KiB x 2 + write 8 KiB x 1
    assert float(kv["traffic_bytes_per_launch"]) == pytest.approx(105 * 1024 * 2 + 8 * 1024)
    # the summary is tied to the kernel sources it was taken from
    assert bench.read_traffic(out) == pytest.approx(105 * 1024 * 2 + 8 * 1024)
    stale = os.path.join(base, "stale.txt")
    with open(stale, "w") as f:
        f.write("".join(l.replace(bench.source_digest(), "0" * 16) for l in open(out)))
    assert bench.read_traffic(stale) is None
    assert bench.read_traffic(os.path.join(base, "missing.txt")) is None
    # plain counter means, for the kernel named by the fragment only
    cnt = os.path.join(base, "cnt.txt")
    _write_csv(os.path.join(base, "c", "x_counter_collection.csv"),
               _counter_rows(k, "SQ_INSTS_VALU", [10.0, 30.0]) + _counter_rows("other", "SQ_INSTS_VALU", [99.0]))
    bench.summarize_counters(os.path.join(base, "c"), cnt, "bt64s", ["demo"])
    assert "SQ_INSTS_VALU: 20  (mean of 2 dispatches)" in open(cnt).read()


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in (r.stdout + r.stderr)
