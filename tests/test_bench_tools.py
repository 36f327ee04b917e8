"""CPU tests of the benchmark's measurement tooling: the algorithmic byte count
of a step, the rocprofv3 csv summaries (kernel trace percentiles, counter
means, traffic checked against calibration kernels of known size), the tie
between a traffic summary and the kernel sources, the CPU-baseline thread
count, and the one-GPU guard. No GPU is touched."""
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
    for k in ("k_bt64s_w4a4", "k_bt64_w4a4"):
        assert bench.step_bytes(dm, N, k, False) == 8 * M * T + payload + block_offsets + N * (K // 2) + 4 * M * N
    # the row-wave kernel reads every tile's offset instead of the block starts
    assert bench.step_bytes(dm, N, "k_rowwave_w4a4", False) == 8 * M * T + 4 * M * T + payload + N * (K // 2) + 4 * M * N
    W16 = (rng.normal(size=(M, K)) * (rng.random((M, K)) < 0.4)).astype(np.float16)
    e16 = bsp.encode(W16)
    d16 = e16.to_device("cpu")
    assert bench.step_bytes(d16, N, "k_bt64_f16", True) == 8 * M * T + 2 * e16.nnz + block_offsets + 2 * N * K + 2 * M * N
    # the eight-row fp16 kernel: one offset per 8-row step plus the end, and one half-row start per row
    step_offsets = 4 * ((M + 7) // 8 + 1 + M)
    assert bench.step_bytes(d16, N, "k_bt8_f16", True) == 8 * M * T + 2 * e16.nnz + step_offsets + 2 * N * K + 2 * M * N
    # odd K: X rows of ceil(K/2) bytes
    W = (rng.integers(-8, 8, size=(5, 77)) * (rng.random((5, 77)) < 0.5)).astype(np.int8)
    e = bsp.encode(W)
    assert bench.step_bytes(e.to_device("cpu"), 2, "k_bt64s_w4a4", False) == \
        8 * 5 * 2 + (e.nnz + 1) // 2 + 4 * 2 + 2 * 39 + 4 * 5 * 2


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


def _rows(kernel, counters):
    return [{"Kernel_Name": kernel, "Dispatch_Id": i, "Counter_Name": c, "Counter_Value": v}
            for c, vals in counters.items() for i, v in enumerate(vals)]


def test_counter_summary_and_traffic_calibration(tmp_path):
    k = "void k_bt64s_w4a4<1, 3, false>(unsigned int const*)"
    probe = "void k_probe_read<0>(unsigned char const*, unsigned int, unsigned int*)"
    cp = "at::native::bitwise_not_kernel_cuda"
    base = str(tmp_path)
    C = bench.COPY_BYTES
    # the probe reads C bytes in 128-byte requests; the copy reads C in 128-byte
    # and writes C in 64-byte requests. The DRAM 32-byte counts see all of it;
    # the by-size counts are made to miss a sixth of the copy's writes, so only
    # the first estimator passes the 5 % check.
    reads = (_rows(probe, {"TCC_EA0_RDREQ_128B_sum": [C / 128] * 3, "TCC_EA0_RDREQ_DRAM_32B_sum": [C / 32] * 3,
                           "TCC_EA0_RDREQ_32B_sum": [0] * 3, "TCC_EA0_RDREQ_64B_sum": [0] * 3})
             + _rows(cp, {"TCC_EA0_RDREQ_128B_sum": [C / 128] * 2, "TCC_EA0_RDREQ_DRAM_32B_sum": [C / 32] * 2,
                          "TCC_EA0_RDREQ_32B_sum": [0] * 2, "TCC_EA0_RDREQ_64B_sum": [0] * 2})
             + _rows(k, {"TCC_EA0_RDREQ_128B_sum": [100.0, 110.0], "TCC_EA0_RDREQ_DRAM_32B_sum": [400.0, 440.0],
                         "TCC_EA0_RDREQ_32B_sum": [0, 0], "TCC_EA0_RDREQ_64B_sum": [0, 0]}))
    writes = (_rows(probe, {"TCC_EA0_WRREQ_sum": [1] * 3, "TCC_EA0_WRREQ_64B_sum": [0] * 3,
                            "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum": [1] * 3, "TCC_BUBBLE_sum": [0] * 3})
              + _rows(cp, {"TCC_EA0_WRREQ_sum": [C / 64 * 5 / 6] * 2, "TCC_EA0_WRREQ_64B_sum": [C / 64 * 5 / 6] * 2,
                           "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum": [C / 32] * 2, "TCC_BUBBLE_sum": [0] * 2})
              + _rows(k, {"TCC_EA0_WRREQ_sum": [8.0, 8.0], "TCC_EA0_WRREQ_64B_sum": [8.0, 8.0],
                          "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum": [16.0, 16.0], "TCC_BUBBLE_sum": [0, 0]})
              + _rows("other", {"TCC_EA0_WRREQ_sum": [99.0], "TCC_EA0_WRREQ_64B_sum": [0],
                                "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum": [99.0], "TCC_BUBBLE_sum": [0]}))
    _write_csv(os.path.join(base, "r", "x_counter_collection.csv"), reads)
    _write_csv(os.path.join(base, "w", "x_counter_collection.csv"), writes)
    out = os.path.join(base, "traffic.txt")
    bench.summarize_traffic(out, os.path.join(base, "r"), os.path.join(base, "w"), "bt64s", ["demo"])
    kv = dict(l.split(":", 1) for l in open(out) if ":" in l and not l.startswith("#"))
    assert kv["estimator"].strip() == "dram_32b"
    # mean DRAM units: reads (400 + 440) / 2 x 32 B, writes 16 x 32 B
    assert float(kv["traffic_bytes_per_launch"]) == pytest.approx(420 * 32 + 16 * 32)
    assert "outside 5 %" in open(out).read()          # the by-size estimator's check failed and is reported
    # the summary is tied to the kernel sources it was taken from
    assert bench.read_traffic(out) == pytest.approx(420 * 32 + 16 * 32)
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


def test_traffic_without_a_calibrated_estimator_is_null(tmp_path):
    probe, cp, k = "k_probe_read<0>", "bitwise_not_kernel", "k_bt64s_w4a4<1, 3, false>"
    C = bench.COPY_BYTES
    reads = [{"Kernel_Name": kk, "Dispatch_Id": 0, "Counter_Name": c, "Counter_Value": C / 64}
             for kk in (probe, cp, k) for c in bench.READ_COUNTERS]
    writes = [{"Kernel_Name": kk, "Dispatch_Id": 0, "Counter_Name": c, "Counter_Value": 1.0}
              for kk in (probe, cp, k) for c in bench.WRITE_COUNTERS]
    _write_csv(os.path.join(str(tmp_path), "r", "x_counter_collection.csv"), reads)
    _write_csv(os.path.join(str(tmp_path), "w", "x_counter_collection.csv"), writes)
    out = os.path.join(str(tmp_path), "t.txt")
    bench.summarize_traffic(out, os.path.join(str(tmp_path), "r"), os.path.join(str(tmp_path), "w"), "bt64s", [])
    assert "estimator: none" in open(out).read()
    assert bench.read_traffic(out) is None


def test_cpu_baseline_thread_count(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "16")
    assert bench.host_threads() == 16
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert bench.host_threads() >= 1
    assert isinstance(bench.cpu_model(), str)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in (r.stdout + r.stderr)
