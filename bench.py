"""Benchmark of the bitmap-tiled sparse x skinny-dense SpMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload qkv] [--n N] [--algo auto]

A step is one call of the SpMM entry point (``spmm_bitmap_w4a4``, or
``spmm_bitmap_f16`` for ``--workload fp16``: host-side argument checks and
kernel selection, then the kernel that streams the compressed tiles, stages
X, decodes, contracts and stores Y) on one batch of synthetic input already
resident in HBM. Encoding is the offline step of the method and runs once,
before timing. Every timed step reads its own device copy of the inputs, and
between a copy's last use and its timed use the GPU reads at least 1 GiB of
other copies (four times the 256 MB Infinity Cache), whatever --steps is: the
K steps use copies 0..K-1, and after the graph's warm-up replay the copies
K..R-1 (>= 1 GiB) are run eagerly before the timed replay.

The K timed steps are captured once in a HIP graph (one kernel node per SpMM
call) and replayed back to back: these kernels last a few microseconds, less
than a Python-level launch, so eager launching would time the host instead.

Prints ONE JSON line. ``value`` is achieved GB/s over the algorithmic bytes of
a step (bitmaps, the offsets the kernel reads, payload, X, Y) divided by the
host wall time per step around the replay; the ``roofline`` object divides the
same bytes by the average launch duration from HIP events recorded on the
replay stream, and ``roofline.achievable`` gives what a plain streaming read
of the same byte count reaches in one launch on this GPU (the best of a few
launch shapes and load forms of ``libbsp_probe.so``), and a read of 1 GiB.
``traffic`` is the HBM byte count of one launch from the counter summary in
``profiles/`` (TCC read/write requests to DRAM, checked against a read-only
probe and a copy of known size) when that summary was taken from the current
kernel sources (else null). ``cpu_baseline`` times the CPU oracle (plain C)
on every host core the process may use, and on one core, on a bounded sample
of the same workload.

Helper modes used to produce the ``profiles/`` summaries:

    python bench.py --sweep                     # N = 1..32 on the qkv weights, N = 16, 32 at 70 % density
    python bench.py --peak-read                 # the read probe alone, at this workload's byte count
    python bench.py --counter-run               # read probe + copy of known size + the SpMM steps (for --pmc)
    python bench.py --summarize-trace DIR OUT   # rocprofv3 --kernel-trace --stats csv -> text
    python bench.py --summarize-traffic OUT --reads DIR --writes DIR --kernel FRAGMENT
    python bench.py --summarize-counters DIR OUT --kernel FRAGMENT   # rocprofv3 --pmc csv -> text
    python bench.py --summarize-selection OUT --side LABEL:TRACE:PMC:READS:WRITES:FRAGMENT ...
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
FLUSH_BYTES = 1 << 30          # other traffic between a copy's last use and its timed use
COPY_BYTES = 256 << 20         # calibration kernels: the copy reads and writes this many bytes, the probe reads it
PROBE_SHAPES = [(256, 512), (512, 512), (1024, 256), (2048, 256)]   # (grid, block) of the read probe
PROBE_MODES = {0: "registers", 1: "registers, non-temporal", 2: "direct-to-LDS, non-temporal"}
# TCC counters of the traffic passes (each pass within the 4-TCC-counter limit)
READ_COUNTERS = ["TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum",
                 "TCC_EA0_RDREQ_DRAM_32B_sum"]
WRITE_COUNTERS = ["TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum", "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum",
                  "TCC_BUBBLE_sum"]
METRIC = "achieved HBM GB/s (frac of peak) + dense-equiv TOPS, bitmap SpMM at N=1..32"

SWEEP = [("qkv", 0, n) for n in (1, 2, 4, 8, 16, 32)] + [("lowsparse", 0, 16), ("lowsparse", 0, 32)]
KERNEL_SYMBOL = {"rowwave": "k_rowwave", "mfma": "k_bt64", "splitk": "k_bsk"}


def algo_name(bsp, a):
    return {bsp.ALGO_AUTO: "auto", bsp.ALGO_ROWWAVE: "rowwave", bsp.ALGO_MFMA: "mfma", bsp.ALGO_SPLITK: "splitk"}[a]


def kernel_symbol(bsp, chosen, dt, M, K, N, nnz, workspace=False):
    """Name of the kernel a launch runs: the library's own description of the
    plan the timed choice (automatic or forced) takes, else the algorithm's
    kernel family."""
    m = re.search(r"kernel=(\S+)", bsp.describe(dt, M, K, N, nnz, workspace=workspace, algo=chosen))
    if m:
        return m.group(1)
    return KERNEL_SYMBOL[algo_name(bsp, chosen)]


def source_digest():
    """sha256 over the library's device and host sources: ties a counter
    summary to the kernel build it was taken from."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "bit_unstructured_sparse_amd", "csrc", "*")) +
                   glob.glob(os.path.join(ROOT, "include", "*.h")))
    for f in files:
        if os.path.isfile(f):
            h.update(os.path.basename(f).encode())
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def offsets_read(kernel, M, T, plan=""):
    """4-byte offsets one launch of `kernel` reads: every tile's (the plain
    row-wave kernel), one per 16-row block plus the end (the 16-row MFMA
    kernels), one per 8-row step plus the end and one half-row start per row
    (the eight-row fp16 kernel), the ends of every row's K ranges (the
    streamed split-K kernel), or the bounds of every row's chunks (the
    chunked split-K kernels: chunks of `chunk_tiles` tiles inside K ranges of
    `tiles_per_split`, from the plan's description)."""
    if kernel.startswith("k_rowwave"):
        return M * T
    if kernel.startswith("k_bt8_f16"):
        return (M + 7) // 8 + 1 + M
    if kernel.startswith("k_bsks"):
        m_s = re.search(r"splits=(\d+)", plan)
        return M * (int(m_s.group(1)) + 1) if m_s else M * T   # the ends of every row's K ranges
    if kernel.startswith("k_bsk"):
        m_tps, m_ct = re.search(r"tiles_per_split=(\d+)", plan), re.search(r"chunk_tiles=(\d+)", plan)
        if not (m_tps and m_ct):
            return M * T          # plan not described (a forced choice): at most every tile's
        tps, ct = int(m_tps.group(1)), int(m_ct.group(1))
        bounds = 1   # the row's start
        t = 0
        while t < T:
            te = min(T, t + tps)
            bounds += -(-(te - t) // ct)
            t = te
        return M * bounds
    return (M + 15) // 16 + 1


def step_bytes(dm, N, kernel, fp16, plan=""):
    """Algorithmic bytes of one SpMM call: words, the offsets the kernel
    reads, payload, X and Y."""
    stream = dm.stream_bytes(with_offsets=False) + 4 * offsets_read(kernel, dm.M, dm.T, plan)
    if fp16:
        return stream + 2 * N * dm.K + 2 * dm.M * N
    return stream + N * ((dm.K + 1) // 2) + 4 * dm.M * N


def _pack(X):
    # test-side packer for the oracle input (pinned by tests/golden/x_int4_packing.json)
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import pins
    return pins._pack_x_for_test(X)


def host_threads():
    """Threads the CPU baseline may use: the process's CPU share (the
    OMP_NUM_THREADS the host sets for it, else the CPUs it may run on)."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _time_oracle(problem, Xin, threads, max_seconds):
    """Rows sampled and median seconds of the oracle on the first rows of W:
    the sample grows until one run takes at least a second (or W is whole),
    then runs repeat until three are taken or the budget is spent (at least
    one second of runs when W is whole)."""
    import numpy as np
    import oracle
    M = problem.M

    def run(s):
        t0 = time.perf_counter()
        if problem.dtype == "fp16":
            oracle.spmm_f16(s, Xin, threads=threads)
        else:
            oracle.spmm_w4a4(s, Xin, problem.N, threads=threads)
        return time.perf_counter() - t0

    rows = min(M, 64)
    while True:
        s = oracle.encode(np.ascontiguousarray(problem.W[:rows]))
        t = run(s)
        if t >= 1.0 or rows >= M:
            break
        rows = min(M, rows * max(2, int(1.5 / max(t, 1e-3))))
    times = [t]
    while (len(times) < 3 or sum(times) < 1.0) and sum(times) + t < max_seconds and len(times) < 50:
        times.append(run(s))
    return rows, statistics.median(times), len(times)


def cpu_baseline(problem, bytes_per_row, max_seconds=12.0):
    """The oracle as it stands (plain C: decode the stream to dense, then the
    exact int64 -- fp64 for fp16 -- triple loop), its rows split over every
    thread the process may use, and again on one thread, on a bounded sample
    of the same workload. Encoding is not timed. GB/s scales the GPU step's
    bytes by the share of rows in the sample."""
    Xin = problem.X if problem.dtype == "fp16" else _pack(problem.X)
    nthr = host_threads()
    rows, t_all, n_all = _time_oracle(problem, Xin, nthr, max_seconds)
    rows1, t_one, n_one = _time_oracle(problem, Xin, 1, max_seconds)
    sample = (f"{{rows}} of {problem.M} rows of {problem.name} (K={problem.K}, N={problem.N}): decode + exact "
              f"triple loop, median of {{n}} runs of {{t:.3f}} s; bytes scaled per row from the GPU step")
    return {"value": round(bytes_per_row * rows / t_all / 1e9, 4), "unit": "GB/s", "cores": nthr, "kind": "oracle",
            "sample": sample.format(rows=rows, n=n_all, t=t_all) + f"; rows split over {nthr} threads",
            "cpu": cpu_model(), "nproc": os.cpu_count(),
            "one_core": {"value": round(bytes_per_row * rows1 / t_one / 1e9, 4), "unit": "GB/s", "cores": 1,
                         "sample": sample.format(rows=rows1, n=n_one, t=t_one)}}


# ---------------------------------------------------------------- read probe

def _probe_lib():
    import ctypes
    path = os.path.join(ROOT, "bit_unstructured_sparse_amd", "libbsp_probe.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is missing; build it with `python -m bit_unstructured_sparse_amd.build`")
    L = ctypes.CDLL(path)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.bsp_probe_read.argtypes, L.bsp_probe_read.restype = [P, I64, P, I32, I32, I32, P], I32
    L.bsp_probe_sink_words.argtypes, L.bsp_probe_sink_words.restype = [I32, I32], I64
    return L


def _probe_launch(L, buf_ptr, nbytes, sink, mode, grid, block):
    import ctypes
    import torch
    rc = L.bsp_probe_read(ctypes.c_void_p(buf_ptr), nbytes, ctypes.c_void_p(sink.data_ptr()), mode, grid, block,
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise RuntimeError(f"bsp_probe_read failed: {rc}")


def probe_achievable(nbytes, steps):
    """What a plain streaming read reaches on this GPU: per launch for
    `nbytes` (each of `steps` launches in a graph reads its own slice, with
    >= 1 GiB of other slices read between a slice's warm-up and timed use,
    as the SpMM steps are timed), best over launch shapes and load forms;
    and one launch over 1 GiB."""
    import torch
    L = _probe_lib()
    dev = torch.device("cuda:0")
    nb = (nbytes + 15) // 16 * 16
    slot = (nb + 4095) // 4096 * 4096
    nflush = -(-FLUSH_BYTES // slot)
    nslots = steps + nflush
    buf = torch.empty(nslots * slot, dtype=torch.uint8, device=dev)
    buf.fill_(0x5A)
    big = max(g * (b // 64) for g, b in PROBE_SHAPES)
    sink = torch.zeros(big, dtype=torch.int32, device=dev)
    base = buf.data_ptr()
    best = None
    for mode in PROBE_MODES:
        for grid, block in PROBE_SHAPES:
            g = torch.cuda.CUDAGraph()
            cs = torch.cuda.Stream()
            cs.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(cs):
                with torch.cuda.graph(g, stream=cs):
                    for i in range(steps):
                        _probe_launch(L, base + i * slot, nb, sink, mode, grid, block)
            torch.cuda.synchronize()
            g.replay()
            for i in range(steps, nslots):
                _probe_launch(L, base + i * slot, nb, sink, mode, grid, block)
            torch.cuda.synchronize()
            stream = torch.cuda.current_stream()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / steps
            if best is None or us < best[0]:
                best = (us, mode, grid, block)
            del g
    # one launch over 1 GiB, alternating between two halves of a 2 GiB buffer
    del buf
    torch.cuda.empty_cache()
    gib = 1 << 30
    buf2 = torch.empty(2 * gib, dtype=torch.uint8, device=dev)
    buf2.fill_(0x33)
    us_big = []
    for rep in range(6):
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        _probe_launch(L, buf2.data_ptr() + (rep % 2) * gib, gib, sink, best[1], best[2], best[3])
        e1.record(stream)
        torch.cuda.synchronize()
        if rep >= 2:
            us_big.append(e0.elapsed_time(e1) * 1e3)
    del buf2
    torch.cuda.empty_cache()
    us, mode, grid, block = best
    t_big = statistics.median(us_big)
    return {"unit": "GB/s", "bytes_per_launch": nb, "one_launch": round(nb / (us * 1e-6) / 1e9, 2),
            "one_launch_us": round(us, 3), "large_read": round(gib / (t_big * 1e-6) / 1e9, 2),
            "large_read_bytes": gib,
            "probe": f"bsp_probe_read mode {mode} ({PROBE_MODES[mode]}), grid {grid} x {block} threads, "
                     f"best of {len(PROBE_MODES) * len(PROBE_SHAPES)} forms; {steps} launches in a graph"}


# ---------------------------------------------------------------- profiles

def _csv_rows(d, suffix):
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _pick(table, fragment):
    hits = [k for k in table if fragment in k]
    if not hits:
        raise SystemExit(f"no kernel matching {fragment!r} in {list(table)[:8]}")
    return max(hits, key=lambda k: table[k][1])


def summarize_trace(d, out, header):
    rows = _csv_rows(d, "kernel_stats.csv")
    # per-dispatch durations (end - start) for the percentiles
    durs = {}
    for r in _csv_rows(d, "kernel_trace.csv"):
        durs.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = [f"# {h}" for h in header]
    lines.append(f"{'kernel':72s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'p10_us':>9s} {'p50_us':>9s} "
                 f"{'p90_us':>9s} {'max_us':>9s} {'share%':>7s}")
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        v = sorted(durs.get(r["Name"], [float("nan")]))
        pct = lambda q: v[min(len(v) - 1, int(q * (len(v) - 1) + 0.5))]
        lines.append(f"{r['Name'][:72]:72s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.3f} "
                     f"{float(r['MinNs']) / 1e3:9.3f} {pct(0.1):9.3f} {pct(0.5):9.3f} {pct(0.9):9.3f} "
                     f"{float(r['MaxNs']) / 1e3:9.3f} {float(r['Percentage']):7.2f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counters_by_kernel(d, names):
    """{kernel: {counter: mean per dispatch}} over a rocprofv3 --pmc csv."""
    per = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        c = r.get("Counter_Name")
        if c not in names:
            continue
        key = (r.get("Kernel_Name", "?"), r.get("Dispatch_Id", r.get("Correlation_Id")), c)
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (k, _, c), v in per.items():
        out.setdefault(k, {}).setdefault(c, []).append(v)
    return {k: {c: (statistics.mean(v), len(v)) for c, v in cs.items()} for k, cs in out.items()}


def traffic_estimators(rd, wr):
    """HBM bytes of one dispatch from the TCC counters, two ways:
    'by_size' -- read requests by size (32/64/128 B) and write requests by
    size (32/64 B) leaving the L2 for memory; 'dram_32b' -- the counts of
    32-byte DRAM units (a 64-byte request counts 2, a 128-byte one 4)."""
    g = lambda t, c: t.get(c, (0.0, 0))[0]
    by_size_r = 32 * g(rd, "TCC_EA0_RDREQ_32B_sum") + 64 * g(rd, "TCC_EA0_RDREQ_64B_sum") \
        + 128 * g(rd, "TCC_EA0_RDREQ_128B_sum")
    by_size_w = 32 * (g(wr, "TCC_EA0_WRREQ_sum") - g(wr, "TCC_EA0_WRREQ_64B_sum")) + 64 * g(wr, "TCC_EA0_WRREQ_64B_sum")
    return {"by_size": (by_size_r, by_size_w),
            "dram_32b": (32 * g(rd, "TCC_EA0_RDREQ_DRAM_32B_sum"), 32 * g(wr, "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum"))}


def traffic_lines(reads, writes, fragment):
    """Counter lines, the calibration check and the traffic of one launch of
    the kernel matching `fragment`, with the estimator that reproduces the
    known bytes of both calibration kernels of the same run (the read probe:
    COPY_BYTES read; the copy: COPY_BYTES read and written) within 5 %.
    Returns (kernel, lines, bytes or None)."""
    R = _counters_by_kernel(reads, set(READ_COUNTERS))
    W = _counters_by_kernel(writes, set(WRITE_COUNTERS))
    kr, kw = _pick({k: (0, v[READ_COUNTERS[0]][1]) for k, v in R.items()}, fragment), \
        _pick({k: (0, v[WRITE_COUNTERS[0]][1]) for k, v in W.items()}, fragment)
    pr = _pick({k: (0, 1) for k in R}, "k_probe_read")
    cr = _pick({k: (0, 1) for k in R}, "bitwise_not")
    pw = _pick({k: (0, 1) for k in W}, "k_probe_read")
    cw = _pick({k: (0, 1) for k in W}, "bitwise_not")
    lines = [f"kernel: {kr}", f"dispatches: reads {R[kr][READ_COUNTERS[0]][1]}, writes {W[kw][WRITE_COUNTERS[0]][1]}"]
    for c in READ_COUNTERS:
        lines.append(f"{c}: {R[kr].get(c, (0.0, 0))[0]:.0f}")
    for c in WRITE_COUNTERS:
        lines.append(f"{c}: {W[kw].get(c, (0.0, 0))[0]:.0f}")
    chosen = None
    for name in ("dram_32b", "by_size"):
        p_r, p_w = traffic_estimators(R[pr], W[pw])[name]
        c_r, c_w = traffic_estimators(R[cr], W[cw])[name]
        ratios = (p_r / COPY_BYTES, c_r / COPY_BYTES, c_w / COPY_BYTES)
        ok = all(abs(x - 1.0) <= 0.05 for x in ratios)
        lines.append(f"estimator {name}: read probe reads {p_r:.0f} of {COPY_BYTES} B ({ratios[0]:.4f}); copy reads "
                     f"{c_r:.0f} ({ratios[1]:.4f}) and writes {c_w:.0f} ({ratios[2]:.4f}) of {COPY_BYTES} B: "
                     f"{'within' if ok else 'outside'} 5 %")
        if ok and chosen is None:
            chosen = name
    total = None
    if chosen is not None:
        k_r, k_w = traffic_estimators(R[kr], W[kw])[chosen]
        total = k_r + k_w
        lines += [f"estimator: {chosen}", f"read_bytes_per_launch: {k_r:.0f}", f"write_bytes_per_launch: {k_w:.0f}",
                  f"traffic_bytes_per_launch: {total:.0f}"]
    else:
        lines += ["estimator: none (no estimator reproduces both calibration kernels within 5 %)"]
    return kr, lines, total


def summarize_traffic(out, reads, writes, fragment, header):
    """Traffic summary file of one launch (see traffic_lines), tied to the
    current kernel sources by their digest."""
    _, body, _ = traffic_lines(reads, writes, fragment)
    lines = [f"# {h}" for h in header] + body + [f"source_digest: {source_digest()}"]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _trace_stats(d, fragment):
    """(kernel, calls, mean us, p50 us) of the kernel matching `fragment` in
    a rocprofv3 kernel trace."""
    durs = {}
    for r in _csv_rows(d, "kernel_trace.csv"):
        durs.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    name = _pick({k: (0, len(v)) for k, v in durs.items()}, fragment)
    v = sorted(durs[name])
    return name, len(v), statistics.mean(v), v[len(v) // 2]


def _counter_means(d, fragment):
    per, name = {}, None
    for r in _csv_rows(d, "counter_collection.csv"):
        if fragment in r["Kernel_Name"]:
            name = r["Kernel_Name"]
            per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return name, {k: sum(v) / len(v) for k, v in per.items()}


def summarize_selection(out, sides, header):
    """A/B of the kernels on either side of a selection threshold, on one
    shape: per side the launch duration (kernel trace), the SQ counters of
    one --pmc pass and the calibrated HBM traffic of one launch. Each side is
    LABEL:TRACE_DIR:PMC_DIR:READS_DIR:WRITES_DIR:FRAGMENT."""
    lines = [f"# {h}" for h in header]
    for side in sides:
        label, tdir, pdir, rdir, wdir, frag = side.split(":")
        kname, calls, avg, p50 = _trace_stats(tdir, frag)
        _, cnt = _counter_means(pdir, frag)
        _, _, traffic = traffic_lines(rdir, wdir, frag)
        lines.append(f"[{label}] kernel: {kname}")
        lines.append(f"[{label}] duration_us: mean {avg:.3f}, p50 {p50:.3f} over {calls} dispatches")
        for c in sorted(cnt):
            lines.append(f"[{label}] {c}: {cnt[c]:.0f}")
        lines.append(f"[{label}] traffic_bytes_per_launch: {'%.0f' % traffic if traffic is not None else 'none'}")
    lines.append(f"source_digest: {source_digest()}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_counters(d, out, fragment, header):
    """Mean per dispatch of every counter in a rocprofv3 --pmc csv, for the
    kernel whose name holds `fragment`."""
    per = {}
    name = None
    for r in _csv_rows(d, "counter_collection.csv"):
        if fragment in r["Kernel_Name"]:
            name = r["Kernel_Name"]
            per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if name is None:
        raise SystemExit(f"no dispatch of a kernel matching {fragment!r} under {d}")
    lines = [f"# {h}" for h in header] + [f"kernel: {name}"]
    lines += [f"{k}: {sum(v) / len(v):.0f}  (mean of {len(v)} dispatches)" for k, v in sorted(per.items())]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def read_traffic(path):
    """Bytes per launch from a traffic summary, or None when the summary is
    missing, has no calibrated estimator, or was taken from other kernel
    sources."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_digest") != source_digest() or "traffic_bytes_per_launch" not in kv:
        return None
    return float(kv["traffic_bytes_per_launch"])


def calibration_kernels():
    """The two kernels of known traffic the counter passes are checked on: the
    read probe over COPY_BYTES (reads them) and an int32 bitwise_not over
    COPY_BYTES (reads and writes them), five launches each, on buffers far
    larger than the Infinity Cache."""
    import numpy as np
    import torch
    n = COPY_BYTES // 4
    src = torch.arange(n, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    other = torch.empty(4 * COPY_BYTES // 4, dtype=torch.int32, device="cuda:0")
    L = _probe_lib()
    sink = torch.zeros(L.bsp_probe_sink_words(1024, 256), dtype=torch.int32, device="cuda:0")
    for _ in range(5):
        other.fill_(1)          # evicts src from the Infinity Cache between launches
        _probe_launch(L, src.data_ptr(), COPY_BYTES, sink, 0, 1024, 256)
    for _ in range(5):
        other.fill_(2)
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    # checked on the host: a device-side check would launch a small kernel
    # of the same name, and the summary averages over that name's dispatches
    ok = bool(np.array_equal(dst[:1024].cpu().numpy(), ~src[:1024].cpu().numpy()))
    print(json.dumps({"calibration_bytes": COPY_BYTES, "dispatches": 5, "ok": ok}), flush=True)


# ---------------------------------------------------------------- main

def prepare(args, workload, index, n):
    """The problem, its encoding and device copies, and a step function."""
    import torch
    import bit_unstructured_sparse_amd as bsp
    import workloads

    dev = torch.device("cuda:0")
    bsp.load_library()
    if workload.startswith("custom:"):
        # custom:DTYPE:M:K:N:DENSITY[:SEED[:rows]] -- a seeded random problem
        # of any shape (selection A/B runs on shapes outside the named
        # workloads); "rows": every row keeps the same count
        parts = workload.split(":")
        dty, Mc, Kc, Nc, dens = parts[1], int(parts[2]), int(parts[3]), int(parts[4]), float(parts[5])
        seed = int(parts[6]) if len(parts) > 6 else 12345
        rows = len(parts) > 7 and parts[7] == "rows"
        tag = "_rows" if rows else ""
        if dty == "int4":
            problems = [workloads.random_int4_problem(seed, Mc, Kc, Nc, keep=dens, rows=rows,
                                                      name=f"custom_int4_{Mc}x{Kc}_d{dens:g}{tag}")]
        else:
            problems = [workloads.random_fp16_problem(seed, Mc, Kc, Nc, sparsity=1.0 - dens, rows=rows,
                                                      name=f"custom_fp16_{Mc}x{Kc}_d{dens:g}{tag}")]
    else:
        problems = workloads.make(workload)
    problem = problems[index]
    if n:
        widest = max(problems, key=lambda p: p.N) if problem.dtype == "fp16" else problem
        X = problem.meta.get("X_full", widest.X)
        problem = workloads.Problem(problem.name.rsplit("_n", 1)[0] if problem.dtype == "fp16" else problem.name,
                                    problem.dtype, problem.W, X[:n], dict(problem.meta, N=n))
    fp16 = problem.dtype == "fp16"
    N, M, K = problem.N, problem.M, problem.K
    if getattr(args, "format", "bt64") == "union":
        return _prepare_union(args, bsp, problem, dev)
    if getattr(args, "format", "bt64") == "cbc":
        return _prepare_cbc(args, bsp, problem, dev)
    if getattr(args, "parts", 0) or getattr(args, "epilogue", "int32") == "dq":
        return _prepare_parts(args, bsp, problem, dev)
    if getattr(args, "wbits", 4) == 2:
        return _prepare_w2(args, bsp, problem, dev)
    enc = bsp.encode(problem.W)
    algo = {"auto": bsp.ALGO_AUTO, "rowwave": bsp.ALGO_ROWWAVE, "mfma": bsp.ALGO_MFMA, "splitk": bsp.ALGO_SPLITK}[args.algo]
    dt = bsp.FP16 if fp16 else bsp.INT4
    chosen = algo
    dm0 = enc.to_device(dev)
    if fp16:
        Xd = torch.from_numpy(problem.X.copy()).to(dev)
        y_dtype = torch.float16
    else:
        Xd = torch.from_numpy(bsp.pack_int4(problem.X)).to(dev)
        y_dtype = torch.int32
    esize = 2 if fp16 else 4
    ws = (dm0.bitmaps.numel() * 8 + dm0.offsets.numel() * 4 + dm0.payload.numel() * dm0.payload.element_size()
          + Xd.numel() * Xd.element_size() + esize * M * N)
    # copies 0..steps-1 are the timed steps'; the rest (>= FLUSH_BYTES) are
    # run between the graph's warm-up replay and its timed replay
    R = args.steps + max(1, -(-FLUSH_BYTES // ws))
    copies = [(dm0, Xd, torch.empty((N, M), dtype=y_dtype, device=dev))]
    for _ in range(R - 1):
        dm = bsp.DeviceMatrix(enc.dtype, M, K, enc.nnz, dm0.bitmaps.clone(), dm0.offsets.clone(), dm0.payload.clone())
        copies.append((dm, Xd.clone(), torch.empty((N, M), dtype=y_dtype, device=dev)))
    torch.cuda.synchronize()

    # the split plans' workspace (calls on one stream share it in order)
    ws = bsp.new_workspace(dt, M, K, N, enc.nnz, device=dev) if args.workspace else None

    def step(i):
        dm, x, y = copies[i % R]
        if fp16:
            bsp.spmm_f16(dm, x, Y=y, algo=chosen, workspace=ws)
        else:
            bsp.spmm_w4a4(dm, x, N, Y=y, algo=chosen, workspace=ws)

    kernel = kernel_symbol(bsp, chosen, dt, M, K, N, enc.nnz, workspace=ws is not None)
    plan = bsp.describe(dt, M, K, N, enc.nnz, workspace=ws is not None, algo=chosen)
    return dict(problem=problem, fp16=fp16, enc=enc, dm0=dm0, copies=copies, R=R, step=step, chosen=chosen,
                name=algo_label(kernel), kernel=kernel, dt=dt, plan=plan)


def union_step_bytes(ue, N):
    """Algorithmic bytes of one union-mask SpMM call: every tile's four mask
    words, rowpos word and offset (plus the end offset), the payload, X and Y."""
    return ue.stream_bytes() + N * ((ue.K + 1) // 2) + 4 * ue.M * N


def _prepare_union(args, bsp, problem, dev):
    """prepare() for the union-mask format (int4 only): 2 x 2 areas, rows of
    every tile reordered unless --no-reorder."""
    import numpy as np
    import torch
    if problem.dtype != "int4":
        raise SystemExit("the union-mask format is int4 only")
    N, M, K = problem.N, problem.M, problem.K
    t0 = time.perf_counter()
    ue = bsp.encode_union_tiles(problem.W, 2, 2, reorder=not args.no_reorder)
    enc_s = time.perf_counter() - t0
    du0 = ue.to_device(dev)
    Xd = torch.from_numpy(bsp.pack_int4(problem.X)).to(dev)
    ws = ue.stream_bytes() + Xd.numel() + 4 * M * N
    R = args.steps + max(1, -(-FLUSH_BYTES // ws))
    copies = [(du0, Xd, torch.empty((N, M), dtype=torch.int32, device=dev))]
    for _ in range(R - 1):
        du = bsp.UnionDevice(M, K, 2, 2, ue.nvals, du0.ubitmaps.clone(), du0.offsets.clone(), du0.rowpos.clone(),
                             du0.payload.clone())
        copies.append((du, Xd.clone(), torch.empty((N, M), dtype=torch.int32, device=dev)))
    torch.cuda.synchronize()

    def step(i):
        du, x, y = copies[i % R]
        bsp.spmm_union_w4a4(du, x, N, Y=y)

    nnz = int(np.count_nonzero(problem.W))

    class _Enc:   # what measure() reads of an encoding
        pass
    enc = _Enc()
    enc.nnz = nnz
    return dict(problem=problem, fp16=False, enc=enc, dm0=None, copies=copies, R=R, step=step, chosen=None,
                name="union", kernel="k_ie_w4a4", dt=bsp.INT4, plan="union 2x2", nbytes=union_step_bytes(ue, N),
                union={"nvals": ue.nvals, "reorder": not args.no_reorder, "encode_seconds": round(enc_s, 3),
                       "stream_bytes": ue.stream_bytes(), "payload_bytes": int(ue.payload.nbytes),
                       "value_fill": round(ue.nvals / max(1, 4 * nnz), 4)})


def _prepare_cbc(args, bsp, problem, dev):
    """prepare() for the Tiled-CBC product with dynamic activation pruning
    (fp16): the threshold is the --dyn-sparsity quantile of |x|, so that
    fraction of the activations (and, at N = 1, of W's columns) is pruned."""
    import numpy as np
    import torch
    if problem.dtype != "fp16":
        raise SystemExit("the Tiled-CBC path is fp16")
    N, M, K = problem.N, problem.M, problem.K
    q = args.dyn_sparsity
    tau = float(np.quantile(np.abs(problem.X.astype(np.float32)), q)) if q > 0 else 0.0
    enc = bsp.encode_cbc_f16(problem.W)
    d0 = enc.to_device(dev)
    Xd = torch.from_numpy(problem.X.copy()).to(dev)
    ws = bsp.new_cbc_workspace(M, K, N, device=dev)
    per_copy = enc.storage_bytes() + Xd.numel() * 2 + 2 * M * N
    R = args.steps + max(1, -(-FLUSH_BYTES // per_copy))
    copies = [(d0, Xd, torch.empty((N, M), dtype=torch.float16, device=dev))]
    for _ in range(R - 1):
        d = bsp.CbcDevice(M, K, enc.nnz, d0.tile_offsets.clone(), d0.colinfo.clone(), d0.bitmaps.clone(),
                          d0.values.clone())
        copies.append((d, Xd.clone(), torch.empty((N, M), dtype=torch.float16, device=dev)))
    torch.cuda.synchronize()

    def step(i):
        d, x, y = copies[i % R]
        bsp.spmspv_cbc_f16(d, x, tau, Y=y, workspace=ws)

    # algorithmic bytes: for every column with an activation kept, its bitmap
    # words, ColInfo and values; every GTile offset; X and Y
    kept = np.abs(problem.X.astype(np.float32)) > np.float32(tau)       # the kernel's rule: |x| > tau
    active = kept.any(axis=0)
    kept_nnz = int(np.count_nonzero(problem.W[:, active]))
    bands = (M + 255) // 256
    nbytes = (4 * (enc.tile_offsets.size) + bands * int(active.sum()) * (4 + 32) + 2 * kept_nnz +
              2 * N * K + 2 * N * M)

    class _Enc:
        pass
    e = _Enc()
    e.nnz = enc.nnz
    return dict(problem=problem, fp16=True, enc=e, dm0=None, copies=copies, R=R, step=step, chosen=None,
                name="cbc", kernel="k_cbc_f16", dt=bsp.FP16, plan="tiled-cbc", nbytes=nbytes,
                cbc={"threshold": tau, "dyn_sparsity": q, "active_columns": int(active.sum()),
                     "kept_nnz": kept_nnz, "storage_bytes": enc.storage_bytes()},
                ref_mask=kept)


def _prepare_w2(args, bsp, problem, dev):
    """prepare() for W2A4: the workload's nonzero pattern with fresh 2-bit
    values in {-2, -1, 1} (workloads.int2_like), its int4 X."""
    import numpy as np
    import torch
    import workloads
    if problem.dtype != "int4":
        raise SystemExit("W2A4 runs on the int4 workloads' shapes")
    N, M, K = problem.N, problem.M, problem.K
    W2 = workloads.int2_like(problem.W, seed=0)
    problem = workloads.Problem(problem.name + "_w2", "int2", W2, problem.X, dict(problem.meta))
    enc = bsp.encode(W2, dtype=bsp.INT2)
    dm0 = enc.to_device(dev)
    Xd = torch.from_numpy(bsp.pack_int4(problem.X)).to(dev)
    algo = {"auto": bsp.ALGO_AUTO, "rowwave": bsp.ALGO_ROWWAVE, "mfma": bsp.ALGO_MFMA}[args.algo]
    per_copy = dm0.stream_bytes() + Xd.numel() + 4 * M * N
    R = args.steps + max(1, -(-FLUSH_BYTES // per_copy))
    copies = [(dm0, Xd, torch.empty((N, M), dtype=torch.int32, device=dev))]
    for _ in range(R - 1):
        dm = bsp.DeviceMatrix(enc.dtype, M, K, enc.nnz, dm0.bitmaps.clone(), dm0.offsets.clone(), dm0.payload.clone())
        copies.append((dm, Xd.clone(), torch.empty((N, M), dtype=torch.int32, device=dev)))
    torch.cuda.synchronize()

    def step(i):
        dm, x, y = copies[i % R]
        bsp.spmm_w2a4(dm, x, N, Y=y, algo=algo)

    kernel = kernel_symbol(bsp, algo, bsp.INT2, M, K, N, enc.nnz)
    nbytes = dm0.stream_bytes(with_offsets=False) + 4 * offsets_read(kernel, M, dm0.T) + N * ((K + 1) // 2) + 4 * M * N
    return dict(problem=problem, fp16=False, enc=enc, dm0=dm0, copies=copies, R=R, step=step, chosen=algo,
                name="w2a4", kernel=kernel, dt=bsp.INT2, plan="w2a4", nbytes=nbytes)


def _prepare_parts(args, bsp, problem, dev):
    """prepare() for the grouped launch and the dequant epilogue (int4): W's
    rows cut into --parts matrices sharing X, run as one grouped launch (or,
    with --separate, one call each); --epilogue dq writes fp16 through the
    dequant epilogue with seeded per-channel and per-token scales."""
    import numpy as np
    import torch
    if problem.dtype != "int4":
        raise SystemExit("the grouped launch and the dequant epilogue are int4 only")
    N, M, K = problem.N, problem.M, problem.K
    P = max(1, args.parts)
    dq = args.epilogue == "dq"
    separate = args.separate or not args.parts   # the epilogue alone: one plain call
    cuts = [M * j // P for j in range(P + 1)]
    encs = [bsp.encode(np.ascontiguousarray(problem.W[cuts[j]:cuts[j + 1]])) for j in range(P)]
    rng = np.random.default_rng(0)
    sx = torch.from_numpy(np.exp(rng.uniform(np.log(1e-2), np.log(2.0), N)).astype(np.float32)).to(dev)
    sws = [torch.from_numpy(np.exp(rng.uniform(np.log(1e-4), np.log(5e-2), e.M)).astype(np.float32)).to(dev)
           for e in encs]
    Xd = torch.from_numpy(bsp.pack_int4(problem.X)).to(dev)
    dms0 = [e.to_device(dev) for e in encs]
    esize = 2 if dq else 4
    per_copy = sum(d.stream_bytes() for d in dms0) + Xd.numel() + esize * M * N
    R = args.steps + max(1, -(-FLUSH_BYTES // per_copy))
    ydt = torch.float16 if dq else torch.int32

    def fresh(dms, x):
        return (dms, x, [torch.empty((N, e.M), dtype=ydt, device=dev) for e in encs])
    copies = [fresh(dms0, Xd)]
    for _ in range(R - 1):
        copies.append(fresh([bsp.DeviceMatrix(e.dtype, e.M, K, e.nnz, d.bitmaps.clone(), d.offsets.clone(),
                                              d.payload.clone()) for e, d in zip(encs, dms0)], Xd.clone()))
    torch.cuda.synchronize()

    def step(i):
        dms, x, ys = copies[i % R]
        if separate:
            for j in range(P):
                if dq:
                    bsp.spmm_bitmap_w4a4_dq(dms[j], x, N, sws[j], sx, Yh=ys[j])
                else:
                    bsp.spmm_w4a4(dms[j], x, N, Y=ys[j])
        else:
            items = []
            for j in range(P):
                it = dict(W=dms[j], X=x, N=N)
                if dq:
                    it.update(scale_w=sws[j], scale_x=sx, Yh=ys[j])
                else:
                    it["Y"] = ys[j]
                items.append(it)
            bsp.spmm_bitmap_w4a4_grouped(items)

    nnz = sum(e.nnz for e in encs)
    # algorithmic bytes: every part's words, block offsets and payload, X once
    # per part (each reads it), Y (fp16 with the epilogue, plus the scales)
    nbytes = 0
    for e, d in zip(encs, dms0):
        nbytes += d.stream_bytes(with_offsets=False) + 4 * ((e.M + 15) // 16 + 1) + N * ((K + 1) // 2)
        nbytes += esize * e.M * N + (4 * e.M + 4 * N if dq else 0)

    class _Enc:
        pass
    enc = _Enc()
    enc.nnz = nnz
    separate = args.separate or not args.parts
    kernel = kernel_symbol(bsp, bsp.ALGO_AUTO, bsp.INT4, encs[0].M, K, N, encs[0].nnz) if separate else "k_bt64s_group"

    def gather(i):
        # Y of copy i as one [N][M] array (int32), or the fp16 values
        return torch.cat([ys.float() if dq else ys for ys in copies[i][2]], dim=1)
    return dict(problem=problem, fp16=False, enc=enc, dm0=None, copies=copies, R=R, step=step, chosen=None,
                name="separate" if separate else "grouped", kernel=kernel, dt=bsp.INT4,
                plan=f"parts={P} {'separate calls' if separate else 'one grouped launch'}"
                     f"{' dequant epilogue' if dq else ''}",
                nbytes=nbytes, gather=gather, dq=(sws, sx) if dq else None,
                parts={"parts": P, "separate": separate, "epilogue": args.epilogue,
                       "launches_per_step": P if separate else 1})


def measure(args, workload, index, n, with_probe=True):
    """Time one workload (n > 0 slices its widest X to N = n); returns the
    bench record without the CPU baseline."""
    import numpy as np
    import torch

    ctx = prepare(args, workload, index, n)
    problem, fp16, enc, dm0, copies, R, step = (ctx[k] for k in ("problem", "fp16", "enc", "dm0", "copies", "R",
                                                                   "step"))
    N, M, K = problem.N, problem.M, problem.K
    for i in range(args.warmup):
        step(args.steps + i % (R - args.steps))
    torch.cuda.synchronize()
    # spot check of the timed configuration against an independent dense
    # product on a sample of rows (exact integers; fp16 within the 1e-2 bound)
    rows = np.random.default_rng(0).choice(M, size=min(M, 256), replace=False)

    def spot_ok(i):
        if "gather" in ctx:
            got = ctx["gather"](i).cpu().numpy()[:, rows]
            ref = (problem.W[rows].astype(np.int64) @ problem.X.astype(np.int64).T).T
            if ctx.get("dq") is not None:
                sws, sx = ctx["dq"]
                sw = torch.cat(sws).cpu().numpy()[rows]
                want = ((ref.astype(np.float32) * sw[None, :]) * sx.cpu().numpy()[:, None]).astype(np.float16)
                return bool(np.array_equal(got.astype(np.float16).view(np.uint16), want.view(np.uint16)))
            return bool(np.array_equal(got, ref))
        got = copies[i][2].cpu().numpy()[:, rows]
        if fp16:
            Xr = problem.X
            if "ref_mask" in ctx:
                Xr = np.where(ctx["ref_mask"], problem.X, np.float16(0))
            ref = (problem.W[rows].astype(np.float64) @ Xr.astype(np.float64).T).T
            floor = 0.01 * np.sqrt(np.mean(ref ** 2))
            err = np.abs(got.astype(np.float64) - ref) / np.maximum(np.abs(ref), floor)
            return bool(np.max(err) <= 1e-2)
        ref = (problem.W[rows].astype(np.int64) @ problem.X.astype(np.int64).T).T
        return bool(np.array_equal(got, ref))

    parity = spot_ok(args.steps)

    # timed region: exactly K steps, captured once in a HIP graph (one node
    # per SpMM call, step i on copy i) and replayed
    capture_stream = torch.cuda.Stream()
    capture_stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(capture_stream):
        with torch.cuda.graph(graph, stream=capture_stream):
            for i in range(args.steps):
                step(i)
    torch.cuda.synchronize()
    graph.replay()                  # first replay is warm-up
    for i in range(args.steps, R):  # >= 1 GiB of other copies: the timed steps' copies leave the caches
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()     # graph.replay() launches on this stream
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    kern_ms = ev0.elapsed_time(ev1) / args.steps     # average launch duration (HIP events)
    parity = parity and spot_ok(0) and spot_ok(args.steps - 1)
    del graph

    kernel = ctx["kernel"]
    nbytes = ctx["nbytes"] if "nbytes" in ctx else step_bytes(dm0, N, kernel, fp16, ctx["plan"])
    union_info = ctx.get("union")
    ctx_parts = ctx.get("parts")
    cbc_info = ctx.get("cbc")
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    dense_ops = 2.0 * M * K * N
    useful_ops = 2.0 * enc.nnz * N
    wl = f"{problem.name}_n{N}" if not problem.name.endswith(f"_n{N}") else problem.name
    traffic = read_traffic(os.path.join(ROOT, "profiles", f"traffic_{ctx['name']}_{wl}.txt"))
    del copies, ctx
    torch.cuda.empty_cache()
    achievable = probe_achievable(nbytes, args.steps) if with_probe else None

    density = enc.nnz / (M * K)
    roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else int(traffic),
            "kernel": kernel, "bytes_per_launch": nbytes}
    if achievable is not None:
        roof["achievable"] = achievable
        roof["frac_of_achievable_one_launch"] = round(achieved / achievable["one_launch"], 4)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 x f16 -> f32 acc -> f16" if fp16 else
                 ("int2 x int4 -> int32" if problem.dtype == "int2" else "int4 x int4 -> int32"),
        "data": "synthetic (seeded iid unstructured mask / magnitude pruning; the pages' model weights "
                "are not available)",
        "config": {"workload": f"{wl}: W {M}x{K} {'fp16' if fp16 else problem.dtype}, density {density:.3f}, N={N}",
                   "M": M, "K": K, "N": N, "nnz": enc.nnz, "kernel": algo_label(kernel),
                   "rotated_copies": R, "bytes_per_step": nbytes},
        "frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        "tops_dense_equiv": round(dense_ops / (ms_per_step * 1e-3) / 1e12, 3),
        "tops_useful": round(useful_ops / (ms_per_step * 1e-3) / 1e12, 3),
        "kernel_us_avg": round(kern_ms * 1e3, 3),
        "timing": "K steps captured in one HIP graph (step i on its own copy i) and replayed back to back after "
                  ">= 1 GiB of other copies; value uses host wall time around the replay, roofline uses HIP "
                  "events on the replay stream",
        "roofline": roof,
        "parity_sample_ok": parity,
    }
    if cbc_info is not None:
        out["config"]["format"] = "Tiled-CBC (256 x 64 GTiles), dynamic activation pruning"
        out["cbc"] = cbc_info
    if ctx_parts is not None:
        out["config"]["grouping"] = ctx_parts
    if union_info is not None:
        out["config"]["format"] = "union-mask 2x2 areas of 16x64 tiles" + (", rows reordered" if union_info["reorder"]
                                                                          else "")
        out["union"] = union_info
    args._problem = problem
    return out


def algo_label(kernel):
    if kernel.startswith("k_ie"):
        return "union"
    return "rowwave" if kernel.startswith("k_rowwave") else "splitk" if kernel.startswith("k_bsk") else "mfma"


def counter_run(args):
    """One process for the --pmc passes: the two calibration kernels, then
    the workload's SpMM steps (eager, each on its own copy)."""
    import torch
    calibration_kernels()
    ctx = prepare(args, args.workload, args.index, args.n)
    for i in range(args.steps):
        ctx["step"](i)
    torch.cuda.synchronize()
    print(json.dumps({"counter_run": ctx["problem"].name, "steps": args.steps, "kernel": ctx["kernel"]}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qkv",
                    help="tiny | qkv | ffn | lowsparse | fp16 | custom:DTYPE:M:K:N:DENSITY[:SEED[:rows]]")
    ap.add_argument("--index", type=int, default=0, help="matrix index inside the workload (ffn: 0 up, 1 down)")
    ap.add_argument("--n", type=int, default=0, help="override N (slices the workload's widest X)")
    ap.add_argument("--algo", default="auto", choices=["auto", "rowwave", "mfma", "splitk"])
    ap.add_argument("--workspace", action="store_true", help="call the *_ws entry point with a workspace")
    ap.add_argument("--format", default="bt64", choices=["bt64", "union", "cbc"],
                    help="weight format: BT64 (1x64 tiles), the union mask (2x2 areas of 16x64 tiles) or Tiled-CBC "
                         "(fp16, dynamic activation pruning)")
    ap.add_argument("--no-reorder", action="store_true", help="union format without row reordering")
    ap.add_argument("--dyn-sparsity", type=float, default=0.5,
                    help="--format cbc: fraction of activations pruned (the threshold is that quantile of |x|)")
    ap.add_argument("--wbits", type=int, default=4, choices=[4, 2], help="2: W2A4 (2-bit weights) on the shape")
    ap.add_argument("--parts", type=int, default=0, help="cut W's rows into this many matrices: one grouped launch")
    ap.add_argument("--separate", action="store_true", help="with --parts: one call per part instead")
    ap.add_argument("--epilogue", default="int32", choices=["int32", "dq"],
                    help="dq: fp16 output through the fused dequant epilogue")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="leave out the read probe (roofline.achievable)")
    ap.add_argument("--sweep", action="store_true", help="one line per (workload, N) of the N sweep")
    ap.add_argument("--peak-read", action="store_true", help="the read probe alone at this workload's byte count")
    ap.add_argument("--counter-run", action="store_true", help="calibration kernels + SpMM steps, for --pmc passes")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("DIR", "OUT"))
    ap.add_argument("--summarize-traffic", metavar="OUT")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("DIR", "OUT"))
    ap.add_argument("--summarize-selection", metavar="OUT")
    ap.add_argument("--side", action="append", default=[],
                    help="--summarize-selection: LABEL:TRACE_DIR:PMC_DIR:READS_DIR:WRITES_DIR:KERNEL_FRAGMENT")
    ap.add_argument("--reads"), ap.add_argument("--writes")
    ap.add_argument("--kernel", default="w4a4", help="kernel name fragment for the summaries")
    ap.add_argument("--note", action="append", default=[], help="header line for a summary")
    args = ap.parse_args()

    if args.summarize_trace:
        return summarize_trace(args.summarize_trace[0], args.summarize_trace[1], args.note)
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters[0], args.summarize_counters[1], args.kernel, args.note)
    if args.summarize_traffic:
        return summarize_traffic(args.summarize_traffic, args.reads, args.writes, args.kernel, args.note)
    if args.summarize_selection:
        return summarize_selection(args.summarize_selection, args.side, args.note)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the path has no "
              f"multi-GPU code; how it would shard is described with the design.", file=sys.stderr)
        sys.exit(2)
    if args.counter_run:
        return counter_run(args)
    if args.peak_read:
        import torch
        ctx = prepare(args, args.workload, args.index, args.n)
        nbytes = step_bytes(ctx["dm0"], ctx["problem"].N, ctx["kernel"], ctx["fp16"], ctx["plan"])
        del ctx
        torch.cuda.empty_cache()
        print(json.dumps({"peak_read": probe_achievable(nbytes, args.steps)}), flush=True)
        return

    if args.sweep:
        # the N sweep on the qkv weights and the 70 %-dense matrix at N = 16, 32
        for wl, idx, n in SWEEP:
            out = measure(args, wl, idx, n, with_probe=False)
            print(json.dumps({"sweep": out["config"]["workload"].split(":")[0], "N": out["config"]["N"],
                              "kernel": out["roofline"]["kernel"], "kernel_us_avg": out["kernel_us_avg"],
                              "GB/s (events)": out["roofline"]["achieved"], "GB/s (wall)": out["value"],
                              "frac_of_peak": out["roofline"]["frac"], "tops_dense_equiv": out["tops_dense_equiv"],
                              "tops_useful": out["tops_useful"], "parity_sample_ok": out["parity_sample_ok"]}),
                  flush=True)
        return
    out = measure(args, args.workload, args.index, args.n, with_probe=not args.no_probe)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args._problem, out["config"]["bytes_per_step"] / out["config"]["M"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
