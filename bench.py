"""Benchmark of the bitmap-tiled sparse x skinny-dense SpMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload qkv] [--n N] [--algo auto]

A step is one call of the SpMM entry point (``spmm_bitmap_w4a4``, or
``spmm_bitmap_f16`` for ``--workload fp16``: host-side argument checks and
kernel selection, then the kernel that streams the compressed tiles, stages
X, decodes, contracts and stores Y) on one batch of synthetic input already
resident in HBM. Encoding is the offline step of the method and runs once,
before timing. The inputs are rotated through enough identical device copies
(>= 1 GiB in total, four times the 256 MB Infinity Cache) that each step reads
its operands from HBM, not from cache.

The K timed steps are captured once in a HIP graph (one kernel node per SpMM
call) and replayed back to back: these kernels last a few microseconds, less
than a Python-level launch, so eager launching would time the host instead.

Prints ONE JSON line. ``value`` is achieved GB/s over the algorithmic bytes of
a step (bitmaps, the offsets the kernel reads, payload, X, Y) divided by the
host wall time per step around the replay; the ``roofline`` object divides the
same bytes by the average launch duration from HIP events recorded on the
replay stream. ``traffic`` is the HBM byte count of one launch from the
FETCH_SIZE / WRITE_SIZE counter summary in ``profiles/`` when that summary was
taken from the current kernel sources (else null). ``cpu_baseline`` times the
CPU oracle (plain C, one thread) on a bounded sample of the same workload.

Helper modes used to produce the ``profiles/`` summaries:

    python bench.py --sweep                     # N = 1..32 on the qkv weights, N = 16, 32 at 70 % density
    python bench.py --copy-calibration          # a plain copy of known size
    python bench.py --summarize-trace DIR OUT   # rocprofv3 --kernel-trace --stats csv -> text
    python bench.py --summarize-traffic OUT --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR
    python bench.py --summarize-counters DIR OUT --kernel FRAGMENT   # rocprofv3 --pmc csv -> text
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
ROTATE_TARGET = 1 << 30
COPY_BYTES = 256 << 20         # calibration copy: reads and writes this many bytes
METRIC = "achieved HBM GB/s (frac of peak) + dense-equiv TOPS, bitmap SpMM at N=1..32"

# kernel symbol fragment per algorithm, and whether it reads one 4-byte
# offset per tile (else one per 16-row block)
SWEEP = [("qkv", 0, n) for n in (1, 2, 4, 8, 16, 32)] + [("lowsparse", 0, 16), ("lowsparse", 0, 32)]
KERNEL_SYMBOL = {"rowwave": "k_rowwave", "valu": "k_valu", "mfma": "k_bt64"}
READS_TILE_OFFSETS = {"rowwave": True, "valu": False, "mfma": False}


def algo_name(bsp, a):
    return {bsp.ALGO_ROWWAVE: "rowwave", bsp.ALGO_VALU: "valu", bsp.ALGO_MFMA: "mfma"}[a]


def kernel_symbol(bsp, chosen, dt, M, K, N, nnz):
    """Name of the kernel a launch runs: the library's own description of its
    plan when the automatic choice is the one timed, else the algorithm's
    kernel family."""
    if chosen == bsp.select(dt, M, K, N, nnz):
        m = re.search(r"kernel=(\S+)", bsp.describe(dt, M, K, N, nnz))
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


def step_bytes(dm, N, algo, fp16):
    """Algorithmic bytes of one SpMM call: stream (+ offsets read) + X + Y."""
    tile_offsets = READS_TILE_OFFSETS[algo]
    stream = dm.stream_bytes(with_offsets=tile_offsets)
    if not tile_offsets:
        stream += 4 * ((dm.M + 15) // 16 + 1)      # one offset per 16-row block
    if fp16:
        return stream + 2 * N * dm.K + 2 * dm.M * N
    return stream + N * ((dm.K + 1) // 2) + 4 * dm.M * N


def _pack(X):
    # test-side packer for the oracle input (pinned by tests/golden/x_int4_packing.json)
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import pins
    return pins._pack_x_for_test(X)


def cpu_baseline(problem, bytes_per_row, max_seconds=20.0):
    """The oracle as it stands (plain C, one thread): decode the stream to
    dense, then the exact int64 (fp64 for fp16) triple loop, on a bounded
    sample of the same workload: the first rows of W, grown until one run
    takes at least a second (or W is whole), then up to three runs within the
    time budget. Encoding is not timed. GB/s scales the GPU step's bytes by
    the share of rows in the sample."""
    import numpy as np
    import oracle
    M = problem.M
    Xin = problem.X if problem.dtype == "fp16" else _pack(problem.X)

    def run(s):
        t0 = time.perf_counter()
        if problem.dtype == "fp16":
            oracle.spmm_f16(s, Xin)
        else:
            oracle.spmm_w4a4(s, Xin, problem.N)
        return time.perf_counter() - t0

    rows = min(M, 64)
    while True:
        s = oracle.encode(np.ascontiguousarray(problem.W[:rows]))
        t = run(s)
        if t >= 1.0 or rows >= M:
            break
        rows = min(M, rows * max(2, int(1.5 / max(t, 1e-3))))
    times = [t]
    while len(times) < 3 and sum(times) + t < max_seconds:
        times.append(run(s))
    t_run = statistics.median(times)
    gbs = bytes_per_row * rows / t_run / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {rows} of {M} rows of {problem.name} (K={problem.K}, N={problem.N}): "
                      f"decode + exact triple loop, median of {len(times)} runs of {t_run:.2f} s; "
                      f"bytes scaled per row from the GPU step",
            "cpu": platform.processor() or platform.machine()}


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


def _counter_per_kernel(d, counter):
    """Mean counter value per dispatch, per kernel name (rocprofv3 csv)."""
    per = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        key = (r.get("Kernel_Name", "?"), r.get("Dispatch_Id", r.get("Correlation_Id")))
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    by_kernel = {}
    for (k, _), v in per.items():
        by_kernel.setdefault(k, []).append(v)
    return {k: (statistics.mean(v), len(v)) for k, v in by_kernel.items()}


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


def summarize_traffic(out, fetch, write, copy_fetch, copy_write, fragment, header):
    f_k = _counter_per_kernel(fetch, "FETCH_SIZE")
    w_k = _counter_per_kernel(write, "WRITE_SIZE")
    cf = _counter_per_kernel(copy_fetch, "FETCH_SIZE")
    cw = _counter_per_kernel(copy_write, "WRITE_SIZE")
    kf, kw = _pick(f_k, fragment), _pick(w_k, fragment)
    ck = _pick(cf, "bitwise_not")
    # counters read KiB per dispatch; the copy reads and writes COPY_BYTES
    fetch_factor = COPY_BYTES / (cf[ck][0] * 1024.0)
    write_factor = COPY_BYTES / (cw[_pick(cw, "bitwise_not")][0] * 1024.0)
    fetch_b = f_k[kf][0] * 1024.0 * fetch_factor
    write_b = w_k[kw][0] * 1024.0 * write_factor
    lines = [f"# {h}" for h in header] + [
        f"kernel: {kf}",
        f"dispatches: fetch {f_k[kf][1]}, write {w_k[kw][1]}",
        f"fetch_kib_per_dispatch: {f_k[kf][0]:.1f}",
        f"write_kib_per_dispatch: {w_k[kw][0]:.1f}",
        f"copy_kernel: {ck}",
        f"copy_fetch_kib_per_dispatch: {cf[ck][0]:.1f}  (copy of {COPY_BYTES} bytes)",
        f"copy_write_kib_per_dispatch: {cw[_pick(cw, 'bitwise_not')][0]:.1f}",
        f"fetch_factor: {fetch_factor:.4f}",
        f"write_factor: {write_factor:.4f}",
        f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}",
        f"source_digest: {source_digest()}",
    ]
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
    missing or was taken from other kernel sources."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_digest") != source_digest():
        return None
    return float(kv["traffic_bytes_per_launch"])


def copy_calibration():
    import torch
    n = COPY_BYTES // 4
    src = torch.arange(n, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.bitwise_not(src, out=dst)
    # a read-only pass of the same bytes (a reduction): the fetch counter's
    # factor for a kernel that streams loads without stores
    total = None
    for _ in range(5):
        total = torch.sum(src, dtype=torch.int64)
    torch.cuda.synchronize()
    assert int(total.item()) == n * (n - 1) // 2
    ok = bool(torch.equal(dst[:1024], ~src[:1024]))
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "dispatches": 5, "ok": ok}), flush=True)


# ---------------------------------------------------------------- main

def measure(args, workload, index, n):
    """Time one workload (n > 0 slices its widest X to N = n); returns the
    bench record without the CPU baseline."""
    import numpy as np
    import torch
    import bit_unstructured_sparse_amd as bsp
    import workloads

    dev = torch.device("cuda:0")
    bsp.load_library()
    problems = workloads.make(workload)
    problem = problems[index]
    if n:
        widest = max(problems, key=lambda p: p.N) if problem.dtype == "fp16" else problem
        X = problem.meta.get("X_full", widest.X)
        problem = workloads.Problem(problem.name.rsplit("_n", 1)[0] if problem.dtype == "fp16" else problem.name,
                                    problem.dtype, problem.W, X[:n], dict(problem.meta, N=n))
    fp16 = problem.dtype == "fp16"
    N, M, K = problem.N, problem.M, problem.K

    enc = bsp.encode(problem.W)
    algo = {"auto": bsp.ALGO_AUTO, "rowwave": bsp.ALGO_ROWWAVE, "valu": bsp.ALGO_VALU, "mfma": bsp.ALGO_MFMA}[args.algo]
    dt = bsp.FP16 if fp16 else bsp.INT4
    chosen = algo if algo != bsp.ALGO_AUTO else bsp.select(dt, M, K, N, enc.nnz)
    name = algo_name(bsp, chosen)
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
    R = max(1, -(-ROTATE_TARGET // ws))
    copies = [(dm0, Xd, torch.empty((N, M), dtype=y_dtype, device=dev))]
    for _ in range(R - 1):
        dm = bsp.DeviceMatrix(enc.dtype, M, K, enc.nnz, dm0.bitmaps.clone(), dm0.offsets.clone(), dm0.payload.clone())
        copies.append((dm, Xd.clone(), torch.empty((N, M), dtype=y_dtype, device=dev)))
    torch.cuda.synchronize()

    def step(i):
        dm, x, y = copies[i % R]
        if fp16:
            bsp.spmm_f16(dm, x, Y=y, algo=chosen)
        else:
            bsp.spmm_w4a4(dm, x, N, Y=y, algo=chosen)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # spot check of the timed configuration against an independent dense
    # product on a sample of rows (exact integers; fp16 within the 1e-2 bound)
    rows = np.random.default_rng(0).choice(M, size=min(M, 256), replace=False)

    def spot_ok():
        got = copies[0][2].cpu().numpy()[:, rows]
        if fp16:
            ref = (problem.W[rows].astype(np.float64) @ problem.X.astype(np.float64).T).T
            floor = 0.01 * np.sqrt(np.mean(ref ** 2))
            err = np.abs(got.astype(np.float64) - ref) / np.maximum(np.abs(ref), floor)
            return bool(np.max(err) <= 1e-2)
        ref = (problem.W[rows].astype(np.int64) @ problem.X.astype(np.int64).T).T
        return bool(np.array_equal(got, ref))

    parity = spot_ok()

    # timed region: exactly K steps, captured once in a HIP graph (one node
    # per SpMM call, cycling through the rotated copies) and replayed
    capture_stream = torch.cuda.Stream()
    capture_stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(capture_stream):
        with torch.cuda.graph(graph, stream=capture_stream):
            for i in range(args.steps):
                step(i)
    torch.cuda.synchronize()
    graph.replay()                  # first replay is warm-up
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
    parity = parity and spot_ok()

    nbytes = step_bytes(dm0, N, name, fp16)
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    dense_ops = 2.0 * M * K * N
    useful_ops = 2.0 * enc.nnz * N
    wl = f"{problem.name}_n{N}" if not problem.name.endswith(f"_n{N}") else problem.name
    traffic = read_traffic(os.path.join(ROOT, "profiles", f"traffic_{name}_{wl}.txt"))

    density = enc.nnz / (M * K)
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
        "dtype": "f16 x f16 -> f32 acc -> f16" if fp16 else "int4 x int4 -> int32",
        "data": "synthetic (seeded iid unstructured mask / magnitude pruning; the pages' model weights "
                "are not available)",
        "config": {"workload": f"{wl}: W {M}x{K} {'fp16' if fp16 else 'int4'}, density {density:.3f}, N={N}",
                   "M": M, "K": K, "N": N, "nnz": enc.nnz, "kernel": name,
                   "rotated_copies": R, "bytes_per_step": nbytes},
        "frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        "tops_dense_equiv": round(dense_ops / (ms_per_step * 1e-3) / 1e12, 3),
        "tops_useful": round(useful_ops / (ms_per_step * 1e-3) / 1e12, 3),
        "kernel_us_avg": round(kern_ms * 1e3, 3),
        "timing": "K steps captured in one HIP graph and replayed back to back; value uses host wall time "
                  "around the replay, roofline uses HIP events on the replay stream",
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else int(traffic),
                     "kernel": kernel_symbol(bsp, chosen, dt, M, K, N, enc.nnz), "bytes_per_launch": nbytes},
        "parity_sample_ok": parity,
    }
    args._problem = problem
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qkv", help="tiny | qkv | ffn | lowsparse | fp16")
    ap.add_argument("--index", type=int, default=0, help="matrix index inside the workload (ffn: 0 up, 1 down)")
    ap.add_argument("--n", type=int, default=0, help="override N (slices the workload's widest X)")
    ap.add_argument("--algo", default="auto", choices=["auto", "rowwave", "valu", "mfma"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true", help="one line per (workload, N) of the N sweep")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("DIR", "OUT"))
    ap.add_argument("--summarize-traffic", metavar="OUT")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("DIR", "OUT"))
    ap.add_argument("--fetch"), ap.add_argument("--write")
    ap.add_argument("--copy-fetch"), ap.add_argument("--copy-write")
    ap.add_argument("--kernel", default="w4a4", help="kernel name fragment for --summarize-traffic")
    ap.add_argument("--note", action="append", default=[], help="header line for a summary")
    args = ap.parse_args()

    if args.summarize_trace:
        return summarize_trace(args.summarize_trace[0], args.summarize_trace[1], args.note)
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters[0], args.summarize_counters[1], args.kernel, args.note)
    if args.summarize_traffic:
        return summarize_traffic(args.summarize_traffic, args.fetch, args.write, args.copy_fetch,
                                 args.copy_write, args.kernel, args.note)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the path has no "
              f"multi-GPU code; how it would shard is described with the design.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        return copy_calibration()

    if args.sweep:
        # the N sweep on the qkv weights and the 70 %-dense matrix at N = 16, 32
        for wl, idx, n in SWEEP:
            out = measure(args, wl, idx, n)
            print(json.dumps({"sweep": out["config"]["workload"].split(":")[0], "N": out["config"]["N"],
                              "kernel": out["roofline"]["kernel"], "kernel_us_avg": out["kernel_us_avg"],
                              "GB/s (events)": out["roofline"]["achieved"], "GB/s (wall)": out["value"],
                              "frac_of_peak": out["roofline"]["frac"], "tops_dense_equiv": out["tops_dense_equiv"],
                              "tops_useful": out["tops_useful"], "parity_sample_ok": out["parity_sample_ok"]}),
                  flush=True)
        return
    out = measure(args, args.workload, args.index, args.n)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args._problem, out["config"]["bytes_per_step"] / out["config"]["M"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
