"""Benchmark of the bitmap-tiled int4 SpMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload qkv] [--algo auto]

A step is one call of the SpMM entry point (``spmm_bitmap_w4a4``: host-side
argument checks and kernel selection, then the kernel that streams the
compressed tiles, stages X, decodes, contracts and stores Y) on one batch of
synthetic input already resident in HBM. Encoding is the offline step of the
method and is done once, before timing. The inputs are rotated through
enough identical device copies (>= 1 GiB in total, four times the 256 MB
Infinity Cache) that each step reads its operands from HBM, not from cache.

The K timed steps are captured once in a HIP graph (one kernel node per SpMM
call) and replayed back to back: these kernels last a few microseconds, less
than a Python-level launch, so eager launching would time the host instead.
The eager per-call time is reported too (``eager_ms_per_step``).

Prints ONE JSON line. ``value`` is achieved GB/s over the algorithmic bytes of
a step (bitmaps, offsets if the kernel reads them per tile, payload, X, Y)
divided by the host wall time per step around the replay; the ``roofline``
object divides the same bytes by the average launch duration taken with HIP
events on the replay stream. ``cpu_baseline`` times the CPU oracle (single
thread, plain C) on the same workload and byte count.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MALL_BYTES = 256 << 20
ROTATE_TARGET = 1 << 30

# Whether a kernel reads one 4-byte offset per tile (else one per row block).
READS_TILE_OFFSETS = {"rowwave": True, "valu": False, "mfma": False}


def algo_name(bsp, a):
    return {bsp.ALGO_ROWWAVE: "rowwave", bsp.ALGO_VALU: "valu", bsp.ALGO_MFMA: "mfma"}[a]


def step_bytes(dm, N, algo):
    """Algorithmic bytes of one SpMM call (int4): stream + X + Y."""
    stream = dm.stream_bytes(with_offsets=READS_TILE_OFFSETS[algo])
    if not READS_TILE_OFFSETS[algo]:
        stream += 4 * (dm.M + 1)       # one offset per row
    return stream + N * ((dm.K + 1) // 2) + 4 * dm.M * N


def cpu_baseline(problem, nbytes, reps):
    """The oracle as it stands (plain C, one thread) on the full workload:
    decode the stream to dense, unpack X, exact int64 product."""
    import numpy as np
    import oracle
    s = oracle.encode(problem.W)
    Xp = _pack(problem.X)
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.spmm_w4a4(s, Xp, problem.N)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    return {"value": round(nbytes / t / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"full {problem.name} workload (M={problem.M}, K={problem.K}, N={problem.N}), "
                      f"median of {reps} runs, {t:.3f} s each, same byte count as the GPU step",
            "seconds": round(t, 4), "cpu": platform.processor() or platform.machine()}


def _pack(X):
    # test-side packer for the oracle input (pinned by tests/golden/x_int4_packing.json)
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import pins
    return pins._pack_x_for_test(X)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qkv", help="tiny | qkv | ffn | lowsparse")
    ap.add_argument("--index", type=int, default=0, help="matrix index inside the workload (ffn: 0 up, 1 down)")
    ap.add_argument("--n", type=int, default=0, help="override N (uses the workload's X drawn at N=32 when present)")
    ap.add_argument("--algo", default="auto", choices=["auto", "rowwave", "valu", "mfma"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=3)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import bit_unstructured_sparse_amd as bsp
    import workloads

    dev = torch.device("cuda:0")
    bsp.load_library()
    problem = workloads.make(args.workload)[args.index]
    if args.n:
        X = problem.meta.get("X_full", problem.X)
        problem = workloads.Problem(problem.name, problem.dtype, problem.W, X[: args.n], dict(problem.meta, N=args.n))
    if problem.dtype != "int4":
        raise SystemExit("bench.py times the int4 path (the headline metric)")
    N, M, K = problem.N, problem.M, problem.K

    enc = bsp.encode(problem.W)
    algo = {"auto": bsp.ALGO_AUTO, "rowwave": bsp.ALGO_ROWWAVE, "valu": bsp.ALGO_VALU, "mfma": bsp.ALGO_MFMA}[args.algo]
    chosen = algo if algo != bsp.ALGO_AUTO else bsp.select(bsp.INT4, M, K, N, enc.nnz)
    name = algo_name(bsp, chosen)
    dm0 = enc.to_device(dev)
    Xp = torch.from_numpy(bsp.pack_int4(problem.X)).to(dev)
    ws = (dm0.bitmaps.numel() * 8 + dm0.offsets.numel() * 4 + dm0.payload.numel() + Xp.numel() + 4 * M * N)
    R = max(1, -(-ROTATE_TARGET // ws))
    copies = [(dm0, Xp, torch.empty((N, M), dtype=torch.int32, device=dev))]
    for _ in range(R - 1):
        dm = bsp.DeviceMatrix(enc.dtype, M, K, enc.nnz, dm0.bitmaps.clone(), dm0.offsets.clone(), dm0.payload.clone())
        copies.append((dm, Xp.clone(), torch.empty((N, M), dtype=torch.int32, device=dev)))
    torch.cuda.synchronize()

    def step(i):
        dm, x, y = copies[i % R]
        bsp.spmm_w4a4(dm, x, N, Y=y, algo=chosen)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # parity spot check of the timed configuration against an independent
    # dense product (exact integers) on a sample of rows
    rows = np.random.default_rng(0).choice(M, size=min(M, 256), replace=False)
    ref = (problem.W[rows].astype(np.int64) @ problem.X.astype(np.int64).T).T
    got = copies[0][2].cpu().numpy()[:, rows]
    parity = bool(np.array_equal(got, ref))

    # eager steps (one host call per step), for reference
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n_eager = min(args.steps, 100)
    for i in range(n_eager):
        step(i)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / n_eager

    # timed region: exactly K steps, captured once in a HIP graph (one node
    # per SpMM call, cycling through the rotated copies) and replayed, so the
    # GPU runs the steps back to back without host launch gaps
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
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    # average launch duration: HIP events on the replay stream over the K launches
    kern_ms = ev0.elapsed_time(ev1) / args.steps
    got2 = copies[0][2].cpu().numpy()[:, rows]
    parity = parity and bool(np.array_equal(got2, ref))

    nbytes = step_bytes(dm0, N, name)
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    dense_ops = 2.0 * M * K * N
    useful_ops = 2.0 * enc.nnz * N
    traffic = None
    tfile = os.path.join(ROOT, "profiles", f"traffic_{name}_{problem.name}_n{N}.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            traffic = json.load(f).get("bytes_per_launch")

    out = {
        "metric": "achieved HBM GB/s (frac of peak) + dense-equiv TOPS, bitmap SpMM at N=1..32",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 x int4 -> int32",
        "data": "synthetic (seeded iid unstructured mask; pages' model weights not available)",
        "config": {"workload": f"{problem.name}: W {M}x{K} int4, density {enc.nnz / (M * K):.3f}, N={N}",
                   "M": M, "K": K, "N": N, "nnz": enc.nnz, "kernel": name,
                   "rotated_copies": R, "bytes_per_step": nbytes},
        "frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        "tops_dense_equiv": round(dense_ops / (ms_per_step * 1e-3) / 1e12, 3),
        "tops_useful": round(useful_ops / (ms_per_step * 1e-3) / 1e12, 3),
        "kernel_us_avg": round(kern_ms * 1e3, 3),
        "eager_ms_per_step": round(eager_ms, 5),
        "timing": "K steps captured in one HIP graph and replayed back to back; value uses host wall time "
                  "around the replay, roofline uses HIP events on the replay stream",
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": f"bsp {name} w4a4", "bytes_per_launch": nbytes},
        "parity_sample_ok": parity,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(problem, nbytes, args.cpu_reps)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
