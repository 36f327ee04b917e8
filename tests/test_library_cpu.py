"""Host-side checks of the product library (no GPU needed): it loads, exports
every symbol the header declares, its encoder is byte-identical to the
oracle's reference encoder, and bad SpMM arguments are rejected on the host
before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import bit_unstructured_sparse_amd as bsp
import oracle
import pins
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions(header="bitmap_spmm.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|int64_t|char\s*\*|const char\s*\*)\s*\*?\s*(\w+)\s*\(",
                                src, re.M)))


def test_library_exports_every_declared_symbol():
    L = bsp.load_library()
    names = _declared_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/bitmap_spmm.h but not exported"
    assert sorted(bsp.EXPORTS) == names
    assert bsp.load_library().bsp_version().decode().count(".") == 2


def test_probe_library_exports_every_declared_symbol():
    # the streaming-read probe the benchmark loads (include/bsp_probe.h)
    L = ctypes.CDLL(os.path.join(ROOT, "bit_unstructured_sparse_amd", "libbsp_probe.so"))
    names = _declared_functions("bsp_probe.h")
    assert names == ["bsp_probe_read", "bsp_probe_sink_words"]
    for n in names:
        assert hasattr(L, n)
    L.bsp_probe_sink_words.restype = ctypes.c_int64
    assert L.bsp_probe_sink_words(256, 512) == 2048
    # invalid arguments are refused before any launch
    L.bsp_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_void_p]
    assert L.bsp_probe_read(None, 1024, FAKE, 0, 256, 512, None) == 1
    assert L.bsp_probe_read(FAKE, 1000, FAKE, 0, 256, 512, None) == 1     # not a multiple of 16
    assert L.bsp_probe_read(FAKE, 1024, FAKE, 3, 256, 512, None) == 1     # unknown mode
    assert L.bsp_probe_read(FAKE, 1024, FAKE, 0, 256, 100, None) == 1     # block not a multiple of 64


def _same(e, s):
    return (e.nnz == s.nnz and np.array_equal(e.bitmaps, s.bitmaps) and np.array_equal(e.offsets, s.offsets)
            and np.array_equal(e.payload, s.payload))


@pytest.mark.parametrize("M,K,keep", [(1, 1, 1.0), (3, 63, 0.5), (2, 64, 0.5), (5, 65, 0.3), (7, 127, 0.7),
                                      (64, 128, 0.5), (129, 300, 0.5), (1000, 77, 0.37), (517, 513, 0.5),
                                      (300, 64, 0.0), (257, 1, 0.5), (0, 10, 0.5), (10, 0, 0.5)])
def test_encoder_byte_identical_to_oracle(M, K, keep):
    p = workloads.random_int4_problem(M * 131 + K, M, K, 1, keep=keep)
    e = bsp.encode(p.W)
    s = oracle.encode(p.W)
    assert _same(e, s)
    assert oracle.validate_arrays(0, e.bitmaps, e.offsets, e.payload, M, K) == 0


def test_encoder_thread_boundaries_odd_rows():
    # every row holds an odd count, so thread blocks start and end mid-byte
    rng = np.random.default_rng(5)
    for M in (128, 129, 640, 1031):
        W = np.zeros((M, 200), np.int8)
        for m in range(M):
            cnt = 2 * int(rng.integers(0, 50)) + 1
            cols = rng.choice(200, cnt, replace=False)
            W[m, cols] = rng.integers(1, 8, cnt) * rng.choice([-1, 1], cnt)
        assert _same(bsp.encode(W), oracle.encode(W))


def test_encoder_fp16_byte_identical():
    for i, (M, K) in enumerate([(33, 200), (200, 64), (5, 1)]):
        p = workloads.random_fp16_problem(50 + i, M, K, 1)
        W = p.W.copy()
        W[0, 0] = np.float16(-0.0)
        e, s = bsp.encode(W), oracle.encode(W)
        assert _same(e, s)


def test_encoder_strided_input():
    p = workloads.random_int4_problem(3, 40, 300, 1)
    big = np.zeros((40, 333), np.int8)
    big[:, :300] = p.W
    assert _same(bsp.encode(big[:, :300]), oracle.encode(p.W))


def test_encoder_errors():
    L = bsp.load_library()
    W = np.zeros((2, 10), np.int8); W[1, 3] = 8
    with pytest.raises(bsp.BspError) as ei:
        bsp.encode(W)
    assert ei.value.status == bsp.E_RANGE
    W = np.ones((2, 10), np.int8)
    nnz, nb = ctypes.c_int64(-1), ctypes.c_int64(-1)
    bm = np.zeros(2, np.uint64); off = np.zeros(3, np.uint32); pl = np.zeros(16, np.uint8)
    P = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    rc = L.encode_bitmap_tiles(0, P(W), 2, 10, 10, P(bm), P(off), P(pl), 9, ctypes.byref(nnz), ctypes.byref(nb))
    assert rc == bsp.E_CAPACITY and nnz.value == 20 and nb.value == 10
    assert L.encode_bitmap_tiles(0, P(W), 2, 10, 9, None, None, None, 0, None, None) == bsp.E_ARG   # ldw < K
    assert L.encode_bitmap_tiles(7, P(W), 2, 10, 10, None, None, None, 0, None, None) == bsp.E_ARG  # dtype
    assert L.encode_bitmap_tiles(0, None, 2, 10, 10, None, None, None, 0, None, None) == bsp.E_ARG  # W null
    assert L.encode_bitmap_tiles(0, P(W), 2, 10, 10, P(bm), None, None, 0, None, None) == bsp.E_ARG


def test_pack_int4_golden():
    g = pins._golden("x_int4_packing.json")
    out = bsp.pack_int4(np.array(g["X_rows"], np.int8)).reshape(-1)
    assert [f"{int(b):02X}" for b in out] == g["packed_hex"]
    # round trip through the oracle's unpacker on a ragged K
    p = workloads.random_int4_problem(4, 1, 77, 5)
    assert np.array_equal(oracle.unpack_x4(bsp.pack_int4(p.X), 5, 77), p.X)
    with pytest.raises(bsp.BspError):
        bsp.pack_int4(np.full((1, 3), 9, np.int8))


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every case below fails on the host


@pytest.mark.parametrize("fn", ["spmm_bitmap_w4a4_algo", "spmm_bitmap_f16_algo"])
def test_spmm_argument_errors_on_host(fn):
    f = getattr(bsp.load_library(), fn)
    ok = dict(bm=FAKE, off=FAKE, pl=FAKE, pb=64, M=4, K=64, X=FAKE, N=1, Y=FAKE, algo=0)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["bm"], a["off"], a["pl"], a["pb"], a["M"], a["K"], a["X"], a["N"], a["Y"], a["algo"], None)

    assert call(N=33) == bsp.E_ARG
    assert call(N=-1) == bsp.E_ARG
    assert call(M=-1) == bsp.E_ARG
    assert call(K=-5) == bsp.E_ARG
    assert call(K=1 << 25) == bsp.E_OVERFLOW
    assert call(M=1 << 31) == bsp.E_OVERFLOW
    assert call(M=1 << 30, K=1 << 20) == bsp.E_OVERFLOW       # M*T beyond 2^31
    assert call(pb=17) == bsp.E_ARG                            # not a multiple of 16
    assert call(pb=-16) == bsp.E_ARG
    assert call(Y=None) == bsp.E_ARG
    assert call(off=None) == bsp.E_ARG
    assert call(bm=None) == bsp.E_ARG
    assert call(X=None) == bsp.E_ARG
    assert call(pl=None) == bsp.E_ARG
    assert call(algo=99) == bsp.E_ARG
    assert call(algo=-1) == bsp.E_ARG
    assert call(algo=4) == bsp.E_ARG                           # no fourth kernel family
    # a forced kernel that cannot run the shape is an error, never a silent
    # fallback to another kernel (the shape is far past the fast path's K range)
    assert call(algo=bsp.ALGO_MFMA, K=1 << 20, pb=1 << 20) == bsp.E_UNSUPPORTED
    assert bsp.status_string(bsp.E_UNSUPPORTED) == "the forced kernel cannot run this shape"
    # empty problems succeed without launching anything
    assert call(M=0) == bsp.OK
    assert call(N=0) == bsp.OK
    assert call(M=0, Y=None, X=None) == bsp.OK


def test_workspace_api_on_host():
    # sizes: no workspace below the split thresholds; the split plans' counters
    # and partials above (independent of nnz); errors before any launch
    # (the size covers the forced split-K plan: 2 K ranges per 2-block set)
    n = bsp.workspace_bytes(bsp.INT4, 4096, 11008, 16)
    # 128 sets of 2 blocks, 2 K ranges: the fixed 64 KiB counter area + 128 * 2 * 2 * 16 columns * 16 rows * 4 B
    assert n == 65536 + 128 * 2 * 2 * 16 * 16 * 4
    assert bsp.workspace_bytes(bsp.INT4, 12288, 4096, 8) > 0
    assert bsp.workspace_bytes(bsp.FP16, 4096, 11008, 8) > 0
    assert bsp.workspace_bytes(bsp.FP16, 4096, 11008, 8, 1000) == bsp.workspace_bytes(bsp.FP16, 4096, 11008, 8)
    L = bsp.load_library()
    out = ctypes.c_int64(-1)
    assert L.bsp_workspace_bytes(7, 1, 1, 1, -1, ctypes.byref(out)) == bsp.E_ARG
    assert L.bsp_workspace_bytes(0, 1, 1, 33, -1, ctypes.byref(out)) == bsp.E_ARG
    assert L.bsp_workspace_bytes(0, 1, 1 << 25, 1, -1, ctypes.byref(out)) == bsp.E_OVERFLOW
    assert L.bsp_workspace_bytes(0, 1, 1, 1, -1, None) == bsp.E_ARG
    # the _ws entry points: a workspace off a 256-byte boundary, NULL with a
    # size, or smaller than the plan needs is refused on the host
    f = L.spmm_bitmap_w4a4_ws
    M, K, N = 4096, 11008, 16
    base = dict(bm=FAKE, off=FAKE, pl=FAKE, pb=16 * (M * K // 32), X=FAKE, Y=FAKE)

    def call(ws, wsb, algo=bsp.ALGO_AUTO):
        return f(base["bm"], base["off"], base["pl"], base["pb"], M, K, base["X"], N, base["Y"], ws, wsb, algo, None)

    assert call(ctypes.c_void_p(0x1010), n) == bsp.E_ARG          # not 256-byte aligned
    assert call(None, 256) == bsp.E_ARG                            # size without a workspace
    assert call(FAKE, -256) == bsp.E_ARG
    # (every call here fails on the host: the pointers are fake, a launch would fault)
    assert call(FAKE, 256, bsp.ALGO_SPLITK) == bsp.E_CAPACITY      # the forced split plan needs more
    g = L.spmm_bitmap_f16_ws
    assert g(FAKE, FAKE, FAKE, 16 * 1000, 4096, 11008, FAKE, 8, FAKE, FAKE, 256, bsp.ALGO_AUTO, None) == bsp.E_CAPACITY
    # fp16 with K % 8 != 0 has no split-K plan
    assert g(FAKE, FAKE, FAKE, 16, 16, 100, FAKE, 8, FAKE, None, 0, bsp.ALGO_SPLITK, None) == bsp.E_UNSUPPORTED


def test_noalloc_entry_point_limits_on_host():
    # a plan needing more than the static scratch is refused before any
    # device call (fake pointers: a launch would fault)
    L = bsp.load_library()
    assert L.bsp_noalloc_scratch_bytes() == 8 << 20
    M, K, N = 1 << 19, 8192, 32          # 16384 sets of 2 blocks (the most the counter area holds)
    assert bsp.workspace_bytes(bsp.FP16, M, K, N) > L.bsp_noalloc_scratch_bytes()
    f = L.spmm_bitmap_f16_noalloc
    assert f(FAKE, FAKE, FAKE, 16 << 20, M, K, FAKE, N, FAKE, bsp.ALGO_AUTO, None) == bsp.E_CAPACITY
    assert f(FAKE, FAKE, FAKE, 16, 4, 64, FAKE, 33, FAKE, bsp.ALGO_AUTO, None) == bsp.E_ARG
    assert f(FAKE, FAKE, FAKE, 16, 4, 100, FAKE, 8, FAKE, bsp.ALGO_SPLITK, None) == bsp.E_UNSUPPORTED


def test_selection_is_defined_for_every_shape():
    for dt in (bsp.INT4, bsp.FP16):
        for N in range(1, 33):
            for (M, K) in [(512, 512), (12288, 4096), (11008, 4096), (4096, 11008), (8192, 8192), (1, 1), (7, 0)]:
                a = bsp.select(dt, M, K, N)
                assert a in (bsp.ALGO_ROWWAVE, bsp.ALGO_MFMA, bsp.ALGO_SPLITK)
                assert bsp.describe(dt, M, K, N).startswith("dtype=")
    assert bsp.select(bsp.INT4, 1, 1, 33) == -1
    assert bsp.select(5, 1, 1, 1) == -1


def test_description_names_the_launched_kernel():
    # the plan's kernel for each family of shapes (host-only planning, no launch)
    d = bsp.describe(bsp.INT4, 12288, 4096, 8, 12288 * 4096 // 2)
    assert "-> mfma kernel=k_bt64s_w4a4 " in d and "grid=256 block=512" in d
    d = bsp.describe(bsp.INT4, 4096, 11008, 16, 4096 * 11008 * 3 // 10)
    assert "-> mfma kernel=k_bt64_w4a4 " in d and "tiles_per_lane=8" in d
    d = bsp.describe(bsp.FP16, 4096, 4096, 1, 4096 * 4096 * 4 // 10)
    assert "-> mfma kernel=k_bt8_f16 " in d and "grid=256 block=512" in d and "step_slots=2" in d
    d = bsp.describe(bsp.FP16, 8003, 1000, 5, 8003 * 1000 // 10)   # four steps per workgroup
    assert "-> mfma kernel=k_bt8_f16 " in d and "step_slots=4" in d
    d = bsp.describe(bsp.FP16, 4096, 4096, 32, 4096 * 4096 * 4 // 10)
    assert "-> mfma kernel=k_bt64_f16 " in d and "block=1024" in d
    # any K up to 16384 takes the MFMA kernels (odd K too); beyond, the split-K
    # kernel walking all of K per workgroup
    assert "-> mfma kernel=k_bt64s_w4a4 " in bsp.describe(bsp.INT4, 64, 100, 4)
    assert "-> mfma kernel=k_bt64_w4a4 " in bsp.describe(bsp.INT4, 64, 64 * 255 + 7, 4, 64 * 16327 // 2)
    # blocks of 128 or more tiles too dense to stage (nnz unknown: planned
    # dense) take the split-K kernel
    assert "-> splitk kernel=k_bsk_w4a4 " in bsp.describe(bsp.INT4, 64, 64 * 255 + 7, 4)
    d = bsp.describe(bsp.INT4, 64, 16385, 4)
    assert "-> splitk kernel=k_bsk_w4a4 " in d and "splits=1 " in d
    # fp16 beyond K = 4096: the split-K kernel (2 K ranges with a workspace)
    d = bsp.describe(bsp.FP16, 4096, 11008, 8)
    assert "-> splitk kernel=k_bsk_f16 " in d and "splits=1 " in d
    d = bsp.describe(bsp.FP16, 4096, 11008, 8, workspace=True)
    assert "-> splitk kernel=k_bsk_f16 " in d and "splits=2 " in d and "blocks_per_set=1 " in d
    # int4 with a workspace: the block kernels up to K = 16384, one K range
    # up to K = 20480, two beyond
    assert "-> mfma kernel=k_bt64_w4a4 " in bsp.describe(bsp.INT4, 4096, 11008, 16, workspace=True)
    d = bsp.describe(bsp.INT4, 4096, 20000, 8, workspace=True)
    assert "-> splitk kernel=k_bsk_w4a4 " in d and "splits=1 " in d
    d = bsp.describe(bsp.INT4, 4096, 20480, 8, workspace=True)
    assert "-> splitk kernel=k_bsk_w4a4 " in d and "splits=1 " in d
    d = bsp.describe(bsp.INT4, 4096, 20481, 8, workspace=True)
    assert "-> splitk kernel=k_bsk_w4a4 " in d and "splits=2 " in d
    d = bsp.describe(bsp.INT4, 4096, 32768, 8)
    assert "-> splitk kernel=k_bsk_w4a4 " in d and "splits=1 " in d
    # fp16 with K % 8 != 0: the plain kernel
    assert bsp.describe(bsp.FP16, 64, 100, 4).endswith("-> rowwave kernel=k_rowwave_f16")
    # nothing to launch
    assert "kernel=" not in bsp.describe(bsp.INT4, 0, 4096, 8)


def test_describe_plan_of_forced_choices():
    # bsp_describe_plan: the plan an explicit choice takes, or E_UNSUPPORTED
    nnz = int(4096 * 11008 * 0.3)
    d = bsp.describe(bsp.INT4, 4096, 11008, 16, nnz, workspace=True, algo=bsp.ALGO_SPLITK)
    assert "kernel=k_bsks_w4a4" in d and "splits=2 " in d and "blocks_per_set=2 " in d and "grid=256 " in d, d
    d = bsp.describe(bsp.INT4, 4096, 11008, 16, nnz, workspace=False, algo=bsp.ALGO_SPLITK)
    assert "kernel=k_bsk_w4a4" in d and "splits=1 " in d, d          # no workspace: one range
    d = bsp.describe(bsp.INT4, 300, 24616, 8, -1, workspace=True, algo=bsp.ALGO_SPLITK)
    assert "kernel=k_bsk_w4a4" in d and "splits=2 " in d, d          # ranges past 96 tiles: chunked
    with pytest.raises(bsp.BspError) as ei:
        bsp.describe(bsp.FP16, 100, 4100, 3, algo=bsp.ALGO_MFMA)
    assert ei.value.status == bsp.E_UNSUPPORTED
    assert bsp.describe(bsp.INT4, 12288, 4096, 8, algo=bsp.ALGO_MFMA) == bsp.describe(bsp.INT4, 12288, 4096, 8)
    assert "kernel=k_rowwave_w4a4" in bsp.describe(bsp.INT4, 64, 640, 2, algo=bsp.ALGO_ROWWAVE)
    for bad in (-1, 4, 99):
        with pytest.raises(bsp.BspError) as ei:
            bsp.describe(bsp.INT4, 64, 640, 2, algo=bad)
        assert ei.value.status == bsp.E_ARG


def test_streamed_splitk_plans_fit():
    # every streamed split-K plan: one workgroup per CU at most, its LDS
    # within 160 KB, each K range within its lanes' tiles, and a workspace
    # of counters plus one int32 partial per (block, range, column, row)
    rng = np.random.default_rng(11)
    seen = 0
    for _ in range(400):
        M = int(rng.integers(1, 9000))
        K = int(rng.integers(64 * 64 + 1, 64 * 200))
        N = int(rng.integers(1, 33))
        keep = float(rng.uniform(0.02, 1.0))
        nnz = int(M * K * keep)
        d = bsp.describe(bsp.INT4, M, K, N, nnz, workspace=True, algo=bsp.ALGO_SPLITK)
        if "k_bsks_w4a4" not in d:
            continue
        seen += 1
        f = {k: int(v) for k, v in re.findall(r"(\w+)=(\d+)", d.split("->")[1])}
        T, blocks = -(-K // 64), -(-M // 16)
        assert f["grid"] <= 256 and f["lds"] <= 160 * 1024 and f["block"] == 512, d
        assert f["tiles_per_split"] <= 32 * f["tiles_per_lane"] and f["tiles_per_lane"] in (2, 3), d
        assert (f["splits"] - 1) * f["tiles_per_split"] < T <= f["splits"] * f["tiles_per_split"], d
        nsets = -(-blocks // f["blocks_per_set"])
        assert f["grid"] == nsets * f["splits"] and 1 <= f["blocks_per_set"] <= 3, d
        assert f["workspace"] == 65536 + nsets * f["blocks_per_set"] * f["splits"] * N * 16 * 4, d
        assert bsp.workspace_bytes(bsp.INT4, M, K, N, nnz) >= f["workspace"], d
    assert seen > 50


def test_every_plan_fits_the_hardware():
    # every described launch (automatic or forced, with or without a
    # workspace, int4 or fp16): LDS within gfx950's 160 KB per workgroup, a
    # whole number of wavefronts up to 1024 threads, at least one workgroup
    rng = np.random.default_rng(5)
    seen = set()
    for _ in range(600):
        u = rng.random()
        dt = bsp.INT4 if u < 0.5 else bsp.FP16 if u < 0.85 else bsp.INT2
        M = int(rng.integers(1, 70000))
        K = int(rng.integers(1, 40000))
        if dt == bsp.FP16 and rng.random() < 0.7:
            K = K // 8 * 8 + 8
        N = int(rng.integers(1, 33))
        nnz = int(M * K * rng.uniform(0.02, 1.0))
        for algo in (bsp.ALGO_AUTO, bsp.ALGO_ROWWAVE, bsp.ALGO_MFMA, bsp.ALGO_SPLITK):
            for ws in (False, True):
                try:
                    d = bsp.describe(dt, M, K, N, nnz, workspace=ws, algo=algo)
                except bsp.BspError as e:
                    assert e.status == bsp.E_UNSUPPORTED and algo != bsp.ALGO_AUTO, d
                    continue
                m = re.search(r"kernel=(\S+)", d)
                assert m, d
                seen.add(m.group(1))
                f = {k: int(v) for k, v in re.findall(r"(\w+)=(\d+)", d.split("->")[1])}
                if f.get("partial_ring"):
                    assert f["step_slots"] == 8, d
                if "lds" in f:
                    assert f["lds"] <= 160 * 1024, d
                    assert 64 <= f["block"] <= 1024 and f["block"] % 64 == 0, d
                    assert f["grid"] >= 1, d
    want = {"k_bt64s_w4a4", "k_bt64_w4a4", "k_bsk_w4a4", "k_bsks_w4a4", "k_bt8_f16", "k_bt64_f16", "k_bsk_f16",
            "k_rowwave_w4a4", "k_rowwave_f16", "k_bt64s_w2a4"}
    assert want <= seen, want - seen


def test_streaming_plan_density_rule():
    # the streaming kernel keeps its staggered staging while the average block
    # fits it, drops the stagger when only the plain layout holds the average
    # block, and leaves fully dense blocks (which fit neither area) to the ring
    # kernel, whose staging holds a whole dense block (staggered: every row
    # is 2048 B long)
    M, K, N = 12288, 4096, 8
    d50 = bsp.describe(bsp.INT4, M, K, N, M * K // 2)
    assert "kernel=k_bt64s_w4a4" in d50 and "stagger=1" in d50, d50
    d99 = bsp.describe(bsp.INT4, M, K, N, int(M * K * 0.99))
    assert "kernel=k_bt64s_w4a4" in d99 and "stagger=0" in d99, d99
    d100 = bsp.describe(bsp.INT4, M, K, N, M * K)
    assert "kernel=k_bt64_w4a4 " in d100 and "stagger=1" in d100 and "stage_bufs=3" in d100, d100


def _kv(d):
    return dict(kv.split("=", 1) for kv in d.split("->", 1)[1].split() if "=" in kv)


def test_ring_plans_stage_past_one_workgroup_per_cu():
    # int4 ring kernel past 256 workgroups: staging sized for one resident
    # workgroup per CU (the grid runs in rounds) rather than global windows
    for M, K, N, dens, grid, bufs in [(8192, 16384, 8, 0.5, 512, 1), (16384, 16384, 8, 0.5, 1024, 1),
                                      (5000, 12000, 3, 0.5, 313, 1), (65536, 4096, 8, 0.5, 1024, 4),
                                      (32768, 8192, 8, 0.5, 1024, 2)]:
        d = bsp.describe(bsp.INT4, M, K, N, int(M * K * dens))
        kv = _kv(d)
        assert "kernel=k_bt64_w4a4 " in d, d
        assert int(kv["grid"]) == grid and int(kv["stage_bufs"]) == bufs, d
        assert int(kv["stage_kb"]) > 0 and 80 * 1024 < int(kv["lds"]) <= 160 * 1024, d
    # two blocks per workgroup that do not fit twice: one block per workgroup
    d = bsp.describe(bsp.INT4, 8192, 8192, 8, int(8192 * 8192 * 0.9))
    kv = _kv(d)
    assert kv["grid"] == "512" and int(kv["stage_kb"]) > 0 and kv["stage_bufs"] == "1", d
    # one dense 256-tile block exceeds the LDS: automatic plans take the
    # split-K kernel, a forced MFMA call reads global windows
    for ws in (False, True):
        d = bsp.describe(bsp.INT4, 4096, 16384, 8, int(4096 * 16384 * 0.85), workspace=ws)
        assert "-> splitk kernel=k_bsk_w4a4 " in d, d
    d = bsp.describe(bsp.INT4, 4096, 16384, 8, int(4096 * 16384 * 0.85), algo=bsp.ALGO_MFMA)
    assert "kernel=k_bt64_w4a4 " in d and "stage_kb=0 " in d, d
    # below that density the block still stages
    d = bsp.describe(bsp.INT4, 4096, 16384, 8, int(4096 * 16384 * 0.75))
    assert "kernel=k_bt64_w4a4 " in d and int(_kv(d)["stage_kb"]) > 100, d


def test_staggered_staging_rules():
    # ring kernel: staggered when the average row is within 12 B of a
    # multiple of 64 B (rows of one length, as row-wise pruning leaves them,
    # would otherwise line a tile of the 16 rows up on the same LDS banks),
    # its buffers 64/61 larger
    for M, K, N, dens, stg in [(4096, 11008, 16, 0.5, 1), (5120, 5120, 8, 0.5, 1), (4096, 14336, 8, 0.5, 1),
                               (4096, 16384, 8, 0.5, 1), (4096, 11008, 16, 0.3, 0), (8192, 8192, 32, 0.7, 0)]:
        d = bsp.describe(bsp.INT4, M, K, N, int(M * K * dens))
        kv = _kv(d)
        assert "kernel=k_bt64_w4a4 " in d and kv["stagger"] == str(stg), d
    plain = _kv(bsp.describe(bsp.INT4, 4096, 16384, 8, 4096 * 16384 // 2, algo=bsp.ALGO_MFMA))
    assert plain["stagger"] == "1" and int(plain["stage_kb"]) * 1024 >= (4096 * 16384 // 4 // 256) * 64 // 61
    # ... but not when the staggered buffers would hold fewer blocks than the
    # plain ones (two 128-tile blocks per workgroup, rows of 3072 B), or
    # lose the single pass, unless the average row is an exact multiple
    # (rows of 2048 B, dense 64-tile blocks, three per workgroup)
    kv = _kv(bsp.describe(bsp.INT4, 8192, 8192, 8, int(8192 * 8192 * 0.75)))
    assert kv["stagger"] == "0" and kv["stage_bufs"] == "2", kv
    kv = _kv(bsp.describe(bsp.INT4, 8192, 8192, 8, int(8192 * 8192 * 0.72)))
    assert kv["stagger"] == "1" and kv["stage_bufs"] == "2", kv
    kv = _kv(bsp.describe(bsp.INT4, 40000, 4096, 8, int(40000 * 4096 * 0.495)))   # rows of ~1014 B
    assert kv["stagger"] == "0" and kv["one_pass"] == "1", kv
    for M, dens in [(40000, 0.5), (12288, 1.0)]:                                    # 1024 B, 2048 B
        kv = _kv(bsp.describe(bsp.INT4, M, 4096, 8, int(M * 4096 * dens)))
        assert kv["stagger"] == "1" and kv["one_pass"] == "0", kv
    # streaming kernel: rows within 28 B of a multiple of 128 B
    for dens, stg in [(0.5, 1), (0.5625, 1), (0.25, 1), (0.35, 0), (0.4, 0)]:
        d = bsp.describe(bsp.INT4, 12288, 4096, 8, int(12288 * 4096 * dens))
        assert "kernel=k_bt64s_w4a4 " in d and _kv(d)["stagger"] == str(stg), (dens, d)


def test_f16_block_plan_partial_sets():
    # the 16-row fp16 kernel keeps one set of per-wavefront partials when a
    # workgroup owns one block (two otherwise), which leaves room to stage
    # denser blocks
    for N, dens in [(32, 0.6), (32, 0.75), (16, 0.95), (12, 1.0)]:
        kv = _kv(bsp.describe(bsp.FP16, 4096, 4096, N, int(4096 * 4096 * dens)))
        assert int(kv["stage_kb"]) > 0 and int(kv["lds"]) <= 160 * 1024, (N, dens, kv)
    # two blocks per workgroup: two sets, two buffers
    kv = _kv(bsp.describe(bsp.FP16, 5000, 4096, 20, int(5000 * 4096 * 0.2)))
    assert kv["stage_bufs"] == "2" and int(kv["lds"]) == 128 + 2048 + 2 * 16 * 2 * 1024 + 2 * 1024 * int(kv["stage_kb"])
    kv = _kv(bsp.describe(bsp.FP16, 4096, 4096, 32, int(4096 * 4096 * 0.4)))
    assert int(kv["lds"]) == 128 + 2048 + 16 * 2 * 1024 + 1024 * int(kv["stage_kb"]), kv


def test_wide_n_past_k8192_takes_split_k():
    # two column blocks at 8 tiles per lane exceed the ring kernel's
    # registers: N > 16 past K = 8192 goes to split-K (two K ranges with a
    # workspace); 4 tiles per lane keeps the ring kernel
    for N in (17, 24, 32):
        assert "-> splitk kernel=k_bsk_w4a4 " in bsp.describe(bsp.INT4, 4096, 11008, N, 4096 * 11008 * 3 // 10)
        d = bsp.describe(bsp.INT4, 4096, 11008, N, 4096 * 11008 * 3 // 10, workspace=True)
        assert "-> splitk kernel=k_bsks_w4a4 " in d and "splits=2 " in d, d
    assert "-> mfma kernel=k_bt64_w4a4 " in bsp.describe(bsp.INT4, 4096, 11008, 16, 4096 * 11008 * 3 // 10)
    assert "-> mfma kernel=k_bt64_w4a4 " in bsp.describe(bsp.INT4, 8192, 8192, 32, 8192 * 8192 * 7 // 10)
    # forced, the ring kernel still runs the shape
    d = bsp.describe(bsp.INT4, 4096, 11008, 32, 4096 * 11008 * 3 // 10, algo=bsp.ALGO_MFMA)
    assert "kernel=k_bt64_w4a4 " in d and "tiles_per_lane=8" in d, d


def test_f16_split_plans_share_cus_past_256_workgroups():
    # fp16 split-K past 256 workgroups: shorter chunks so that the workgroups
    # share the CUs instead of running in rounds of one per CU
    for M, K, maxlds, block in [(5120, 5120, 80, 512), (13824, 5120, 40, 256), (8192, 8192, 80, 512)]:
        kv = _kv(bsp.describe(bsp.FP16, M, K, 1, int(M * K * 0.4)))
        assert int(kv["lds"]) <= maxlds * 1024 and kv["block"] == str(block), (M, K, kv)
    kv = _kv(bsp.describe(bsp.FP16, 4096, 11008, 1, int(4096 * 11008 * 0.4)))
    assert kv["grid"] == "256" and kv["block"] == "1024", kv


def test_f16_eight_row_plans_take_up_to_eight_steps():
    # up to 8 steps per workgroup on one workgroup per CU (no rounds) when
    # the LDS holds them; 4-step rounds otherwise
    for M, slots, grid in [(4096, 2, 256), (8192, 4, 256), (8200, 8, 256), (11008, 8, 256), (12288, 8, 256),
                           (16384, 4, 512)]:
        kv = _kv(bsp.describe(bsp.FP16, M, 4096, 1, int(M * 4096 * 0.4)))
        assert kv["step_slots"] == str(slots) and kv["grid"] == str(grid), (M, kv)
        assert int(kv["lds"]) <= 160 * 1024
        assert kv["partial_ring"] == "0", (M, kv)
    # 8 steps with every step's partials would not fit: the partials in a
    # ring of two slots, where a workgroup has 5 to 7 steps
    kv = _kv(bsp.describe(bsp.FP16, 11008, 4096, 1, int(11008 * 4096 * 0.5)))
    assert kv["step_slots"] == "8" and kv["partial_ring"] == "1" and kv["grid"] == "256", kv
    kv = _kv(bsp.describe(bsp.FP16, 16384, 4096, 1, int(16384 * 4096 * 0.5)))   # 8 steps each: rounds of 4
    assert kv["step_slots"] == "4" and kv["grid"] == "512", kv


def test_ring_plans_take_eight_blocks_at_two_tiles_per_lane():
    # K <= 4096 past 1024 blocks: up to 8 blocks per workgroup on 256
    # workgroups instead of rounds of 4
    for M, grid in [(16384, 256), (16400, 256), (20000, 256), (32768, 256), (33000, 516)]:
        kv = _kv(bsp.describe(bsp.INT4, M, 4096, 8, M * 2048))
        assert "kernel=k_bt64_w4a4 " in bsp.describe(bsp.INT4, M, 4096, 8, M * 2048)
        assert kv["grid"] == str(grid) and int(kv["lds"]) <= 160 * 1024, (M, kv)


def test_ring_plans_take_four_blocks_at_four_tiles_per_lane():
    # 4096 < K <= 8192, N <= 16, past 512 blocks: up to 4 blocks per workgroup
    # on 256 workgroups; two column blocks keep 2 (4 would spill)
    for M, K, N, grid in [(8200, 8192, 8, 256), (10240, 8192, 8, 256), (13824, 5120, 16, 256), (10240, 8192, 32, 320),
                          (16400, 8192, 8, 513)]:
        kv = _kv(bsp.describe(bsp.INT4, M, K, N, M * K // 2))
        assert kv["tiles_per_lane"] == "4" and kv["grid"] == str(grid) and int(kv["lds"]) <= 160 * 1024, (M, kv)


def test_f16_block_plan_one_set_for_several_blocks():
    # several blocks per workgroup: one set of partials (and a barrier per
    # block) when two sets would leave no room for two staging buffers
    for M, N, dens in [(8192, 16, 0.4), (16384, 16, 0.4), (8192, 32, 0.3), (9000, 10, 0.4)]:
        kv = _kv(bsp.describe(bsp.FP16, M, 4096, N, int(M * 4096 * dens)))
        nb = 1 if N <= 16 else 2
        assert kv["stage_bufs"] == "2", (M, N, kv)
        assert int(kv["lds"]) == 128 + 2048 + 16 * nb * 1024 + 2 * 1024 * int(kv["stage_kb"]), (M, N, kv)
