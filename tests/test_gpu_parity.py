"""GPU parity: every kernel of the library against the CPU oracle.

int4 results must match bit for bit; fp16 results must meet the documented
tolerance (max floored relative error <= 1e-2 against the fp64 reference).
Inputs are the seeded workloads; expected values come only from ``oracle``.
Every call goes through the C ABI (``libbitmap_spmm.so``) via the binding.
A call that forces the MFMA kernels first checks, from the library's own
launch plan, which kernel runs; a shape outside them must be refused with
BSP_E_UNSUPPORTED (a forced kernel never falls back to another one).
"""
import functools
import re

import numpy as np
import pytest

import bit_unstructured_sparse_amd as bsp
import oracle
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

INT4_ALGOS = [bsp.ALGO_AUTO, bsp.ALGO_ROWWAVE, bsp.ALGO_MFMA]
F16_ALGOS = [bsp.ALGO_AUTO, bsp.ALGO_ROWWAVE, bsp.ALGO_MFMA]
_NAMES = {bsp.ALGO_AUTO: "auto", bsp.ALGO_ROWWAVE: "rowwave", bsp.ALGO_MFMA: "mfma"}
SENTINEL = -0x21524111   # 0xDEADBEEF as int32
F16_TOL = 1e-2
MFMA_KERNELS = {bsp.INT4: ("k_bt64s_w4a4", "k_bt64_w4a4"), bsp.FP16: ("k_bt8_f16", "k_bt64_f16")}


def int4_kernel_for(K, N):
    """The int4 MFMA kernel the plan picks for the small shapes below (at
    most three 16-row blocks per workgroup): the streaming kernel up to
    K = 4096, the ring kernel past it."""
    return "k_bt64s_w4a4" if K <= 4096 else "k_bt64_w4a4"


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def mfma_kernel(dtype, M, K, N, nnz):
    """The MFMA kernel a forced-MFMA call launches, from the library's plan
    for that choice, or None for a shape outside the MFMA path."""
    try:
        d = bsp.describe(dtype, M, K, N, nnz, algo=bsp.ALGO_MFMA)
    except bsp.BspError as e:
        assert e.status == bsp.E_UNSUPPORTED, e
        return None
    k = re.search(r"kernel=(\w+)", d).group(1)
    assert k in MFMA_KERNELS[dtype], d
    return k


def _y_with_canary(N, M, dtype, dev):
    """Output buffer followed by 256 sentinel elements (out-of-bounds write check)."""
    big = torch.full((N * M + 256,), SENTINEL if dtype == torch.int32 else -1, dtype=torch.int32, device=dev)
    if dtype == torch.int32:
        return big, big[: N * M].view(N, M)
    raw = big.view(torch.int16)
    return raw, raw[: N * M].view(torch.float16).view(N, M)


def _canary_ok(big, N, M, dtype):
    if dtype == torch.int32:
        return bool((big[N * M:] == SENTINEL).all().item())
    return bool((big[N * M:] == -1).all().item())


def run_w4a4(W_int8, X_int8, algo, dev, enc=None, expect_kernel=None):
    """Y from the library, or None when a forced MFMA call is refused as
    unsupported (which is then asserted). expect_kernel: the MFMA kernel the
    caller intends to exercise (asserted when forcing MFMA)."""
    enc = enc or bsp.encode(W_int8)
    N = X_int8.shape[0]
    k = None
    if algo == bsp.ALGO_MFMA and N > 0 and enc.M > 0:
        k = mfma_kernel(bsp.INT4, enc.M, enc.K, N, enc.nnz)
        if expect_kernel is not None:
            assert k == expect_kernel, (k, expect_kernel)
    dm = enc.to_device(dev)
    Xd = torch.from_numpy(bsp.pack_int4(X_int8)).to(dev)
    big, Y = _y_with_canary(N, enc.M, torch.int32, dev)
    if algo == bsp.ALGO_MFMA and N > 0 and enc.M > 0 and k is None:
        with pytest.raises(bsp.BspError) as ei:
            bsp.spmm_w4a4(dm, Xd, N, Y=Y, algo=algo)
        assert ei.value.status == bsp.E_UNSUPPORTED
        torch.cuda.synchronize()
        assert bool((big == SENTINEL).all()), "a refused call wrote Y"
        return None
    bsp.spmm_w4a4(dm, Xd, N, Y=Y, algo=algo)
    torch.cuda.synchronize()
    assert _canary_ok(big, N, enc.M, torch.int32), "write past the end of Y"
    return Y.cpu().numpy()


def run_f16(W_f16, X_f16, algo, dev, enc=None, expect_kernel=None):
    enc = enc or bsp.encode(W_f16)
    N = X_f16.shape[0]
    k = None
    if algo == bsp.ALGO_MFMA:
        k = mfma_kernel(bsp.FP16, enc.M, enc.K, N, enc.nnz)
        if expect_kernel is not None:
            assert k == expect_kernel, (k, expect_kernel)
    dm = enc.to_device(dev)
    Xd = torch.from_numpy(np.ascontiguousarray(X_f16)).to(dev)
    big, Y = _y_with_canary(N, enc.M, torch.float16, dev)
    if algo == bsp.ALGO_MFMA and k is None:
        with pytest.raises(bsp.BspError) as ei:
            bsp.spmm_f16(dm, Xd, Y=Y, algo=algo)
        assert ei.value.status == bsp.E_UNSUPPORTED
        return None
    bsp.spmm_f16(dm, Xd, Y=Y, algo=algo)
    torch.cuda.synchronize()
    assert _canary_ok(big.view(torch.int16), N, enc.M, torch.float16), "write past the end of Y"
    return Y.cpu().numpy()


def assert_w4a4(Y, W, X, ref=None):
    """Bit-exact against the oracle (nothing to compare for a refused call)."""
    if Y is None:
        return
    assert np.array_equal(Y, oracle_w4a4(W, X) if ref is None else ref)


def oracle_w4a4(W, X):
    s = oracle.encode(W)
    return oracle.spmm_w4a4(s, _pack_for_oracle(X), X.shape[0], threads=16)   # rows over 16 threads: the same result


def _pack_for_oracle(X):
    # the oracle consumes the packed layout; pack with the test-side packer that the
    # golden layout file pins (tests/pins.py), independent of the library's packer
    import pins
    return pins._pack_x_for_test(X)


SMALL_INT4 = [  # (M, K, N, keep)
    (1, 1, 1, 1.0), (1, 64, 1, 0.5), (3, 63, 2, 0.5), (5, 65, 3, 0.5), (64, 64, 8, 0.5),
    (65, 130, 3, 0.5), (17, 127, 31, 0.5), (257, 1000, 16, 0.3), (129, 64 * 67 + 17, 32, 0.7),
    (300, 64 * 40, 5, 0.5), (97, 4096, 8, 0.5), (1024, 512, 4, 0.5), (33, 777, 7, 1.0),
    (48, 64 * 67 + 24, 20, 0.5), (31, 64 * 33 + 8, 16, 1.0), (16, 64 * 65, 32, 0.5), (250, 64 * 5 + 56, 13, 0.6),
    (40, 64 * 320, 5, 0.5), (17, 64 * 330 + 32, 24, 0.9),   # K beyond the MFMA kernels' 16384: refused there
    (40, 333, 9, 0.0), (2, 2048, 32, 0.05), (512, 64 * 172, 16, 0.3),
    (70, 64 * 256, 8, 0.5), (33, 64 * 255 + 7, 17, 0.5),   # the largest K of the MFMA kernels, and an odd one
]


@pytest.mark.parametrize("algo", INT4_ALGOS, ids=lambda a: _NAMES[a])
@pytest.mark.parametrize("M,K,N,keep", SMALL_INT4)
def test_w4a4_small(dev, algo, M, K, N, keep):
    p = workloads.random_int4_problem(M * 7 + K * 3 + N, M, K, N, keep=keep)
    assert_w4a4(run_w4a4(p.W, p.X, algo, dev), p.W, p.X)


# every weight and activation at -8 or +7: the largest-magnitude products,
# through the x16 int8 form and the >> 8 of the MFMA kernels (K = 64 * 33:
# rows on a 4-byte boundary; K = 2117: odd K, rows off any boundary)
@pytest.mark.parametrize("algo", INT4_ALGOS, ids=lambda a: _NAMES[a])
@pytest.mark.parametrize("K", [64 * 33, 2117, 64 * 256])
def test_w4a4_extremes(dev, algo, K):
    M, N = 70, 32
    W = np.full((M, K), -8, np.int8)
    W[::3, ::5] = 7
    X = np.full((N, K), -8, np.int8)
    X[1::2] = 7
    kern = int4_kernel_for(K, N)
    assert_w4a4(run_w4a4(W, X, algo, dev, expect_kernel=kern if algo == bsp.ALGO_MFMA else None), W, X)


@pytest.mark.parametrize("algo", INT4_ALGOS, ids=lambda a: _NAMES[a])
@pytest.mark.parametrize("dense_block", [0, 3, 9])
def test_w4a4_uneven_block_density(dev, algo, dense_block):
    # One 16-row block at full density among blocks at 2 %: its payload is far
    # larger than the average block the staging area is sized for, so the MFMA
    # kernel must take its global-memory window path for that block only.
    rng = np.random.default_rng(100 + dense_block)
    M, K, N = 160, 64 * 40, 8
    keep = np.full((M, 1), 0.02)
    keep[16 * dense_block:16 * dense_block + 16] = 1.0
    W = workloads._int4_weights(rng, M, K, keep)
    X = workloads.int4_activations(rng, (N, K))
    assert_w4a4(run_w4a4(W, X, algo, dev), W, X)


@pytest.mark.parametrize("algo", INT4_ALGOS, ids=lambda a: _NAMES[a])
@pytest.mark.parametrize("M,K,N", [(4100, 512, 8), (4098, 1024, 3), (8200, 4096, 20), (5000, 64 * 130, 5)])
@pytest.mark.parametrize("y_shift", [0, 1])
def test_w4a4_many_blocks_ragged_y(dev, algo, M, K, N, y_shift):
    # several 16-row blocks per workgroup (the all-blocks-staged path and the
    # ring), M not a multiple of 4 or 16, and Y placed 4 bytes off a 16-byte
    # boundary: the 16-byte stores of Y must fall back to single stores
    p = workloads.random_int4_problem(M + K + N, M, K, N, keep=0.5)
    enc = bsp.encode(p.W)
    if algo == bsp.ALGO_MFMA:
        assert mfma_kernel(bsp.INT4, M, K, N, enc.nnz) is not None
    dm = enc.to_device(dev)
    Xd = torch.from_numpy(bsp.pack_int4(p.X)).to(dev)
    big = torch.full((N * M + 8 + y_shift,), SENTINEL, dtype=torch.int32, device=dev)
    Y = big[y_shift: y_shift + N * M].view(N, M)
    bsp.spmm_w4a4(dm, Xd, N, Y=Y, algo=algo)
    torch.cuda.synchronize()
    assert bool((big[:y_shift] == SENTINEL).all()) and bool((big[y_shift + N * M:] == SENTINEL).all())
    assert np.array_equal(Y.cpu().numpy(), oracle_w4a4(p.W, p.X))


@pytest.mark.parametrize("M,K,N", [(1000, 64 * 100 + 32, 17), (2050, 8192, 32), (300, 11008, 20), (70, 8256, 24),
                                   (200, 16384, 32), (333, 64 * 70 + 32, 3), (301, 64 * 90 + 13, 20),
                                   (77, 64 * 150 + 40, 7)])
def test_w4a4_ring_x_runs(dev, M, K, N):
    # the ring kernel loads X in 64-byte runs of 16 rows and hands each lane
    # its slices by a transpose across lane groups; K % 64 == 32 leaves the
    # last tile half in X, K % 8 != 0 puts X rows off a 4-byte boundary
    # (funnel-shifted loads), and rows n >= N read zeros
    p = workloads.random_int4_problem(M + K + N, M, K, N, keep=0.4)
    assert_w4a4(run_w4a4(p.W, p.X, bsp.ALGO_MFMA, dev, expect_kernel="k_bt64_w4a4"), p.W, p.X)


@pytest.mark.parametrize("algo", INT4_ALGOS, ids=lambda a: _NAMES[a])
@pytest.mark.parametrize("M,K,N,keep,dense_block", [(4100, 2048, 20, 0.5, -1), (3000, 1024, 24, 0.5, -1),
                                                    (2048, 4096, 20, 0.25, -1), (1600, 4096, 17, 0.5, -1),
                                                    (1600, 4096, 17, 0.5, 7), (1600, 4096, 17, 0.5, 99)])
def test_w4a4_staggered_staging(dev, algo, M, K, N, keep, dense_block):
    # the streaming kernel (N > 16) with rows whose payload is close to a
    # multiple of 256 bytes (half density at K = 1024, 2048 and 4096, quarter
    # density at 4096): the plan stages them in staggered runs; one fully
    # dense block (or the last, ragged one) is too large for the staggered
    # area and reads its windows from global memory
    rng = np.random.default_rng(M + K + N + dense_block)
    keep = np.full((M, 1), keep)
    if dense_block >= 0:
        b = min(dense_block, (M - 1) // 16)
        keep[16 * b:16 * b + 16] = 1.0
    W = workloads._int4_weights(rng, M, K, keep)
    X = workloads.int4_activations(rng, (N, K))
    enc = bsp.encode(W)
    if algo == bsp.ALGO_MFMA:
        assert "stagger=1" in bsp.describe(bsp.INT4, M, K, N, enc.nnz)
    assert_w4a4(run_w4a4(W, X, algo, dev, enc=enc, expect_kernel="k_bt64s_w4a4" if algo == bsp.ALGO_MFMA else None),
                W, X)


@pytest.mark.parametrize("algo", INT4_ALGOS, ids=lambda a: _NAMES[a])
@pytest.mark.parametrize("M,K,N,pattern", [(64, 4096, 8, "alternate"), (4100, 4096, 16, "alternate"),
                                           (300, 2048, 5, "every_fifth"), (48, 512, 1, "one_row"),
                                           (16 * 768, 4096, 8, "alternate")])
def test_w4a4_mixed_dense_rows(dev, algo, M, K, N, pattern):
    # nearly dense rows beside sparse ones in the same 16-row blocks: blocks
    # larger than the staging area sized from the average read their windows
    # from global memory, the others from LDS
    rng = np.random.default_rng(M + K + N)
    keep = np.full((M, 1), 0.3)
    if pattern == "alternate":
        keep[::2] = 0.97
    elif pattern == "every_fifth":
        keep[::5] = 1.0
    else:
        keep[7] = 1.0
    W = workloads._int4_weights(rng, M, K, keep)
    X = workloads.int4_activations(rng, (N, K))
    Y = run_w4a4(W, X, algo, dev, expect_kernel="k_bt64s_w4a4" if algo == bsp.ALGO_MFMA else None)
    assert_w4a4(Y, W, X)


@pytest.mark.parametrize("algo", INT4_ALGOS, ids=lambda a: _NAMES[a])
def test_w4a4_k_zero(dev, algo):
    W = np.zeros((9, 0), np.int8)
    X = np.zeros((3, 0), np.int8)
    enc = bsp.encode(W)
    dm = enc.to_device(dev)
    Xd = torch.zeros(0, dtype=torch.uint8, device=dev)
    Y = torch.full((3, 9), SENTINEL, dtype=torch.int32, device=dev)
    if algo == bsp.ALGO_MFMA:
        # K = 0 has no tile to decode: only the plain kernel writes its zeros
        with pytest.raises(bsp.BspError) as ei:
            bsp.spmm_w4a4(dm, Xd, 3, Y=Y, algo=algo)
        assert ei.value.status == bsp.E_UNSUPPORTED
        return
    bsp.spmm_w4a4(dm, Xd, 3, Y=Y, algo=algo)
    torch.cuda.synchronize()
    assert not Y.cpu().numpy().any()


# every N in 1..32 through the MFMA kernels: the streaming kernel at K = 608
# (rows on a 4-byte boundary) and K = 609 (odd), the ring kernel at K = 6432
@pytest.mark.parametrize("algo", INT4_ALGOS, ids=lambda a: _NAMES[a])
@pytest.mark.parametrize("K", [64 * 9 + 32, 64 * 9 + 33, 64 * 100 + 32])
@pytest.mark.parametrize("N", list(range(1, 33)))
def test_w4a4_every_n(dev, algo, K, N):
    if K > 4096 and algo != bsp.ALGO_MFMA:
        pytest.skip("the ring-kernel shape is checked through the forced MFMA path only")
    p = workloads.random_int4_problem(77 + K, 200, K, 32, keep=0.5)
    kern = int4_kernel_for(K, N) if algo == bsp.ALGO_MFMA else None
    Y = run_w4a4(p.W, p.X[:N], algo, dev, expect_kernel=kern)
    assert_w4a4(Y, p.W, p.X[:N])


SMALL_F16 = [(1, 1, 1), (3, 63, 2), (65, 130, 32), (257, 1000, 1), (129, 64 * 67 + 17, 17), (64, 4096, 8),
             (500, 64 * 20, 32), (16, 8, 1), (33, 4088, 16), (48, 4096, 32), (20, 64 * 65, 4),
             (5000, 256, 3),    # several 16-row blocks per workgroup
             (4100, 64, 17)]    # ragged last block, two column blocks


def _assert_f16(y, r):
    if y is None:
        return
    e = oracle.fp16_error(y.astype(np.float64), r)
    assert e["nonfinite"] == 0, e
    assert e["max_rel_floored"] <= F16_TOL, e


@pytest.mark.parametrize("algo", F16_ALGOS, ids=lambda a: _NAMES[a])
@pytest.mark.parametrize("M,K,N", SMALL_F16)
def test_f16_small(dev, algo, M, K, N):
    p = workloads.random_fp16_problem(M + K + N, M, K, N)
    _assert_f16(run_f16(p.W, p.X, algo, dev), oracle.spmm_f16(oracle.encode(p.W), p.X, threads=16))


@pytest.mark.parametrize("algo", F16_ALGOS, ids=lambda a: _NAMES[a])
@pytest.mark.parametrize("dense_block", [0, 5])
def test_f16_uneven_block_density(dev, algo, dense_block):
    # one dense 16-row block among sparse ones: it overflows the staging
    # buffer sized from the average block and takes the global-window path
    rng = np.random.default_rng(11 + dense_block)
    M, K, N = 128, 2048, 8
    W = rng.normal(0, 0.02, size=(M, K)).astype(np.float16)
    keep = rng.random((M, K)) < 0.03
    keep[16 * dense_block: 16 * dense_block + 16] = True
    W = np.where(keep, W, np.float16(0))
    X = rng.normal(0, 1, size=(N, K)).astype(np.float16)
    _assert_f16(run_f16(W, X, algo, dev), oracle.spmm_f16(oracle.encode(W), X))


@pytest.mark.parametrize("algo", F16_ALGOS, ids=lambda a: _NAMES[a])
@pytest.mark.parametrize("M,K,N,dense_rows", [(8003, 1000, 5, -1),   # 4 steps per workgroup: the ring wraps
                                              (4096, 4096, 1, -1), (4099, 4088, 8, -1), (1000, 2048, 7, 3),
                                              (77, 520, 2, 9), (9, 4096, 1, 0), (2048, 64, 6, -1)])
def test_f16_eight_row_steps(dev, algo, M, K, N, dense_rows):
    # N <= 8 and K <= 4096: the kernel that walks rows eight at a time (one
    # step in flight, MFMA rows 8-15 holding the second half of K); ragged M
    # and K, every step count per workgroup up to four, and an optional dense
    # group of 8 rows that overflows its staging area (global-window path)
    rng = np.random.default_rng(M + K + N)
    W = rng.normal(0, 0.02, size=(M, K)).astype(np.float16)
    keep = rng.random((M, K)) < 0.4
    if dense_rows >= 0:
        keep[8 * dense_rows: 8 * dense_rows + 8] = True
    W = np.where(keep, W, np.float16(0))
    X = rng.normal(0, 1, size=(N, K)).astype(np.float16)
    enc = bsp.encode(W)
    y = run_f16(W, X, algo, dev, enc=enc, expect_kernel="k_bt8_f16" if algo == bsp.ALGO_MFMA else None)
    _assert_f16(y, oracle.spmm_f16(oracle.encode(W), X))


@pytest.mark.parametrize("algo", F16_ALGOS, ids=lambda a: _NAMES[a])
def test_f16_zero_and_dense(dev, algo):
    W = np.zeros((33, 100), np.float16)
    X = np.ones((2, 100), np.float16)
    y = run_f16(W, X, algo, dev)
    assert y is None or not y.any()
    p = workloads.random_fp16_problem(3, 40, 256, 4, sparsity=0.0)
    _assert_f16(run_f16(p.W, p.X, algo, dev), oracle.spmm_f16(oracle.encode(p.W), p.X, threads=16))


# --- the named workloads at their full sizes -------------------------------------------------

@functools.lru_cache(maxsize=None)
def _full_int4(config, idx, nmax):
    p = workloads.make(config)[idx]
    X = p.meta.get("X_full", p.X)[:nmax] if nmax else p.X
    s = oracle.encode(p.W)
    return p, X, oracle.spmm_w4a4(s, _pack_for_oracle(X), X.shape[0])


@functools.lru_cache(maxsize=None)
def _full_f16(idx):
    p = workloads.make("fp16")[idx]
    return p, oracle.spmm_f16(oracle.encode(p.W), p.X, threads=16)


FULL_INT4 = [("tiny", 0), ("qkv", 0), ("ffn", 0), ("ffn", 1), ("lowsparse", 0)]


@pytest.mark.parametrize("algo", INT4_ALGOS, ids=lambda a: _NAMES[a])
@pytest.mark.parametrize("config,idx", FULL_INT4)
def test_w4a4_full_workload(dev, algo, config, idx):
    p, X, ref = _full_int4(config, idx, 0)
    assert_w4a4(run_w4a4(p.W, X, algo, dev), p.W, X, ref=ref)


@pytest.mark.parametrize("algo", INT4_ALGOS, ids=lambda a: _NAMES[a])
@pytest.mark.parametrize("N", [1, 2, 4, 8, 16, 32])
def test_w4a4_qkv_n_sweep(dev, algo, N):
    p, X, ref = _full_int4("qkv", 0, 32)
    assert_w4a4(run_w4a4(p.W, X[:N], algo, dev), p.W, X[:N], ref=ref[:N])


@pytest.mark.parametrize("algo", INT4_ALGOS, ids=lambda a: _NAMES[a])
def test_w4a4_lowsparse_n16(dev, algo):
    # the 70 %-dense 8192 x 8192 workload at N = 16 (the N sweep's other point)
    p, X, ref = _full_int4("lowsparse", 0, 32)
    assert_w4a4(run_w4a4(p.W, X[:16], algo, dev), p.W, X[:16], ref=ref[:16])


@pytest.mark.parametrize("algo", F16_ALGOS, ids=lambda a: _NAMES[a])
@pytest.mark.parametrize("idx", [0, 1])
def test_f16_full_workload(dev, algo, idx):
    p, r = _full_f16(idx)
    _assert_f16(run_f16(p.W, p.X, algo, dev), r)


@pytest.mark.parametrize("algo", INT4_ALGOS, ids=lambda a: _NAMES[a])
def test_w4a4_x_off_a_dword_boundary(dev, algo):
    # X one byte into an allocation: the MFMA kernels read X in whole dwords
    # from its start, so such an X runs the plain kernel (automatic choice) or
    # is refused (forced MFMA)
    p = workloads.random_int4_problem(4242, 300, 777, 5, keep=0.5)
    enc = bsp.encode(p.W)
    dm = enc.to_device(dev)
    Xp = bsp.pack_int4(p.X).reshape(-1)
    raw = torch.zeros(Xp.size + 1, dtype=torch.uint8, device=dev)
    raw[1:] = torch.from_numpy(Xp).to(dev)
    Xd = raw[1:]
    Y = torch.full((5, 300), SENTINEL, dtype=torch.int32, device=dev)
    if algo == bsp.ALGO_MFMA:
        with pytest.raises(bsp.BspError) as ei:
            bsp.spmm_w4a4(dm, Xd, 5, Y=Y, algo=algo)
        assert ei.value.status == bsp.E_UNSUPPORTED
        return
    bsp.spmm_w4a4(dm, Xd, 5, Y=Y, algo=algo)
    torch.cuda.synchronize()
    assert np.array_equal(Y.cpu().numpy(), oracle_w4a4(p.W, p.X))


# --- the split-K kernels (K ranges of block sets; partials meet in a workspace) --------------

def _ws(dtype, M, K, N, nnz, dev, extra=0):
    n = bsp.workspace_bytes(dtype, M, K, N, nnz)
    return torch.zeros(max(n, 256) + extra, dtype=torch.uint8, device=dev) if n else None


SPLITK_INT4 = [  # (M, K, N, keep)
    (48, 20000, 5, 0.5),         # K past the MFMA block kernels
    (100, 64 * 300 + 17, 16, 0.3),
    (4100, 11008, 16, 0.3),      # ragged last block, last set of one block
    (33, 8192, 32, 0.7), (257, 64 * 130 + 32, 8, 0.5), (16, 128, 1, 0.5), (70, 300, 17, 0.9),
    (200, 64 * 140, 24, 0.05),
]


@pytest.mark.parametrize("with_ws", [False, True], ids=["plain", "workspace"])
@pytest.mark.parametrize("M,K,N,keep", SPLITK_INT4)
def test_splitk_w4a4(dev, M, K, N, keep, with_ws):
    p = workloads.random_int4_problem(M * 5 + K + N, M, K, N, keep=keep)
    enc = bsp.encode(p.W)
    dm = enc.to_device(dev)
    Xd = torch.from_numpy(bsp.pack_int4(p.X)).to(dev)
    ws = _ws(bsp.INT4, M, K, N, enc.nnz, dev) if with_ws else None
    ref = oracle_w4a4(p.W, p.X)
    for rep in range(2):   # the second call reuses the workspace (its counters were reset)
        big, Y = _y_with_canary(N, M, torch.int32, dev)
        bsp.spmm_w4a4(dm, Xd, N, Y=Y, algo=bsp.ALGO_SPLITK, workspace=ws)
        torch.cuda.synchronize()
        assert _canary_ok(big, N, M, torch.int32), "write past the end of Y"
        assert np.array_equal(Y.cpu().numpy(), ref), f"call {rep}"
    if ws is not None:
        assert not ws[:65536].any(), "arrival counters left nonzero"


LARGE_GRIDS = [  # (M, K, N, keep, rows): int4 plans past 256 workgroups, dense blocks, equal-length rows
    (8192, 16384, 8, 0.5, False),    # one resident workgroup per CU, two rounds
    (5000, 12001, 3, 0.5, False),    # 313 workgroups, ragged last block, X rows off a 4-byte boundary
    (8192, 8192, 8, 0.9, False),     # one block per workgroup
    (65536, 4096, 8, 0.5, False),    # four blocks per workgroup, four rounds
    (16400, 4096, 8, 0.5, False),    # up to 8 blocks per workgroup (2 tiles per lane), 5 buffers refilled
    (22016, 4096, 32, 0.5, False),   # the same with two column blocks
    (20000, 4091, 5, 0.5, True),     # the same, rows of one length, X rows off a 4-byte boundary
    (10240, 8192, 8, 0.5, False),    # up to 4 blocks per workgroup (4 tiles per lane), 3 buffers refilled
    (11008, 5121, 16, 0.5, True),    # the same, one pass, rows of one length, X off a 4-byte boundary
    (4096, 16384, 8, 0.9, False),    # too dense to stage: split-K (auto), global windows (forced)
    (4096, 16384, 8, 0.5, True),     # every row 4096 B long
    (12288, 4096, 8, 0.5, True),     # every row 1024 B long: staggered streaming
]


@functools.lru_cache(maxsize=2)
def _large_case(M, K, N, keep, rows):
    p = workloads.random_int4_problem(M + K + N, M, K, N, keep=keep, rows=rows)
    return p, oracle_w4a4(p.W, p.X)


@pytest.mark.parametrize("algo", [bsp.ALGO_AUTO, bsp.ALGO_MFMA], ids=["auto", "mfma"])
@pytest.mark.parametrize("M,K,N,keep,rows", LARGE_GRIDS)
def test_w4a4_large_grids_and_equal_rows(dev, M, K, N, keep, rows, algo):
    p, ref = _large_case(M, K, N, keep, rows)
    assert_w4a4(run_w4a4(p.W, p.X, algo, dev), p.W, p.X, ref=ref)


@pytest.mark.parametrize("algo", F16_ALGOS, ids=lambda a: _NAMES[a])
@pytest.mark.parametrize("N", [1, 8, 32])
def test_f16_equal_rows(dev, algo, N):
    # every row pruned to the same count (rows 4096 B long)
    p = workloads.random_fp16_problem(77 + N, 4096, 4096, N, sparsity=0.5, rows=True)
    _assert_f16(run_f16(p.W, p.X, algo, dev), oracle.spmm_f16(oracle.encode(p.W), p.X, threads=16))


EQUAL_ROWS = [  # (M, K, N, keep): every row keeps the same count; staggered staging
    (4096, 11008, 16, 0.5),    # ring, 8 tiles per lane
    (5120, 5120, 8, 0.5),      # ring, 4 tiles per lane, one pass
    (1000, 11008, 32, 0.5),    # ring, two column blocks, ragged last block
    (13824, 5120, 8, 0.5),     # ring, 432 workgroups in rounds
    (2000, 8193, 5, 0.5),      # ring, X rows off a 4-byte boundary
    (8192, 8192, 8, 0.72),     # ring, two buffers per workgroup, refilled
    (40000, 4096, 8, 0.25),    # ring, 2 tiles per lane, four blocks per workgroup, one pass
    (20000, 4096, 8, 0.25),    # ring, 2 tiles per lane, three buffers for four blocks
    (12288, 4096, 8, 1.0),     # ring, every row dense: staggered, buffers refilled instead of one pass
    (12288, 4096, 8, 0.5625),  # streaming kernel, rows of 1152 B
    (3000, 4096, 17, 0.5),     # streaming kernel, two column blocks
]


@pytest.mark.parametrize("algo", [bsp.ALGO_AUTO, bsp.ALGO_MFMA], ids=["auto", "mfma"])
@pytest.mark.parametrize("M,K,N,keep", EQUAL_ROWS)
def test_w4a4_staggered_equal_rows(dev, M, K, N, keep, algo):
    p, ref = _large_case(M, K, N, keep, True)
    enc = bsp.encode(p.W)
    d = bsp.describe(bsp.INT4, M, K, N, enc.nnz, algo=bsp.ALGO_MFMA)
    assert "stagger=1" in d, d
    assert_w4a4(run_w4a4(p.W, p.X, algo, dev, enc=enc), p.W, p.X, ref=ref)


F16_STAGED = [  # (M, K, N, density): the 16-row fp16 kernel staging dense blocks
    (4096, 4096, 32, 0.75),   # one set of partials, two column blocks
    (4096, 4096, 16, 1.0),    # every block dense
    (4096, 4096, 12, 0.95),
    (1000, 4096, 32, 0.75),   # ragged last block
    (5000, 4096, 20, 0.2),    # two blocks per workgroup: two sets, two buffers
    (8192, 4096, 16, 0.4),    # two blocks per workgroup, one set (a barrier before each block's partials)
    (16384, 4096, 16, 0.4),   # four blocks per workgroup, one set, two buffers refilled
    (8192, 4096, 32, 0.3),    # the same with two column blocks
    (9000, 4096, 10, 0.4),    # two or three blocks per workgroup, ragged last block
]


@pytest.mark.parametrize("algo", [bsp.ALGO_AUTO, bsp.ALGO_MFMA], ids=["auto", "mfma"])
@pytest.mark.parametrize("M,K,N,dens", F16_STAGED)
def test_f16_block_staging(dev, M, K, N, dens, algo):
    p = workloads.random_fp16_problem(M + K + N, M, K, N, sparsity=1.0 - dens)
    enc = bsp.encode(p.W)
    d = bsp.describe(bsp.FP16, M, K, N, enc.nnz, algo=bsp.ALGO_MFMA)
    assert "kernel=k_bt64_f16 " in d and "stage_kb=0 " not in d, d
    _assert_f16(run_f16(p.W, p.X, algo, dev, enc=enc), oracle.spmm_f16(oracle.encode(p.W), p.X, threads=16))


@pytest.mark.parametrize("with_ws", [False, True], ids=["plain", "workspace"])
@pytest.mark.parametrize("M,K,N", [(2000, 11008, 32), (1000, 16384, 17), (300, 9000, 24)])
def test_w4a4_wide_n_past_k8192_auto(dev, M, K, N, with_ws):
    # N > 16 at 8 tiles per lane: the automatic plan is split-K
    p, ref = _large_case(M, K, N, 0.3, False)
    enc = bsp.encode(p.W)
    d = bsp.describe(bsp.INT4, M, K, N, enc.nnz, workspace=with_ws)
    assert "-> splitk " in d, d
    dm = enc.to_device(dev)
    Xd = torch.from_numpy(bsp.pack_int4(p.X)).to(dev)
    ws = _ws(bsp.INT4, M, K, N, enc.nnz, dev) if with_ws else None
    big, Y = _y_with_canary(N, M, torch.int32, dev)
    bsp.spmm_w4a4(dm, Xd, N, Y=Y, workspace=ws)
    torch.cuda.synchronize()
    assert _canary_ok(big, N, M, torch.int32), "write past the end of Y"
    assert np.array_equal(Y.cpu().numpy(), ref), d
    if with_ws:
        assert not ws[:65536].any(), "arrival counters left nonzero"


@pytest.mark.parametrize("M,K,N", [(5120, 5120, 1), (13824, 5120, 3), (8200, 8192, 8), (4500, 6000, 17)])
def test_splitk_f16_shared_cus(dev, M, K, N):
    # fp16 split-K past 256 workgroups, two to four sharing a CU (shorter chunks)
    p = workloads.random_fp16_problem(M + K + N, M, K, N, sparsity=0.6)
    enc = bsp.encode(p.W)
    d = bsp.describe(bsp.FP16, M, K, N, enc.nnz)
    assert "-> splitk kernel=k_bsk_f16 " in d and "block=1024" not in d, d
    _assert_f16(run_f16(p.W, p.X, bsp.ALGO_AUTO, dev, enc=enc), oracle.spmm_f16(oracle.encode(p.W), p.X, threads=16))


@pytest.mark.parametrize("algo", [bsp.ALGO_AUTO, bsp.ALGO_MFMA], ids=["auto", "mfma"])
@pytest.mark.parametrize("M,N,dens,ring", [(8200, 1, 0.4, 0), (11008, 8, 0.4, 0), (12288, 3, 0.4, 0),
                                           (11008, 8, 0.5, 1), (9000, 1, 0.5, 1), (12288, 5, 0.5, 1)])
def test_f16_eight_row_eight_steps(dev, M, N, dens, ring, algo):
    # the eight-row fp16 kernel with up to 8 steps per workgroup (8200 rows:
    # one workgroup of 5 steps, the rest 4), every step's partials kept or
    # in a ring of two slots
    p = workloads.random_fp16_problem(M + N, M, 4096, N, sparsity=1.0 - dens)
    enc = bsp.encode(p.W)
    d = bsp.describe(bsp.FP16, M, 4096, N, enc.nnz)
    assert "kernel=k_bt8_f16 " in d and "step_slots=8" in d and f"partial_ring={ring}" in d, d
    _assert_f16(run_f16(p.W, p.X, algo, dev, enc=enc), oracle.spmm_f16(oracle.encode(p.W), p.X, threads=16))


SPLITK_STREAMED = [  # (M, K, N, keep): the streamed split-K kernel (one pass per block and K range)
    (100, 64 * 65, 3, 0.5),      # two tiles per lane, ragged last block
    (513, 6000, 17, 0.5),        # two column blocks, ragged last tile
    (2000, 12287, 32, 0.3),      # three tiles per lane, X rows off a 4-byte boundary, 250 workgroups
    (48, 8200, 1, 0.95),         # 2 KB slots
    (4096, 8192, 8, 0.5),        # two blocks per set, 256 workgroups
    (16, 64 * 65 + 4, 1, 0.5),   # one block
    (4100, 11008, 16, 0.3),      # three blocks per set, the last set of two, the last block of 4 rows
]


@pytest.mark.parametrize("M,K,N,keep", SPLITK_STREAMED)
def test_splitk_streamed_w4a4(dev, M, K, N, keep):
    p = workloads.random_int4_problem(M * 7 + K + N, M, K, N, keep=keep)
    enc = bsp.encode(p.W)
    d = bsp.describe(bsp.INT4, M, K, N, enc.nnz, workspace=True, algo=bsp.ALGO_SPLITK)
    assert "kernel=k_bsks_w4a4" in d, d
    dm = enc.to_device(dev)
    Xd = torch.from_numpy(bsp.pack_int4(p.X)).to(dev)
    ws = _ws(bsp.INT4, M, K, N, enc.nnz, dev)
    ref = oracle_w4a4(p.W, p.X)
    for rep in range(2):   # the second call reuses the workspace (its counters were reset)
        big, Y = _y_with_canary(N, M, torch.int32, dev)
        bsp.spmm_w4a4(dm, Xd, N, Y=Y, algo=bsp.ALGO_SPLITK, workspace=ws)
        torch.cuda.synchronize()
        assert _canary_ok(big, N, M, torch.int32), "write past the end of Y"
        assert np.array_equal(Y.cpu().numpy(), ref), f"call {rep}: {d}"
    assert not ws[:65536].any(), "arrival counters left nonzero"


SPLITK_F16 = [(4096, 11008, 8), (100, 5000, 1), (257, 64 * 130 + 8, 16), (33, 8192, 32), (64, 4096, 32),
              (4100, 4096, 17), (17, 64 * 65, 3)]


@pytest.mark.parametrize("with_ws", [False, True], ids=["plain", "workspace"])
@pytest.mark.parametrize("M,K,N", SPLITK_F16)
def test_splitk_f16(dev, M, K, N, with_ws):
    p = workloads.random_fp16_problem(M + 3 * K + N, M, K, N)
    enc = bsp.encode(p.W)
    dm = enc.to_device(dev)
    Xd = torch.from_numpy(p.X).to(dev)
    ws = _ws(bsp.FP16, M, K, N, enc.nnz, dev) if with_ws else None
    r = oracle.spmm_f16(oracle.encode(p.W), p.X, threads=16)
    first = None
    for rep in range(2):
        big, Y = _y_with_canary(N, M, torch.float16, dev)
        bsp.spmm_f16(dm, Xd, Y=Y, algo=bsp.ALGO_SPLITK, workspace=ws)
        torch.cuda.synchronize()
        assert _canary_ok(big.view(torch.int16), N, M, torch.float16), "write past the end of Y"
        y = Y.cpu().numpy()
        _assert_f16(y, r)
        if first is None:
            first = y.view(np.uint16).copy()
        else:   # partials are added in a fixed order: the same bits every call
            assert np.array_equal(first, y.view(np.uint16))


@pytest.mark.parametrize("dtype", ["int4", "fp16"])
def test_splitk_dense_block_global_windows(dev, dtype):
    # one fully dense 16-row block among sparse ones: its segments exceed the
    # slots sized from the average, and that block reads its windows from
    # global memory (with and without a workspace)
    rng = np.random.default_rng(7)
    M, K, N = 96, 64 * 150, 8
    keep = np.full((M, 1), 0.05)
    keep[32:48] = 1.0
    for with_ws in (False, True):
        if dtype == "int4":
            W = workloads._int4_weights(rng, M, K, keep)
            X = workloads.int4_activations(rng, (N, K))
            enc = bsp.encode(W)
            ws = _ws(bsp.INT4, M, K, N, enc.nnz, dev) if with_ws else None
            Y = bsp.spmm_w4a4(enc.to_device(dev), torch.from_numpy(bsp.pack_int4(X)).to(dev), N,
                              algo=bsp.ALGO_SPLITK, workspace=ws)
            torch.cuda.synchronize()
            assert np.array_equal(Y.cpu().numpy(), oracle_w4a4(W, X))
        else:
            W = np.where(rng.random((M, K)) < keep, rng.normal(0, 0.02, (M, K)), 0).astype(np.float16)
            X = rng.normal(0, 1, (N, K)).astype(np.float16)
            enc = bsp.encode(W)
            ws = _ws(bsp.FP16, M, K, N, enc.nnz, dev) if with_ws else None
            Y = bsp.spmm_f16(enc.to_device(dev), torch.from_numpy(X).to(dev), algo=bsp.ALGO_SPLITK, workspace=ws)
            torch.cuda.synchronize()
            _assert_f16(Y.cpu().numpy(), oracle.spmm_f16(oracle.encode(W), X))


@pytest.mark.parametrize("config,idx,N", [("ffn", 1, 16), ("lowsparse", 0, 32)])
def test_splitk_full_workloads_forced_with_workspace(dev, config, idx, N):
    # the split-K kernel with 2 K ranges per 2-block set on the named workloads
    p, X, ref = _full_int4(config, idx, 32 if config == "lowsparse" else 0)
    X = X[:N]
    enc = bsp.encode(p.W)
    ws = _ws(bsp.INT4, p.M, p.K, N, enc.nnz, dev)
    Y = bsp.spmm_w4a4(enc.to_device(dev), torch.from_numpy(bsp.pack_int4(X)).to(dev), N, algo=bsp.ALGO_SPLITK,
                      workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(Y.cpu().numpy(), ref[:N])


def test_splitk_f16_full_workload_n32_with_workspace(dev):
    p, r = _full_f16(1)
    enc = bsp.encode(p.W)
    ws = _ws(bsp.FP16, p.M, p.K, p.N, enc.nnz, dev)
    Y = bsp.spmm_f16(enc.to_device(dev), torch.from_numpy(p.X).to(dev), algo=bsp.ALGO_SPLITK, workspace=ws)
    torch.cuda.synchronize()
    _assert_f16(Y.cpu().numpy(), r)


@pytest.mark.parametrize("M,K,N", [(4096, 11008, 8), (300, 64 * 100, 1)])
def test_f16_past_k4096_auto(dev, M, K, N):
    # fp16 past K = 4096: the automatic plan is the split-K kernel (2 K ranges
    # with a workspace, 1 without), never the plain kernel
    p = workloads.random_fp16_problem(M + K + N, M, K, N)
    enc = bsp.encode(p.W)
    r = oracle.spmm_f16(oracle.encode(p.W), p.X, threads=16)
    for ws in (None, _ws(bsp.FP16, M, K, N, enc.nnz, dev)):
        d = bsp.describe(bsp.FP16, M, K, N, enc.nnz, workspace=ws is not None)
        assert "-> splitk kernel=k_bsk_f16" in d and ("splits=2 " in d) == (ws is not None), d
        Y = bsp.spmm_f16(enc.to_device(dev), torch.from_numpy(p.X).to(dev), workspace=ws)
        torch.cuda.synchronize()
        _assert_f16(Y.cpu().numpy(), r)


@pytest.mark.parametrize("M,K,N,split_with_ws", [(300, 24576 + 40, 8, 2), (130, 20480, 5, 1), (64, 32768, 32, 2)])
def test_w4a4_past_k16384_auto(dev, M, K, N, split_with_ws):
    # int4 past K = 16384: the automatic plan is the split-K kernel, with 2 K
    # ranges past K = 20480 when given a workspace, 1 otherwise; bit-exact
    p = workloads.random_int4_problem(M + K + N, M, K, N, keep=0.5)
    enc = bsp.encode(p.W)
    ref = oracle_w4a4(p.W, p.X)
    for ws in (None, _ws(bsp.INT4, M, K, N, enc.nnz, dev)):
        d = bsp.describe(bsp.INT4, M, K, N, enc.nnz, workspace=ws is not None)
        want = split_with_ws if ws is not None else 1
        assert "-> splitk kernel=k_bsk_w4a4" in d and f"splits={want} " in d, d
        big, Y = _y_with_canary(N, M, torch.int32, dev)
        bsp.spmm_w4a4(enc.to_device(dev), torch.from_numpy(bsp.pack_int4(p.X)).to(dev), N, Y=Y, workspace=ws)
        torch.cuda.synchronize()
        assert _canary_ok(big, N, M, torch.int32), "write past the end of Y"
        assert np.array_equal(Y.cpu().numpy(), ref), d


@pytest.mark.parametrize("dtype", ["int4", "fp16"])
def test_splitk_workspace_reused_across_shapes(dev, dtype):
    # one caller workspace for a large problem, then a smaller one, then the
    # large one again: the smaller call's partials must not land on counters
    # the larger plan uses (the counter area has a fixed size)
    shapes = [(4096, 11008, 8), (1000, 64 * 100, 3), (4096, 11008, 8)]
    need = max(bsp.workspace_bytes(bsp.INT4 if dtype == "int4" else bsp.FP16, M, K, N) for M, K, N in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    for i, (M, K, N) in enumerate(shapes):
        if dtype == "int4":
            p = workloads.random_int4_problem(60 + i, M, K, N, keep=0.5)
            enc = bsp.encode(p.W)
            Y = bsp.spmm_w4a4(enc.to_device(dev), torch.from_numpy(bsp.pack_int4(p.X)).to(dev), N,
                              algo=bsp.ALGO_SPLITK, workspace=ws)
            torch.cuda.synchronize()
            assert np.array_equal(Y.cpu().numpy(), oracle_w4a4(p.W, p.X)), f"call {i}"
        else:
            p = workloads.random_fp16_problem(60 + i, M, K, N)
            enc = bsp.encode(p.W)
            Y = bsp.spmm_f16(enc.to_device(dev), torch.from_numpy(p.X).to(dev), algo=bsp.ALGO_SPLITK, workspace=ws)
            torch.cuda.synchronize()
            _assert_f16(Y.cpu().numpy(), oracle.spmm_f16(oracle.encode(p.W), p.X, threads=16))
    assert not ws[:65536].any()
