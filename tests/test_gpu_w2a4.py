"""GPU parity of the W2A4 SpMM (2-bit weights in the bitmap-tiled format,
int4 activations, int32 Y) against the W2A4 oracle, bit for bit, through the
C ABI. Both kernels (the streaming MFMA kernel and the plain one) on every
shape they take; the automatic choice past the streaming kernel's K."""
import numpy as np
import pytest

import bit_unstructured_sparse_amd as bsp
import workloads
from oracle import w2

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
SENTINEL = -0x21524111


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def run(W, X, algo, dev):
    enc = bsp.encode(W, dtype=bsp.INT2)
    N = X.shape[0]
    dm = enc.to_device(dev)
    Xd = torch.from_numpy(bsp.pack_int4(X)).to(dev)
    big = torch.full((N * enc.M + 256,), SENTINEL, dtype=torch.int32, device=dev)
    Y = big[:N * enc.M].view(N, enc.M)
    bsp.spmm_w2a4(dm, Xd, N, Y=Y, algo=algo)
    torch.cuda.synchronize()
    assert bool((big[N * enc.M:] == SENTINEL).all()), "write past the end of Y"
    return Y.cpu().numpy()


def ref(W, X):
    return w2.spmm_w2a4(w2.decode(w2.encode(W)) if W.size <= 200000 else W, X)


SHAPES = [  # (M, K, N, keep)
    (16, 64, 1, 0.5), (1, 1, 1, 1.0), (37, 150, 5, 0.3), (33, 129, 17, 0.7), (100, 1000, 32, 0.5),
    (64, 4096, 8, 0.5), (48, 4091, 16, 0.6), (20, 70, 4, 0.0), (130, 520, 9, 0.05), (256, 2048, 32, 1.0),
    (40, 4032, 3, 0.95),
]


@pytest.mark.parametrize("M,K,N,keep", SHAPES)
@pytest.mark.parametrize("algo", [bsp.ALGO_AUTO, bsp.ALGO_MFMA, bsp.ALGO_ROWWAVE])
def test_w2a4_small(M, K, N, keep, algo, dev):
    p = workloads.random_int2_problem(M * 977 + K * 3 + N, M, K, N, keep=keep)
    Y = run(p.W, p.X, algo, dev)
    assert np.array_equal(Y, ref(p.W, p.X))


def test_w2a4_extremes(dev):
    for K in (64, 4096):
        W = np.full((48, K), -2, np.int8)
        X = np.full((5, K), -8, np.int8)
        assert (run(W, X, bsp.ALGO_MFMA, dev) == 16 * K).all()


def test_w2a4_past_mfma_kernels(dev):
    # past K = 16384 only the plain kernel runs W2A4; a forced MFMA call is refused
    p = workloads.random_int2_problem(3, 40, 16400, 4, keep=0.4)
    assert np.array_equal(run(p.W, p.X, bsp.ALGO_AUTO, dev), ref(p.W, p.X))
    enc = bsp.encode(p.W, dtype=bsp.INT2)
    with pytest.raises(bsp.BspError) as ei:
        bsp.spmm_w2a4(enc.to_device(dev), torch.from_numpy(bsp.pack_int4(p.X)).to(dev), 4, algo=bsp.ALGO_MFMA)
    assert ei.value.status == bsp.E_UNSUPPORTED


RING = [  # (M, K, N, keep): past the streaming kernel, the ring kernel with 2-bit values
    (40, 8192, 4, 0.4),       # 4 tiles per lane
    (300, 11008, 16, 0.3),    # 8 tiles per lane
    (100, 5000, 32, 0.5),     # two column blocks, ragged last tile
    (50, 6001, 5, 0.5),       # X rows off a 4-byte boundary
    (70, 16384, 17, 0.95),    # two column blocks at 8 tiles per lane, near dense
    (20000, 4096, 8, 0.5),    # more than three blocks per workgroup: the ring at 2 tiles per lane
]


@pytest.mark.parametrize("M,K,N,keep", RING)
@pytest.mark.parametrize("algo", [bsp.ALGO_AUTO, bsp.ALGO_MFMA])
def test_w2a4_ring_kernel(M, K, N, keep, algo, dev):
    p = workloads.random_int2_problem(M * 31 + K + N, M, K, N, keep=keep)
    d = bsp.describe(bsp.INT2, M, K, N, int(np.count_nonzero(p.W)), algo=bsp.ALGO_MFMA)
    assert "kernel=k_bt64_w4a4 " in d, d
    assert np.array_equal(run(p.W, p.X, algo, dev), ref(p.W, p.X))


def test_w2a4_ring_extremes(dev):
    for K in (4160, 8192, 16384):
        W = np.full((48, K), -2, np.int8)
        X = np.full((5, K), -8, np.int8)
        assert (run(W, X, bsp.ALGO_MFMA, dev) == 16 * K).all()


@pytest.mark.parametrize("config,index,N", [("qkv", 0, 8), ("qkv", 0, 32), ("qkv", 0, 1), ("ffn", 0, 16), ("ffn", 1, 16),
                                            ("lowsparse", 0, 32)])
def test_w2a4_full_workloads(config, index, N, dev):
    p = workloads.make(config)[index]
    X = p.meta.get("X_full", p.X)[:N]
    W = workloads.int2_like(p.W, seed=N)
    assert np.array_equal(run(W, X, bsp.ALGO_AUTO, dev), w2.spmm_w2a4(W, X))
