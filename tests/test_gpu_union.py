"""GPU parity of the union-mask (IE-BME, 2 x 2 areas of 16 x 64 tiles) SpMM
against the oracle, bit for bit. Small shapes compare the full Y with the
IE-BME oracle's own decode times X; the full workloads compare the full Y
with the C oracle's product (the same plain definition, threaded). The
encodings come from the library encoder, which the CPU suite checks byte for
byte against the oracle's; calls go through the C ABI via the binding."""
import numpy as np
import pytest

import bit_unstructured_sparse_amd as bsp
import oracle
import pins
import workloads
from oracle import union as U

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
SENTINEL = -0x21524111


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _w(seed, M, K, keep):
    rng = np.random.default_rng(seed)
    v = rng.integers(-8, 8, size=(M, K))
    W = np.where(rng.random((M, K)) < keep, v, 0).astype(np.int8)
    return W, rng


def run_union(W, X, dev, reorder=True, enc=None):
    enc = enc or bsp.encode_union_tiles(W, 2, 2, reorder)
    N = X.shape[0]
    du = enc.to_device(dev)
    Xd = torch.from_numpy(bsp.pack_int4(X)).to(dev)
    big = torch.full((N * enc.M + 256,), SENTINEL, dtype=torch.int32, device=dev)
    Y = big[:N * enc.M].view(N, enc.M)
    bsp.spmm_union_w4a4(du, Xd, N, Y=Y)
    torch.cuda.synchronize()
    assert bool((big[N * enc.M:] == SENTINEL).all()), "write past the end of Y"
    return Y.cpu().numpy()


def ref_union(W, X, reorder):
    """Y from the IE-BME oracle: encode (with its own reordering), decode, multiply."""
    perms = U.reorder(W, 2, 2) if reorder else None
    Wd = U.decode(U.encode(W, 2, 2, perms=perms))
    return (Wd.astype(np.int64) @ X.astype(np.int64).T).T.astype(np.int32)


SMALL = [  # (M, K, N, keep)
    (16, 64, 1, 0.5), (1, 1, 1, 1.0), (37, 150, 5, 0.3), (33, 129, 17, 0.7), (5, 65, 3, 0.2),
    (100, 1000, 32, 0.5), (64, 512, 16, 1.0), (48, 4096, 8, 0.5), (20, 70, 4, 0.0), (130, 520, 9, 0.05),
    (16, 8256, 2, 0.5), (40, 4104, 31, 0.95), (17, 4099, 16, 0.6),
]


@pytest.mark.parametrize("M,K,N,keep", SMALL)
@pytest.mark.parametrize("reorder", [False, True])
def test_union_small(M, K, N, keep, reorder, dev):
    W, rng = _w(M * 7919 + K * 31 + N, M, K, keep)
    X = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    Y = run_union(W, X, dev, reorder)
    assert np.array_equal(Y, ref_union(W, X, reorder))


def test_union_extremes(dev):
    # every weight -8 against every activation -8: |Y| = 64 K at the largest
    # K the kernel takes, and fully dense tiles (the largest chunk payload)
    for K in (64, 4096, bsp.UNION_MAX_K):
        M, N = 32, 3
        W = np.full((M, K), -8, np.int8)
        X = np.full((N, K), -8, np.int8)
        Y = run_union(W, X, dev, reorder=False)
        assert (Y == 64 * K).all(), K


def test_union_every_n(dev):
    W, rng = _w(77, 70, 700, 0.4)
    X = rng.integers(-8, 8, size=(32, 700)).astype(np.int8)
    enc = bsp.encode_union_tiles(W, 2, 2, True)
    ref = ref_union(W, X, True)
    for N in range(1, 33):
        assert np.array_equal(run_union(W, X[:N], dev, enc=enc), ref[:N]), N


def test_union_k_zero_and_empty(dev):
    W = np.zeros((20, 0), np.int8)
    enc = bsp.encode_union_tiles(W, 2, 2, True)
    du = enc.to_device(dev)
    Y = torch.full((3, 20), 5, dtype=torch.int32, device=dev)
    bsp.spmm_union_w4a4(du, torch.zeros(0, dtype=torch.uint8, device=dev), 3, Y=Y)
    torch.cuda.synchronize()
    assert (Y.cpu().numpy() == 0).all()


@pytest.mark.parametrize("config,index,N", [("qkv", 0, 8), ("qkv", 0, 32), ("qkv", 0, 1), ("ffn", 0, 16),
                                            ("ffn", 1, 16), ("lowsparse", 0, 32)])
def test_union_full_workloads(config, index, N, dev):
    p = workloads.make(config)[index]
    X = p.meta.get("X_full", p.X)[:N] if config == "qkv" else p.X[:N]
    enc = bsp.encode_union_tiles(p.W, 2, 2, True)
    Y = run_union(p.W, X, dev, enc=enc)
    ref = oracle.spmm_w4a4(oracle.encode(p.W), pins._pack_x_for_test(X), N, threads=16)
    assert np.array_equal(Y, ref)


def test_union_reordered_and_plain_agree(dev):
    # reordering changes the stream, not the product
    p = workloads.make("qkv")[0]
    W = p.W[:2048]
    X = p.X[:8]
    e0, e1 = bsp.encode_union_tiles(W, 2, 2, False), bsp.encode_union_tiles(W, 2, 2, True)
    assert e1.nvals < e0.nvals
    assert np.array_equal(run_union(W, X, dev, enc=e0), run_union(W, X, dev, enc=e1))
