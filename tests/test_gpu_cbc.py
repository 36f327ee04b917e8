"""GPU parity of the Tiled-CBC product with dynamic activation pruning (fp16)
against the oracle's fp64 reference of the thresholded product, within the
fp16 bound (max floored relative error <= 1e-2), through the C ABI. Columns
whose activations are all pruned must not be read: changing W there leaves
Y bit for bit the same."""
import numpy as np
import pytest

import bit_unstructured_sparse_amd as bsp
import oracle
import workloads
from oracle import cbc

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _w(seed, M, K, keep):
    rng = np.random.default_rng(seed)
    W = rng.normal(0, 1, (M, K)).astype(np.float16)
    W[rng.random((M, K)) >= keep] = 0
    return W, rng


def run(W, X, tau, dev, workspace=True, enc=None):
    enc = enc or bsp.encode_cbc_f16(W)
    D = enc.to_device(dev)
    N = X.shape[0]
    ws = bsp.new_cbc_workspace(W.shape[0], W.shape[1], N, device=dev) if workspace else None
    big = torch.full((N * W.shape[0] + 64,), 0x7E00, dtype=torch.int16, device=dev)
    Y = big[:N * W.shape[0]].view(torch.float16).view(N, W.shape[0])
    bsp.spmspv_cbc_f16(D, torch.from_numpy(X).to(dev), tau, Y=Y, workspace=ws)
    torch.cuda.synchronize()
    assert bool((big[N * W.shape[0]:] == 0x7E00).all()), "write past the end of Y"
    return Y.cpu().numpy()


def check(Y, W, X, tau):
    r = cbc.spmspv_reference(W, X, tau)
    e = oracle.fp16_error(Y, r)
    assert e["nonfinite"] == 0 and e["max_rel_floored"] <= TOL, e


SHAPES = [(256, 64, 1, 0.4), (300, 130, 1, 0.3), (1, 1, 1, 1.0), (513, 1000, 2, 0.4), (1024, 4096, 8, 0.4),
          (77, 4099, 3, 0.9), (4096, 512, 1, 0.05)]


@pytest.mark.parametrize("M,K,N,keep", SHAPES)
@pytest.mark.parametrize("quantile", [0.0, 0.5, 0.9])
@pytest.mark.parametrize("workspace", [True, False])
def test_cbc_thresholds(M, K, N, keep, quantile, workspace, dev):
    W, rng = _w(M * 31 + K + N, M, K, keep)
    X = rng.normal(0, 1, (N, K)).astype(np.float16)
    tau = float(np.quantile(np.abs(X.astype(np.float32)), quantile)) if quantile else 0.0
    check(run(W, X, tau, dev, workspace), W, X, tau)


@pytest.mark.parametrize("workspace", [True, False])
def test_cbc_every_n(workspace, dev):
    # every width from 1 to BSP_CBC_MAX_N (the kernel instances hold 1, 2, 4 or 8 activation columns)
    W, rng = _w(91, 700, 1500, 0.4)
    X = rng.normal(0, 1, (8, 1500)).astype(np.float16)
    tau = float(np.quantile(np.abs(X.astype(np.float32)), 0.5))
    enc = bsp.encode_cbc_f16(W)
    for N in range(1, 9):
        check(run(W, X[:N], tau, dev, workspace, enc=enc), W, X[:N], tau)


def test_cbc_all_pruned_and_k_zero(dev):
    W, rng = _w(1, 300, 200, 0.5)
    X = rng.normal(0, 1, (2, 200)).astype(np.float16)
    assert (run(W, X, 1e6, dev) == 0).all()
    W0 = np.zeros((10, 0), np.float16)
    assert (run(W0, np.zeros((1, 0), np.float16), 0.0, dev) == 0).all()


def test_cbc_pruned_columns_are_not_read(dev):
    W, rng = _w(2, 1024, 2048, 0.4)
    X = rng.normal(0, 1, (1, 2048)).astype(np.float16)
    tau = float(np.quantile(np.abs(X.astype(np.float32)), 0.6))
    skip = cbc.skipped_columns(X, tau)
    W2 = W.copy()
    W2[:, skip] = rng.normal(0, 100, (1024, int(skip.sum()))).astype(np.float16)
    y1, y2 = run(W, X, tau, dev), run(W2, X, tau, dev)
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))


def test_cbc_fp16_workload_half_pruned(dev):
    p = workloads.make("fp16")[0]          # W 4096 x 4096, 60 % magnitude-pruned, N = 1
    X = p.X
    tau = float(np.quantile(np.abs(X.astype(np.float32)), 0.5))
    enc = bsp.encode_cbc_f16(p.W)
    check(run(p.W, X, tau, dev, enc=enc), p.W, X, tau)
    check(run(p.W, X, 0.0, dev, enc=enc), p.W, X, 0.0)


def test_cbc_workspace_reused(dev):
    # one workspace across calls and shapes: the counters return to zero
    M, K = 1024, 4096
    ws = bsp.new_cbc_workspace(M, K, 8, device=dev)
    for (m, k, n) in [(1024, 4096, 8), (512, 4096, 1), (1024, 2048, 2), (1024, 4096, 8)]:
        W, rng = _w(m + k + n, m, k, 0.4)
        X = rng.normal(0, 1, (n, k)).astype(np.float16)
        D = bsp.encode_cbc_f16(W).to_device(dev)
        Y = bsp.spmspv_cbc_f16(D, torch.from_numpy(X).to(dev), 0.3, workspace=ws)
        torch.cuda.synchronize()
        check(Y.cpu().numpy(), W, X, 0.3)
