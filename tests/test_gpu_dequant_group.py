"""GPU parity of the dequant epilogue (int32 -> fp16 with per-channel and
per-token scales, fused into the int4 MFMA kernels) and of the grouped launch
(several matrices of one K in one dispatch), bit for bit against the oracle:
the oracle's int32 product, then its dequant step. Calls go through the C ABI
via the binding."""
import numpy as np
import pytest

import bit_unstructured_sparse_amd as bsp
import oracle
import pins
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _scales(rng, M, N):
    sw = np.exp(rng.uniform(np.log(1e-4), np.log(5e-2), size=M)).astype(np.float32)
    sw[rng.random(M) < 0.1] *= -1
    sx = np.exp(rng.uniform(np.log(1e-2), np.log(2.0), size=N)).astype(np.float32)
    return sw, sx


def _oracle_y(W, X):
    return oracle.spmm_w4a4(oracle.encode(W), pins._pack_x_for_test(X), X.shape[0], threads=16)


def _run_dq(W, X, sw, sx, dev, enc=None):
    enc = enc or bsp.encode(W)
    N = X.shape[0]
    dm = enc.to_device(dev)
    Xd = torch.from_numpy(bsp.pack_int4(X)).to(dev)
    big = torch.full((N * enc.M + 64,), 0x7E00, dtype=torch.int16, device=dev)
    Yh = big[:N * enc.M].view(torch.float16).view(N, enc.M)
    bsp.spmm_bitmap_w4a4_dq(dm, Xd, N, torch.from_numpy(sw).to(dev), torch.from_numpy(sx).to(dev), Yh=Yh)
    torch.cuda.synchronize()
    assert bool((big[N * enc.M:] == 0x7E00).all()), "write past the end of Yh"
    return Yh.cpu().numpy()


DQ_SHAPES = [  # (M, K, N, keep): streaming (K <= 4096), ring (K > 4096), K % 8 != 0, ragged M
    (16, 64, 1, 0.5), (37, 150, 5, 0.3), (100, 1000, 32, 0.5), (64, 4096, 8, 0.5), (33, 4099, 17, 0.4),
    (48, 8192, 16, 0.5), (20, 16384, 3, 0.3), (1, 1, 1, 1.0), (130, 520, 9, 0.05), (256, 2048, 32, 0.7),
]


@pytest.mark.parametrize("M,K,N,keep", DQ_SHAPES)
def test_dequant_epilogue(M, K, N, keep, dev):
    p = workloads.random_int4_problem(M * 131 + K + N, M, K, N, keep=keep)
    rng = np.random.default_rng(M + 7 * K + N)
    sw, sx = _scales(rng, M, N)
    got = _run_dq(p.W, p.X, sw, sx, dev)
    want = oracle.dequant_f16(_oracle_y(p.W, p.X), sw, sx)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def test_dequant_overflow_and_signed_zero(dev):
    # large sums with a large channel scale overflow to +-inf; zero sums keep the sign of the scales
    M, K, N = 32, 4096, 4
    W = np.full((M, K), -8, np.int8)
    W[::2] = 0
    X = np.full((N, K), -8, np.int8)
    sw = np.full(M, 1.0, np.float32)
    sw[1::4] = -1.0
    sx = np.array([1.0, 0.5, -1.0, 2.0 ** -20], np.float32)
    got = _run_dq(W, X, sw, sx, dev)
    want = oracle.dequant_f16(_oracle_y(W, X), sw, sx)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))
    assert np.isinf(got[0, 1]) and got.view(np.uint16)[2, 0] == 0x8000


def test_dequant_k_zero(dev):
    W = np.zeros((10, 0), np.int8)
    X = np.zeros((3, 0), np.int8)
    rng = np.random.default_rng(1)
    sw, sx = _scales(rng, 10, 3)
    enc = bsp.encode(W)
    dm = enc.to_device(dev)
    Yh = torch.full((3, 10), 7.0, dtype=torch.float16, device=dev)
    bsp.spmm_bitmap_w4a4_dq(dm, torch.zeros(0, dtype=torch.uint8, device=dev), 3, torch.from_numpy(sw).to(dev),
                            torch.from_numpy(sx).to(dev), Yh=Yh)
    torch.cuda.synchronize()
    want = oracle.dequant_f16(np.zeros((3, 10), np.int32), sw, sx)
    assert np.array_equal(Yh.cpu().numpy().view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("config,index,N", [("qkv", 0, 8), ("ffn", 1, 16), ("qkv", 0, 32)])
def test_dequant_full_workloads(config, index, N, dev):
    p = workloads.make(config)[index]
    X = p.meta.get("X_full", p.X)[:N]
    rng = np.random.default_rng(N)
    sw, sx = _scales(rng, p.M, N)
    got = _run_dq(p.W, X, sw, sx, dev)
    want = oracle.dequant_f16(_oracle_y(p.W, X), sw, sx)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def _grouped(specs, dev):
    """specs: (W, X, scales or None). Runs one grouped call; returns outputs as numpy."""
    items = []
    for (W, X, sc) in specs:
        enc = bsp.encode(W)
        it = dict(W=enc.to_device(dev), X=torch.from_numpy(bsp.pack_int4(X)).to(dev), N=X.shape[0])
        if sc is not None:
            it["scale_w"] = torch.from_numpy(sc[0]).to(dev)
            it["scale_x"] = torch.from_numpy(sc[1]).to(dev)
        items.append(it)
    outs = bsp.spmm_bitmap_w4a4_grouped(items)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs]


def _want(W, X, sc):
    y = _oracle_y(W, X)
    return y if sc is None else oracle.dequant_f16(y, *sc)


def test_grouped_qkv_projections(dev):
    # the fused 12288 x 4096 QKV matrix as three 4096 x 4096 projections with
    # one X: Q and V through the dequant epilogue, K as int32
    p = workloads.make("qkv")[0]
    X = p.X
    rng = np.random.default_rng(3)
    specs = []
    for j in range(3):
        W = p.W[4096 * j:4096 * (j + 1)]
        specs.append((W, X, None if j == 1 else _scales(rng, 4096, X.shape[0])))
    outs = _grouped(specs, dev)
    for (W, Xj, sc), o in zip(specs, outs):
        w = _want(W, Xj, sc)
        assert np.array_equal(o.view(w.dtype if sc is None else np.uint16),
                              w if sc is None else w.view(np.uint16))


@pytest.mark.parametrize("K", [1000, 999, 64, 4096])
def test_grouped_eight_ragged_items(K, dev):
    rng = np.random.default_rng(K)
    Ms = [1, 17, 100, 2048, 33, 0, 640, 1500]
    Ns = [1, 32, 8, 16, 3, 5, 24, 7]
    specs = []
    for i, (M, N) in enumerate(zip(Ms, Ns)):
        p = workloads.random_int4_problem(K * 10 + i, M, K, N, keep=[0.5, 0.1, 0.9, 0.3][i % 4])
        specs.append((p.W, p.X, _scales(rng, M, N) if i % 2 else None))
    outs = _grouped(specs, dev)
    for (W, X, sc), o in zip(specs, outs):
        if W.shape[0] == 0:
            continue
        w = _want(W, X, sc)
        if sc is None:
            assert np.array_equal(o, w)
        else:
            assert np.array_equal(o.view(np.uint16), w.view(np.uint16))


def test_grouped_refuses_other_kernels(dev):
    p = workloads.random_int4_problem(5, 64, 8192, 4)
    enc = bsp.encode(p.W)
    it = dict(W=enc.to_device(dev), X=torch.from_numpy(bsp.pack_int4(p.X)).to(dev), N=4)
    with pytest.raises(bsp.BspError) as ei:
        bsp.spmm_bitmap_w4a4_grouped([it, it])
    assert ei.value.status == bsp.E_UNSUPPORTED
