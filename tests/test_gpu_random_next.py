"""Seeded random parity sweep over the next rows through the C ABI: per case
one of the union-mask SpMM (2 x 2 areas, rows reordered or not), W2A4, the
dequant epilogue and the Tiled-CBC product with dynamic pruning, on a random
shape (ragged M and K), density and N. Union and W2A4 results must equal the
oracle's plain product W.X bit for bit (both formats are lossless), the
dequant output the oracle's closed form bit for bit, and the Tiled-CBC output
the fp64 reference of the thresholded product within the fp16 bound. A canary
behind every output catches writes past its end."""
import numpy as np
import pytest

import bit_unstructured_sparse_amd as bsp
import oracle
import pins
import workloads
from oracle import cbc

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
SENTINEL = -0x2A2A2A2B
ROWS = ("union", "w2a4", "dq", "cbc")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _plain(W, X):
    return oracle.spmm_w4a4(oracle.encode(W), pins._pack_x_for_test(X), X.shape[0], threads=16)


def _case(i):
    rng = np.random.default_rng(4242 + i)
    row = ROWS[i % len(ROWS)]
    M = int(np.exp(rng.uniform(0, np.log(3000))))
    K = int(np.exp(rng.uniform(0, np.log(12000 if row != "union" else 6000))))
    N = int(rng.integers(1, 9 if row == "cbc" else 33))
    while M * K * max(N, 8) > 2e8:
        K = max(1, K // 2)
    keep = float(rng.choice([0.02, 0.1, 0.3, 0.5, 0.7, 0.95]))
    return row, M, K, N, keep, rng


def _int32_out(N, M, dev):
    big = torch.full((N * M + 256,), SENTINEL, dtype=torch.int32, device=dev)
    return big, big[:N * M].view(N, M)


@pytest.mark.parametrize("i", range(80))
def test_random_next_case(i, dev):
    row, M, K, N, keep, rng = _case(i)
    seed = 30000 + i
    if row == "union":
        p = workloads.random_int4_problem(seed, M, K, N, keep=keep)
        reorder = bool(rng.random() < 0.5)
        du = bsp.encode_union_tiles(p.W, 2, 2, reorder).to_device(dev)
        big, Y = _int32_out(N, M, dev)
        bsp.spmm_union_w4a4(du, torch.from_numpy(bsp.pack_int4(p.X)).to(dev), N, Y=Y)
        torch.cuda.synchronize()
        assert bool((big[N * M:] == SENTINEL).all().item()), "write past the end of Y"
        assert np.array_equal(Y.cpu().numpy(), _plain(p.W, p.X)), (M, K, N, keep, reorder)
    elif row == "w2a4":
        p = workloads.random_int2_problem(seed, M, K, N, keep=keep)
        dm = bsp.encode(p.W, dtype=bsp.INT2).to_device(dev)
        big, Y = _int32_out(N, M, dev)
        bsp.spmm_w2a4(dm, torch.from_numpy(bsp.pack_int4(p.X)).to(dev), N, Y=Y)
        torch.cuda.synchronize()
        assert bool((big[N * M:] == SENTINEL).all().item()), "write past the end of Y"
        assert np.array_equal(Y.cpu().numpy(), _plain(p.W, p.X)), (M, K, N, keep)
    elif row == "dq":
        p = workloads.random_int4_problem(seed, M, K, N, keep=keep)
        sw = np.exp(rng.uniform(np.log(1e-4), np.log(5e-2), size=M)).astype(np.float32)
        sw[rng.random(M) < 0.1] *= -1
        sx = np.exp(rng.uniform(np.log(1e-2), np.log(2.0), size=N)).astype(np.float32)
        dm = bsp.encode(p.W).to_device(dev)
        big = torch.full((N * M + 64,), 0x7E00, dtype=torch.int16, device=dev)
        Yh = big[:N * M].view(torch.float16).view(N, M)
        try:
            bsp.spmm_bitmap_w4a4_dq(dm, torch.from_numpy(bsp.pack_int4(p.X)).to(dev), N, torch.from_numpy(sw).to(dev),
                                    torch.from_numpy(sx).to(dev), Yh=Yh)
        except bsp.BspError as e:   # past the int4 MFMA kernels' K bound
            assert e.status == bsp.E_UNSUPPORTED and K > 16384
            return
        torch.cuda.synchronize()
        assert bool((big[N * M:] == 0x7E00).all().item()), "write past the end of Yh"
        want = oracle.dequant_f16(_plain(p.W, p.X), sw, sx)
        assert np.array_equal(Yh.cpu().numpy().view(np.uint16), want.view(np.uint16)), (M, K, N, keep)
    else:
        W = rng.normal(0, 1, (M, K)).astype(np.float16)
        W[rng.random((M, K)) >= keep] = 0
        X = rng.normal(0, 1, (N, K)).astype(np.float16)
        q = float(rng.choice([0.0, 0.3, 0.5, 0.9]))
        tau = float(np.quantile(np.abs(X.astype(np.float32)), q)) if q else 0.0
        D = bsp.encode_cbc_f16(W).to_device(dev)
        ws = bsp.new_cbc_workspace(M, K, N, device=dev) if rng.random() < 0.7 else None
        big = torch.full((N * M + 64,), 0x7E00, dtype=torch.int16, device=dev)
        Y = big[:N * M].view(torch.float16).view(N, M)
        bsp.spmspv_cbc_f16(D, torch.from_numpy(X).to(dev), tau, Y=Y, workspace=ws)
        torch.cuda.synchronize()
        assert bool((big[N * M:] == 0x7E00).all().item()), "write past the end of Y"
        e = oracle.fp16_error(Y.cpu().numpy().astype(np.float64), cbc.spmspv_reference(W, X, tau))
        assert e["nonfinite"] == 0 and e["max_rel_floored"] <= 1e-2, (e, M, K, N, keep, tau)
        if ws is not None:
            assert not ws[:65536].any().item(), "arrival counters left nonzero"
