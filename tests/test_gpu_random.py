"""Seeded random parity sweep through the C ABI: shapes (M up to 6000, K up
to 30000, ragged everywhere), densities from 2 % to 95 % and every N from 1
to 32, drawn per case; each case runs every plan the library offers for it
(automatic, forced MFMA and forced split-K, each without and with a
workspace) and compares the full Y with the oracle's: int4 bit for bit,
fp16 within the documented bound (max floored relative error <= 1e-2). A
canary behind Y catches writes past its end, and the workspace's arrival
counters must be back at zero after every call."""
import numpy as np
import pytest

import bit_unstructured_sparse_amd as bsp
import oracle
import pins
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
SENTINEL = -123456789


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _case(i):
    rng = np.random.default_rng(31337 + i)
    dt = bsp.INT4 if rng.random() < 0.7 else bsp.FP16
    M = int(np.exp(rng.uniform(0, np.log(6000))))
    K = int(np.exp(rng.uniform(0, np.log(30000))))
    if dt == bsp.FP16 and rng.random() < 0.8:
        K = max(8, K // 8 * 8)
    N = int(rng.integers(1, 33))
    while M * K * N > 3e8:
        K = max(1, K // 2)
    keep = float(rng.choice([0.02, 0.1, 0.3, 0.5, 0.7, 0.95]))
    rows = bool(rng.random() < 0.3)   # every row keeps the same count (drawn last: the shapes stay)
    return dt, M, K, N, keep, rows


@pytest.mark.parametrize("i", range(120))
def test_random_case(i, dev):
    dt, M, K, N, keep, rows = _case(i)
    if dt == bsp.INT4:
        p = workloads.random_int4_problem(20000 + i, M, K, N, keep=keep, rows=rows)
        enc = bsp.encode(p.W)
        ref = oracle.spmm_w4a4(oracle.encode(p.W), pins._pack_x_for_test(p.X), N, threads=16)
        Xd = torch.from_numpy(bsp.pack_int4(p.X)).to(dev)
    else:
        p = workloads.random_fp16_problem(20000 + i, M, K, N, sparsity=1.0 - keep, rows=rows)
        enc = bsp.encode(p.W)
        ref = oracle.spmm_f16(oracle.encode(p.W), p.X, threads=16)
        Xd = torch.from_numpy(p.X).to(dev)
    dm = enc.to_device(dev)
    wsz = bsp.workspace_bytes(dt, M, K, N, enc.nnz)
    ws = torch.zeros(max(wsz, 256), dtype=torch.uint8, device=dev) if wsz else None
    ran = 0
    for algo in (bsp.ALGO_AUTO, bsp.ALGO_MFMA, bsp.ALGO_SPLITK):
        for w in ((None, ws) if ws is not None else (None,)):
            try:
                d = bsp.describe(dt, M, K, N, enc.nnz, workspace=w is not None, algo=algo)
            except bsp.BspError as e:
                assert e.status == bsp.E_UNSUPPORTED
                continue
            big = torch.full((N * M + 256,), SENTINEL if dt == bsp.INT4 else -1, dtype=torch.int32, device=dev)
            if dt == bsp.INT4:
                Y = big[:N * M].view(N, M)
                bsp.spmm_w4a4(dm, Xd, N, Y=Y, algo=algo, workspace=w)
                torch.cuda.synchronize()
                assert bool((big[N * M:] == SENTINEL).all().item()), f"write past the end of Y: {d}"
                assert np.array_equal(Y.cpu().numpy(), ref), d
            else:
                Y = big.view(torch.int16)[:N * M].view(torch.float16).view(N, M)
                bsp.spmm_f16(dm, Xd, Y=Y, algo=algo, workspace=w)
                torch.cuda.synchronize()
                assert bool((big.view(torch.int16)[N * M:] == -1).all().item()), f"write past the end of Y: {d}"
                e = oracle.fp16_error(Y.cpu().numpy().astype(np.float64), ref)
                assert e["nonfinite"] == 0 and e["max_rel_floored"] <= 1e-2, (e, d)
            if w is not None:
                assert not w[:65536].any().item(), f"arrival counters left nonzero: {d}"
            ran += 1
    assert ran >= 1
