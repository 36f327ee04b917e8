"""The allocation-free fp16 entry point (spmm_bitmap_f16_noalloc): its
split-K plans use the library's static per-GPU scratch instead of a caller
workspace. Checked through the C ABI against spmm_bitmap_f16_ws with a
caller workspace (the same plan, so the same bits), on two calls in a row,
the second with a smaller input, and against the oracle's tolerance."""
import ctypes

import numpy as np
import pytest

import bit_unstructured_sparse_amd as bsp
import oracle
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _call_noalloc(dm, X, Y, algo=bsp.ALGO_AUTO):
    L = bsp.load_library()
    rc = L.spmm_bitmap_f16_noalloc(dm.bitmaps.data_ptr(), dm.offsets.data_ptr(), dm.payload.data_ptr(),
                                   dm.payload.numel(), dm.M, dm.K, X.data_ptr(), X.shape[0], Y.data_ptr(), algo,
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return rc


def _call_ws(dm, X, Y, ws, algo=bsp.ALGO_AUTO):
    L = bsp.load_library()
    return L.spmm_bitmap_f16_ws(dm.bitmaps.data_ptr(), dm.offsets.data_ptr(), dm.payload.data_ptr(),
                                dm.payload.numel(), dm.M, dm.K, X.data_ptr(), X.shape[0], Y.data_ptr(),
                                ws.data_ptr(), ws.numel(), algo, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("algo", [bsp.ALGO_AUTO, bsp.ALGO_SPLITK])
def test_noalloc_matches_workspace_entry_point(algo):
    dev = torch.device("cuda:0")
    # a larger problem, then a smaller one: the second call reuses the scratch
    # the first left behind (its arrival counters back at zero)
    for seed, (M, K, N) in enumerate([(4096, 11008, 8), (1000, 64 * 100, 3)]):
        p = workloads.random_fp16_problem(900 + seed, M, K, N)
        enc = bsp.encode(p.W)
        dm = enc.to_device(dev)
        X = torch.from_numpy(p.X).to(dev)
        need = bsp.workspace_bytes(bsp.FP16, M, K, N, enc.nnz)
        assert 0 < need <= bsp.load_library().bsp_noalloc_scratch_bytes()
        d = bsp.describe(bsp.FP16, M, K, N, enc.nnz, workspace=True)
        assert "splits=2 " in d, d     # the plan uses the scratch
        Y0 = torch.full((N, M), -1, dtype=torch.int16, device=dev).view(torch.float16)
        Y1 = torch.full((N, M), -1, dtype=torch.int16, device=dev).view(torch.float16)
        ws = torch.zeros(need, dtype=torch.uint8, device=dev)
        assert _call_ws(dm, X, Y0, ws, algo) == bsp.OK
        assert _call_noalloc(dm, X, Y1, algo) == bsp.OK
        torch.cuda.synchronize()
        assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16)), f"call {seed}: not the same bits"
        e = oracle.fp16_error(Y1.cpu().numpy().astype(np.float64), oracle.spmm_f16(oracle.encode(p.W), p.X))
        assert e["nonfinite"] == 0 and e["max_rel_floored"] <= 1e-2, e
    # a plan without a workspace (K <= 4096) does not touch the scratch
    p = workloads.random_fp16_problem(950, 300, 2048, 4)
    dm = bsp.encode(p.W).to_device(dev)
    X = torch.from_numpy(p.X).to(dev)
    Y = torch.empty((4, 300), dtype=torch.float16, device=dev)
    assert _call_noalloc(dm, X, Y) == bsp.OK
    torch.cuda.synchronize()
    e = oracle.fp16_error(Y.cpu().numpy().astype(np.float64), oracle.spmm_f16(oracle.encode(p.W), p.X))
    assert e["max_rel_floored"] <= 1e-2, e
