"""Concurrent calls on different streams: the entry points keep no state of
their own (the split-K and Tiled-CBC plans use the caller's workspace), so
calls of several kernel families issued on four streams, interleaved and
repeated without synchronising in between, must each give the result they
give alone. Every output is checked against the oracle."""
import numpy as np
import pytest

import bit_unstructured_sparse_amd as bsp
import oracle
import pins
import workloads
from oracle import cbc
from oracle import union as U

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
TOL = 1e-2
REPS = 3


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def test_four_streams_interleaved(dev):
    rng = np.random.default_rng(2024)
    # int4, block kernel
    p4 = workloads.random_int4_problem(11, 2000, 3000, 8, keep=0.5)
    e4 = bsp.encode(p4.W)
    d4 = e4.to_device(dev)
    x4 = torch.from_numpy(bsp.pack_int4(p4.X)).to(dev)
    ref4 = oracle.spmm_w4a4(oracle.encode(p4.W), pins._pack_x_for_test(p4.X), 8, threads=16)
    # fp16 past K = 4096: split-K with a workspace
    p16 = workloads.random_fp16_problem(12, 500, 6000, 4)
    e16 = bsp.encode(p16.W)
    d16 = e16.to_device(dev)
    x16 = torch.from_numpy(p16.X).to(dev)
    ws16 = bsp.new_workspace(bsp.FP16, 500, 6000, 4, e16.nnz, device=dev)
    assert ws16 is not None and "splitk" in bsp.describe(bsp.FP16, 500, 6000, 4, e16.nnz, workspace=True)
    ref16 = oracle.spmm_f16(oracle.encode(p16.W), p16.X)
    # Tiled-CBC with dynamic pruning and a workspace
    Wc = rng.normal(0, 1, (600, 2000)).astype(np.float16)
    Wc[rng.random((600, 2000)) >= 0.4] = 0
    Xc = rng.normal(0, 1, (1, 2000)).astype(np.float16)
    tau = float(np.median(np.abs(Xc.astype(np.float32))))
    ec = bsp.encode_cbc_f16(Wc)
    dc = ec.to_device(dev)
    xc = torch.from_numpy(Xc).to(dev)
    wsc = bsp.new_cbc_workspace(600, 2000, 1, device=dev)
    refc = cbc.spmspv_reference(Wc, Xc, tau)
    # union mask
    Wu = rng.integers(-8, 8, size=(300, 1000)).astype(np.int8)
    Wu[rng.random((300, 1000)) >= 0.5] = 0
    Xu = rng.integers(-8, 8, size=(5, 1000)).astype(np.int8)
    du = bsp.encode_union_tiles(Wu, 2, 2, True).to_device(dev)
    xu = torch.from_numpy(bsp.pack_int4(Xu)).to(dev)
    refu = (U.decode(U.encode(Wu, 2, 2, perms=U.reorder(Wu, 2, 2))).astype(np.int64)
            @ Xu.astype(np.int64).T).T.astype(np.int32)

    streams = [torch.cuda.Stream() for _ in range(4)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = {k: [] for k in ("int4", "fp16", "cbc", "union")}
    for _ in range(REPS):
        with torch.cuda.stream(streams[0]):
            outs["int4"].append(bsp.spmm_w4a4(d4, x4, 8, stream=streams[0]))
        with torch.cuda.stream(streams[1]):
            outs["fp16"].append(bsp.spmm_f16(d16, x16, stream=streams[1], workspace=ws16))
        with torch.cuda.stream(streams[2]):
            outs["cbc"].append(bsp.spmspv_cbc_f16(dc, xc, tau, workspace=wsc, stream=streams[2]))
        with torch.cuda.stream(streams[3]):
            outs["union"].append(bsp.spmm_union_w4a4(du, xu, 5, stream=streams[3]))
    torch.cuda.synchronize()
    for y in outs["int4"]:
        assert np.array_equal(y.cpu().numpy(), ref4)
    first = None
    for y in outs["fp16"]:
        yn = y.cpu().numpy()
        e = oracle.fp16_error(yn.astype(np.float64), ref16)
        assert e["nonfinite"] == 0 and e["max_rel_floored"] <= TOL, e
        if first is None:
            first = yn.view(np.uint16).copy()
        else:   # partials meet in a fixed order: the same bits every call
            assert np.array_equal(first, yn.view(np.uint16))
    for y in outs["cbc"]:
        e = oracle.fp16_error(y.cpu().numpy().astype(np.float64), refc)
        assert e["nonfinite"] == 0 and e["max_rel_floored"] <= TOL, e
    for y in outs["union"]:
        assert np.array_equal(y.cpu().numpy(), refu)
    # the workspaces' arrival counters are back to zero
    assert not ws16[:65536].any() and not wsc[:65536].any()
