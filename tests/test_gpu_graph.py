"""SpMM calls captured in a HIP graph: every replay, with eager work and
synchronisation between replays, must reproduce the eager result exactly
(the benchmark times graph replays). The kernels issue no memset or other
library call of their own, so a graph holds only their kernel nodes."""
import pytest

torch = pytest.importorskip("torch")

import bit_unstructured_sparse_amd as bsp
import workloads

pytestmark = pytest.mark.gpu

SENTINEL = -0x21524111   # 0xDEADBEEF as int32


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _capture(calls):
    """Capture calls() on a side stream; returns the graph."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            calls()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("M,K,N,algo", [(12288, 4096, 8, bsp.ALGO_AUTO), (4100, 2048, 20, bsp.ALGO_AUTO),
                                        (4096, 11008, 16, bsp.ALGO_AUTO), (1000, 520, 3, bsp.ALGO_ROWWAVE)])
def test_w4a4_graph_replays_match_eager(dev, M, K, N, algo):
    p = workloads.random_int4_problem(M ^ K ^ N, M, K, N, keep=0.5)
    enc = bsp.encode(p.W)
    dms = [enc.to_device(dev) for _ in range(2)]   # two copies, as the benchmark rotates them
    Xd = torch.from_numpy(bsp.pack_int4(p.X)).to(dev)
    Ys = [torch.empty((N, M), dtype=torch.int32, device=dev) for _ in range(2)]
    eager = torch.empty((N, M), dtype=torch.int32, device=dev)
    bsp.spmm_w4a4(dms[0], Xd, N, Y=eager, algo=algo)
    torch.cuda.synchronize()
    want = eager.cpu()

    def calls():
        for dm, Y in zip(dms, Ys):
            bsp.spmm_w4a4(dm, Xd, N, Y=Y, algo=algo)

    g = _capture(calls)
    for rep in range(3):
        for Y in Ys:
            Y.fill_(SENTINEL)   # eager work between replays; a replay must rewrite Y
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for Y in Ys:
            assert torch.equal(Y.cpu(), want), f"replay {rep} differs from the eager result"


@pytest.mark.parametrize("M,K,N", [(4096, 4096, 1), (4096, 4096, 32), (1000, 2048, 7)])
def test_f16_graph_replays_match_eager(dev, M, K, N):
    p = workloads.random_fp16_problem(M + K + N, M, K, N, sparsity=0.6)
    dm = bsp.encode(p.W).to_device(dev)
    Xd = torch.from_numpy(p.X).to(dev)
    Y = torch.empty((N, M), dtype=torch.float16, device=dev)
    eager = torch.empty((N, M), dtype=torch.float16, device=dev)
    bsp.spmm_f16(dm, Xd, Y=eager)
    torch.cuda.synchronize()
    want = eager.cpu().view(torch.int16)   # bitwise: the partial sums are added in a fixed order

    g = _capture(lambda: bsp.spmm_f16(dm, Xd, Y=Y))
    for rep in range(3):
        Y.view(torch.int16).fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y.cpu().view(torch.int16), want), f"replay {rep} differs from the eager result"
