"""Host-side checks of the W2A4 part of the product library (no GPU needed):
the int2 encoder is byte-identical to the W2A4 oracle's, and bad SpMM calls
are refused on the host before any HIP call."""
import ctypes

import numpy as np
import pytest

import bit_unstructured_sparse_amd as bsp
import workloads
from oracle import w2

F = ctypes.c_void_p(0x1000)


@pytest.mark.parametrize("M,K,keep", [(1, 1, 1.0), (9, 65, 0.5), (17, 300, 0.3), (40, 1000, 0.9), (6, 63, 0.0),
                                      (130, 4096, 0.5), (3, 129, 1.0)])
def test_int2_encoder_matches_oracle(M, K, keep):
    p = workloads.random_int2_problem(M + K, M, K, 1, keep=keep)
    e = bsp.encode(p.W, dtype=bsp.INT2)
    o = w2.encode(p.W)
    assert e.nnz == o.nnz
    assert e.bitmaps.tolist() == [int(x) for x in o.bitmaps]
    assert e.offsets.tolist() == [int(x) for x in o.offsets]
    assert bytes(e.payload) == o.payload
    assert e.payload.nbytes == (o.nnz + 3) // 4


def test_int2_encoder_range():
    for bad in (2, -3):
        with pytest.raises(bsp.BspError) as ei:
            bsp.encode(np.array([[0, bad]], np.int8), dtype=bsp.INT2)
        assert ei.value.status == bsp.E_RANGE


def test_w2a4_host_errors():
    L = bsp.load_library()

    def call(M=16, K=64, N=1, X=F, Y=F, pb=16, algo=0):
        return L.spmm_bitmap_w2a4_algo(F, F, F, pb, M, K, X, N, Y, algo, None)

    assert call(N=33) == bsp.E_ARG
    assert call(Y=None) == bsp.E_ARG
    assert call(pb=12) == bsp.E_ARG
    assert call(algo=bsp.ALGO_SPLITK) == bsp.E_UNSUPPORTED
    assert call(algo=bsp.ALGO_MFMA, K=16385) == bsp.E_UNSUPPORTED       # past the MFMA block kernels
    assert call(algo=bsp.ALGO_MFMA, X=ctypes.c_void_p(0x1001)) == bsp.E_UNSUPPORTED
    assert call(algo=9) == bsp.E_ARG
    assert call(M=0) == bsp.OK and call(N=0) == bsp.OK


def test_w2a4_plan_descriptions():
    # the W2A4 plans: the streaming kernel up to K = 4096, the ring kernel up to
    # 16384 (2-bit values, never staggered), the plain kernel past it; no split-K
    d = bsp.describe(bsp.INT2, 12288, 4096, 8, 12288 * 4096 // 2)
    assert d.startswith("dtype=int2 ") and "-> mfma kernel=k_bt64s_w2a4 " in d, d
    for K in (4097, 11008, 16384):
        d = bsp.describe(bsp.INT2, 4096, K, 16, 4096 * K * 3 // 10)
        assert "-> mfma kernel=k_bt64_w4a4 " in d and "stagger=0" in d, d
    d = bsp.describe(bsp.INT2, 4096, 16385, 16, 4096 * 16385 * 3 // 10)
    assert "-> rowwave kernel=k_rowwave_w4a4" in d, d
    assert "-> rowwave " in bsp.describe(bsp.INT2, 4096, 11008, 16, -1, algo=bsp.ALGO_ROWWAVE)
    for algo, K in [(bsp.ALGO_SPLITK, 11008), (bsp.ALGO_MFMA, 16385)]:
        with pytest.raises(bsp.BspError) as ei:
            bsp.describe(bsp.INT2, 4096, K, 16, -1, algo=algo)
        assert ei.value.status == bsp.E_UNSUPPORTED
