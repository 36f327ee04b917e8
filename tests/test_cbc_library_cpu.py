"""Host-side checks of the Tiled-CBC part of the product library (no GPU
needed): its encoder is byte-identical to the oracle's, and bad calls are
refused on the host before any HIP call."""
import ctypes

import numpy as np
import pytest

import bit_unstructured_sparse_amd as bsp
from oracle import cbc

F = ctypes.c_void_p(0x1000)


@pytest.mark.parametrize("M,K,keep", [(1, 1, 1.0), (300, 130, 0.3), (256, 64, 0.0), (77, 200, 0.9), (257, 65, 0.5)])
def test_cbc_encoder_matches_oracle(M, K, keep):
    rng = np.random.default_rng(M * K)
    W = rng.normal(0, 1, (M, K)).astype(np.float16)
    W[rng.random((M, K)) >= keep] = 0
    W.reshape(-1)[::13] = np.float16(-0.0)
    e = bsp.encode_cbc_f16(W)
    o = cbc.encode(W)
    assert e.nnz == o.values.size
    assert e.tile_offsets.tolist() == [int(x) for x in o.tile_offsets]
    assert e.colinfo.tolist() == [int(x) for x in o.colinfo.reshape(-1)]
    assert e.bitmaps.tolist() == [int(x) for x in o.bitmaps.reshape(-1)]
    assert np.array_equal(e.values, o.values.view(np.uint16))
    assert e.storage_bytes() == o.storage_bytes()


def test_cbc_host_errors():
    L = bsp.load_library()

    def call(M=256, K=64, N=1, tau=0.5, X=F, Y=F, vb=16, ws=None, wsb=0):
        return L.spmspv_cbc_f16(F, F, F, F, vb, M, K, X, N, ctypes.c_float(tau), Y, ws, wsb, None)

    assert call(N=9) == bsp.E_ARG
    assert call(tau=-1.0) == bsp.E_ARG
    assert call(tau=float("nan")) == bsp.E_ARG
    assert call(tau=float("inf")) == bsp.E_ARG
    assert call(vb=10) == bsp.E_ARG
    assert call(Y=None) == bsp.E_ARG
    assert call(X=None) == bsp.E_ARG
    assert call(ws=ctypes.c_void_p(0x1010), wsb=1 << 20) == bsp.E_ARG          # workspace off a 256-byte boundary
    assert call(M=4096, K=4096, ws=ctypes.c_void_p(0x10000), wsb=1024) == bsp.E_CAPACITY
    assert call(M=0) == bsp.OK and call(N=0) == bsp.OK
    b = ctypes.c_int64(-1)
    assert L.spmspv_cbc_workspace_bytes(4096, 4096, 1, ctypes.byref(b)) == bsp.OK and b.value > 65536
    assert L.spmspv_cbc_workspace_bytes(4096, 4096, 9, ctypes.byref(b)) == bsp.E_ARG
    assert bsp.cbc_gtile_count(300, 130) == 2 * 3 and bsp.cbc_gtile_count(-1, 1) == -1
