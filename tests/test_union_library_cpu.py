"""Host-side checks of the union-mask (IE-BME) part of the product library (no
GPU needed): its encoder, row reordering included, is byte-identical to the
oracle's, and bad SpMM arguments are refused on the host before any HIP call."""
import ctypes

import numpy as np
import pytest

import bit_unstructured_sparse_amd as bsp
from oracle import union as U

FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every case below fails on the host


def _w(seed, M, K, keep):
    rng = np.random.default_rng(seed)
    v = rng.integers(-8, 8, size=(M, K))
    return np.where(rng.random((M, K)) < keep, v, 0).astype(np.int8)


@pytest.mark.parametrize("M,K,keep", [(1, 1, 1.0), (16, 64, 0.5), (37, 150, 0.3), (33, 129, 0.7),
                                      (50, 300, 0.05), (20, 70, 0.0), (17, 64, 1.0)])
@pytest.mark.parametrize("ra,ca", [(2, 2), (1, 1), (2, 1), (1, 2), (4, 1), (4, 4), (2, 8)])
@pytest.mark.parametrize("reorder", [False, True])
def test_union_encoder_matches_oracle(M, K, keep, ra, ca, reorder):
    W = _w(M * 1000 + K, M, K, keep)
    e = bsp.encode_union_tiles(W, ra, ca, reorder)
    perms = U.reorder(W, ra, ca) if reorder else None
    o = U.encode(W, ra, ca, perms=perms)
    assert e.nvals == o.nvals
    assert e.ubitmaps.tolist() == [int(x) for x in o.ubitmaps.reshape(-1)]
    assert e.offsets.tolist() == [int(x) for x in o.offsets]
    assert e.rowpos.tolist() == [int(x) for x in o.rowpos]
    assert bytes(e.payload) == o.payload()
    assert np.array_equal(U.decode(o), W)


def test_union_reordering_shrinks_a_structured_matrix():
    # rows 2i and 2i+8 of every band share a pattern: pairing them (what the DP
    # finds) halves the active positions of the identity grouping (rows r, r+8)
    rng = np.random.default_rng(3)
    W = np.zeros((64, 256), np.int8)
    for band in range(4):
        perm = rng.permutation(16)
        for k in range(8):
            cols = rng.choice(256, 40, replace=False)
            for r in (perm[2 * k], perm[2 * k + 1]):
                W[16 * band + r, cols] = rng.integers(1, 8, 40)
    e0, e1 = bsp.encode_union_tiles(W, 2, 2, False), bsp.encode_union_tiles(W, 2, 2, True)
    o1 = U.encode(W, 2, 2, perms=U.reorder(W, 2, 2))
    assert e1.nvals == o1.nvals < e0.nvals


def test_union_encoder_errors():
    L = bsp.load_library()
    nv, nb = ctypes.c_int64(0), ctypes.c_int64(0)
    W = np.array([[9]], np.int8)
    p = W.ctypes.data_as(ctypes.c_void_p)
    assert L.encode_union_tiles(p, 1, 1, 1, 2, 2, 1, None, None, None, None, 0, ctypes.byref(nv),
                                ctypes.byref(nb)) == bsp.E_RANGE
    W = np.array([[1]], np.int8)
    p = W.ctypes.data_as(ctypes.c_void_p)
    for ra, ca in [(3, 1), (0, 1), (1, 0), (4, 8), (32, 1), (2, 128)]:
        assert L.encode_union_tiles(p, 1, 1, 1, ra, ca, 0, None, None, None, None, 0, ctypes.byref(nv),
                                    ctypes.byref(nb)) == bsp.E_ARG
        assert bsp.union_mask_words(ra, ca) == 0
    assert bsp.union_mask_words(2, 2) == 4 and bsp.union_mask_words(1, 1) == 16
    assert L.encode_union_tiles(p, 1, 2, 1, 2, 2, 0, None, None, None, None, 0, None, None) == bsp.E_ARG  # ldw < K
    ub, off, rp = np.zeros(4, np.uint64), np.zeros(2, np.uint32), np.zeros(1, np.uint64)
    pl = np.zeros(1, np.uint8)
    args = [ub.ctypes.data_as(ctypes.c_void_p), off.ctypes.data_as(ctypes.c_void_p), None]
    assert L.encode_union_tiles(p, 1, 1, 1, 2, 2, 0, *args, None, 0, None, None) == bsp.E_ARG   # rowpos missing
    W = np.full((16, 64), 3, np.int8)
    p = W.ctypes.data_as(ctypes.c_void_p)
    args = [x.ctypes.data_as(ctypes.c_void_p) for x in (ub, off, rp)]
    rc = L.encode_union_tiles(p, 16, 64, 64, 2, 2, 0, *args, pl.ctypes.data_as(ctypes.c_void_p), 1,
                              ctypes.byref(nv), ctypes.byref(nb))
    assert rc == bsp.E_CAPACITY and nv.value == 1024 and nb.value == 512
    assert bsp.union_tile_count(33, 129) == 3 * 3 and bsp.union_tile_count(-1, 5) == -1


def test_union_spmm_host_errors():
    L = bsp.load_library()
    F = FAKE

    def call(ub=F, off=F, rp=F, pl=F, pb=16, ra=2, ca=2, M=16, K=64, X=F, N=1, Y=F):
        return L.spmm_union_w4a4(ub, off, rp, pl, pb, ra, ca, M, K, X, N, Y, None)

    assert call(ra=3) == bsp.E_ARG
    assert call(ra=1, ca=1) == bsp.E_UNSUPPORTED            # valid format, no kernel for it
    assert call(K=bsp.UNION_MAX_K + 1) == bsp.E_UNSUPPORTED
    assert call(N=33) == bsp.E_ARG
    assert call(N=-1) == bsp.E_ARG
    assert call(pb=17) == bsp.E_ARG                          # not a multiple of 16
    assert call(pb=1 << 33) == bsp.E_OVERFLOW
    assert call(Y=None) == bsp.E_ARG
    assert call(off=None) == bsp.E_ARG
    assert call(rp=None) == bsp.E_ARG
    assert call(X=None) == bsp.E_ARG
    assert call(pl=None) == bsp.E_ARG
    assert call(X=ctypes.c_void_p(0x1002)) == bsp.E_UNSUPPORTED   # X off a 4-byte boundary
    assert call(M=0) == bsp.OK and call(N=0) == bsp.OK      # nothing to launch
    assert call(M=1 << 31) == bsp.E_OVERFLOW
