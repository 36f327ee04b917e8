"""Host-side argument checks of the dequant-epilogue and grouped entry points
(no GPU needed): every call below is refused on the host, before any HIP call."""
import ctypes

import bit_unstructured_sparse_amd as bsp

F = ctypes.c_void_p(0x1000)          # never dereferenced
FX = ctypes.c_void_p(0x1002)         # off a 4-byte boundary


def _dq(M=16, K=64, N=1, X=F, sw=F, sx=F, Yh=F, pb=16):
    return bsp.load_library().spmm_bitmap_w4a4_dq(F, F, F, pb, M, K, X, N, sw, sx, Yh, None)


def test_dq_host_errors():
    assert _dq(sw=None) == bsp.E_ARG
    assert _dq(sx=None) == bsp.E_ARG
    assert _dq(Yh=None) == bsp.E_ARG
    assert _dq(N=33) == bsp.E_ARG
    assert _dq(pb=20) == bsp.E_ARG
    assert _dq(K=16384 + 64) == bsp.E_UNSUPPORTED          # past the MFMA kernels
    assert _dq(X=FX) == bsp.E_UNSUPPORTED                  # X off a 4-byte boundary
    assert _dq(M=0) == bsp.OK and _dq(N=0) == bsp.OK       # nothing to do


def _item(**kw):
    d = dict(bitmaps=F, offsets=F, payload=F, payload_bytes=16, M=16, X=F, N=1, Y=F, Yh=None, scale_w=None,
             scale_x=None)
    d.update(kw)
    return bsp.W4A4Item(**d)


def _group(items, K=64):
    arr = (bsp.W4A4Item * max(1, len(items)))(*items)
    return bsp.load_library().spmm_bitmap_w4a4_grouped(ctypes.cast(arr, ctypes.c_void_p), len(items), K, None)


def test_grouped_host_errors():
    L = bsp.load_library()
    assert L.spmm_bitmap_w4a4_grouped(None, 1, 64, None) == bsp.E_ARG
    assert _group([]) == bsp.E_ARG
    assert _group([_item()] * (bsp.GROUP_MAX + 1)) == bsp.E_ARG
    assert _group([_item(), _item(Y=F, Yh=F, scale_w=F, scale_x=F)]) == bsp.E_ARG     # two outputs
    assert _group([_item(), _item(Y=None)]) == bsp.E_ARG                              # no output
    assert _group([_item(Y=None, Yh=F, scale_w=F)]) == bsp.E_ARG                      # token scales missing
    assert _group([_item(), _item(N=40)]) == bsp.E_ARG
    assert _group([_item(), _item(payload_bytes=8)]) == bsp.E_ARG
    assert _group([_item(), _item(X=FX)]) == bsp.E_UNSUPPORTED
    assert _group([_item(), _item()], K=4096 + 64) == bsp.E_UNSUPPORTED               # not the streaming kernel
    assert _group([_item(), _item()], K=-1) == bsp.E_ARG
    assert _group([_item(M=0), _item(N=0)]) == bsp.OK                                 # nothing to launch
