"""Bitmap-tiled int4 / fp16 sparse x dense matmul on AMD MI355X (gfx950).

A thin ctypes binding over ``libbitmap_spmm.so`` (C ABI in
``include/bitmap_spmm.h``). Host arrays are numpy; device memory and streams
come from PyTorch tensors. Every step of the SpMM runs in the library's HIP
kernels; there is no CPU fallback: if the library is missing, importing the
SpMM functions raises.

    import bit_unstructured_sparse_amd as bsp
    enc = bsp.encode(W_int8)                 # host, UnionSparse Sec. V-A with Q = 1
    dev = enc.to_device("cuda")              # torch tensors
    Xp  = bsp.pack_int4(X_int8)              # [N][ceil(K/2)] bytes
    Y   = bsp.spmm_w4a4(dev, torch.from_numpy(Xp).cuda(), N)   # int32 [N][M]
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

__all__ = ["load_library", "encode", "pack_int4", "Encoded", "DeviceMatrix", "spmm_w4a4", "spmm_f16",
           "select", "describe", "workspace_bytes", "BspError", "ALGO_AUTO", "ALGO_ROWWAVE", "ALGO_MFMA",
           "ALGO_SPLITK",
           "INT4", "FP16", "PAYLOAD_ALIGN", "MAX_N", "library_path"]

HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(HERE, "libbitmap_spmm.so")

OK, E_ARG, E_RANGE, E_CAPACITY, E_OVERFLOW, E_HIP, E_UNSUPPORTED = 0, 1, 2, 3, 4, 5, 6
INT4, FP16, INT2 = 0, 1, 2
ALGO_AUTO, ALGO_ROWWAVE, ALGO_MFMA, ALGO_SPLITK = 0, 1, 2, 3
PAYLOAD_ALIGN = 16
MAX_N = 32

# Every symbol include/bitmap_spmm.h declares.
EXPORTS = ["encode_bitmap_tiles", "pack_int4_activations", "spmm_bitmap_w4a4", "spmm_bitmap_w4a4_algo",
           "spmm_bitmap_w4a4_ws", "spmm_bitmap_f16", "spmm_bitmap_f16_algo", "spmm_bitmap_f16_ws",
           "bsp_workspace_bytes", "bsp_select", "bsp_describe_selection", "bsp_describe_selection_ws", "bsp_describe_plan",
           "bsp_status_string", "bsp_version", "spmm_bitmap_f16_noalloc", "bsp_noalloc_scratch_bytes",
           "union_tile_count", "union_mask_words", "encode_union_tiles", "spmm_union_w4a4",
           "spmm_bitmap_w4a4_dq", "spmm_bitmap_w4a4_grouped", "spmm_bitmap_w2a4", "spmm_bitmap_w2a4_algo",
           "cbc_gtile_count", "encode_cbc_f16", "spmspv_cbc_workspace_bytes", "spmspv_cbc_f16"]


class BspError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


_lib = None


def load_library():
    """Load libbitmap_spmm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise ImportError(f"{library_path} is missing; build it with "
                              "`python -m bit_unstructured_sparse_amd.build`")
        L = ctypes.CDLL(library_path)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.encode_bitmap_tiles.argtypes = [I32, P, I64, I64, I64, P, P, P, I64, P, P]
        L.encode_bitmap_tiles.restype = I32
        L.pack_int4_activations.argtypes, L.pack_int4_activations.restype = [P, I64, I64, I64, P], I32
        L.spmm_bitmap_w4a4.argtypes = [P, P, P, I64, I64, I64, P, I64, P, P]
        L.spmm_bitmap_w4a4.restype = I32
        L.spmm_bitmap_w4a4_algo.argtypes = [P, P, P, I64, I64, I64, P, I64, P, I32, P]
        L.spmm_bitmap_w4a4_algo.restype = I32
        L.spmm_bitmap_f16.argtypes = [P, P, P, I64, I64, I64, P, I64, P, P]
        L.spmm_bitmap_f16.restype = I32
        L.spmm_bitmap_f16_algo.argtypes = [P, P, P, I64, I64, I64, P, I64, P, I32, P]
        L.spmm_bitmap_f16_algo.restype = I32
        L.spmm_bitmap_w4a4_ws.argtypes = [P, P, P, I64, I64, I64, P, I64, P, P, I64, I32, P]
        L.spmm_bitmap_w4a4_ws.restype = I32
        L.spmm_bitmap_f16_ws.argtypes = [P, P, P, I64, I64, I64, P, I64, P, P, I64, I32, P]
        L.spmm_bitmap_f16_ws.restype = I32
        L.bsp_workspace_bytes.argtypes, L.bsp_workspace_bytes.restype = [I32, I64, I64, I64, I64, P], I32
        L.spmm_bitmap_f16_noalloc.argtypes = [P, P, P, I64, I64, I64, P, I64, P, I32, P]
        L.spmm_bitmap_f16_noalloc.restype = I32
        L.bsp_noalloc_scratch_bytes.argtypes, L.bsp_noalloc_scratch_bytes.restype = [], I64
        L.bsp_describe_selection_ws.argtypes = [I32, I64, I64, I64, I64, ctypes.c_char_p, ctypes.c_size_t]
        L.bsp_describe_selection_ws.restype = I32
        L.bsp_describe_plan.argtypes = [I32, I64, I64, I64, I64, I32, I32, ctypes.c_char_p, ctypes.c_size_t]
        L.bsp_describe_plan.restype = I32
        L.bsp_select.argtypes, L.bsp_select.restype = [I32, I64, I64, I64, I64], I32
        L.bsp_describe_selection.argtypes = [I32, I64, I64, I64, I64, ctypes.c_char_p, ctypes.c_size_t]
        L.bsp_describe_selection.restype = I32
        L.bsp_status_string.argtypes, L.bsp_status_string.restype = [I32], ctypes.c_char_p
        L.bsp_version.argtypes, L.bsp_version.restype = [], ctypes.c_char_p
        L.union_tile_count.argtypes, L.union_tile_count.restype = [I64, I64], I64
        L.union_mask_words.argtypes, L.union_mask_words.restype = [I32, I32], I32
        L.encode_union_tiles.argtypes = [P, I64, I64, I64, I32, I32, I32, P, P, P, P, I64, P, P]
        L.encode_union_tiles.restype = I32
        L.spmm_union_w4a4.argtypes = [P, P, P, P, I64, I32, I32, I64, I64, P, I64, P, P]
        L.spmm_union_w4a4.restype = I32
        L.spmm_bitmap_w4a4_dq.argtypes = [P, P, P, I64, I64, I64, P, I64, P, P, P, P]
        L.spmm_bitmap_w4a4_dq.restype = I32
        L.spmm_bitmap_w4a4_grouped.argtypes = [P, I32, I64, P]
        L.spmm_bitmap_w4a4_grouped.restype = I32
        L.spmm_bitmap_w2a4.argtypes = [P, P, P, I64, I64, I64, P, I64, P, P]
        L.spmm_bitmap_w2a4.restype = I32
        L.spmm_bitmap_w2a4_algo.argtypes = [P, P, P, I64, I64, I64, P, I64, P, I32, P]
        L.spmm_bitmap_w2a4_algo.restype = I32
        L.cbc_gtile_count.argtypes, L.cbc_gtile_count.restype = [I64, I64], I64
        L.encode_cbc_f16.argtypes = [P, I64, I64, I64, P, P, P, P, I64, P]
        L.encode_cbc_f16.restype = I32
        L.spmspv_cbc_workspace_bytes.argtypes, L.spmspv_cbc_workspace_bytes.restype = [I64, I64, I64, P], I32
        L.spmspv_cbc_f16.argtypes = [P, P, P, P, I64, I64, I64, P, I64, ctypes.c_float, P, P, I64, P]
        L.spmspv_cbc_f16.restype = I32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return load_library().bsp_status_string(status).decode()


def _np_ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != OK:
        raise BspError(rc, what)


@dataclass
class Encoded:
    """Host-side BT64 stream: bitmaps uint64[M*T], offsets uint32[M*T+1],
    payload uint8[ceil(nnz/2)] (int4) or uint16[nnz] (fp16)."""
    dtype: int
    M: int
    K: int
    nnz: int
    bitmaps: np.ndarray
    offsets: np.ndarray
    payload: np.ndarray

    @property
    def T(self) -> int:
        return (self.K + 63) // 64

    @property
    def payload_bytes(self) -> int:
        return int(self.payload.nbytes)

    def to_device(self, device="cuda") -> "DeviceMatrix":
        import torch
        pad = (-self.payload_bytes) % PAYLOAD_ALIGN
        raw = np.zeros(self.payload_bytes + pad, np.uint8)
        raw[: self.payload_bytes] = self.payload.view(np.uint8)
        if raw.size == 0:
            raw = np.zeros(PAYLOAD_ALIGN, np.uint8)
        return DeviceMatrix(
            dtype=self.dtype, M=self.M, K=self.K, nnz=self.nnz,
            bitmaps=torch.from_numpy(self.bitmaps.view(np.int64)).to(device),
            offsets=torch.from_numpy(self.offsets.view(np.int32)).to(device),
            payload=torch.from_numpy(raw).to(device))


@dataclass
class DeviceMatrix:
    """The BT64 stream in device memory (torch tensors). ``payload`` is padded
    with zeros to a whole number of PAYLOAD_ALIGN bytes."""
    dtype: int
    M: int
    K: int
    nnz: int
    bitmaps: "object"
    offsets: "object"
    payload: "object"

    @property
    def T(self) -> int:
        return (self.K + 63) // 64

    def stream_bytes(self, with_offsets: bool = True) -> int:
        """Bytes of the encoded stream proper (unpadded payload)."""
        G = self.M * self.T
        pb = {INT4: (self.nnz + 1) // 2, INT2: (self.nnz + 3) // 4}.get(self.dtype, 2 * self.nnz)
        return 8 * G + (4 * (G + 1) if with_offsets else 0) + pb


def encode(W: np.ndarray, dtype: Optional[int] = None) -> Encoded:
    """Encode a dense host matrix: int8 (int4 values in [-8, 7]; with
    dtype=INT2, 2-bit values in [-2, 1]) or float16."""
    L = load_library()
    if W.dtype == np.int8:
        dt = INT2 if dtype == INT2 else INT4
    elif W.dtype == np.float16:
        dt = FP16
        W = W.view(np.uint16)
    elif W.dtype == np.uint16:
        dt = FP16
    else:
        raise TypeError("W must be int8 (int4 values) or float16")
    if W.ndim != 2:
        raise ValueError("W must be 2-D")
    M, K = W.shape
    ldw = W.strides[0] // W.itemsize if W.strides[1] == W.itemsize else None
    if ldw is None or ldw < K:
        W = np.ascontiguousarray(W)
        ldw = K
    nnz, nbytes = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(L.encode_bitmap_tiles(dt, _np_ptr(W), M, K, ldw, None, None, None, 0,
                                 ctypes.byref(nnz), ctypes.byref(nbytes)), "encode_bitmap_tiles (size)")
    T = (K + 63) // 64
    bitmaps = np.empty(M * T, np.uint64)
    offsets = np.empty(M * T + 1, np.uint32)
    payload = np.empty(nnz.value if dt == FP16 else nbytes.value, np.uint16 if dt == FP16 else np.uint8)
    _check(L.encode_bitmap_tiles(dt, _np_ptr(W), M, K, ldw, _np_ptr(bitmaps), _np_ptr(offsets),
                                 _np_ptr(payload), payload.nbytes, ctypes.byref(nnz), ctypes.byref(nbytes)),
           "encode_bitmap_tiles")
    return Encoded(dt, M, K, int(nnz.value), bitmaps, offsets, payload)


def spmm_w2a4(W: DeviceMatrix, X, N: int, Y=None, algo: int = ALGO_AUTO, stream=None):
    """Y[n][m] = sum_k W[m][k] X[k][n] (int32) with 2-bit weights (a stream
    encoded with dtype=INT2). X: uint8 [N][ceil(K/2)] packed int4."""
    import torch
    if W.dtype != INT2:
        raise TypeError("spmm_w2a4 needs an INT2 DeviceMatrix")
    _check_dev(X, "X", torch.uint8, N * ((W.K + 1) // 2))
    if Y is None:
        Y = torch.empty((N, W.M), dtype=torch.int32, device=X.device)
    _check_dev(Y, "Y", torch.int32, N * W.M)
    rc = load_library().spmm_bitmap_w2a4_algo(
        _dptr(W.bitmaps), _dptr(W.offsets), _dptr(W.payload), W.payload.numel(), W.M, W.K,
        _dptr(X), N, _dptr(Y), algo, _stream_handle(stream))
    _check(rc, "spmm_bitmap_w2a4")
    return Y


def pack_int4(X: np.ndarray) -> np.ndarray:
    """int8 [N][K] activations in [-8, 7] -> packed uint8 [N][ceil(K/2)]."""
    if X.dtype != np.int8 or X.ndim != 2:
        raise TypeError("X must be a 2-D int8 array")
    X = np.ascontiguousarray(X)
    N, K = X.shape
    out = np.zeros((N, (K + 1) // 2), np.uint8)
    _check(load_library().pack_int4_activations(_np_ptr(X), N, K, K, _np_ptr(out)), "pack_int4_activations")
    return out


def _dptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check_dev(t, name, dtype, numel=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


def _ws_args(workspace):
    if workspace is None:
        return None, 0
    import torch
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous CUDA (HIP) tensor")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def spmm_w4a4(W: DeviceMatrix, X, N: int, Y=None, algo: int = ALGO_AUTO, stream=None, workspace=None):
    """Y[n][m] = sum_k W[m][k] X[k][n] (int32) on the GPU. X: uint8 [N][ceil(K/2)].
    workspace: an optional zero-initialised device tensor of at least
    workspace_bytes(...) bytes, 256-byte aligned (enables the split plans)."""
    import torch
    if W.dtype != INT4:
        raise TypeError("spmm_w4a4 needs an int4 DeviceMatrix")
    _check_dev(X, "X", torch.uint8, N * ((W.K + 1) // 2))
    if Y is None:
        Y = torch.empty((N, W.M), dtype=torch.int32, device=X.device)
    _check_dev(Y, "Y", torch.int32, N * W.M)
    wp, wb = _ws_args(workspace)
    rc = load_library().spmm_bitmap_w4a4_ws(
        _dptr(W.bitmaps), _dptr(W.offsets), _dptr(W.payload), W.payload.numel(), W.M, W.K,
        _dptr(X), N, _dptr(Y), wp, wb, algo, _stream_handle(stream))
    _check(rc, "spmm_bitmap_w4a4")
    return Y


def spmm_f16(W: DeviceMatrix, X, Y=None, algo: int = ALGO_AUTO, stream=None, workspace=None):
    """fp16 Y [N][M] = W X with fp32 accumulation. X: float16 [N][K]."""
    import torch
    if W.dtype != FP16:
        raise TypeError("spmm_f16 needs an fp16 DeviceMatrix")
    if X.dim() != 2 or X.shape[1] != W.K:
        raise ValueError("X must be [N][K]")
    N = int(X.shape[0])
    _check_dev(X, "X", torch.float16)
    if Y is None:
        Y = torch.empty((N, W.M), dtype=torch.float16, device=X.device)
    _check_dev(Y, "Y", torch.float16, N * W.M)
    wp, wb = _ws_args(workspace)
    rc = load_library().spmm_bitmap_f16_ws(
        _dptr(W.bitmaps), _dptr(W.offsets), _dptr(W.payload), W.payload.numel(), W.M, W.K,
        _dptr(X), N, _dptr(Y), wp, wb, algo, _stream_handle(stream))
    _check(rc, "spmm_bitmap_f16")
    return Y


# ---- dequant epilogue and grouped launch ----

GROUP_MAX = 8


class W4A4Item(ctypes.Structure):
    """bsp_w4a4_item of include/bitmap_spmm.h."""
    _fields_ = [("bitmaps", ctypes.c_void_p), ("offsets", ctypes.c_void_p), ("payload", ctypes.c_void_p),
                ("payload_bytes", ctypes.c_int64), ("M", ctypes.c_int64), ("X", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("Y", ctypes.c_void_p), ("Yh", ctypes.c_void_p),
                ("scale_w", ctypes.c_void_p), ("scale_x", ctypes.c_void_p)]


def spmm_bitmap_w4a4_dq(W: DeviceMatrix, X, N: int, scale_w, scale_x, Yh=None, stream=None):
    """fp16 Yh [N][M] = fp16(fp32(fp32(W X) * scale_w[m]) * scale_x[n]), the
    dequant step fused into the int4 SpMM. scale_w: float32 [M], scale_x:
    float32 [N] (device)."""
    import torch
    if W.dtype != INT4:
        raise TypeError("spmm_bitmap_w4a4_dq needs an int4 DeviceMatrix")
    _check_dev(X, "X", torch.uint8, N * ((W.K + 1) // 2))
    _check_dev(scale_w, "scale_w", torch.float32, W.M)
    _check_dev(scale_x, "scale_x", torch.float32, N)
    if Yh is None:
        Yh = torch.empty((N, W.M), dtype=torch.float16, device=X.device)
    _check_dev(Yh, "Yh", torch.float16, N * W.M)
    rc = load_library().spmm_bitmap_w4a4_dq(
        _dptr(W.bitmaps), _dptr(W.offsets), _dptr(W.payload), W.payload.numel(), W.M, W.K, _dptr(X), N,
        _dptr(scale_w), _dptr(scale_x), _dptr(Yh), _stream_handle(stream))
    _check(rc, "spmm_bitmap_w4a4_dq")
    return Yh


def spmm_bitmap_w4a4_grouped(items, stream=None):
    """One launch for several int4 matrices of one K. items: a list of dicts
    with W (DeviceMatrix), X (uint8 [N][ceil(K/2)]), N, and either Y (int32
    [N][M]) or Yh (fp16 [N][M]) with scale_w (float32 [M]) and scale_x
    (float32 [N]). Returns the list of outputs."""
    import torch
    if not items:
        raise ValueError("no items")
    K = items[0]["W"].K
    arr = (W4A4Item * len(items))()
    outs = []
    for i, it in enumerate(items):
        W, X, N = it["W"], it["X"], int(it["N"])
        if W.K != K or W.dtype != INT4:
            raise ValueError("grouped items must be int4 matrices of one K")
        _check_dev(X, "X", torch.uint8, N * ((K + 1) // 2))
        Y, Yh = it.get("Y"), it.get("Yh")
        sw, sx = it.get("scale_w"), it.get("scale_x")
        if sw is not None:
            _check_dev(sw, "scale_w", torch.float32, W.M)
            _check_dev(sx, "scale_x", torch.float32, N)
            if Yh is None:
                Yh = torch.empty((N, W.M), dtype=torch.float16, device=X.device)
            _check_dev(Yh, "Yh", torch.float16, N * W.M)
            outs.append(Yh)
        else:
            if Y is None:
                Y = torch.empty((N, W.M), dtype=torch.int32, device=X.device)
            _check_dev(Y, "Y", torch.int32, N * W.M)
            outs.append(Y)
        arr[i] = W4A4Item(_dptr(W.bitmaps), _dptr(W.offsets), _dptr(W.payload), W.payload.numel(), W.M, _dptr(X), N,
                          _dptr(Y) if sw is None else None, _dptr(Yh) if sw is not None else None, _dptr(sw),
                          _dptr(sx))
    rc = load_library().spmm_bitmap_w4a4_grouped(ctypes.cast(arr, ctypes.c_void_p), len(items), K,
                                                 _stream_handle(stream))
    _check(rc, "spmm_bitmap_w4a4_grouped")
    return outs


# ---- Tiled-CBC format with dynamic activation pruning (fp16) ----

CBC_TILE = (256, 64)
CBC_MAX_N = 8


@dataclass
class CbcEncoded:
    """Host-side Tiled-CBC stream: tile_offsets uint32[n_gt + 1], colinfo
    uint32[n_gt * 64], bitmaps uint64[n_gt * 256], values fp16 bits [nnz]."""
    M: int
    K: int
    nnz: int
    tile_offsets: np.ndarray
    colinfo: np.ndarray
    bitmaps: np.ndarray
    values: np.ndarray

    def storage_bytes(self) -> int:
        return int(self.tile_offsets.nbytes + self.colinfo.nbytes + self.bitmaps.nbytes + self.values.nbytes)

    def to_device(self, device="cuda") -> "CbcDevice":
        import torch
        vb = self.values.nbytes
        raw = np.zeros(max(PAYLOAD_ALIGN, vb + (-vb) % PAYLOAD_ALIGN), np.uint8)
        raw[:vb] = self.values.view(np.uint8)
        return CbcDevice(self.M, self.K, self.nnz,
                         torch.from_numpy(self.tile_offsets.view(np.int32)).to(device),
                         torch.from_numpy(self.colinfo.view(np.int32)).to(device),
                         torch.from_numpy(self.bitmaps.view(np.int64)).to(device),
                         torch.from_numpy(raw).to(device))


@dataclass
class CbcDevice:
    M: int
    K: int
    nnz: int
    tile_offsets: "object"
    colinfo: "object"
    bitmaps: "object"
    values: "object"       # uint8, padded to PAYLOAD_ALIGN


def cbc_gtile_count(M: int, K: int) -> int:
    return int(load_library().cbc_gtile_count(M, K))


def encode_cbc_f16(W: np.ndarray) -> CbcEncoded:
    L = load_library()
    W = np.ascontiguousarray(W)
    if W.dtype == np.float16:
        W = W.view(np.uint16)
    if W.dtype != np.uint16 or W.ndim != 2:
        raise TypeError("W must be a 2-D float16 (or uint16 bits) array")
    M, K = W.shape
    nnz = ctypes.c_int64(0)
    _check(L.encode_cbc_f16(_np_ptr(W), M, K, K, None, None, None, None, 0, ctypes.byref(nnz)), "encode_cbc_f16 (size)")
    ngt = cbc_gtile_count(M, K)
    to = np.zeros(ngt + 1, np.uint32)
    ci = np.zeros(ngt * 64, np.uint32)
    bm = np.zeros(ngt * 256, np.uint64)
    vals = np.zeros(nnz.value, np.uint16)
    _check(L.encode_cbc_f16(_np_ptr(W), M, K, K, _np_ptr(to), _np_ptr(ci), _np_ptr(bm), _np_ptr(vals), vals.size,
                            ctypes.byref(nnz)), "encode_cbc_f16")
    return CbcEncoded(M, K, int(nnz.value), to, ci, bm, vals)


def spmspv_cbc_workspace_bytes(M: int, K: int, N: int) -> int:
    b = ctypes.c_int64(0)
    _check(load_library().spmspv_cbc_workspace_bytes(M, K, N, ctypes.byref(b)), "spmspv_cbc_workspace_bytes")
    return int(b.value)


def new_cbc_workspace(M: int, K: int, N: int, device="cuda"):
    import torch
    n = spmspv_cbc_workspace_bytes(M, K, N)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device) if n else None


def spmspv_cbc_f16(D: CbcDevice, X, threshold: float, Y=None, workspace=None, stream=None):
    """fp16 Y [N][M] = W X' with X' = X where |x| > threshold, else 0 (dynamic
    activation pruning; the all-pruned columns of W are not read)."""
    import torch
    if X.dim() != 2 or X.shape[1] != D.K:
        raise ValueError("X must be [N][K]")
    N = int(X.shape[0])
    _check_dev(X, "X", torch.float16)
    if Y is None:
        Y = torch.empty((N, D.M), dtype=torch.float16, device=X.device)
    _check_dev(Y, "Y", torch.float16, N * D.M)
    wp, wb = _ws_args(workspace)
    rc = load_library().spmspv_cbc_f16(
        _dptr(D.tile_offsets), _dptr(D.colinfo), _dptr(D.bitmaps), _dptr(D.values), D.values.numel(), D.M, D.K,
        _dptr(X), N, ctypes.c_float(threshold), _dptr(Y), wp, wb, _stream_handle(stream))
    _check(rc, "spmspv_cbc_f16")
    return Y


# ---- union-mask (IE-BME) format: 16 x 64 local tiles, ra x ca areas ----

UNION_MAX_K = 32768


@dataclass
class UnionEncoded:
    """Host-side union-mask stream: ubitmaps uint64[nlt * words], offsets
    uint32[nlt + 1], rowpos uint64[nlt], payload uint8[ceil(nvals / 2)]."""
    M: int
    K: int
    ra: int
    ca: int
    nvals: int
    ubitmaps: np.ndarray
    offsets: np.ndarray
    rowpos: np.ndarray
    payload: np.ndarray

    @property
    def nlt(self) -> int:
        return int(self.rowpos.size)

    def stream_bytes(self) -> int:
        """Bytes of the encoded stream proper: mask words, offsets, rowpos, payload."""
        return int(self.ubitmaps.nbytes + self.offsets.nbytes + self.rowpos.nbytes + self.payload.nbytes)

    def to_device(self, device="cuda") -> "UnionDevice":
        import torch
        pb = self.payload.nbytes
        raw = np.zeros(max(PAYLOAD_ALIGN, pb + (-pb) % PAYLOAD_ALIGN), np.uint8)
        raw[:pb] = self.payload
        return UnionDevice(self.M, self.K, self.ra, self.ca, self.nvals,
                           torch.from_numpy(self.ubitmaps.view(np.int64)).to(device),
                           torch.from_numpy(self.offsets.view(np.int32)).to(device),
                           torch.from_numpy(self.rowpos.view(np.int64)).to(device),
                           torch.from_numpy(raw).to(device))


@dataclass
class UnionDevice:
    """The union-mask stream in device memory; payload padded with zeros to a
    whole number of PAYLOAD_ALIGN bytes."""
    M: int
    K: int
    ra: int
    ca: int
    nvals: int
    ubitmaps: "object"
    offsets: "object"
    rowpos: "object"
    payload: "object"


def union_tile_count(M: int, K: int) -> int:
    return int(load_library().union_tile_count(M, K))


def union_mask_words(ra: int, ca: int) -> int:
    return int(load_library().union_mask_words(ra, ca))


def encode_union_tiles(W: np.ndarray, ra: int = 2, ca: int = 2, reorder: bool = True) -> UnionEncoded:
    """Union-mask encoding of an int8 (int4 values) host matrix, with
    bitmap-aware row reordering of every local tile when ``reorder``."""
    L = load_library()
    if W.dtype != np.int8 or W.ndim != 2:
        raise TypeError("W must be a 2-D int8 array of int4 values")
    W = np.ascontiguousarray(W)
    M, K = W.shape
    nv, nb = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(L.encode_union_tiles(_np_ptr(W), M, K, K, ra, ca, int(reorder), None, None, None, None, 0,
                                ctypes.byref(nv), ctypes.byref(nb)), "encode_union_tiles (size)")
    nlt, words = union_tile_count(M, K), union_mask_words(ra, ca)
    ub = np.zeros(nlt * words, np.uint64)
    off = np.zeros(nlt + 1, np.uint32)
    rp = np.zeros(nlt, np.uint64)
    pl = np.zeros(nb.value, np.uint8)
    _check(L.encode_union_tiles(_np_ptr(W), M, K, K, ra, ca, int(reorder), _np_ptr(ub), _np_ptr(off), _np_ptr(rp),
                                _np_ptr(pl), pl.nbytes, ctypes.byref(nv), ctypes.byref(nb)), "encode_union_tiles")
    return UnionEncoded(M, K, ra, ca, int(nv.value), ub, off, rp, pl)


def spmm_union_w4a4(U: UnionDevice, X, N: int, Y=None, stream=None):
    """Y[n][m] = sum_k W[m][k] X[k][n] (int32) with W in the union-mask
    format. X: uint8 [N][ceil(K/2)] packed int4."""
    import torch
    _check_dev(X, "X", torch.uint8, N * ((U.K + 1) // 2))
    if Y is None:
        Y = torch.empty((N, U.M), dtype=torch.int32, device=X.device)
    _check_dev(Y, "Y", torch.int32, N * U.M)
    rc = load_library().spmm_union_w4a4(
        _dptr(U.ubitmaps), _dptr(U.offsets), _dptr(U.rowpos), _dptr(U.payload), U.payload.numel(), U.ra, U.ca,
        U.M, U.K, _dptr(X), N, _dptr(Y), _stream_handle(stream))
    _check(rc, "spmm_union_w4a4")
    return Y


def select(dtype: int, M: int, K: int, N: int, nnz: int = -1) -> int:
    return int(load_library().bsp_select(dtype, M, K, N, nnz))


def describe(dtype: int, M: int, K: int, N: int, nnz: int = -1, workspace: bool = False,
             algo: int = ALGO_AUTO) -> str:
    """The plan (kernel and launch shape) of the plain entry points, or with
    workspace=True of the *_ws entry points given a workspace; for an
    explicit algo, the plan that choice takes (BspError if it cannot run)."""
    buf = ctypes.create_string_buffer(384)
    if algo != ALGO_AUTO:
        _check(load_library().bsp_describe_plan(dtype, M, K, N, nnz, algo, int(workspace), buf, 384),
               "bsp_describe_plan")
        return buf.value.decode()
    fn = load_library().bsp_describe_selection_ws if workspace else load_library().bsp_describe_selection
    _check(fn(dtype, M, K, N, nnz, buf, 384), "bsp_describe_selection")
    return buf.value.decode()


def workspace_bytes(dtype: int, M: int, K: int, N: int, nnz: int = -1) -> int:
    """Bytes of workspace the *_ws entry points want for a problem (0: none)."""
    out = ctypes.c_int64(0)
    _check(load_library().bsp_workspace_bytes(dtype, M, K, N, nnz, ctypes.byref(out)), "bsp_workspace_bytes")
    return int(out.value)


def new_workspace(dtype: int, M: int, K: int, N: int, nnz: int = -1, device="cuda"):
    """A zero-filled device workspace for the split plans (None if none is needed)."""
    import torch
    n = workspace_bytes(dtype, M, K, N, nnz)
    if n == 0:
        return None
    return torch.zeros(n, dtype=torch.uint8, device=device)
