"""CPU oracle for the bitmap-tiled sparse matmul -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product library never loads it and
shares no code with it.

The arithmetic lives in ``bsp_oracle.c`` (plain C, no intrinsics), compiled
with gcc into ``liboracle.so`` next to this file; this module only marshals
numpy arrays into it. See the header of ``bsp_oracle.c`` for the definitions
it follows and the readings it takes where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bsp_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, E_ARG, E_RANGE, E_CAPACITY, E_OVERFLOW = 0, 1, 2, 3, 4
DT_INT4, DT_FP16 = 0, 1


def build(force: bool = True) -> str:
    """Compile bsp_oracle.c with gcc. Returns the library path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-shared", "-fPIC", "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = _configure(ctypes.CDLL(_LIB))
    return _lib


def swap_library(path: Optional[str]):
    """Load another build of bsp_oracle.c (used only by the mutation tests, which
    plant mistakes in a copy of the oracle). ``None`` restores the normal build.
    Returns the previously active handle."""
    global _lib
    prev = _lib
    _lib = None if path is None else _configure(ctypes.CDLL(path))
    return prev


def _configure(L):
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.or_tiles_per_row.argtypes, L.or_tiles_per_row.restype = [I64], I64
    L.or_popcount64.argtypes, L.or_popcount64.restype = [ctypes.c_uint64], I32
    L.or_rank.argtypes, L.or_rank.restype = [ctypes.c_uint64, I32], I32
    L.or_f16_to_f64.argtypes, L.or_f16_to_f64.restype = [ctypes.c_uint16], ctypes.c_double
    L.or_encode.argtypes = [I32, P, I64, I64, I64, P, P, P, I64, P, P]
    L.or_encode.restype = I32
    L.or_validate.argtypes, L.or_validate.restype = [I32, P, P, P, I64, I64, I64], I32
    L.or_decode.argtypes, L.or_decode.restype = [I32, P, P, P, I64, I64, P], None
    L.or_unpack_x4.argtypes, L.or_unpack_x4.restype = [P, I64, I64, P], None
    L.or_matmul_i64.argtypes, L.or_matmul_i64.restype = [P, I64, I64, P, I64, P], None
    L.or_matmul_f64.argtypes, L.or_matmul_f64.restype = [P, I64, I64, P, I64, P], None
    L.or_spmm_w4a4.argtypes, L.or_spmm_w4a4.restype = [P, P, P, I64, I64, P, I64, P], I32
    L.or_spmm_f16.argtypes, L.or_spmm_f16.restype = [P, P, P, I64, I64, P, I64, P], I32
    L.or_spmm_w4a4_mt.argtypes, L.or_spmm_w4a4_mt.restype = [P, P, P, I64, I64, P, I64, P, I32], I32
    L.or_spmm_f16_mt.argtypes, L.or_spmm_f16_mt.restype = [P, P, P, I64, I64, P, I64, P, I32], I32
    L.or_spmm_w4a4_one.argtypes, L.or_spmm_w4a4_one.restype = [P, P, P, I64, P, I64, I64], I64
    L.or_spmm_f16_one.argtypes, L.or_spmm_f16_one.restype = [P, P, P, I64, P, I64, I64], ctypes.c_double
    return L


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


@dataclass
class Stream:
    """An encoded matrix: bitmaps[M*T], offsets[M*T+1], payload (uint8 or uint16)."""
    dtype: int
    M: int
    K: int
    bitmaps: np.ndarray
    offsets: np.ndarray
    payload: np.ndarray
    nnz: int

    @property
    def T(self) -> int:
        return (self.K + 63) // 64

    @property
    def payload_bytes(self) -> int:
        return int(self.payload.nbytes)


def tiles_per_row(K: int) -> int:
    return int(lib().or_tiles_per_row(K))


def popcount64(w: int) -> int:
    return int(lib().or_popcount64(w))


def rank(w: int, j: int) -> int:
    return int(lib().or_rank(w, j))


def f16_to_f64(bits: int) -> float:
    return float(lib().or_f16_to_f64(bits))


def encode(W: np.ndarray) -> Stream:
    """Reference encoder. int8 W -> int4 stream; float16 W -> fp16 stream."""
    if W.dtype == np.int8:
        dt = DT_INT4
    elif W.dtype == np.float16:
        dt = DT_FP16
    else:
        raise TypeError("W must be int8 (int4 values) or float16")
    W = np.ascontiguousarray(W)
    M, K = W.shape
    nnz, nbytes = ctypes.c_int64(0), ctypes.c_int64(0)
    rc = lib().or_encode(dt, _p(W), M, K, K, None, None, None, 0, ctypes.byref(nnz), ctypes.byref(nbytes))
    if rc != OK:
        raise ValueError(f"oracle encode failed: code {rc}")
    T = (K + 63) // 64
    bitmaps = np.zeros(M * T, np.uint64)
    offsets = np.zeros(M * T + 1, np.uint32)
    payload = np.zeros(nbytes.value if dt == DT_INT4 else nnz.value, np.uint8 if dt == DT_INT4 else np.uint16)
    rc = lib().or_encode(dt, _p(W), M, K, K, _p(bitmaps), _p(offsets), _p(payload),
                         payload.nbytes, ctypes.byref(nnz), ctypes.byref(nbytes))
    if rc != OK:
        raise ValueError(f"oracle encode failed: code {rc}")
    return Stream(dt, M, K, bitmaps, offsets, payload, int(nnz.value))


def encode_rc(W: np.ndarray, dtype: int, payload_cap: Optional[int] = None):
    """Raw return code of the reference encoder (for error-path tests)."""
    W = np.ascontiguousarray(W)
    M, K = W.shape
    nnz, nbytes = ctypes.c_int64(-1), ctypes.c_int64(-1)
    T = (K + 63) // 64
    if payload_cap is None:
        rc = lib().or_encode(dtype, _p(W), M, K, K, None, None, None, 0, ctypes.byref(nnz), ctypes.byref(nbytes))
    else:
        bm = np.zeros(M * T, np.uint64)
        off = np.zeros(M * T + 1, np.uint32)
        pl = np.zeros(max(payload_cap, 1), np.uint8)
        rc = lib().or_encode(dtype, _p(W), M, K, K, _p(bm), _p(off), _p(pl), payload_cap,
                             ctypes.byref(nnz), ctypes.byref(nbytes))
    return int(rc), int(nnz.value), int(nbytes.value)


def validate(s: Stream) -> int:
    return int(lib().or_validate(s.dtype, _p(s.bitmaps), _p(s.offsets), _p(s.payload),
                                 s.payload_bytes, s.M, s.K))


def validate_arrays(dtype: int, bitmaps, offsets, payload, M: int, K: int) -> int:
    return int(lib().or_validate(dtype, _p(bitmaps), _p(offsets), _p(payload), payload.nbytes, M, K))


def decode(s: Stream) -> np.ndarray:
    out = np.zeros((s.M, s.K), np.int8 if s.dtype == DT_INT4 else np.uint16)
    lib().or_decode(s.dtype, _p(s.bitmaps), _p(s.offsets), _p(s.payload), s.M, s.K, _p(out))
    return out if s.dtype == DT_INT4 else out.view(np.float16)


def unpack_x4(Xp: np.ndarray, N: int, K: int) -> np.ndarray:
    Xp = np.ascontiguousarray(Xp, dtype=np.uint8)
    if Xp.size != N * ((K + 1) // 2):
        raise ValueError("packed X has the wrong size")
    out = np.zeros((N, K), np.int8)
    lib().or_unpack_x4(_p(Xp), N, K, _p(out))
    return out


def matmul_i64(Wd: np.ndarray, Xd: np.ndarray) -> np.ndarray:
    """Y[n][m] = sum_k W[m][k] X[n][k], int64."""
    Wd = np.ascontiguousarray(Wd, np.int8)
    Xd = np.ascontiguousarray(Xd, np.int8)
    M, K = Wd.shape
    N = Xd.shape[0]
    Y = np.zeros((N, M), np.int64)
    lib().or_matmul_i64(_p(Wd), M, K, _p(Xd), N, _p(Y))
    return Y


def matmul_f64(Wd: np.ndarray, Xh: np.ndarray) -> np.ndarray:
    Wd = np.ascontiguousarray(Wd, np.float16).view(np.uint16)
    Xh = np.ascontiguousarray(Xh, np.float16).view(np.uint16)
    M, K = Wd.shape
    N = Xh.shape[0]
    Y = np.zeros((N, M), np.float64)
    lib().or_matmul_f64(_p(Wd), M, K, _p(Xh), N, _p(Y))
    return Y


def spmm_w4a4(s: Stream, Xp: np.ndarray, N: int, threads: int = 0) -> np.ndarray:
    """Y int32 [N][M] from the stream and packed int4 X ([N][ceil(K/2)] bytes).
    threads > 0 splits the rows of Y over that many threads (same result)."""
    Xp = np.ascontiguousarray(Xp, dtype=np.uint8)
    Y = np.zeros((N, s.M), np.int32)
    if threads > 0:
        rc = lib().or_spmm_w4a4_mt(_p(s.bitmaps), _p(s.offsets), _p(s.payload), s.M, s.K, _p(Xp), N, _p(Y), threads)
    else:
        rc = lib().or_spmm_w4a4(_p(s.bitmaps), _p(s.offsets), _p(s.payload), s.M, s.K, _p(Xp), N, _p(Y))
    if rc != OK:
        raise ValueError(f"oracle spmm_w4a4 failed: code {rc}")
    return Y


def spmm_f16(s: Stream, Xh: np.ndarray, threads: int = 0) -> np.ndarray:
    """fp64 reference r[N][M] for an fp16 stream and fp16 X [N][K].
    threads > 0 splits the rows over that many threads (same result)."""
    Xh = np.ascontiguousarray(Xh, np.float16).view(np.uint16)
    N = Xh.shape[0]
    Y = np.zeros((N, s.M), np.float64)
    if threads > 0:
        rc = lib().or_spmm_f16_mt(_p(s.bitmaps), _p(s.offsets), _p(s.payload), s.M, s.K, _p(Xh), N, _p(Y), threads)
    else:
        rc = lib().or_spmm_f16(_p(s.bitmaps), _p(s.offsets), _p(s.payload), s.M, s.K, _p(Xh), N, _p(Y))
    if rc != OK:
        raise ValueError(f"oracle spmm_f16 failed: code {rc}")
    return Y


def spmm_w4a4_one(s: Stream, Xp: np.ndarray, m: int, n: int) -> int:
    Xp = np.ascontiguousarray(Xp, dtype=np.uint8)
    return int(lib().or_spmm_w4a4_one(_p(s.bitmaps), _p(s.offsets), _p(s.payload), s.K, _p(Xp), m, n))


def spmm_f16_one(s: Stream, Xh: np.ndarray, m: int, n: int) -> float:
    Xh = np.ascontiguousarray(Xh, np.float16).view(np.uint16)
    return float(lib().or_spmm_f16_one(_p(s.bitmaps), _p(s.offsets), _p(s.payload), s.K, _p(Xh), m, n))


def fp16_error(y: np.ndarray, r: np.ndarray) -> dict:
    """Tolerance metric for an fp16 result y against the fp64 reference r.

    err_i = |y_i - r_i| / max(|r_i|, 0.01 * rms(r)); the bar is max err <= 1e-2.
    The floor keeps outputs that cancel to near zero (whose relative error is
    unbounded for any fp32-accumulated, fp16-rounded result) from deciding
    the verdict; the unfloored maximum and the normwise error are reported
    alongside.
    """
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    if r.size == 0:
        return dict(max_rel_floored=0.0, max_rel_unfloored=0.0, normwise=0.0, nonfinite=0)
    rms = float(np.sqrt(np.mean(r * r)))
    floor = max(0.01 * rms, np.finfo(np.float64).tiny)
    d = np.abs(y - r)
    floored = d / np.maximum(np.abs(r), floor)
    with np.errstate(divide="ignore", invalid="ignore"):
        unf = np.where(r != 0, d / np.abs(r), np.where(d == 0, 0.0, np.inf))
    rn = float(np.max(np.abs(r)))
    return dict(max_rel_floored=float(np.max(floored)), max_rel_unfloored=float(np.max(unf)),
                normwise=float(np.max(d) / rn) if rn > 0 else float(np.max(d)),
                nonfinite=int(np.count_nonzero(~np.isfinite(y))))


def dequant_f16(Y: np.ndarray, scale_w: np.ndarray, scale_x: np.ndarray) -> np.ndarray:
    """The Dequant step after the int4 SpMM (UnionSparse, Fig. 2: the int32
    result goes back to fp16), with one fp32 scale per output channel (row m
    of W) and one per token (column n of X), as the fused epilogue computes it:

        Yh[n][m] = fp16( fp32( fp32(Y[n][m]) * scale_w[m] ) * scale_x[n] )

    each operation rounded to nearest even, in this order. numpy's float32
    arithmetic is IEEE binary32 with that rounding, and its float32 -> float16
    conversion rounds to nearest even; overflow gives +-inf. Returns the fp16
    array [N][M]."""
    Y = np.asarray(Y)
    sw = np.asarray(scale_w, np.float32)
    sx = np.asarray(scale_x, np.float32)
    N, M = Y.shape
    assert sw.shape == (M,) and sx.shape == (N,)
    out = np.empty((N, M), np.float16)
    with np.errstate(over="ignore"):
        for n in range(N):
            a = Y[n].astype(np.float32) * sw          # fp32(y) * scale_w, rounded in fp32
            b = a * sx[n]                             # ... * scale_x, rounded in fp32
            out[n] = b.astype(np.float16)             # one rounding to fp16
    return out
