"""Tiled-CBC oracle with dynamic activation pruning (SPDP) -- TEST
INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module. The product library never loads it and
shares no code with it.

What it follows (SPDP, "Unified Static-Dynamic Pruning for Efficient LLM
Inference", Sec. 4.1 "Tiled-CBC", Fig. 4(a), and Sec. 4.2, the decode-phase
spMspV kernel):

* The weight matrix is cut into GTiles of TILE_M x TILE_K, stored in
  row-major order. Inside a GTile each column is a TILE_M x 1 column tile:
  its nonzero pattern is TILE_M / 64 64-bit bitmap words (bit j of word w is
  row 64 w + j, the first row in the lowest bit), and its nonzeros are stored
  in row order; the columns of a GTile follow one another (column-major
  values inside the GTile).
* TileOffset[g] is the position of GTile g's first value in the Values array
  (N_GT + 1 entries, the last one NNZ).
* ColInfo packs two 16-bit fields per column of each GTile: the upper half is
  the column's first value relative to its GTile (TileOffset_Col), the lower
  half its number of nonzeros (NNZ_Column).
* Storage: 4 (N_GT + 1) + 4 N_GT TILE_K + 8 N_BM + 2 NNZ bytes.
* Decode with dynamic pruning: activation x[n][k] takes part only when its
  magnitude passes the threshold; a column none of whose activations pass is
  skipped (its bitmaps and values are not needed). The result is the product
  of W with the thresholded X.

Readings taken where the pages are silent (also listed in the design notes):

* TILE_M = 256 (the pages' column tile) and TILE_K = 64; a GTile past M or K
  is padded with zero rows and columns.
* An activation is kept when |x| > tau (tau >= 0, compared in fp32): tau = 0
  gives the plain product.
* fp16 values; the reference sum is exact (fp16 x fp16 products are exact in
  fp64).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Tuple

import numpy as np

TILE = (256, 64)


def _f16_nonzero(W: np.ndarray) -> np.ndarray:
    """fp16 +0 and -0 are zero; every other value (NaN included) is stored."""
    bits = np.asarray(W, np.float16).view(np.uint16)
    return (bits & 0x7FFF) != 0


@dataclass
class CBC:
    M: int
    K: int
    tile: Tuple[int, int]
    tile_offsets: np.ndarray   # int64 [N_GT + 1]
    colinfo: np.ndarray        # uint32 [N_GT, TILE_K]
    bitmaps: np.ndarray        # uint64 [N_GT, TILE_K, TILE_M // 64]
    values: np.ndarray         # float16 [NNZ]

    @property
    def n_gt(self) -> int:
        return int(self.colinfo.shape[0])

    def storage_bytes(self) -> int:
        """Bytes of the four arrays as stored (4-byte offsets and ColInfo,
        8-byte bitmap words, 2-byte values)."""
        return 4 * self.tile_offsets.size + 4 * self.colinfo.size + 8 * self.bitmaps.size + 2 * self.values.size


def grid(M: int, K: int, tile=TILE) -> Tuple[int, int]:
    tm, tk = tile
    return (M + tm - 1) // tm, (K + tk - 1) // tk


def encode(W: np.ndarray, tile=TILE) -> CBC:
    W = np.asarray(W, np.float16)
    M, K = W.shape
    tm, tk = tile
    assert tm % 64 == 0 or tm < 64
    nwords = max(1, tm // 64)
    gr, gc = grid(M, K, tile)
    nz = _f16_nonzero(W)
    offs = [0]
    ci = np.zeros((gr * gc, tk), np.uint32)
    bm = np.zeros((gr * gc, tk, nwords), np.uint64)
    vals = []
    for a in range(gr):
        for b in range(gc):
            g = a * gc + b
            start = len(vals)
            for c in range(tk):
                k = b * tk + c
                col_start = len(vals) - start
                count = 0
                words = [0] * nwords
                for r in range(tm):
                    m = a * tm + r
                    if m < M and k < K and nz[m, k]:
                        words[r // 64] |= 1 << (r % 64)
                        vals.append(W[m, k])
                        count += 1
                bm[g, c, :] = words
                ci[g, c] = (col_start << 16) | count
            offs.append(len(vals))
    return CBC(M, K, tuple(tile), np.array(offs, np.int64), ci, bm, np.array(vals, np.float16))


def decode(s: CBC) -> np.ndarray:
    """Dense fp16 matrix: value of row r, column c of GTile g is
    Values[TileOffset[g] + TileOffset_Col + (set bits of the column before r)]."""
    tm, tk = s.tile
    gr, gc = grid(s.M, s.K, s.tile)
    out = np.zeros((gr * tm, gc * tk), np.float16)
    for a in range(gr):
        for b in range(gc):
            g = a * gc + b
            for c in range(tk):
                base = int(s.tile_offsets[g]) + (int(s.colinfo[g, c]) >> 16)
                rank = 0
                for r in range(tm):
                    if (int(s.bitmaps[g, c, r // 64]) >> (r % 64)) & 1:
                        out[a * tm + r, b * tk + c] = s.values[base + rank]
                        rank += 1
                assert rank == int(s.colinfo[g, c]) & 0xFFFF
    return out[:s.M, :s.K]


def active_mask(X: np.ndarray, tau: float) -> np.ndarray:
    """Which activations take part: |x| > tau, compared in fp32."""
    return np.abs(np.asarray(X, np.float16).astype(np.float32)) > np.float32(tau)


def spmspv_reference(W: np.ndarray, X: np.ndarray, tau: float) -> np.ndarray:
    """fp64 reference [N][M] of W times the thresholded X (exact products,
    exact sum up to fp64 rounding)."""
    Xm = np.where(active_mask(X, tau), np.asarray(X, np.float16), np.float16(0)).astype(np.float64)
    return (np.asarray(W, np.float16).astype(np.float64) @ Xm.T).T


def skipped_columns(X: np.ndarray, tau: float) -> np.ndarray:
    """Columns none of whose activations pass the threshold."""
    return ~active_mask(X, tau).any(axis=0)
