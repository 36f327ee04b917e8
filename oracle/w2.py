"""W2A4 oracle: the bitmap-tiled format with 2-bit weights and int4
activations -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module. The product library never loads it and
shares no code with it.

UnionSparse evaluates its kernel under W2A4 quantization as well as W4A4
(Sec. VII, Fig. 11): the weights are 2-bit signed codes, the activations
4-bit. The format is the one of Sec. V-A with a single area per 1 x 64 tile,
exactly as for int4: one 64-bit word per tile (bit j set when column 64 t + j
holds a nonzero; the leftmost column in the lowest bit, Fig. 7), a prefix
offset per tile counting values, and the nonzeros in tile order. Only the
width of a stored value changes.

Readings taken where the pages are silent (also listed in the design notes):

* a 2-bit weight is a two's-complement code: 0b01 = 1, 0b10 = -2, 0b11 = -1
  (0 is never stored: a stored value is nonzero);
* payload element e sits in byte e // 4, at bits 2 (e % 4) and up (the
  lowest bits first, as the int4 payload puts element 0 in the low nibble);
  ceil(nnz / 4) bytes, unused high bits of the last byte zero;
* the product is the exact integer sum Y[n][m] = sum_k W[m][k] X[k][n].
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List

import numpy as np


@dataclass
class W2Stream:
    M: int
    K: int
    bitmaps: np.ndarray      # uint64 [M * T]
    offsets: np.ndarray      # int64 [M * T + 1]
    values: List[int]        # the nonzeros in tile order
    payload: bytes           # packed 2-bit codes

    @property
    def nnz(self) -> int:
        return len(self.values)


def pack2(values) -> bytes:
    """Element e in byte e // 4 at bit 2 (e % 4); code v & 3."""
    out = bytearray((len(values) + 3) // 4)
    for e, v in enumerate(values):
        out[e // 4] |= (int(v) & 3) << (2 * (e % 4))
    return bytes(out)


def unpack2(data: bytes, n: int) -> List[int]:
    vals = []
    for e in range(n):
        code = (data[e // 4] >> (2 * (e % 4))) & 3
        vals.append(code - 4 if code >= 2 else code)
    return vals


def encode(W: np.ndarray) -> W2Stream:
    """Words, offsets and payload of a 2-bit weight matrix (values in [-2, 1])."""
    W = np.asarray(W)
    if W.size and (W.min() < -2 or W.max() > 1):
        raise ValueError("2-bit weights must lie in [-2, 1]")
    M, K = W.shape
    T = (K + 63) // 64
    words, offs, vals = [], [0], []
    for m in range(M):
        for t in range(T):
            word = 0
            for j in range(64):
                k = 64 * t + j
                if k < K and W[m, k] != 0:
                    word |= 1 << j
                    vals.append(int(W[m, k]))
            words.append(word)
            offs.append(len(vals))
    return W2Stream(M, K, np.array(words, dtype=np.uint64), np.array(offs, dtype=np.int64), vals, pack2(vals))


def decode(s: W2Stream) -> np.ndarray:
    """Dense matrix of a stream: value of column 64 t + j is element
    offsets[g] + (set bits of the word below j)."""
    T = (s.K + 63) // 64
    vals = unpack2(s.payload, s.nnz)
    out = np.zeros((s.M, s.K), np.int64)
    for m in range(s.M):
        for t in range(T):
            g = m * T + t
            word = int(s.bitmaps[g])
            e = int(s.offsets[g])
            for j in range(64):
                if (word >> j) & 1:
                    out[m, 64 * t + j] = vals[e]
                    e += 1
    return out


def spmm_w2a4(W: np.ndarray, X: np.ndarray) -> np.ndarray:
    """Y int32 [N][M] = W X exactly (int64 sums, then int32)."""
    Y = np.asarray(W, np.int64) @ np.asarray(X, np.int64).T
    assert np.abs(Y).max(initial=0) < 2 ** 31
    return Y.T.astype(np.int32)
