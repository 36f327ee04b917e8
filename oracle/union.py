"""IE-BME oracle: the union-mask encoding and bitmap-aware row reordering of
UnionSparse, written out plainly in numpy and Python -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module. The product library never loads it and
shares no code with it.

What it follows (UnionSparse, Sec. V-A "IE-BME Representation", Fig. 7, and
Sec. V-B "Bitmap-Aware Row Reordering", Eq. 3-5 and Algorithm 1):

* A weight matrix is cut into local tiles (LTs) of H_L x K_L (16 x 64; the
  figure draws 8 x 32). Each LT is split into an R_A x C_A grid of Q = R_A C_A
  areas of (H_L / R_A) x (K_L / C_A). Area q = a C_A + c holds tile rows
  [a H_L/R_A, (a+1) H_L/R_A) and columns [c K_L/C_A, (c+1) K_L/C_A).
* Logical position (i, j) groups the Q values at (i, j) of every area. Its
  union-mask bit is set when any of them is nonzero; P_t is the number of set
  bits.
* The mask is scanned row-major and packed into 64-bit words, the leftmost
  position of a row in the least significant bit.
* Every set position gets a compact rank (the number of set positions before
  it in row-major order) and emits one value from every area, zeros
  included; area q's value goes to CV[o_t + q P_t + rank].
* o_t = sum of Q P over the LTs before t.
* Row reordering groups the tile's rows into H_L / R_A groups of R_A rows; the
  cost of a group is the number of logical positions it activates (Eq. 3-4);
  a subset DP (Eq. 5) finds a partition of minimum total cost; groups are
  sorted and the permutation lists, partition by partition, the p-th row of
  every group.

Readings taken where the pages leave a step open (each also listed in the
design notes):

* LTs are ordered row-major over the matrix (band of H_L rows, then column
  of K_L), as the BT64 tiles are. A tile that runs past M or K is padded
  with zero rows and columns, which never set a mask bit.
* Area numbering is row-major over the R_A x C_A grid.
* Ties in the DP are broken by taking, at every state, the first candidate
  group in ascending lexicographic order that attains the minimum. The
  partition found is then the lexicographically first optimal one, and it
  is already in the canonical order.
* The permutation is stored by its inverse: ``rowpos`` nibble r is the
  reordered position of original tile row r (four bits per row, so
  H_L <= 16). Without reordering rowpos is the identity.
* int4 values are packed two per byte, element e in byte e // 2, low nibble
  first, as the BT64 payload is.
"""
from __future__ import annotations

import itertools
from dataclasses import dataclass
from functools import lru_cache
from typing import List, Optional, Sequence, Tuple

import numpy as np

LT = (16, 64)


def lt_grid(M: int, K: int, lt: Tuple[int, int] = LT) -> Tuple[int, int]:
    """(row bands, tile columns) of an M x K matrix cut into LTs."""
    H, KL = lt
    return (M + H - 1) // H, (K + KL - 1) // KL


def local_tile(W: np.ndarray, band: int, col: int, lt: Tuple[int, int] = LT) -> np.ndarray:
    """LT (band, col) of W as an H_L x K_L array, zero past the matrix."""
    H, KL = lt
    t = np.zeros((H, KL), dtype=W.dtype)
    blk = W[band * H:(band + 1) * H, col * KL:(col + 1) * KL]
    t[:blk.shape[0], :blk.shape[1]] = blk
    return t


def areas(tile: np.ndarray, ra: int, ca: int) -> List[np.ndarray]:
    """The Q = ra * ca areas of a tile, area q = a * ca + c."""
    H, KL = tile.shape
    h, w = H // ra, KL // ca
    return [tile[a * h:(a + 1) * h, c * w:(c + 1) * w] for a in range(ra) for c in range(ca)]


def union_mask(tile: np.ndarray, ra: int, ca: int) -> np.ndarray:
    """B_t(i, j): whether any area has a nonzero at logical position (i, j)."""
    acc = None
    for ar in areas(tile, ra, ca):
        nz = ar != 0
        acc = nz if acc is None else (acc | nz)
    return acc


def tile_streams(tile: np.ndarray, ra: int, ca: int):
    """(mask, P_t, streams): streams[q] lists area q's value at every set
    logical position in row-major order (zeros included)."""
    mask = union_mask(tile, ra, ca)
    ars = areas(tile, ra, ca)
    h, w = mask.shape
    streams: List[List[int]] = [[] for _ in ars]
    for i in range(h):
        for j in range(w):
            if mask[i, j]:
                for q, ar in enumerate(ars):
                    streams[q].append(int(ar[i, j]))
    return mask, int(mask.sum()), streams


def pack_mask(mask: np.ndarray) -> List[int]:
    """Row-major scan of the mask into 64-bit words, the first position of a
    row in the lowest bit."""
    flat = mask.reshape(-1)
    nwords = (flat.size + 63) // 64
    words = [0] * nwords
    for f, bit in enumerate(flat):
        if bit:
            words[f // 64] |= 1 << (f % 64)
    return words


def unpack_mask(words: Sequence[int], shape: Tuple[int, int]) -> np.ndarray:
    h, w = shape
    out = np.zeros(h * w, dtype=bool)
    for f in range(h * w):
        out[f] = (int(words[f // 64]) >> (f % 64)) & 1
    return out.reshape(h, w)


def pack_int4(values: Sequence[int]) -> bytes:
    """Element e in byte e // 2, the low nibble for even e; v & 0xF."""
    out = bytearray((len(values) + 1) // 2)
    for e, v in enumerate(values):
        code = int(v) & 0xF
        if e % 2 == 0:
            out[e // 2] |= code
        else:
            out[e // 2] |= code << 4
    return bytes(out)


def unpack_int4(data: bytes, n: int) -> List[int]:
    vals = []
    for e in range(n):
        b = data[e // 2]
        code = b & 0xF if e % 2 == 0 else b >> 4
        vals.append(code - 16 if code >= 8 else code)
    return vals


def rowpos_word(pi: Sequence[int]) -> int:
    """The inverse of a permutation pi (pi[p] = original row at reordered
    position p) as nibbles: nibble r = the position of row r."""
    w = 0
    for p, r in enumerate(pi):
        w |= (p & 0xF) << (4 * int(r))
    return w


def rowpos_perm(word: int, H: int) -> List[int]:
    """pi from a rowpos word."""
    pi = [0] * H
    for r in range(H):
        pi[(int(word) >> (4 * r)) & 0xF] = r
    return pi


@dataclass
class UnionEncoding:
    ra: int
    ca: int
    lt: Tuple[int, int]
    M: int
    K: int
    ubitmaps: np.ndarray     # uint64 [nLT, words per LT]
    offsets: np.ndarray      # int64 [nLT + 1], in values (the format stores them as uint32)
    rowpos: np.ndarray       # uint64 [nLT]
    values: List[int]        # the Compressed Values array, one entry per value
    perms: List[List[int]]   # pi per LT (reordered position -> original row)

    @property
    def nvals(self) -> int:
        return len(self.values)

    def payload(self) -> bytes:
        return pack_int4(self.values)


def encode(W: np.ndarray, ra: int, ca: int, lt: Tuple[int, int] = LT,
           perms: Optional[Sequence[Sequence[int]]] = None) -> UnionEncoding:
    """IE-BME of W (M x K). perms[t] (optional) is the row permutation of LT t:
    row p of the reordered tile is row perms[t][p] of the original tile."""
    H, KL = lt
    assert H % ra == 0 and KL % ca == 0 and H <= 16
    M, K = W.shape
    bands, T = lt_grid(M, K, lt)
    Q = ra * ca
    words_per_lt = ((H // ra) * (KL // ca) + 63) // 64
    ub, offs, rp, vals, used = [], [0], [], [], []
    for b in range(bands):
        for c in range(T):
            t = b * T + c
            tile = local_tile(W, b, c, lt)
            pi = list(range(H)) if perms is None else [int(r) for r in perms[t]]
            assert sorted(pi) == list(range(H))
            tile = tile[pi, :]
            mask, P, streams = tile_streams(tile, ra, ca)
            words = pack_mask(mask)
            assert len(words) == words_per_lt
            ub.append(words)
            for q in range(Q):
                vals.extend(streams[q])
            offs.append(offs[-1] + Q * P)
            rp.append(rowpos_word(pi))
            used.append(pi)
    return UnionEncoding(ra, ca, lt, M, K, np.array(ub, dtype=np.uint64).reshape(bands * T, words_per_lt),
                         np.array(offs, dtype=np.int64),
                         np.array(rp, dtype=np.uint64), vals, used)


def decode(enc: UnionEncoding) -> np.ndarray:
    """Dense M x K matrix of an encoding: value CV[o_t + q P_t + rank] goes to
    logical position (i, j) of area q, then the reordering is undone."""
    H, KL = enc.lt
    ra, ca = enc.ra, enc.ca
    h, w = H // ra, KL // ca
    bands, T = lt_grid(enc.M, enc.K, enc.lt)
    out = np.zeros((bands * H, T * KL), dtype=np.int64)
    for b in range(bands):
        for c in range(T):
            t = b * T + c
            mask = unpack_mask([int(x) for x in enc.ubitmaps[t]], (h, w))
            P = int(mask.sum())
            o = int(enc.offsets[t])
            assert int(enc.offsets[t + 1]) - o == ra * ca * P
            re = np.zeros((H, KL), dtype=np.int64)
            rank = 0
            for i in range(h):
                for j in range(w):
                    if mask[i, j]:
                        for a in range(ra):
                            for cc in range(ca):
                                q = a * ca + cc
                                re[a * h + i, cc * w + j] = enc.values[o + q * P + rank]
                        rank += 1
            pi = rowpos_perm(int(enc.rowpos[t]), H)
            tile = np.zeros_like(re)
            tile[pi, :] = re
            out[b * H:(b + 1) * H, c * KL:(c + 1) * KL] = tile
    return out[:enc.M, :enc.K]


# ---- bitmap-aware row reordering (Sec. V-B) ----

def grouped_cost(nzmask: np.ndarray, rows: Sequence[int], ca: int) -> int:
    """c_t(r) of Eq. 3-4: the number of grouped columns j < K_L / C_A at which
    any of the group's rows has a nonzero at column j + c K_L / C_A."""
    H, KL = nzmask.shape
    w = KL // ca
    cost = 0
    for j in range(w):
        phi = False
        for r in rows:
            for c in range(ca):
                phi = phi or bool(nzmask[r, j + c * w])
        cost += int(phi)
    return cost


def reorder_tile(nzmask: np.ndarray, ra: int, ca: int) -> Tuple[List[int], int]:
    """Eq. 5 and Algorithm 1 of the pages for one tile: returns (pi, F(all rows)).
    pi[p * G + g] is row p of group g, G = H_L / R_A groups sorted
    lexicographically, rows inside a group ascending."""
    H = nzmask.shape[0]
    assert H % ra == 0
    cost = {}
    for grp in itertools.combinations(range(H), ra):
        cost[grp] = grouped_cost(nzmask, grp, ca)

    @lru_cache(maxsize=None)
    def F(S: int) -> Tuple[int, Tuple[int, ...]]:
        # (minimum cost on the rows in S, the chosen group containing min(S))
        if S == 0:
            return 0, ()
        rows = [r for r in range(H) if (S >> r) & 1]
        r0 = rows[0]
        best, arg = None, None
        for others in itertools.combinations(rows[1:], ra - 1):
            grp = (r0,) + others
            rest = S
            for r in grp:
                rest &= ~(1 << r)
            v = cost[grp] + F(rest)[0]
            if best is None or v < best:
                best, arg = v, grp
        return best, arg

    full = (1 << H) - 1
    total = F(full)[0]
    groups = []
    S = full
    while S:
        grp = F(S)[1]
        groups.append(tuple(sorted(grp)))
        for r in grp:
            S &= ~(1 << r)
    groups.sort()
    G = H // ra
    pi = [groups[g][p] for p in range(ra) for g in range(G)]
    return pi, total


def reorder(W: np.ndarray, ra: int, ca: int, lt: Tuple[int, int] = LT) -> List[List[int]]:
    """pi of every LT of W (row-major LT order)."""
    M, K = W.shape
    bands, T = lt_grid(M, K, lt)
    out = []
    for b in range(bands):
        for c in range(T):
            pi, _ = reorder_tile(local_tile(W, b, c, lt) != 0, ra, ca)
            out.append(pi)
    return out


def union_payload_values(W: np.ndarray, ra: int, ca: int, lt: Tuple[int, int] = LT,
                         perms: Optional[Sequence[Sequence[int]]] = None) -> int:
    """Sum of Q P_t over the LTs of W: the length of the Compressed Values array."""
    return encode(W, ra, ca, lt, perms).nvals
