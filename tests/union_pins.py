"""Pins for the IE-BME oracle (``oracle.union``): facts fixed by the pages'
worked example of Fig. 7, by closed forms and by brute force on tiny tiles.

Each ``pin_*`` takes the oracle module as ``U`` and raises AssertionError when
it disagrees with the fact it checks. ``test_union_oracle.py`` runs them on
the oracle, and on copies of it with planted mistakes, each of which must be
caught by at least one pin.
"""
from __future__ import annotations

import itertools
import json
import os

import numpy as np

import oracle
from oracle import union as _union

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_int4(rng, M, K, keep):
    v = rng.integers(1, 8, size=(M, K)) * rng.choice([-1, 1], size=(M, K))
    v = np.where(v == -8, -8, v)
    return np.where(rng.random((M, K)) < keep, v, 0).astype(np.int8)


def _union_count_direct(tile, ra, ca):
    """Active logical positions of a tile, counted position by position."""
    H, KL = tile.shape
    h, w = H // ra, KL // ca
    n = 0
    for i in range(h):
        for j in range(w):
            if any(tile[a * h + i, c * w + j] != 0 for a in range(ra) for c in range(ca)):
                n += 1
    return n


def pin_union_fig7_words_and_offset(U=_union):
    """Fig. 7: mask rows 0x36DB, 0x6DB6, 0x5B6D, 0xB6DA (leftmost bit lowest)
    in an 8 x 32 tile with 2 x 2 areas: P_t = 40 and the next offset is 160."""
    g = _golden("fig7_union_bitmap_words.json")
    words = [int(x, 16) for x in g["words"]]
    H, KL = 8, 32
    h, w = H // 2, KL // 2
    tile = np.zeros((H, KL), np.int16)
    for i, word in enumerate(words):
        for j in range(w):
            if (word >> j) & 1:
                q = (i + j) % 4                      # spread the nonzeros over the areas
                a, c = divmod(q, 2)
                tile[a * h + i, c * w + j] = 1 + q
    enc = U.encode(tile, 2, 2, lt=(H, KL))
    packed = sum(wd << (16 * i) for i, wd in enumerate(words))
    assert [int(x) for x in enc.ubitmaps[0]] == [packed], "union bitmap differs from the Fig. 7 words"
    assert [int(o) for o in enc.offsets] == [0, g["next_offset_Q4"]]
    assert enc.nvals == g["Q"] * g["P_t"]
    # a second, empty tile to the right keeps the offset (no payload for it)
    enc2 = U.encode(np.concatenate([tile, np.zeros_like(tile)], axis=1), 2, 2, lt=(H, KL))
    assert [int(o) for o in enc2.offsets] == [0, g["next_offset_Q4"], g["next_offset_Q4"]]


def pin_union_aligned_zero_emission(U=_union):
    """Fig. 7's red-framed position [1, 30, 59, 0]: one rank, four aligned
    values, the zero stored; an all-zero position emits nothing."""
    g = _golden("fig7_aligned_zero_emission.json")
    H, KL = g["illustrated_lt"]
    ra, ca = g["R_A"], g["C_A"]
    h, w = H // ra, KL // ca
    tile = np.zeros((H, KL), np.int16)
    tile[0 * h + 0, 0 * w + 3] = 2                   # an earlier active position: rank 0
    pos = (1, 5)                                     # the framed position: rank 1
    for q, v in enumerate(g["area_values"]):
        a, c = divmod(q, ca)
        tile[a * h + pos[0], c * w + pos[1]] = v
    zpos = (2, 7)
    for q, v in enumerate(g["all_zero_values"]):
        a, c = divmod(q, ca)
        tile[a * h + zpos[0], c * w + zpos[1]] = v
    enc = U.encode(tile, ra, ca, lt=(H, KL))
    word = int(enc.ubitmaps[0][0])
    assert (word >> (pos[0] * w + pos[1])) & 1 == g["union_bit"]
    assert (word >> (zpos[0] * w + zpos[1])) & 1 == g["all_zero_union_bit"]
    P = 2
    assert [int(o) for o in enc.offsets] == [0, ra * ca * P]
    for q, v in enumerate(g["emitted_per_area"]):
        assert enc.values[0 + q * P + 1] == v, f"area {q} stream at rank 1"
    assert enc.values == [2, 1, 0, 30, 0, 59, 0, 0]


def pin_union_popcount_inclusion_exclusion(U=_union):
    """P_t equals |union of the areas' nonzero sets| by inclusion-exclusion."""
    rng = np.random.default_rng(11)
    for ra, ca in [(2, 2), (1, 1), (2, 1), (1, 2), (4, 1), (1, 4), (2, 4), (4, 4)]:
        for keep in (0.02, 0.1, 0.3, 0.7):
            tile = _rand_int4(rng, 16, 64, keep)
            h, w = 16 // ra, 64 // ca
            sets = [tile[a * h:(a + 1) * h, c * w:(c + 1) * w] != 0 for a in range(ra) for c in range(ca)]
            total = 0
            for k in range(1, len(sets) + 1):
                for S in itertools.combinations(range(len(sets)), k):
                    inter = np.logical_and.reduce([sets[s] for s in S])
                    total += (-1) ** (k + 1) * int(inter.sum())
            enc = U.encode(tile, ra, ca)
            P = (int(enc.offsets[1]) - int(enc.offsets[0])) // (ra * ca)
            assert P == total
            assert sum(bin(int(x)).count("1") for x in enc.ubitmaps[0]) == total


def pin_union_q1_is_bt64(U=_union):
    """One area over 1 x 64 tiles is the plain bitmap format: words, offsets
    and payload equal the BT64 oracle encoder's."""
    rng = np.random.default_rng(5)
    for (M, K, keep) in [(3, 64, 0.5), (5, 130, 0.3), (7, 1, 0.9), (2, 200, 0.05)]:
        W = _rand_int4(rng, M, K, keep)
        enc = U.encode(W, 1, 1, lt=(1, 64))
        ref = oracle.encode(W)
        assert [int(x) for x in enc.ubitmaps.reshape(-1)] == [int(x) for x in ref.bitmaps]
        assert [int(x) for x in enc.offsets] == [int(x) for x in ref.offsets]
        assert enc.payload() == bytes(np.asarray(ref.payload, dtype=np.uint8)[:(enc.nvals + 1) // 2])


def pin_union_value_addresses(U=_union):
    """CV[o_t + q P_t + rank] holds area q's value at the rank-th active
    position (rank from numpy's flat nonzero index of the mask)."""
    rng = np.random.default_rng(3)
    W = _rand_int4(rng, 37, 150, 0.2)
    ra, ca = 2, 2
    enc = U.encode(W, ra, ca)
    bands, T = U.lt_grid(37, 150)
    h, w = 8, 32
    for b in range(bands):
        for c in range(T):
            t = b * T + c
            tile = np.zeros((16, 64), np.int64)
            blk = W[16 * b:16 * b + 16, 64 * c:64 * c + 64]
            tile[:blk.shape[0], :blk.shape[1]] = blk
            nz = np.zeros((h, w), bool)
            for a in range(ra):
                for cc in range(ca):
                    nz |= tile[a * h:(a + 1) * h, cc * w:(cc + 1) * w] != 0
            active = np.flatnonzero(nz.reshape(-1))
            P = active.size
            o = int(enc.offsets[t])
            assert int(enc.offsets[t + 1]) - o == 4 * P
            for rank, f in enumerate(active):
                i, j = divmod(int(f), w)
                for a in range(ra):
                    for cc in range(ca):
                        assert enc.values[o + (a * ca + cc) * P + rank] == tile[a * h + i, cc * w + j]


def pin_union_roundtrip(U=_union):
    """decode(encode(W)) == W, ragged shapes, with and without permutations."""
    rng = np.random.default_rng(7)
    for (M, K) in [(16, 64), (37, 150), (1, 1), (5, 65), (33, 129)]:
        W = _rand_int4(rng, M, K, 0.3)
        for ra, ca in [(2, 2), (1, 1), (2, 1), (1, 2), (4, 4)]:
            assert np.array_equal(U.decode(U.encode(W, ra, ca)), W)
            bands, T = U.lt_grid(M, K)
            perms = [list(rng.permutation(16)) for _ in range(bands * T)]
            enc = U.encode(W, ra, ca, perms=perms)
            assert np.array_equal(U.decode(enc), W)
            assert [U.rowpos_perm(int(x), 16) for x in enc.rowpos] == [[int(v) for v in p] for p in perms]


def _partitions(rows, ra):
    """Every partition of `rows` into groups of ra, each group sorted, groups in
    order of their first row (the canonical order), lexicographic order."""
    if not rows:
        yield ()
        return
    r0 = rows[0]
    for others in itertools.combinations(rows[1:], ra - 1):
        grp = (r0,) + others
        rest = [r for r in rows if r not in grp]
        for tail in _partitions(rest, ra):
            yield (grp,) + tail


def _perm_costs(tile, perms, ra, ca):
    """Active logical positions of tile[perm] for a batch of row permutations,
    counted with a reshape of the whole batch (no per-position loop)."""
    H, KL = tile.shape
    h, w = H // ra, KL // ca
    nz = (tile != 0)[np.asarray(perms)]                  # (P, H, KL)
    act = nz.reshape(len(perms), ra, h, ca, w).any(axis=(1, 3))
    return act.sum(axis=(1, 2))


def _perm_cost(tile, pi, ra, ca):
    return int(_perm_costs(tile, [list(pi)], ra, ca)[0])


def pin_reorder_dp_equals_bruteforce(U=_union):
    """The DP optimum equals the minimum over every row permutation (tiny
    tiles), its permutation attains it, and its partition is the
    lexicographically first optimal one (the tie rule)."""
    rng = np.random.default_rng(13)
    cases = [(4, 8, 2, 1), (4, 8, 2, 2), (6, 8, 2, 2), (6, 12, 3, 1), (8, 16, 2, 2), (8, 8, 4, 1),
             (8, 16, 2, 4), (8, 16, 4, 2)]
    for (H, KL, ra, ca) in cases:
        allp = np.array(list(itertools.permutations(range(H))))
        for keep in (0.1, 0.25, 0.5):
            tile = _rand_int4(rng, H, KL, keep)
            pi, cost = U.reorder_tile(tile != 0, ra, ca)
            assert sorted(pi) == list(range(H))
            best = int(_perm_costs(tile, allp, ra, ca).min())
            assert cost == best, (H, KL, ra, ca, keep)
            assert _perm_cost(tile, pi, ra, ca) == cost
            assert _perm_cost(tile, pi, ra, ca) == _union_count_direct(tile[pi, :], ra, ca)
            G = H // ra
            parts = list(_partitions(list(range(H)), ra))
            perms = [[part[g][p] for p in range(ra) for g in range(G)] for part in parts]
            costs = _perm_costs(tile, perms, ra, ca)
            first = perms[int(np.flatnonzero(costs == best)[0])]
            assert pi == first, "DP partition is not the lexicographically first optimum"


def pin_reorder_identity_at_one_row_partition(U=_union):
    """With R_A = 1 every grouping costs the same; the result is the identity."""
    rng = np.random.default_rng(17)
    for ca in (1, 2, 4):
        tile = _rand_int4(rng, 16, 64, 0.3)
        pi, cost = U.reorder_tile(tile != 0, 1, ca)
        assert pi == list(range(16))
        assert cost == _union_count_direct(tile, 1, ca)


def pin_reorder_pairs_identical_rows(U=_union):
    """Closed form: 16 rows carrying 8 disjoint 4-column patterns, each on two
    rows placed apart. Pairing equal rows costs 8 x 4 = 32, any other pairing
    more; the DP must find exactly those pairs."""
    rng = np.random.default_rng(19)
    sigma = np.array([0, 1, 2, 3, 4, 5, 6, 7] * 2)
    rng.shuffle(sigma)
    tile = np.zeros((16, 64), np.int8)
    for r in range(16):
        k = int(sigma[r])
        tile[r, 4 * k:4 * k + 4] = 3
    pi, cost = U.reorder_tile(tile != 0, 2, 2)
    assert cost == 32
    groups = {tuple(sorted((pi[g], pi[8 + g]))) for g in range(8)}
    want = {tuple(sorted(np.flatnonzero(sigma == k).tolist())) for k in range(8)}
    assert groups == want
    # the identity grouping pairs row r with row r + 8
    ident = sum(4 if sigma[r] == sigma[r + 8] else 8 for r in range(8))
    assert U.encode(tile, 2, 2).nvals == 4 * ident
    assert U.encode(tile, 2, 2, perms=[pi]).nvals == 4 * 32


def pin_reorder_keeps_values_and_never_grows(U=_union):
    rng = np.random.default_rng(23)
    W = _rand_int4(rng, 40, 200, 0.15)
    perms = U.reorder(W, 2, 2)
    e0, e1 = U.encode(W, 2, 2), U.encode(W, 2, 2, perms=perms)
    assert e1.nvals <= e0.nvals
    nz0 = sorted(v for v in e0.values if v != 0)
    nz1 = sorted(v for v in e1.values if v != 0)
    assert nz0 == nz1 == sorted(int(v) for v in W[W != 0])
    assert np.array_equal(U.decode(e1), W)


def pin_union_int4_packing(U=_union):
    """Payload bytes: element e in byte e // 2, low nibble first (the layout
    golden of the BT64 payload)."""
    g = _golden("payload_nibble_layout.json")
    vals = [v for v in g["W_row"] if v != 0]
    assert [f"{b:02X}" for b in U.pack_int4(vals)] == g["payload_bytes_hex"]
    assert U.unpack_int4(U.pack_int4(vals), len(vals)) == vals


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
