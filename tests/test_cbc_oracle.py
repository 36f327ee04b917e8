"""The Tiled-CBC / dynamic-pruning oracle against the pages' Fig. 4(a)
example, the storage formula, round trips and closed forms of the
thresholded product; and planted mistakes in copies of it."""
import inspect
import json
import os
import sys
import types

import numpy as np
import pytest

from oracle import cbc as _cbc

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand_w(seed, M, K, keep):
    rng = np.random.default_rng(seed)
    W = rng.normal(0, 1, size=(M, K)).astype(np.float16)
    W[rng.random((M, K)) >= keep] = 0
    return W


def pin_cbc_fig4a(C=_cbc):
    g = json.load(open(os.path.join(GOLDEN, "fig4a_colinfo.json")))
    tm, tk = g["tile"]
    W = np.zeros((tm, tk), np.float16)
    v = 1.0
    for c, bm in enumerate(g["column_bitmaps"]):
        b = int(bm, 16)
        for r in range(tm):
            if (b >> r) & 1:
                W[r, c] = v
                v += 1
    s = C.encode(W, tile=(tm, tk))
    assert [int(s.bitmaps[0, c, 0]) for c in range(tk)] == [int(b, 16) for b in g["column_bitmaps"]]
    assert [[int(x) >> 16, int(x) & 0xFFFF] for x in s.colinfo[0]] == g["colinfo_offset_nnz"]
    # values in tile-column order: column by column, rows ascending
    assert [float(x) for x in s.values] == [float(i) for i in range(1, 12)]


def pin_cbc_storage_formula(C=_cbc):
    for (M, K, keep) in [(256, 64, 0.4), (512, 192, 0.1), (256, 128, 1.0)]:
        s = C.encode(_rand_w(M + K, M, K, keep))
        tm, tk = C.TILE
        n_gt = (M // tm) * (K // tk)
        n_bm = M * K // 64
        nnz = int(np.count_nonzero(_rand_w(M + K, M, K, keep)))
        assert s.storage_bytes() == 4 * (n_gt + 1) + 4 * n_gt * tk + 8 * n_bm + 2 * nnz


def pin_cbc_roundtrip_and_metadata(C=_cbc):
    for (M, K, keep) in [(1, 1, 1.0), (300, 130, 0.3), (256, 64, 0.0), (77, 200, 0.9)]:
        W = _rand_w(M * 3 + K, M, K, keep)
        W.reshape(-1)[::17] = np.float16(-0.0)          # negative zeros are not stored
        s = C.encode(W)
        assert np.array_equal(C.decode(s), W)
        counts = [[bin(int(w)).count("1") for w in s.bitmaps[g, c]] for g in range(s.n_gt) for c in range(C.TILE[1])]
        cnt = np.array([sum(x) for x in counts]).reshape(s.n_gt, C.TILE[1])
        assert np.array_equal(s.colinfo & 0xFFFF, cnt)
        starts = np.concatenate([np.zeros((s.n_gt, 1), np.int64), np.cumsum(cnt, axis=1)[:, :-1]], axis=1)
        assert np.array_equal(s.colinfo >> 16, starts)
        assert np.array_equal(np.diff(s.tile_offsets), cnt.sum(axis=1))
    # IEEE -0.0 compares equal to 0: a matrix of negative zeros stores no value
    assert C.encode(np.full((4, 8), -0.0, np.float16)).values.size == 0


def pin_cbc_thresholded_product(C=_cbc):
    rng = np.random.default_rng(9)
    M, K, N = 9, 40, 3
    W = _rand_w(1, M, K, 0.5)
    X = rng.normal(0, 1, size=(N, K)).astype(np.float16)
    tau = float(np.median(np.abs(X.astype(np.float32))))
    r = C.spmspv_reference(W, X, tau)
    for n in range(N):
        for m in range(M):
            want = sum(float(W[m, k]) * float(X[n, k]) for k in range(K) if abs(float(X[n, k])) > tau)
            assert abs(r[n, m] - want) <= 1e-12 * max(1.0, abs(want))
    # tau = 0 is the plain product; an unreachable threshold gives zeros
    plain = (W.astype(np.float64) @ X.astype(np.float64).T).T
    assert np.allclose(C.spmspv_reference(W, X, 0.0), plain, rtol=0, atol=1e-12)
    assert (C.spmspv_reference(W, X, 1e9) == 0).all()
    # a value exactly at the threshold is pruned
    X2 = np.zeros((1, K), np.float16)
    X2[0, 3] = 0.5
    W2 = np.ones((2, K), np.float16)
    assert (C.spmspv_reference(W2, X2, 0.5) == 0).all() and (C.spmspv_reference(W2, X2, 0.49) == 0.5).all()


def pin_cbc_skipped_columns_do_not_matter(C=_cbc):
    rng = np.random.default_rng(4)
    M, K, N = 20, 100, 2
    W = _rand_w(2, M, K, 0.6)
    X = rng.normal(0, 1, size=(N, K)).astype(np.float16)
    tau = 0.8
    skip = C.skipped_columns(X, tau)
    assert skip.any() and (~skip).any()
    W2 = W.copy()
    W2[:, skip] = rng.normal(0, 5, size=(M, int(skip.sum()))).astype(np.float16)
    assert np.array_equal(C.spmspv_reference(W, X, tau), C.spmspv_reference(W2, X, tau))


PINS = [pin_cbc_fig4a, pin_cbc_storage_formula, pin_cbc_roundtrip_and_metadata, pin_cbc_thresholded_product,
        pin_cbc_skipped_columns_do_not_matter]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_cbc_pin(pin):
    pin()


CBC_MUTANTS = [
    ("threshold_keeps_equal", [("> np.float32(tau)", ">= np.float32(tau)")]),
    ("colinfo_fields_swapped", [("ci[g, c] = (col_start << 16) | count", "ci[g, c] = (count << 16) | col_start"),
                                ("base = int(s.tile_offsets[g]) + (int(s.colinfo[g, c]) >> 16)",
                                 "base = int(s.tile_offsets[g]) + (int(s.colinfo[g, c]) & 0xFFFF)"),
                                ("assert rank == int(s.colinfo[g, c]) & 0xFFFF", "assert rank == int(s.colinfo[g, c]) >> 16")]),
    ("bitmap_msb_first", [("words[r // 64] |= 1 << (r % 64)", "words[r // 64] |= 1 << (63 - r % 64)"),
                          ("if (int(s.bitmaps[g, c, r // 64]) >> (r % 64)) & 1:",
                           "if (int(s.bitmaps[g, c, r // 64]) >> (63 - r % 64)) & 1:")]),
    ("offset_per_gtile_dropped", [("offs.append(len(vals))", "offs.append(len(vals) - start)")]),
    ("negative_zero_stored", [("return (bits & 0x7FFF) != 0", "return bits != 0")]),
    ("mask_ignores_magnitude", [("np.abs(np.asarray(X, np.float16).astype(np.float32))",
                                 "np.asarray(X, np.float16).astype(np.float32)")]),
]


@pytest.mark.parametrize("name,edits", CBC_MUTANTS, ids=[m[0] for m in CBC_MUTANTS])
def test_cbc_pins_catch_mutant(name, edits):
    src = inspect.getsource(_cbc)
    for old, new in edits:
        assert old in src, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("cbc_mutant")
    sys.modules["cbc_mutant"] = mod
    caught = []
    try:
        exec(compile(src, "<cbc mutant>", "exec"), mod.__dict__)
        for pin in PINS:
            try:
                pin(C=mod)
            except (AssertionError, IndexError, ValueError):
                caught.append(pin.__name__)
    finally:
        del sys.modules["cbc_mutant"]
    assert caught, f"no pin catches mutant {name}"
