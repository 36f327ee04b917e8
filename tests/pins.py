"""Pins for the CPU oracle: facts fixed by the pages or by mathematics.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
the fact it checks. ``test_oracle.py`` runs them against the oracle;
``test_oracle_mutants.py`` runs them against deliberately broken copies of
the oracle to show that each planted mistake is caught by at least one pin.

None of these re-types the oracle's own formulas: the expected values come
from the pages' worked examples (golden files), from numpy's exact integer
matmul / float64 matmul / float16 conversion (library routines), from
brute-force Python loops on tiny inputs, or from closed forms.
"""
from __future__ import annotations

import json
import os

import numpy as np

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _row_from_words(words, value=1):
    """A 1 x 64*len(words) int4 row with nonzero `value` exactly where the words have set bits
    (bit j of word t <-> column 64t+j, the LSB-first order of the Fig. 7 example)."""
    K = 64 * len(words)
    W = np.zeros((1, K), np.int8)
    for t, w in enumerate(words):
        for j in range(64):
            if (w >> j) & 1:
                W[0, 64 * t + j] = value
    return W


def pin_fig7_offsets():
    g = _golden("fig7_union_bitmap_words.json")
    words = [int(x, 16) for x in g["words"]]
    for w in words:
        assert oracle.popcount64(w) == g["active_per_word"]
    assert sum(oracle.popcount64(w) for w in words) == g["P_t"]
    assert g["Q"] * g["P_t"] == g["next_offset_Q4"]
    s = oracle.encode(_row_from_words(words))
    assert [int(b) for b in s.bitmaps] == words, "bitmap words differ from the Fig. 7 packing"
    assert [int(o) for o in s.offsets] == g["single_area_offsets_if_each_word_is_one_tile"]
    assert oracle.validate(s) == 0


def pin_fig9c_segment():
    g = _golden("fig9c_segment_rank.json")
    word = int(g["word_value_lsb_first"], 16)
    # the display string, position 0 first, is the LSB-first reading of the word
    assert word == sum(1 << j for j, c in enumerate(g["segment_display"]) if c == "1")
    for j, r in zip(g["active_positions"], g["ranks"]):
        assert oracle.rank(word, j) == r
    # encode a row with distinct values at the active positions: the word and the
    # payload order (b, b+1, b+2, b+3) must follow
    vals = [3, -5, 7, -8]
    W = np.zeros((1, 64), np.int8)
    for j, v in zip(g["active_positions"], vals):
        W[0, j] = v
    s = oracle.encode(W)
    assert int(s.bitmaps[0]) == word
    assert [int(v) for v in oracle.decode(s)[0, g["active_positions"]]] == vals
    codes = [v & 0xF for v in vals]
    assert [int(b) for b in s.payload] == [codes[0] | codes[1] << 4, codes[2] | codes[3] << 4]


def pin_payload_layout():
    g = _golden("payload_nibble_layout.json")
    W = np.array([g["W_row"]], np.int8)
    s = oracle.encode(W)
    assert int(s.bitmaps[0]) == int(g["bitmap"], 16)
    assert [int(o) for o in s.offsets] == g["offsets"]
    assert [f"{int(b):02X}" for b in s.payload] == g["payload_bytes_hex"]


def pin_x_unpack():
    g = _golden("x_int4_packing.json")
    Xp = np.array([int(h, 16) for h in g["packed_hex"]], np.uint8)
    X = oracle.unpack_x4(Xp, g["N"], g["K"])
    assert X.tolist() == g["X_rows"]


def pin_popcount_rank_bruteforce():
    rng = np.random.default_rng(123)
    words = [0, 1, 1 << 63, (1 << 64) - 1, 0x2D, 0xAAAAAAAAAAAAAAAA]
    words += [int(x) for x in rng.integers(0, 2**63, size=40, dtype=np.uint64)]
    words += [int(x) | (1 << 63) for x in rng.integers(0, 2**63, size=10, dtype=np.uint64)]
    for w in words:
        assert oracle.popcount64(w) == bin(w).count("1")
        for j in range(64):
            assert oracle.rank(w, j) == bin(w & ((1 << j) - 1)).count("1")


_SHAPES = [(1, 1), (1, 63), (3, 64), (2, 65), (4, 127), (5, 128), (3, 130), (7, 200), (1, 0), (0, 5)]


def pin_roundtrip_and_invariants():
    for i, (M, K) in enumerate(_SHAPES):
        for keep in (0.0, 0.3, 0.5, 1.0):
            p = workloads.random_int4_problem(1000 + i, M, K, 1, keep=keep)
            s = oracle.encode(p.W)
            assert oracle.validate(s) == 0
            assert np.array_equal(oracle.decode(s), p.W)
            nnz = int(np.count_nonzero(p.W))
            assert s.nnz == nnz
            assert sum(bin(int(w)).count("1") for w in s.bitmaps) == nnz
            assert s.payload.nbytes == (nnz + 1) // 2
            if keep == 1.0 and K % 64 == 0 and M * K > 0:
                assert all(int(w) == (1 << 64) - 1 for w in s.bitmaps)


def _naive(W, X):
    M, K = W.shape
    N = X.shape[0]
    Y = [[0] * M for _ in range(N)]
    for n in range(N):
        for m in range(M):
            acc = 0
            for k in range(K):
                acc += int(W[m, k]) * int(X[n, k])
            Y[n][m] = acc
    return np.array(Y, np.int64).reshape(N, M)


def _pack_x_for_test(X):
    """Packs int4 activations for the oracle input, from the layout golden's rule
    (checked against the golden file below before use)."""
    N, K = X.shape
    out = np.zeros((N, (K + 1) // 2), np.uint8)
    for n in range(N):
        for k in range(K):
            c = int(X[n, k]) & 0xF
            out[n, k // 2] |= c if k % 2 == 0 else c << 4
    return out


def pin_test_packer_matches_golden():
    g = _golden("x_int4_packing.json")
    got = _pack_x_for_test(np.array(g["X_rows"], np.int8)).reshape(-1)
    assert [f"{int(b):02X}" for b in got] == g["packed_hex"]


def pin_matmul_tiny_bruteforce():
    for i, (M, K, N) in enumerate([(1, 1, 1), (3, 63, 2), (4, 64, 5), (2, 65, 3), (5, 127, 1), (3, 130, 4)]):
        p = workloads.random_int4_problem(2000 + i, M, K, N, keep=0.5)
        s = oracle.encode(p.W)
        Y = oracle.spmm_w4a4(s, _pack_x_for_test(p.X), N)
        assert np.array_equal(Y.astype(np.int64), _naive(p.W, p.X))


def pin_matmul_numpy():
    for i, (M, K, N, keep) in enumerate([(64, 512, 8, 0.5), (37, 1000, 3, 0.3), (16, 64 * 9 + 17, 32, 0.7)]):
        p = workloads.random_int4_problem(3000 + i, M, K, N, keep=keep)
        s = oracle.encode(p.W)
        Y = oracle.spmm_w4a4(s, _pack_x_for_test(p.X), N)
        ref = (p.W.astype(np.int64) @ p.X.astype(np.int64).T).T
        assert np.array_equal(Y.astype(np.int64), ref)
        # one-element sampler agrees with the full product
        rng = np.random.default_rng(i)
        for _ in range(10):
            m, n = int(rng.integers(0, M)), int(rng.integers(0, N))
            assert oracle.spmm_w4a4_one(s, _pack_x_for_test(p.X), m, n) == ref[n, m]


def pin_special_cases():
    # W = 0: empty payload, Y = 0
    W = np.zeros((5, 130), np.int8)
    s = oracle.encode(W)
    assert s.nnz == 0 and s.payload.nbytes == 0 and all(int(o) == 0 for o in s.offsets)
    X = workloads.random_int4_problem(7, 1, 130, 3).X
    assert not oracle.spmm_w4a4(s, _pack_x_for_test(X), 3).any()
    # W = c * I: Y = c * X (restricted to the first M columns of K)
    for c in (-8, -1, 3, 7):
        M = K = 96
        W = (np.eye(M, K, dtype=np.int64) * c).astype(np.int8)
        X = workloads.random_int4_problem(8, 1, K, 4).X
        Y = oracle.spmm_w4a4(oracle.encode(W), _pack_x_for_test(X), 4)
        assert np.array_equal(Y.astype(np.int64), c * X.astype(np.int64)[:, :M])
    # all -8 weights at a random mask, X all -8: Y[n][m] = 64 * nnz(row m)
    p = workloads.random_int4_problem(9, 11, 200, 2, keep=0.6)
    W = np.where(p.W != 0, np.int8(-8), np.int8(0)).astype(np.int8)
    X = np.full((2, 200), -8, np.int8)
    Y = oracle.spmm_w4a4(oracle.encode(W), _pack_x_for_test(X), 2)
    rownnz = np.count_nonzero(W, axis=1)
    assert np.array_equal(Y.astype(np.int64), np.stack([64 * rownnz] * 2))
    # density 1 -> dense product
    p = workloads.random_int4_problem(10, 9, 192, 3, keep=1.0)
    Y = oracle.spmm_w4a4(oracle.encode(p.W), _pack_x_for_test(p.X), 3)
    assert np.array_equal(Y.astype(np.int64), (p.W.astype(np.int64) @ p.X.astype(np.int64).T).T)


def pin_validator_rejects_corruption():
    p = workloads.random_int4_problem(11, 6, 150, 1, keep=0.5)
    s = oracle.encode(p.W)
    assert oracle.validate(s) == 0
    bm = s.bitmaps.copy(); bm[3] ^= np.uint64(1 << 5)
    assert oracle.validate_arrays(0, bm, s.offsets, s.payload, s.M, s.K) == 2
    off = s.offsets.copy(); off[0] = 1
    assert oracle.validate_arrays(0, s.bitmaps, off, s.payload, s.M, s.K) == 1
    assert oracle.validate_arrays(0, s.bitmaps, s.offsets, np.concatenate([s.payload, [0]]).astype(np.uint8), s.M, s.K) == 3
    # a bit past K in a last tile (K=150 -> columns 150..191 of tile 2 must be zero)
    W = np.zeros((1, 150), np.int8); W[0, 149] = 1
    s2 = oracle.encode(W)
    bm = s2.bitmaps.copy(); bm[2] |= np.uint64(1 << 30)
    off = s2.offsets.copy(); off[3] += 1
    pl = np.array([0x11], np.uint8)
    assert oracle.validate_arrays(0, bm, off, pl, 1, 150) == 4
    # odd count with a nonzero trailing high nibble
    W = np.zeros((1, 64), np.int8); W[0, 0] = 1
    s3 = oracle.encode(W)
    pl = s3.payload.copy(); pl[0] |= 0x50
    assert oracle.validate_arrays(0, s3.bitmaps, s3.offsets, pl, 1, 64) == 5
    # a stored zero value
    W = np.zeros((1, 64), np.int8); W[0, 0] = 1; W[0, 1] = 2
    s4 = oracle.encode(W)
    pl = s4.payload.copy(); pl[0] &= 0x0F
    assert oracle.validate_arrays(0, s4.bitmaps, s4.offsets, pl, 1, 64) == 6


def pin_encoder_errors():
    W = np.zeros((2, 10), np.int8); W[1, 3] = 8
    assert oracle.encode_rc(W, 0)[0] == oracle.E_RANGE
    W[1, 3] = -9
    assert oracle.encode_rc(W, 0)[0] == oracle.E_RANGE
    W = np.ones((2, 10), np.int8)
    rc, nnz, nbytes = oracle.encode_rc(W, 0, payload_cap=9)
    assert rc == oracle.E_CAPACITY and nnz == 20 and nbytes == 10
    rc, nnz, nbytes = oracle.encode_rc(W, 0, payload_cap=10)
    assert rc == oracle.OK


def pin_f16_conversion_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits], np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def pin_f16_zero_semantics():
    W = np.array([[0.0, -0.0, 1.5, np.nan, 6.1e-5, -2.0]], np.float16)
    s = oracle.encode(W)
    assert int(s.bitmaps[0]) == 0b111100
    assert s.nnz == 4
    d = oracle.decode(s)
    assert np.array_equal(d[0, [2, 4, 5]], W[0, [2, 4, 5]]) and np.isnan(d[0, 3])
    assert d[0, 0] == 0 and d[0, 1] == 0


def pin_f16_matmul_numpy():
    for i, (M, K, N) in enumerate([(33, 200, 1), (17, 64 * 5, 32), (8, 63, 4)]):
        p = workloads.random_fp16_problem(4000 + i, M, K, N)
        s = oracle.encode(p.W)
        assert oracle.validate(s) == 0
        r = oracle.spmm_f16(s, p.X)
        ref = (p.W.astype(np.float64) @ p.X.astype(np.float64).T).T
        assert np.allclose(r, ref, rtol=1e-12, atol=1e-15)
        rng = np.random.default_rng(i)
        for _ in range(5):
            m, n = int(rng.integers(0, M)), int(rng.integers(0, N))
            assert abs(oracle.spmm_f16_one(s, p.X, m, n) - ref[n, m]) <= 1e-12 * (abs(ref[n, m]) + 1e-3)



def pin_fp16_error():
    """The fp16 pass/fail metric (floored elementwise relative error, its
    unfloored maximum, the normwise error and the non-finite count) on vectors
    whose values are worked out by hand here."""
    import math
    fn = oracle.fp16_error
    # the floor decides: rms(r) = sqrt(84 / 4) = sqrt(21), floor = 0.01 sqrt(21);
    # the zero reference with |y - r| = 0.01 gives 0.01 / (0.01 sqrt(21)) = 1 / sqrt(21)
    e = fn(np.array([2.02, -4.0, 0.01, 7.9]), np.array([2.0, -4.0, 0.0, 8.0]))
    assert math.isclose(e["max_rel_floored"], 1.0 / math.sqrt(21.0), rel_tol=1e-12), e
    assert e["max_rel_unfloored"] == math.inf, e           # a zero reference with a nonzero error
    assert math.isclose(e["normwise"], 0.1 / 8.0, rel_tol=1e-9), e
    assert e["nonfinite"] == 0, e
    # signs: the largest error is y below a negative r (|-2.5 - (-2)| / |-2| = 0.25);
    # rms(r) = sqrt(7) puts the floor (0.026) below every |r|, so floored = unfloored
    e = fn(np.array([0.9, -2.5, 4.0]), np.array([1.0, -2.0, 4.0]))
    assert math.isclose(e["max_rel_floored"], 0.25, rel_tol=1e-12), e
    assert math.isclose(e["max_rel_unfloored"], 0.25, rel_tol=1e-12), e
    assert math.isclose(e["normwise"], 0.5 / 4.0, rel_tol=1e-12), e
    # non-finite outputs are counted (and never pass as small errors)
    e = fn(np.array([np.inf, np.nan, 1.0]), np.array([1.0, 1.0, 1.0]))
    assert e["nonfinite"] == 2, e
    # exact results, and the empty case
    e = fn(np.array([0.0, 0.0]), np.array([0.0, 0.0]))
    assert e == dict(max_rel_floored=0.0, max_rel_unfloored=0.0, normwise=0.0, nonfinite=0), e
    e = fn(np.zeros(0), np.zeros(0))
    assert e == dict(max_rel_floored=0.0, max_rel_unfloored=0.0, normwise=0.0, nonfinite=0), e
    # a 2-D result is judged over all its elements
    e = fn(np.array([[1.0, 2.0], [3.0, 4.4]]), np.array([[1.0, 2.0], [3.0, 4.0]]))
    assert math.isclose(e["max_rel_floored"], 0.1, rel_tol=1e-12), e


# ---- dequant epilogue (int32 -> fp16 with per-channel and per-token scales) ----

def _ulp16(x):
    """Spacing of binary16 numbers at magnitude x (subnormal spacing 2^-24 below 2^-14)."""
    x = abs(float(x))
    if x < 2.0 ** -14:
        return 2.0 ** -24
    return 2.0 ** (np.floor(np.log2(x)) - 10)


def pin_dequant_closed_form():
    """Against the exact product y * scale_w * scale_x (fp64 holds it to 2^-53):
    three roundings to fp32 (int -> fp32 and two products) and one to fp16
    leave at most half an fp16 ulp plus 3 fp32 units in the last place."""
    rng = np.random.default_rng(31)
    N, M = 7, 300
    Y = rng.integers(-(1 << 26), 1 << 26, size=(N, M)).astype(np.int32)
    Y[:, :50] = rng.integers(-3000, 3000, size=(N, 50))
    sw = np.exp(rng.uniform(np.log(1e-6), np.log(1e-2), size=M)).astype(np.float32)
    sx = np.exp(rng.uniform(np.log(1e-3), np.log(1.0), size=N)).astype(np.float32)
    out = oracle.dequant_f16(Y, sw, sx).astype(np.float64)
    exact = Y.astype(np.float64) * sw.astype(np.float64)[None, :] * sx.astype(np.float64)[:, None]
    checked = 0
    for n in range(N):
        for m in range(M):
            e = exact[n, m]
            if abs(e) > 65504.0:
                assert np.isinf(out[n, m]) or abs(out[n, m]) == 65504.0
                continue
            tol = 0.5 * _ulp16(e) * (1 + 2.0 ** -10) + 3 * 2.0 ** -24 * abs(e)
            assert abs(out[n, m] - e) <= tol, (n, m, out[n, m], e)
            checked += 1
    assert checked > N * M // 2


# Hand-derived binary16 results (IEEE 754 round to nearest, ties to even):
# (y, scale_w, scale_x, expected bits)
DEQUANT_CASES = [
    (1, 1.0, 1 + 2.0 ** -11, 0x3C00),        # halfway between 1 and 1 + 2^-10: even mantissa, 1.0
    (1, 1.0, 1 + 3 * 2.0 ** -11, 0x3C02),    # halfway between 1 + 2^-10 and 1 + 2^-9: to 1 + 2^-9
    (3, 1.0, 2.0 ** -26, 0x0001),            # 0.75 x 2^-24 rounds to the smallest subnormal
    (1, 2.0 ** -25, 1.0, 0x0000),            # exactly half the smallest subnormal: ties to +0
    (65504, 1.0, 1.0, 0x7BFF),               # largest finite fp16
    (65519, 1.0, 1.0, 0x7BFF),               # below the halfway point to 2^16
    (65520, 1.0, 1.0, 0x7C00),               # halfway: ties to even, 2^16, overflows to +inf
    (-2, 0.5, -1.0, 0x3C00),                 # signs: (-2 * 0.5) * -1 = +1
    (0, -1.0, 1.0, 0x8000),                  # 0 * -1 = -0.0
    (7, -0.25, 2.0, 0xC300),                 # -3.5 = -1.75 x 2^1: sign 1, exponent 16, fraction 0b11 << 8
    (1 << 30, 2.0 ** 100, 2.0 ** -120, 0x7C00),   # 2^130 overflows fp32 before the token scale: +inf
]


def pin_dequant_rounding_cases():
    for (y, sw, sx, bits) in DEQUANT_CASES:
        got = oracle.dequant_f16(np.array([[y]], np.int32), np.array([sw], np.float32),
                                 np.array([sx], np.float32)).view(np.uint16)[0, 0]
        assert int(got) == bits, (y, sw, sx, hex(int(got)), hex(bits))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
