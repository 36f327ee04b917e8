"""The W2A4 oracle (2-bit weights, int4 activations) against its pins: the
layout golden, the BT64 oracle's index part, round trips, brute force and
closed forms; and planted mistakes in copies of it that the pins must catch."""
import inspect
import json
import os
import sys
import types

import numpy as np
import pytest

import oracle
import workloads
from oracle import w2 as _w2

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pin_w2_layout_golden(W2=_w2):
    g = json.load(open(os.path.join(GOLDEN, "w2_payload_layout.json")))
    s = W2.encode(np.array([g["W_row"]], np.int8))
    assert int(s.bitmaps[0]) == int(g["bitmap"], 16)
    assert [int(o) for o in s.offsets] == g["offsets"]
    assert [f"{b:02X}" for b in s.payload] == g["payload_bytes_hex"]
    codes = [int(c, 2) for c in g["codes"]]
    assert [v & 3 for v in s.values] == codes


def pin_w2_index_equals_bt64(W2=_w2):
    """The words and offsets do not depend on the value width: they equal the
    int4 oracle encoder's for the same nonzero pattern."""
    for seed, (M, K, keep) in enumerate([(3, 64, 0.5), (5, 130, 0.3), (7, 1, 0.9), (4, 200, 0.05)]):
        p = workloads.random_int2_problem(seed, M, K, 1, keep=keep)
        s = W2.encode(p.W)
        ref = oracle.encode(p.W)       # the same pattern, read as int4 values
        assert [int(x) for x in s.bitmaps] == [int(x) for x in ref.bitmaps]
        assert [int(x) for x in s.offsets] == [int(x) for x in ref.offsets]


def pin_w2_roundtrip(W2=_w2):
    for seed, (M, K, keep) in enumerate([(1, 1, 1.0), (9, 65, 0.5), (17, 300, 0.3), (4, 128, 1.0), (6, 63, 0.0)]):
        p = workloads.random_int2_problem(100 + seed, M, K, 1, keep=keep)
        s = W2.encode(p.W)
        assert len(s.payload) == (s.nnz + 3) // 4
        assert np.array_equal(W2.decode(s), p.W)
        if s.nnz % 4:
            assert s.payload[-1] >> (2 * (s.nnz % 4)) == 0


def pin_w2_matmul_bruteforce(W2=_w2):
    p = workloads.random_int2_problem(7, 5, 70, 3, keep=0.6)
    Y = W2.spmm_w2a4(W2.decode(W2.encode(p.W)), p.X)
    for n in range(3):
        for m in range(5):
            assert Y[n, m] == sum(int(p.W[m, k]) * int(p.X[n, k]) for k in range(70))


def pin_w2_closed_forms(W2=_w2):
    # every weight -2 against every activation -8: 16 per column; the identity-like -1 diagonal
    W = np.full((3, 100), -2, np.int8)
    X = np.full((2, 100), -8, np.int8)
    assert (W2.spmm_w2a4(W2.decode(W2.encode(W)), X) == 1600).all()
    I = -np.eye(40, dtype=np.int8)
    X = workloads.int4_activations(np.random.default_rng(2), (4, 40))
    assert np.array_equal(W2.spmm_w2a4(W2.decode(W2.encode(I)), X), -X.astype(np.int32))


def pin_w2_range():
    for bad in (2, -3, 7):
        with pytest.raises(ValueError):
            _w2.encode(np.array([[bad]], np.int8))


PINS = [pin_w2_layout_golden, pin_w2_index_equals_bt64, pin_w2_roundtrip, pin_w2_matmul_bruteforce,
        pin_w2_closed_forms]


@pytest.mark.parametrize("pin", PINS + [pin_w2_range], ids=lambda f: f.__name__)
def test_w2_pin(pin):
    pin()


W2_MUTANTS = [
    ("high_bits_first", [("out[e // 4] |= (int(v) & 3) << (2 * (e % 4))", "out[e // 4] |= (int(v) & 3) << (6 - 2 * (e % 4))"),
                         ("code = (data[e // 4] >> (2 * (e % 4))) & 3", "code = (data[e // 4] >> (6 - 2 * (e % 4))) & 3")]),
    ("no_sign_extension", [("vals.append(code - 4 if code >= 2 else code)", "vals.append(code)")]),
    ("bit_order_reversed", [("word |= 1 << j\n", "word |= 1 << (63 - j)\n"), ("if (word >> j) & 1:", "if (word >> (63 - j)) & 1:")]),
    ("offset_before_append", [("            offs.append(len(vals))", "            offs.append(len(vals) - (1 if vals else 0))")]),
    ("x_transposed", [("Y = np.asarray(W, np.int64) @ np.asarray(X, np.int64).T", "Y = np.asarray(W, np.int64) @ np.asarray(X, np.int64)[:, ::-1].T")]),
]


@pytest.mark.parametrize("name,edits", W2_MUTANTS, ids=[m[0] for m in W2_MUTANTS])
def test_w2_pins_catch_mutant(name, edits):
    src = inspect.getsource(_w2)
    for old, new in edits:
        assert old in src, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("w2_mutant")
    sys.modules["w2_mutant"] = mod
    caught = []
    try:
        exec(compile(src, "<w2 mutant>", "exec"), mod.__dict__)
        for pin in PINS:
            try:
                pin(W2=mod)
            except (AssertionError, IndexError, ValueError):
                caught.append(pin.__name__)
    finally:
        del sys.modules["w2_mutant"]
    assert caught, f"no pin catches mutant {name}"
