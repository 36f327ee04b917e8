"""The IE-BME oracle against the pages' Fig. 7 example, closed forms and brute
force, and planted mistakes in copies of it that the pins must catch."""
import inspect
import sys
import types

import pytest

import union_pins
from oracle import union


@pytest.mark.parametrize("pin", union_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_union_pin(pin):
    pin()


# (name, [(original text, mutated text), ...]); every original must occur in oracle/union.py.
UNION_MUTANTS = [
    ("zero_emission_dropped", [("                for q, ar in enumerate(ars):\n                    streams[q].append(int(ar[i, j]))",
                                "                for q, ar in enumerate(ars):\n                    if ar[i, j] != 0:\n"
                                "                        streams[q].append(int(ar[i, j]))")]),
    ("offset_counts_positions_not_values", [("offs.append(offs[-1] + Q * P)", "offs.append(offs[-1] + P)")]),
    ("mask_bit_order_msb_first", [("words[f // 64] |= 1 << (f % 64)", "words[f // 64] |= 1 << (63 - f % 64)")]),
    ("areas_column_major", [("for a in range(ra) for c in range(ca)]", "for c in range(ca) for a in range(ra)]")]),
    ("union_is_intersection", [("acc = nz if acc is None else (acc | nz)", "acc = nz if acc is None else (acc & nz)")]),
    ("mask_scanned_column_major", [("flat = mask.reshape(-1)", "flat = mask.T.reshape(-1)")]),
    ("cost_ignores_other_column_areas", [("for c in range(ca):\n                phi = phi or bool(nzmask[r, j + c * w])",
                                          "for c in range(1):\n                phi = phi or bool(nzmask[r, j + c * w])")]),
    ("permutation_concatenated_by_group", [("pi = [groups[g][p] for p in range(ra) for g in range(G)]",
                                            "pi = [groups[g][p] for g in range(G) for p in range(ra)]")]),
    ("dp_keeps_last_minimum", [("if best is None or v < best:", "if best is None or v <= best:")]),
    ("dp_drops_group_cost", [("v = cost[grp] + F(rest)[0]", "v = F(rest)[0] + (cost[grp] if len(grp) > 99 else 0)")]),
    ("dp_maximises", [("if best is None or v < best:", "if best is None or v > best:")]),
    ("rowpos_stores_forward_perm", [("w |= (p & 0xF) << (4 * int(r))", "w |= (int(r) & 0xF) << (4 * p)")]),
    ("int4_high_nibble_first", [("        if e % 2 == 0:\n            out[e // 2] |= code\n",
                                 "        if e % 2 == 1:\n            out[e // 2] |= code\n"),
                                ("        else:\n            out[e // 2] |= code << 4",
                                 "        else:\n            out[e // 2] |= code << 4  # m")]),
]


@pytest.mark.parametrize("name,edits", UNION_MUTANTS, ids=[m[0] for m in UNION_MUTANTS])
def test_union_pins_catch_mutant(name, edits):
    src = inspect.getsource(union)
    for old, new in edits:
        assert old in src, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("union_mutant")
    mod.__file__ = union.__file__
    sys.modules["union_mutant"] = mod
    caught = []
    try:
        exec(compile(src, "<union mutant>", "exec"), mod.__dict__)
        for pin in union_pins.ALL_PINS:
            try:
                pin(U=mod)
            except (AssertionError, IndexError, KeyError, ValueError):
                caught.append(pin.__name__)
    finally:
        del sys.modules["union_mutant"]
    assert caught, f"no pin catches mutant {name}"
