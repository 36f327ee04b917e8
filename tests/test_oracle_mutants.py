"""Plants plausible mistakes in a copy of the oracle (on the CPU) and checks
that the pins catch each one: a dropped term, a wrong sign, index or bit
order, a transposed operand, a wrong constant."""
import os
import subprocess

import pytest

import oracle
import pins

_SRC = os.path.join(os.path.dirname(os.path.abspath(oracle.__file__)), "bsp_oracle.c")

# (name, [(original text, mutated text), ...]); every original must occur in the source.
MUTANTS = [
    ("nibble_order_swapped", [
        ("if (e % 2 == 0) payload[e / 2]", "if (e % 2 == 1) payload[e / 2]"),
        ("int code = (e % 2 == 0) ?", "int code = (e % 2 == 1) ?"),
        ("else            payload[e / 2] = (uint8_t)((payload[e / 2] & 0x0F) | (code << 4));",
         "else            payload[e / 2] = (uint8_t)((payload[e / 2] & 0x0F) | (code << 4)); /*m*/"),
    ]),
    ("rank_skips_bit0", [("for (int i = 0; i < j; ++i)", "for (int i = 1; i < j; ++i)")]),
    ("bit_order_reversed", [
        ("word |= (uint64_t)1 << j;", "word |= (uint64_t)1 << (63 - j);"),
        ("int bit = (int)((word >> j) & 1u);", "int bit = (int)((word >> (63 - j)) & 1u);"),
    ]),
    ("sign_extension_off_by_one", [("return code >= 8 ? code - 16 : code;", "return code > 8 ? code - 16 : code;")]),
    ("x_transposed", [("acc += (int64_t)Wd[m * K + k] * (int64_t)Xd[n * K + k];",
                       "acc += (int64_t)Wd[m * K + k] * (int64_t)Xd[(k % N) * K + (k / N) + 0 * n];")]),
    ("matmul_drops_last_k", [("for (int64_t k = 0; k < K; ++k)\n                acc += (int64_t)Wd",
                              "for (int64_t k = 0; k + 1 < K; ++k)\n                acc += (int64_t)Wd")]),
    ("decode_uses_previous_offset", [("int64_t e = (int64_t)offsets[g] + or_rank(word, j);",
                                      "int64_t e = (int64_t)offsets[g > 0 ? g - 1 : 0] + or_rank(word, j);")]),
    ("offsets_shifted_by_one", [("if (offsets) offsets[g] = (uint32_t)off;",
                                   "if (offsets) offsets[g] = (uint32_t)(off > 0 ? off - 1 : 0);")]),
    ("popcount_misses_bit63", [("for (int j = 0; j < 64; ++j)\n        if ((w >> j) & 1u) c++;",
                                "for (int j = 0; j < 63; ++j)\n        if ((w >> j) & 1u) c++;")]),
    ("f16_exponent_bias", [("expo - 25", "expo - 24")]),
    ("f16_subnormal_scale", [("ldexp((double)frac, -24)", "ldexp((double)frac, -25)")]),
    ("f16_negative_zero_stored", [("return (h & 0x7FFF) == 0;", "return h == 0;")]),
    ("f16_product_sign_dropped", [("acc += or_f16_to_f64(Wd[m * K + k]) * or_f16_to_f64(Xh[n * K + k]);",
                                   "acc += fabs(or_f16_to_f64(Wd[m * K + k])) * or_f16_to_f64(Xh[n * K + k]);")]),
]


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, edits, tmp_path):
    src = open(_SRC).read()
    for old, new in edits:
        assert old in src, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new)
    c = tmp_path / "mutant.c"
    c.write_text(src)
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-shared", "-fPIC", str(c), "-o", str(so), "-lm"])
    prev = oracle.swap_library(str(so))
    caught = []
    try:
        for pin in pins.ALL_PINS:
            try:
                pin()
            except AssertionError:
                caught.append(pin.__name__)
            except ValueError:
                caught.append(pin.__name__ + "(error)")
    finally:
        oracle.swap_library(None)
        oracle._lib = prev
    assert caught, f"no pin catches mutant {name}"


# Planted mistakes in the fp16 tolerance metric (a Python function of the
# oracle): each must make at least one pin fail.
F16_METRIC_MUTANTS = [
    ("rms_of_y", "np.mean(r * r)", "np.mean(y * y)"),
    ("floor_on_numerator", "floored = d / np.maximum(np.abs(r), floor)",
     "floored = np.maximum(d, floor) / np.maximum(np.abs(r), floor)"),
    ("abs_dropped_from_difference", "d = np.abs(y - r)", "d = (y - r)"),
    ("abs_dropped_from_reference", "floored = d / np.maximum(np.abs(r), floor)",
     "floored = d / np.maximum(r, floor)"),
    ("floor_factor", "0.01 * rms", "0.1 * rms"),
    ("normwise_over_y", "rn = float(np.max(np.abs(r)))", "rn = float(np.max(np.abs(y)))"),
    ("nonfinite_not_counted", "np.count_nonzero(~np.isfinite(y))", "np.count_nonzero(np.isnan(y))"),
]


@pytest.mark.parametrize("name,old,new", F16_METRIC_MUTANTS, ids=[m[0] for m in F16_METRIC_MUTANTS])
def test_pins_catch_fp16_metric_mutant(name, old, new):
    import inspect
    import textwrap
    src = textwrap.dedent(inspect.getsource(oracle.fp16_error))
    assert old in src, f"mutation anchor not found: {old!r}"
    ns = dict(oracle.__dict__)
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    real = oracle.fp16_error
    oracle.fp16_error = ns["fp16_error"]
    try:
        with pytest.raises(AssertionError):
            pins.pin_fp16_error()
    finally:
        oracle.fp16_error = real


# Planted mistakes in the dequant epilogue's oracle (a Python function).
DEQUANT_MUTANTS = [
    ("scales_applied_in_other_order", [("a = Y[n].astype(np.float32) * sw ", "a = Y[n].astype(np.float32) * sx[n] "),
                                       ("b = a * sx[n] ", "b = a * sw ")]),
    ("token_scale_dropped", [("b = a * sx[n] ", "b = a * 1 ")]),
    ("channel_scale_reversed", [("a = Y[n].astype(np.float32) * sw ", "a = Y[n].astype(np.float32) * sw[::-1] ")]),
    ("truncated_to_fp16", [("out[n] = b.astype(np.float16)", "out[n] = np.trunc(b * 1024) / 1024")]),
    ("saturates_instead_of_inf", [("out[n] = b.astype(np.float16)", "out[n] = np.clip(b, -65504, 65504).astype(np.float16)")]),
]


@pytest.mark.parametrize("name,edits", DEQUANT_MUTANTS, ids=[m[0] for m in DEQUANT_MUTANTS])
def test_pins_catch_dequant_mutant(name, edits):
    import inspect
    import textwrap
    src = textwrap.dedent(inspect.getsource(oracle.dequant_f16))
    for old, new in edits:
        assert old in src, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new)
    ns = dict(oracle.__dict__)
    exec(compile(src, "<mutant>", "exec"), ns)
    real = oracle.dequant_f16
    oracle.dequant_f16 = ns["dequant_f16"]
    caught = []
    try:
        for pin in (pins.pin_dequant_closed_form, pins.pin_dequant_rounding_cases):
            try:
                pin()
            except (AssertionError, ValueError, IndexError):
                caught.append(pin.__name__)
    finally:
        oracle.dequant_f16 = real
    assert caught, f"no pin catches mutant {name}"
