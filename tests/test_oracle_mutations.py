"""Planted mistakes in a copy of the oracle must turn the pins red.

Each mutation edits one expression of oracle.c in a temporary copy, builds
it with gcc, swaps it in for the oracle's library, and runs the pin suite.
A mutation that no pin catches would mean the pins do not cover that part
of the oracle.  Nothing here touches a GPU.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_argmax as argmax_pins
from tests import test_oracle_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTATIONS = {
    "swap_nibbles": ("(k % 2 == 0) ? (byte & 0x0f) : (byte >> 4)",
                     "(k % 2 == 0) ? (byte >> 4) : (byte & 0x0f)"),
    "q8_group_index": ("scale[n * groups + k / 64]", "scale[n * groups + (k / 64 + 1) % groups]"),
    "q4_group_index": ("scale[n * groups + k / 32]", "scale[n * groups + k / 64]"),
    "drop_min": ("(double)c * s + mn", "(double)c * s"),
    "min_sign": ("(double)c * s + mn", "(double)c * s - mn"),
    "reverse_x": ("x[i * ldx + k]", "x[i * ldx + (K - 1 - k)]"),
    "fp16_exponent": ("expo - 25", "expo - 24"),
    "fp16_subnormal": ("ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    "bf16_implicit_one": ("(128 + frac)", "(frac)"),
    "abs_sum": ("abs_sum += fabs(w * xv);", "abs_sum += fabs(w) * xv;"),
    "code_as_unsigned": ("double code = (double)q[n * K + k];",
                         "double code = (double)(uint8_t)q[n * K + k];"),
    "row_stride": ("y[i * ldy + n] = sum;", "y[i * ldy + (n0 + n1 - 1 - n)] = sum;"),
    "q8g128_group_index": ("scale[n * groups + k / 128]", "scale[n * groups + (k / 64) % groups]"),
    "q8pc_row_scale": ("double s = f32_bits_to_double(scale[n]);",
                       "double s = f32_bits_to_double(scale[N - 1 - n]);"),
    "f32_exponent": ("expo - 150", "expo - 149"),
    "f32_implicit_one": ("(0x800000u + frac)", "(frac)"),
    "argmax_last_on_ties": ("} else if (v > best_v) {", "} else if (v >= best_v) {"),
    "argmax_ignores_nan": ("            if (isnan(v)) {", "            if (0) {"),
    "argmax_scans_past_nan": ("for (int64_t n = 1; n < N && !best_nan; ++n)",
                              "for (int64_t n = 1; n < N; ++n)"),
    "argmax_row_stride": ("double v = f32_bits_to_double(x[i * ldx + n]);",
                          "double v = f32_bits_to_double(x[n]);"),
}

PIN_TESTS = [
    (pins.test_fp16_decoder_matches_numpy_on_every_pattern, False),
    (pins.test_bf16_decoder_matches_numpy_on_every_pattern, False),
    (pins.test_q8g64_two_group_worked_example, True),
    (pins.test_q4g32_two_group_worked_example, True),
    (pins.test_zero_scales_give_exact_zero, False),
    (pins.test_q4_zero_scale_reduces_to_min_times_group_sums, False),
    (pins.test_constant_codes_closed_form, False),
    (pins.test_brute_force_q8_every_int8_value, False),
    (pins.test_brute_force_q4_every_code, False),
    (pins.test_one_hot_pins_group_and_nibble_index, False),
    (pins.test_abs_sum_bounds_and_sign_cases, False),
    (pins.test_f32_decoder_matches_numpy, False),
    (pins.test_q8g128_two_group_worked_example, True),
    (pins.test_q8pc_two_row_worked_example, True),
    (pins.test_q8g128_equals_q8g64_with_duplicated_scales, False),
    (pins.test_q8pc_equals_q8g64_with_row_constant_scales, False),
    (pins.test_q8g128_one_hot_group_index, False),
    (argmax_pins.test_argmax_hand_written_rows, False),
    (lambda: argmax_pins.test_argmax_matches_numpy_on_random_rows(1000), False),
    (argmax_pins.test_argmax_split_and_combine_gives_the_row_winner, False),
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path, golden_dir):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor not found: " + old
    mutated = tmp_path / ("oracle_%s.c" % name)
    mutated.write_text(src.replace(old, new))
    so = tmp_path / ("liboracle_%s.so" % name)
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c99", "-o", str(so),
                           str(mutated), "-lm"])
    real = oracle._load()
    lib = ctypes.CDLL(str(so))
    for fn in ("oracle_q8g64", "oracle_q4g32", "oracle_q8g128", "oracle_q8pc",
               "oracle_half_to_double", "oracle_bf16_to_double", "oracle_f32_to_double",
               "oracle_argmax_f32"):
        getattr(lib, fn).argtypes = getattr(real, fn).argtypes
        getattr(lib, fn).restype = getattr(real, fn).restype
    caught = []
    oracle._lib = lib
    try:
        for fn, wants_dir in PIN_TESTS:
            try:
                fn(golden_dir) if wants_dir else fn()
            except AssertionError:
                caught.append(getattr(fn, "__name__", "pin"))
    finally:
        oracle._lib = real
    assert caught, "no pin caught mutation " + name
