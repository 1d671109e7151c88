"""Mutation check of the pins: plant plausible mistakes in a copy of the
oracle (on the CPU), build it, and require that some pin fails for each.

This shows the pins are sensitive to a dropped term, a wrong sign, a swapped
index or operand, a byte-lane slip and a precision loss -- not only that the
oracle agrees with itself.
"""
import os

import pytest

import oracle
import pins_ncc
import pins_xcorr

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    # u8 normalized correlation
    "ncc_lane_reversed": ("uint64_t t = trow[i];", "uint64_t t = trow[i ^ 3];", "ncc"),
    "ncc_signed_pixels": ("uint64_t p = row[i];", "uint64_t p = (uint64_t)(int64_t)(int8_t)row[i];", "ncc"),
    "ncc_dropped_mean_term": ("int64_t num = n * (int64_t)st - (int64_t)si * (int64_t)sum_t;",
                              "int64_t num = n * (int64_t)st;", "ncc"),
    "ncc_wrong_sign_var": ("int64_t vi = n * (int64_t)sq - (int64_t)si * (int64_t)si;",
                           "int64_t vi = n * (int64_t)sq + (int64_t)si * (int64_t)si;", "ncc"),
    "ncc_template_row_index": ("const uint8_t *trow = tmpl + (size_t)j * tw;",
                               "const uint8_t *trow = tmpl + (size_t)(th - 1 - j) * tw;", "ncc"),
    "ncc_square_uses_template": ("sq += p * p;", "sq += p * t;", "ncc"),
    "ncc_zero_var_rule": ("if (vi != 0 && vt != 0)", "if (vt != 0)", "ncc"),
    "ncc_single_precision": ("c = (double)num / sqrt((double)vi * (double)vt);",
                             "c = (float)num / sqrtf((float)vi * (float)vt);", "ncc"),
    "ncc_peak_last_of_ties": ("if (coef[k] > coef[best])", "if (coef[k] >= coef[best])", "ncc"),
    "ncc_peak_minimum": ("if (coef[k] > coef[best])", "if (coef[k] < coef[best])", "ncc"),
    # fp32 cross-correlation
    "xcorr_operands_swapped": ("one_shift(L, R, rows, cols, y - (rows - 1), x - (cols - 1), out + base + x,",
                               "one_shift(R, L, rows, cols, y - (rows - 1), x - (cols - 1), out + base + x,", "xcorr"),
    "xcorr_dy_sign": ("one_shift(L, R, rows, cols, y - (rows - 1), x - (cols - 1), out + base + x,",
                      "one_shift(L, R, rows, cols, (rows - 1) - y, x - (cols - 1), out + base + x,", "xcorr"),
    "xcorr_dropped_last_row": ("int i1 = dy > 0 ? rows - dy : rows;", "int i1 = dy > 0 ? rows - dy - 1 : rows - 1;", "xcorr"),
    "xcorr_float_accumulator": ("double s = 0.0, a = 0.0;", "float s = 0.0f; double a = 0.0;", "xcorr"),
    "xcorr_abs_signed": ("a += fabs(p);", "a += p;", "xcorr"),
}


def _build_mutant(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation site for {name} not found"
    src = tmp_path / f"{name}.c"
    src.write_text(text.replace(old, new))
    out = str(tmp_path / f"lib{name}.so")
    oracle.build(src=str(src), out=out, extra_flags=("-Wno-unused-variable", "-Wno-unused-but-set-variable"))
    return oracle._bind(out)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches_mutant(tmp_path, name):
    old, new, which = MUTANTS[name]
    lib = _build_mutant(tmp_path, name, old, new)
    pins = pins_ncc.ALL_PINS if which == "ncc" else pins_xcorr.ALL_PINS
    caught = []
    for pin in pins:
        try:
            pin(lib=lib)
        except (AssertionError, OverflowError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {name}"


def test_unmutated_copy_passes(tmp_path):
    """The harness itself: an identical copy passes every pin."""
    lib = _build_mutant(tmp_path, "identity", "#include <math.h>", "#include <math.h>")
    for pin in pins_ncc.ALL_PINS + pins_xcorr.ALL_PINS:
        pin(lib=lib)
