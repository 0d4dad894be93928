"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is a copy of ``oracle/oracle.c`` with one plausible mistake
written into it (a dropped term, a wrong index, a transposed operand, a
narrower accumulator, a wrong magnitude, a wrong starting value).  The copy is
compiled into a temporary directory and the whole pin suite runs against it;
the test requires at least one pin to fail for every mutant.  The real oracle
is never modified.
"""
import os
import subprocess

import pytest

import oracle
from tests import oracle_pins

MUTANTS = {
    # full reduce
    "drops_last_element": (
        "for (int64_t i = 0; i < n; ++i) {", "for (int64_t i = 0; i + 1 < n; ++i) {"),
    "drops_first_element": (
        "for (int64_t i = 0; i < n; ++i) {", "for (int64_t i = 1; i < n; ++i) {"),
    "fp32_accumulator": (
        "        double v = (double)x[i];\n        s += v;",
        "        float v = x[i];\n        s = (float)((float)s + v);"),
    "signed_magnitude_1d": (
        "        s += v;\n        a += fabs(v);\n    }\n    *sum",
        "        s += v;\n        a += v;\n    }\n    *sum"),
    "negative_zero_start": (
        "    double s = 0.0;\n    double a = 0.0;\n    for (int64_t i = 0; i < n;",
        "    double s = -0.0;\n    double a = 0.0;\n    for (int64_t i = 0; i < n;"),
    # axis reduce
    "transposed_outer_and_R": (
        "const float* row = x + (o * R + r) * inner;\n                for (int64_t i = 0; i < inner; ++i) {",
        "const float* row = x + (r * outer + o) * inner;\n                for (int64_t i = 0; i < inner; ++i) {"),
    "drops_last_row": (
        "for (int64_t r = 0; r < R; ++r) {\n                const float* row = x + (o * R + r) * inner;\n                for (int64_t i = 0; i < inner; ++i) {",
        "for (int64_t r = 0; r + 1 < R; ++r) {\n                const float* row = x + (o * R + r) * inner;\n                for (int64_t i = 0; i < inner; ++i) {"),
    "shifted_column": (
        "double v = (double)row[i];",
        "double v = (double)row[(i + 1) % inner];"),
    "row_stride_R_instead_of_inner": (
        "const float* row = x + (o * R + r) * inner;\n                for (int64_t i = 0; i < inner; ++i) {",
        "const float* row = x + o * R * inner + r * (inner > 1 ? inner - 1 : 1);\n                for (int64_t i = 0; i < inner; ++i) {"),
    "signed_magnitude_axis": (
        "s[i] += v;\n                    a[i] += fabs(v);",
        "s[i] += v;\n                    a[i] += v;"),
    # the other reductions
    "max_starts_at_zero": (
        "    if (op == 2)\n        return -INFINITY;", "    if (op == 2)\n        return 0.0;"),
    "min_starts_at_zero": (
        "    if (op == 3)\n        return INFINITY;", "    if (op == 3)\n        return 0.0;"),
    "max_keeps_smaller": (
        "    return v > m ? v : m;", "    return v < m ? v : m;"),
    "max_prefers_negative_zero": (
        "return signbit(m) ? v : m; /* +0 over -0 */", "return signbit(m) ? m : v; /* +0 over -0 */"),
    "max_ignores_nan": (
        "static double maximum754(double m, double v)\n{\n    if (isnan(m) || isnan(v))",
        "static double maximum754(double m, double v)\n{\n    if (0)"),
    "min_ignores_nan": (
        "static double minimum754(double m, double v)\n{\n    if (isnan(m) || isnan(v))",
        "static double minimum754(double m, double v)\n{\n    if (0)"),
    "sumsq_adds_magnitude": (
        "        *s += v * v;\n        *a += v * v;", "        *s += fabs(v);\n        *a += v * v;"),
    "reduce_transposed_outer_and_R": (
        "const float* row = x + (o * R + r) * inner;\n                for (int64_t i = 0; i < inner; ++i)\n                    reduce_step",
        "const float* row = x + (r * outer + o) * inner;\n                for (int64_t i = 0; i < inner; ++i)\n                    reduce_step"),
    "reduce_drops_last_row": (
        "for (int64_t r = 0; r < R; ++r) {\n                const float* row = x + (o * R + r) * inner;\n                for (int64_t i = 0; i < inner; ++i)\n                    reduce_step",
        "for (int64_t r = 0; r + 1 < R; ++r) {\n                const float* row = x + (o * R + r) * inner;\n                for (int64_t i = 0; i < inner; ++i)\n                    reduce_step"),
    "reduce_at_reversed_column": (
        "reduce_step(op, (double)x[(o_idx[k] * R + r) * inner + i_idx[k]], &s, &a);",
        "reduce_step(op, (double)x[(o_idx[k] * R + r) * inner + (inner - 1 - i_idx[k])], &s, &a);"),
    # cumulative sums
    "cumsum_wrong_direction": (
        "const int64_t r = reverse ? R - 1 - k : k;", "const int64_t r = reverse ? k : R - 1 - k;"),
    "cumsum_exclusive": (
        "                s += v;\n                a += fabs(v);\n                out[e] = s;",
        "                out[e] = s;\n                s += v;\n                a += fabs(v);"),
    "cumsum_drops_far_end": (
        "            for (int64_t k = 0; k < R; ++k) {\n                const int64_t r = reverse",
        "            for (int64_t k = 1; k < R; ++k) {\n                const int64_t r = reverse"),
    "cumsum_transposed": (
        "const int64_t e = (o * R + r) * inner + i;", "const int64_t e = (r * outer + o) * inner + i;"),
    # softmax denominator
    "softmax_exp_sign_flipped": (
        "s += exp((double)x[(o * R + r) * inner + i] - c);",
        "s += exp(c - (double)x[(o * R + r) * inner + i]);"),
    "softmax_no_shift": (
        "m = maximum754(m, (double)x[(o * R + r) * inner + i]);\n            const double c = softmax_shift(m);",
        "m = maximum754(m, (double)x[(o * R + r) * inner + i]);\n            const double c = 0.0;"),
    "softmax_shift_by_infinite_max": (
        "return isfinite(m) ? m : 0.0;", "return m;"),
    "softmax_max_starts_at_zero": (
        "double m = -INFINITY;\n            for (int64_t r = 0; r < R; ++r)\n                m = maximum754(m, (double)x[",
        "double m = 0.0;\n            for (int64_t r = 0; r < R; ++r)\n                m = maximum754(m, (double)x["),
    "softmax_drops_last_term": (
        "for (int64_t r = 0; r < R; ++r)\n                s += exp((double)x[",
        "for (int64_t r = 0; r + 1 < R; ++r)\n                s += exp((double)x["),
    "softmax_transposed": (
        "s += exp((double)x[(o * R + r) * inner + i] - c);",
        "s += exp((double)x[(r * outer + o) * inner + i] - c);"),
    "softmax_shift_by_first_term": (
        "m = maximum754(m, (double)x[(o * R + r) * inner + i]);\n            const double c = softmax_shift(m);",
        "m = maximum754(m, (double)x[(o * R + r) * inner + i]);\n            const double c = R ? (double)x[o * R * inner + i] : 0.0;"),
    "softmax_at_reversed_column": (
        "const float* col = x + o_idx[k] * R * inner + i_idx[k];",
        "const float* col = x + o_idx[k] * R * inner + (inner - 1 - i_idx[k]);"),
    # per-output entry point
    "at_reversed_column": (
        "double v = (double)x[(o * R + r) * inner + i];",
        "double v = (double)x[(o * R + r) * inner + (inner - 1 - i)];"),
    "at_drops_first_row": (
        "        for (int64_t r = 0; r < R; ++r) {\n            double v",
        "        for (int64_t r = 1; r < R; ++r) {\n            double v"),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, "mutation site not unique: %s" % name
    src = tmp_path / ("oracle_%s.c" % name)
    src.write_text(source.replace(old, new))
    lib = str(tmp_path / ("liboracle_%s.so" % name))
    oracle.build(source=str(src), library=lib)
    orc = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "mutant %s passed every pin" % name
