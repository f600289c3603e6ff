"""Each plausible mistake planted in a copy of the oracle fails at least one pin (CPU only).

The mistakes are planted in the oracle's C source, on the CPU, in a temporary copy; the
oracle under oracle/ is never modified.
"""
import os

import pytest

import oracle
import oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "argreduce_oracle.c")

# (name, original text, planted mistake)
MAX_CASE = "case ORACLE_ARGMAX: better = a > best;"
MUTANTS = [
    ("ties_to_last_index", MAX_CASE, "case ORACLE_ARGMAX: better = a >= best;"),
    ("argmin_compares_the_wrong_way", "case ORACLE_ARGMIN: better = a < best;",
     "case ORACLE_ARGMIN: better = a > best;"),
    ("nan_unsafe_compare", MAX_CASE, "case ORACLE_ARGMAX: better = !(a <= best);"),
    ("signed_zero_ordered", MAX_CASE,
     "case ORACLE_ARGMAX: better = a > best || (a == best && signbit(best) && !signbit(a));"),
    ("last_index_ties_to_first", "case ORACLE_ARGMAX_LAST: better = a >= best;",
     "case ORACLE_ARGMAX_LAST: better = a > best;"),
    ("min_last_strict", "default: better = a <= best;", "default: better = a < best;"),
    ("last_index_nan_unsafe", "case ORACLE_ARGMAX_LAST: better = a >= best;",
     "case ORACLE_ARGMAX_LAST: better = !(a < best);"),
    ("identity_seed_instead_of_element0",
     "double best = element(x, dtype, row0);",
     "double best = (op == ORACLE_ARGMAX) ? -INFINITY : INFINITY;"),
    ("row_stride_off_by_one", "const int64_t row0 = r * cols;\n        double best",
     "const int64_t row0 = r * (cols - 1);\n        double best"),
    ("f16_subnormals_flushed", "mag = ldexp((double)frac, -24);", "mag = 0.0;"),
    ("f16_exponent_bias", "expo - 25);", "expo - 24);"),
    ("bf16_wrong_shift", "(uint32_t)b << 16;", "(uint32_t)b << 15;"),
    ("f64_read_as_f32_stride", "memcpy(&d, (const char *)x + k * 8, 8);",
     "memcpy(&d, (const char *)x + k * 4, 8);"),
    ("last_column_skipped", "for (int64_t j = 1; j < cols; ++j)", "for (int64_t j = 1; j < cols - 1; ++j)"),
    ("empty_rows_accepted", "cols < 1 || dtype", "cols < 0 || dtype"),
    ("axis_stride_wrong", "element(x, dtype, base + r * inner)", "element(x, dtype, base + r * len)"),
    ("axis_output_transposed", "out[o * inner + i] = idx;", "out[i * outer + o] = idx;"),
    # cumulative extremum with indices
    ("cum_int_ties_to_later_index", "return op == ORACLE_ARGMAX ? a > b : a < b;",
     "return op == ORACLE_ARGMAX ? a >= b : a < b;"),
    ("cum_int_cummin_as_cummax", "return op == ORACLE_ARGMAX ? a > b : a < b;", "return a > b;"),
    ("cum_float_ties_to_later_index", "return moves(op, element(x, dtype, ka), element(x, dtype, kb));",
     "return moves(op + 2, element(x, dtype, ka), element(x, dtype, kb));"),
    ("cum_nan_propagates", "return moves(op, element(x, dtype, ka), element(x, dtype, kb));",
     "return isnan(element(x, dtype, ka)) || moves(op, element(x, dtype, ka), element(x, dtype, kb));"),
    ("cum_value_from_position_not_index", "(const char *)x + (row0 + best) * size",
     "(const char *)x + (row0 + j) * size"),
    ("cum_integers_compared_as_double",
     "const int64_t a = int_element(x, dtype, ka), b = int_element(x, dtype, kb);",
     "const double a = (double)int_element(x, dtype, ka), b = (double)int_element(x, dtype, kb);"),
    ("cum_i32_read_as_i64", "if (dtype == ORACLE_I32) {", "if (dtype == -1) {"),
    ("cum_position_1_skipped", "if (j > 0 && scan_moves", "if (j > 1 && scan_moves"),
    ("cum_empty_rows_accepted", "cols < 1 || size == 0", "cols < 0 || size == 0"),
    ("cum_row_stride_off_by_one", "const int64_t row0 = r * cols;\n        int64_t best = 0;",
     "const int64_t row0 = r * (cols - 1);\n        int64_t best = 0;"),
    ("cum_i64_read_with_i32_stride", "memcpy(&v, (const char *)x + k * 8, 8);",
     "memcpy(&v, (const char *)x + k * 4, 8);"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.build(str(mutated), str(tmp_path / "libmutant.so"))
    o = oracle.Oracle(lib)
    caught = []
    for pin_name, pin in P.all_pins(o, fast=True):
        try:
            pin()
        except AssertionError:
            caught.append(pin_name)
        except Exception as exc:  # a crash or refusal is a catch too
            caught.append(f"{pin_name}:{type(exc).__name__}")
    assert caught, f"mutant {name} passed every pin"
