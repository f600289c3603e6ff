"""The CPU oracle against what the pages and the mathematics fix (CPU only)."""
import numpy as np
import pytest

import oracle_pins as P

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_widen_f16_every_bit_pattern(oracle_lib):
    P.pin_widen_f16(oracle_lib)


def test_widen_bf16_every_bit_pattern(oracle_lib):
    P.pin_widen_bf16(oracle_lib)


def test_widen_f32_f64_sampled_bit_patterns(oracle_lib):
    P.pin_widen_f32_f64(oracle_lib)


@pytest.mark.parametrize("dtype", P.DTYPES)
@pytest.mark.parametrize("op", P.OPS)
def test_brute_force_against_closed_form(oracle_lib, dtype, op):
    P.pin_brute_force(oracle_lib, dtype, op, max_len=5)


def test_pages_fixed_cases(oracle_lib):
    P.pin_fixed_cases(oracle_lib, "cases")


def test_readings_of_cases_the_pages_leave_open(oracle_lib):
    P.pin_fixed_cases(oracle_lib, "readings")


@pytest.mark.parametrize("dtype", P.DTYPES)
@pytest.mark.parametrize("op", P.OPS)
def test_numpy_first_occurrence_on_nan_free_rows(oracle_lib, dtype, op):
    P.pin_numpy_first_occurrence(oracle_lib, dtype, op)


@pytest.mark.parametrize("dtype", P.DTYPES)
@pytest.mark.parametrize("op", P.OPS)
def test_middle_axis_against_closed_form(oracle_lib, dtype, op):
    P.pin_axis(oracle_lib, dtype, op)


@pytest.mark.parametrize("dtype", P.DTYPES)
@pytest.mark.parametrize("op", P.OPS)
def test_raw_bit_patterns_with_signalling_nans(oracle_lib, dtype, op):
    P.pin_raw_bit_patterns(oracle_lib, dtype, op)


def test_rejects_empty_rows(oracle_lib):
    P.pin_rejects_empty_rows(oracle_lib)


def test_closed_form_itself_on_hand_rows():
    """The independent closed form on rows small enough to verify by eye."""
    nan, inf = float("nan"), float("inf")
    rows = np.array([[1, 3, 3, 2], [nan, 5, 6, 7], [-inf, -inf, nan, -inf],
                     [2, nan, 9, 9], [-0.0, 0.0, -1, 0.0]])
    assert P.closed_form(rows, "max").tolist() == [1, 0, 0, 2, 0]
    assert P.closed_form(rows, "min").tolist() == [0, 0, 0, 0, 2]
    assert P.closed_form(rows, "max_last").tolist() == [2, 0, 3, 3, 3]
    assert P.closed_form(rows, "min_last").tolist() == [0, 0, 3, 0, 2]


# cumulative extremum with indices


@pytest.mark.parametrize("dtype", P.CUM_DTYPES)
@pytest.mark.parametrize("op", P.CUM_OPS)
def test_cumulative_brute_force_against_prefix_closed_form(oracle_lib, dtype, op):
    P.pin_cum_brute_force(oracle_lib, dtype, op, max_len=4)


@pytest.mark.parametrize("dtype", P.CUM_DTYPES)
@pytest.mark.parametrize("op", P.CUM_OPS)
def test_cumulative_against_numpy_accumulate(oracle_lib, dtype, op):
    P.pin_cum_numpy_accumulate(oracle_lib, dtype, op)


@pytest.mark.parametrize("dtype", [d for d in P.CUM_DTYPES if d not in P.INT_NP])
@pytest.mark.parametrize("op", P.CUM_OPS)
def test_cumulative_raw_bit_patterns_with_signalling_nans(oracle_lib, dtype, op):
    P.pin_cum_raw_bit_patterns(oracle_lib, dtype, op)


@pytest.mark.parametrize("dtype", P.CUM_DTYPES)
@pytest.mark.parametrize("op", P.CUM_OPS)
def test_cumulative_values_against_two_pass_recipe(oracle_lib, dtype, op):
    P.pin_cum_two_pass(oracle_lib, dtype, op)


def test_cumulative_page_examples(oracle_lib):
    P.pin_cum_page_examples(oracle_lib)


def test_cumulative_fixed_cases(oracle_lib):
    P.pin_cum_fixed_cases(oracle_lib, "cases")


def test_cumulative_readings(oracle_lib):
    P.pin_cum_fixed_cases(oracle_lib, "readings")


def test_cumulative_rejects(oracle_lib):
    P.pin_cum_rejects(oracle_lib)


def test_cumulative_last_position_is_the_reduction(oracle_lib):
    """Consistency of the two oracle entry points on one definition (not a pin: both are
    this oracle): the index at the last position is the row's ArgMax / ArgMin."""
    rng = np.random.default_rng(5)
    for dtype in P.DTYPES:
        for op in P.CUM_OPS:
            v = P.alphabet9(dtype)[rng.integers(0, 9, size=(50, 13))]
            x = P.exact_storage(v, dtype)
            _, idx = oracle_lib.cumulative(x, dtype, op)
            assert np.array_equal(idx[:, -1], oracle_lib.argreduce_lastaxis(x, dtype, op))
