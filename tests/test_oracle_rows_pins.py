"""Pins of the oracle's row softmax and row sum to facts outside it (CPU
only).

The lecture's ladder before the matmul ("Kernels, Triton, XLA", section
"Reductions and tiling"; the Chinese notes' sections 5.3 and 5.4): softmax
exponentiates and normalises each row after subtracting its maximum, and the
row sum adds a row that does not fit one block in tiles. The pins: scipy's
float64 softmax, closed forms (a constant row is uniform, a two-column row is
the logistic function of the difference), rows summing to one, invariance
under adding a constant to a row, finite results for large inputs, exact
integer row sums and the arithmetic-series closed form, bf16 widening, and
padding that is never read. Deliberately broken versions at the bottom must
each fail at least one pin.
"""
import math

import numpy as np
import pytest
import scipy.special

import datagen
import oracle


def _pad(x, extra, fill=np.nan):
    out = np.full((x.shape[0], x.shape[1] + extra), fill, dtype=x.dtype)
    out[:, :x.shape[1]] = x
    return out


# --- softmax ------------------------------------------------------------------

def sm_oracle(x, n=None):
    """Softmax of the first n columns of each row of x (default: all)."""
    if n is None:
        return oracle.softmax_rows(x)
    return oracle.softmax_rows(x, M=x.shape[0], N=n, ldx=x.shape[1])


def pin_softmax_matches_scipy(impl):
    x = datagen.normal_f32(501, 37, 301, 3.0)
    ref = scipy.special.softmax(x.astype(np.float64), axis=1)
    assert np.all(np.abs(impl(x) - ref) <= 1e-14 * ref + 1e-300)


def pin_softmax_closed_forms(impl):
    x = np.zeros((3, 7), np.float32)
    x[1] = 2.5
    x[2] = -40.0
    assert np.all(np.abs(impl(x) - 1 / 7) <= 1e-16)
    d = np.linspace(-20, 20, 81, dtype=np.float32)
    two = np.stack([d, np.zeros_like(d)], axis=1)
    r = impl(two)
    logistic = 1 / (1 + np.exp(-d.astype(np.float64)))
    assert np.all(np.abs(r[:, 0] - logistic) <= 1e-15)
    assert np.all(np.abs(r[:, 1] - (1 - logistic)) <= 1e-15)


def pin_softmax_rows_sum_to_one_and_order(impl):
    x = datagen.normal_f32(502, 19, 1000, 2.0)
    r = impl(x)
    assert np.all(np.abs(r.sum(axis=1) - 1) <= 1e-12)
    assert np.all(r > 0)
    order = np.argsort(x, axis=1, kind="stable")
    assert np.all(np.diff(np.take_along_axis(r, order, axis=1), axis=1) >= 0)


def pin_softmax_shift_invariance_and_large_inputs(impl):
    x = datagen.small_int_f32(503, 11, 64)                 # integers: x + c is exact in fp32
    r = impl(x)
    assert np.all(np.abs(impl(x + 96.0) - r) <= 1e-15)
    big = impl(x + 1000.0)                                 # exp(1000) overflows double without the max
    assert np.all(np.isfinite(big)) and np.all(np.abs(big - r) <= 1e-15)
    assert np.all(np.isfinite(impl(x - 1000.0)))


def pin_softmax_bf16_widening_and_padding(impl):
    x32 = datagen.small_int_f32(504, 9, 40) / 4
    xb = datagen.f32_to_bf16_bits(x32)
    assert np.array_equal(impl(xb), impl(x32))             # quarters are exact in bf16
    padded = _pad(x32, 8)
    assert np.array_equal(impl(padded, n=40), impl(x32))


SOFTMAX_PINS = [pin_softmax_matches_scipy, pin_softmax_closed_forms, pin_softmax_rows_sum_to_one_and_order,
                pin_softmax_shift_invariance_and_large_inputs, pin_softmax_bf16_widening_and_padding]


# --- row sum ------------------------------------------------------------------

def rs_oracle(x, n=None):
    """Sum of the first n columns of each row of x (default: all)."""
    if n is None:
        return oracle.row_sum(x)
    return oracle.row_sum(x, M=x.shape[0], N=n, ldx=x.shape[1])


def pin_row_sum_exact_integers(impl):
    x = datagen.small_int_f32(511, 23, 4099)
    assert np.array_equal(impl(x), x.astype(np.int64).sum(axis=1).astype(np.float64))
    assert np.array_equal(impl(datagen.f32_to_bf16_bits(x)), impl(x))


def pin_row_sum_arithmetic_series(impl):
    M, N = 6, 4096
    x = (np.arange(N)[None, :] + np.arange(M)[:, None]).astype(np.float32)
    expect = N * (N - 1) / 2 + N * np.arange(M)
    assert np.array_equal(impl(x), expect.astype(np.float64))


def pin_row_sum_padding_and_floats(impl):
    x = datagen.normal_f32(512, 13, 777, 1.0)
    ref = x.astype(np.float64).sum(axis=1)
    assert np.all(np.abs(impl(x) - ref) <= 777 * np.finfo(np.float64).eps * np.abs(x).astype(np.float64).sum(axis=1))
    assert np.array_equal(impl(_pad(x, 5, fill=123.0), n=777), impl(x))   # padding never added


ROWSUM_PINS = [pin_row_sum_exact_integers, pin_row_sum_arithmetic_series, pin_row_sum_padding_and_floats]


@pytest.mark.parametrize("pin", SOFTMAX_PINS, ids=lambda p: p.__name__)
def test_oracle_softmax_pin(pin):
    pin(sm_oracle)


@pytest.mark.parametrize("pin", ROWSUM_PINS, ids=lambda p: p.__name__)
def test_oracle_row_sum_pin(pin):
    pin(rs_oracle)


def test_rows_edge_cases_and_checks():
    assert oracle.softmax_rows(np.zeros((0, 5), np.float32)).shape == (0, 5)
    assert oracle.row_sum(np.zeros((4, 0), np.float32)).tolist() == [0.0] * 4
    assert oracle.softmax_rows(np.array([[3.5]], np.float32)).tolist() == [[1.0]]
    with pytest.raises(ValueError):
        oracle.softmax_rows(np.zeros(10, np.float32), M=3, N=4, ldx=4)
    with pytest.raises(ValueError):
        oracle.row_sum(np.zeros(12, np.float32), M=3, N=4, ldx=3)


# ---------------------------------------------------------------------------
# Planted mistakes (numpy re-implementations on the CPU): each must fail a pin.
# ---------------------------------------------------------------------------

def _widen(x):
    return datagen.bf16_bits_to_f32(x).astype(np.float64) if x.dtype == np.uint16 else x.astype(np.float64)


def _sm_mutant(f):
    def impl(x, n=None):
        v = _widen(x)
        if n is not None:
            v = v[:, :n]
        with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
            return f(v)
    return impl


def _rs_mutant(f):
    def impl(x, n=None):
        v = _widen(x)
        if n is not None:
            v = v[:, :n]
        return f(v)
    return impl


SOFTMAX_MUTANTS = {
    "no_max_subtraction": _sm_mutant(lambda v: np.exp(v) / np.exp(v).sum(1, keepdims=True)),
    "column_softmax": _sm_mutant(lambda v: scipy.special.softmax(v, axis=0)),
    "not_normalised": _sm_mutant(lambda v: np.exp(v - v.max(1, keepdims=True))),
    "min_subtracted_unnormalised": _sm_mutant(lambda v: np.exp(v - v.min(1, keepdims=True)) / v.shape[1]),
    "last_column_dropped_from_sum": _sm_mutant(
        lambda v: np.exp(v - v.max(1, keepdims=True)) / np.exp(v - v.max(1, keepdims=True))[:, :-1].sum(1, keepdims=True)),
    "padding_read": lambda x, n=None: scipy.special.softmax(np.nan_to_num(_widen(x)), axis=1),
}

ROWSUM_MUTANTS = {
    "last_column_dropped": _rs_mutant(lambda v: v[:, :-1].sum(1)),
    "column_sum": _rs_mutant(lambda v: np.resize(v.sum(0), v.shape[0])),
    "scaled_sum": _rs_mutant(lambda v: 1.001 * v.sum(1)),
    "padding_read": lambda x, n=None: np.nan_to_num(_widen(x)).sum(1),
}


def _caught(impl, pins):
    failed = []
    for pin in pins:
        try:
            pin(impl)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(SOFTMAX_MUTANTS))
def test_softmax_pins_catch_planted_mistake(name):
    assert _caught(SOFTMAX_MUTANTS[name], SOFTMAX_PINS), f"no pin caught {name}"


@pytest.mark.parametrize("name", sorted(ROWSUM_MUTANTS))
def test_row_sum_pins_catch_planted_mistake(name):
    assert _caught(ROWSUM_MUTANTS[name], ROWSUM_PINS), f"no pin caught {name}"


def test_correct_numpy_versions_pass_every_pin():
    good_sm = _sm_mutant(lambda v: scipy.special.softmax(v, axis=1))
    good_rs = _rs_mutant(lambda v: v.sum(1))
    assert not _caught(good_sm, SOFTMAX_PINS)
    assert not _caught(good_rs, ROWSUM_PINS)
