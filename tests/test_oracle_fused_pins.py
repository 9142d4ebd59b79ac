"""Pins of the oracle's fused epilogues, act(A·B + bias), to facts outside it
(CPU only).

The pages define GeLU by its tanh form, 0.5 x (1 + tanh(0.79788456 (x +
0.044715 x^3))), and state that this naive formula and PyTorch's built-in
gelu(approximate="tanh") agree numerically ("Kernels, Triton, XLA", section
"GeLU three ways: the case for fusion"); they apply any elementwise
activation to the finished output tile before its one store (section
"Reductions and tiling"). A per-column bias (a linear layer x·W + b) is this
repository's reading; the pages name the linear layer but print no bias.

The pins: the library GeLU in float64; the identity gelu(x) - gelu(-x) = x
of the tanh form; its known distance from the exact erf form x·Phi(x) (at
most 4.74e-4, reached near |x| = 2.7), computed with math.erf; limits; exact
integer sums with a bias per output column; bf16 widening of the bias; and
the identity activation against a float64 BLAS product. Deliberately broken
variants at the bottom must each fail at least one pin.
"""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle


def oracle_impl(act, a, b, bias):
    return oracle.fused(act, a, b, bias)


def oracle_at_impl(act, a, b, bias):
    M, K = a.shape
    N = b.shape[1]
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    return oracle.fused_at(act, a, b, bias, ii.ravel(), jj.ravel(), K, K, N).reshape(M, N)


def _as_column(x):
    """A (len(x) x 1) and B (1 x 1) with B = 1: the product is x itself."""
    a = np.ascontiguousarray(np.asarray(x, np.float32).reshape(-1, 1))
    return a, np.ones((1, 1), np.float32)


GRID = np.linspace(-8.0, 8.0, 4001, dtype=np.float32)


def pin_gelu_matches_library(impl):
    a, b = _as_column(GRID)
    r = impl("gelu_tanh", a, b, None)[:, 0]
    ref = torch.nn.functional.gelu(torch.from_numpy(GRID.astype(np.float64)), approximate="tanh").numpy()
    assert np.all(np.abs(r - ref) <= 1e-9 * (1 + np.abs(ref))), np.abs(r - ref).max()


def pin_gelu_odd_identity(impl):
    a, b = _as_column(np.concatenate([GRID, -GRID]))
    r = impl("gelu_tanh", a, b, None)[:, 0]
    n = GRID.size
    x = GRID.astype(np.float64)
    assert np.all(np.abs(r[:n] - r[n:] - x) <= 1e-12 * (1 + np.abs(x)))


def pin_gelu_distance_from_erf_form(impl):
    a, b = _as_column(GRID)
    r = impl("gelu_tanh", a, b, None)[:, 0]
    exact = np.array([0.5 * float(v) * (1 + math.erf(float(v) / math.sqrt(2))) for v in GRID])
    d = np.abs(r - exact).max()
    assert 4.0e-4 <= d <= 5.0e-4, d


def pin_gelu_limits(impl):
    a, b = _as_column([0.0, 10.0, -10.0, 1.0])
    r = impl("gelu_tanh", a, b, None)[:, 0]
    assert r[0] == 0.0
    assert abs(r[1] - 10.0) <= 1e-6 and abs(r[2]) <= 1e-6
    assert 0.84 < r[3] < 0.85          # gelu(1) = 0.8412 (tanh form)


def _small_ints(seed, rows, cols):
    return datagen.small_int_f32(seed, rows, cols)


def pin_bias_exact_integers(impl):
    """Integers: every sum is exact, so R equals the integer result."""
    M, N, K = 7, 11, 9
    a, b = _small_ints(301, M, K), _small_ints(302, K, N)
    bias = _small_ints(303, 1, N).ravel() * 4
    s = a.astype(np.int64) @ b.astype(np.int64) + bias.astype(np.int64)[None, :]
    assert np.array_equal(impl("none", a, b, bias), s.astype(np.float64))
    assert np.array_equal(impl("relu", a, b, bias), np.maximum(s, 0).astype(np.float64))
    assert np.array_equal(impl("relu", a, b, None),
                          np.maximum(a.astype(np.int64) @ b.astype(np.int64), 0).astype(np.float64))
    assert (s < 0).any() and (s > 0).any()


def pin_bias_bf16_widening(impl):
    M, N, K = 5, 6, 4
    a = datagen.f32_to_bf16_bits(_small_ints(311, M, K))
    b = datagen.f32_to_bf16_bits(_small_ints(312, K, N))
    bias_vals = np.array([0.5, -1.25, 3.0, -7.0, 96.0, -0.125], np.float32)
    bias = datagen.f32_to_bf16_bits(bias_vals)
    s = (datagen.bf16_bits_to_f32(a).astype(np.float64) @ datagen.bf16_bits_to_f32(b).astype(np.float64)
         + bias_vals.astype(np.float64)[None, :])
    assert np.array_equal(impl("none", a, b, bias), s)


def pin_identity_is_the_product(impl):
    """act = none without a bias is the plain product (float64 BLAS, within
    the rounding of K additions)."""
    M, N, K = 33, 17, 129
    a = datagen.normal_f32(321, M, K, 1.0)
    b = datagen.normal_f32(322, K, N, 1.0)
    ref = a.astype(np.float64) @ b.astype(np.float64)
    bound = 4 * K * np.finfo(np.float64).eps * (np.abs(a).astype(np.float64) @ np.abs(b).astype(np.float64))
    assert np.all(np.abs(impl("none", a, b, None) - ref) <= bound)
    assert (ref < 0).any()


PINS = [pin_gelu_matches_library, pin_gelu_odd_identity, pin_gelu_distance_from_erf_form, pin_gelu_limits,
        pin_bias_exact_integers, pin_bias_bf16_widening, pin_identity_is_the_product]


@pytest.mark.parametrize("impl", [oracle_impl, oracle_at_impl], ids=["full", "at"])
@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_fused_pin(pin, impl):
    pin(impl)


def test_relu_without_bias_is_mmrelu():
    a = datagen.normal_f32(331, 40, 24, 0.2)
    b = datagen.normal_f32(332, 24, 30, 0.2)
    assert np.array_equal(oracle.fused("relu", a, b), oracle.mmrelu(a, b))


def test_bias_arguments_are_checked():
    a, b = _small_ints(341, 3, 4), _small_ints(342, 4, 5)
    with pytest.raises(ValueError):
        oracle.fused("relu", a, b, np.zeros(4, np.float32))        # too short
    with pytest.raises(ValueError):
        oracle.fused("relu", a, b, np.zeros(5, np.float64))        # wrong dtype
    with pytest.raises(KeyError):
        oracle.fused("tanh", a, b)


# ---------------------------------------------------------------------------
# Planted mistakes (numpy re-implementations on the CPU): each must fail a pin.
# ---------------------------------------------------------------------------

def _widen(x):
    return datagen.bf16_bits_to_f32(x).astype(np.float64) if x.dtype == np.uint16 else x.astype(np.float64)


def _mutant(act_fn, bias_mode="column"):
    def impl(act, a, b, bias):
        s = _widen(a) @ _widen(b)
        if bias is not None:
            bv = _widen(bias)
            if bias_mode == "column":
                s = s + bv[None, :]
            elif bias_mode == "row":
                s = s + bv[: s.shape[0], None] if bv.size >= s.shape[0] else s + bv[None, :]
            elif bias_mode == "after":
                return act_fn(act, s) + bv[None, :]
        return act_fn(act, s)
    return impl


def _act(gelu):
    def f(act, s):
        if act == "relu":
            return np.maximum(s, 0)
        if act == "gelu_tanh":
            return gelu(s)
        return s
    return f


def _gelu(c1=0.79788456, c3=0.044715, half=0.5):
    return lambda x: half * x * (1 + np.tanh(c1 * (x + c3 * x ** 3)))


_erf = np.vectorize(math.erf)

MUTANTS = {
    "gelu_cubic_constant_typo": _mutant(_act(_gelu(c3=0.04715))),
    "gelu_wrong_sqrt_2_over_pi": _mutant(_act(_gelu(c1=0.7071))),
    "gelu_missing_half": _mutant(_act(_gelu(half=1.0))),
    "gelu_exact_erf_form": _mutant(_act(lambda x: 0.5 * x * (1 + _erf(x / math.sqrt(2))))),
    "gelu_is_relu": _mutant(_act(lambda x: np.maximum(x, 0))),
    "bias_per_row": _mutant(_act(_gelu()), bias_mode="row"),
    "bias_after_activation": _mutant(_act(_gelu()), bias_mode="after"),
    "bias_dropped": _mutant(_act(_gelu()), bias_mode="none"),
    "none_is_relu": _mutant(lambda act, s: np.maximum(s, 0) if act in ("relu", "none") else _gelu()(s)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    impl = MUTANTS[name]
    failed = []
    for pin in PINS:
        try:
            pin(impl)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {name}"
