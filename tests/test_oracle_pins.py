"""Pins of the fp64 oracle to facts outside itself (CPU only).

The pages print no numeric result for a matrix product, so the oracle is
pinned by exact arithmetic on tiny inputs, closed forms, the ReLU invariants
against an independent float64 BLAS product, exact-integer inputs, statistics
of the workloads' distributions, and calibration of the fp32 tolerance.

Every pin is written as a check on an ``impl(a, b) -> R`` callable so that the
same checks can be run against deliberately broken variants of the oracle
(planted on the CPU, at the bottom of this file): each of those must fail at
least one pin, which shows the pins would catch that kind of mistake.
"""
from fractions import Fraction
import math

import numpy as np
import pytest
import torch

import datagen
import oracle


def oracle_impl(a, b):
    return oracle.mmrelu(a, b)


def oracle_at_impl(a, b):
    M, K = a.shape
    N = b.shape[1]
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    return oracle.mmrelu_at(a, b, ii.ravel(), jj.ravel(), K, K, N).reshape(M, N)


# ---------------------------------------------------------------------------
# Pins. Each returns None on success and raises AssertionError otherwise.
# ---------------------------------------------------------------------------

def pin_bruteforce_4x4x4(impl):
    """Exact rational sums of fp32 inputs (every float is a dyadic rational)."""
    for seed, kind in [(11, "mixed"), (12, "neg"), (13, "pos"), (14, "mixed")]:
        a = datagen.normal_f32(seed, 4, 4)
        b = datagen.normal_f32(seed + 100, 4, 4)
        if kind == "neg":
            a, b = -np.abs(a), np.abs(b)
        elif kind == "pos":
            a, b = np.abs(a), np.abs(b)
        r = impl(a, b)
        for i in range(4):
            for j in range(4):
                terms = [Fraction(float(a[i, k])) * Fraction(float(b[k, j])) for k in range(4)]
                exact = sum(terms, Fraction(0))
                want = max(exact, Fraction(0))
                mag = sum(abs(t) for t in terms)
                # three fp64 additions: |error| <= 3 * 2^-53 * sum|terms|
                bound = Fraction(3, 2 ** 53) * mag
                assert abs(Fraction(float(r[i, j])) - want) <= bound, (kind, i, j)
                if exact <= -bound:
                    assert r[i, j] == 0.0
        if kind == "neg":
            assert np.all(r == 0.0)


def pin_bruteforce_ragged(impl):
    """Tiny non-square shapes, exact rationals, small-integer inputs: exact equality."""
    for (m, n, k, s) in [(3, 5, 2, 21), (5, 2, 7, 22), (1, 6, 3, 23), (6, 1, 1, 24)]:
        a = datagen.small_int_f32(s, m, k)
        b = datagen.small_int_f32(s + 50, k, n)
        r = impl(a, b)
        assert r.shape == (m, n)
        for i in range(m):
            for j in range(n):
                e = sum(int(a[i, t]) * int(b[t, j]) for t in range(k))
                assert r[i, j] == max(e, 0), (m, n, k, i, j)


def pin_zero(impl):
    a = np.zeros((5, 6), np.float32)
    b = datagen.normal_f32(31, 6, 4)
    assert np.all(impl(a, b) == 0.0)
    assert np.all(impl(datagen.normal_f32(32, 4, 6), np.zeros((6, 5), np.float32)) == 0.0)


def pin_identity(impl):
    b = datagen.normal_f32(41, 6, 5)
    assert np.array_equal(impl(np.eye(6, dtype=np.float32), b), np.maximum(b.astype(np.float64), 0))
    a = datagen.normal_f32(42, 5, 7)
    assert np.array_equal(impl(a, np.eye(7, dtype=np.float32)), np.maximum(a.astype(np.float64), 0))


def pin_permutation(impl):
    a = datagen.normal_f32(51, 6, 5)
    b = datagen.normal_f32(52, 5, 7)
    rng = np.random.default_rng(53)
    p = np.eye(6, dtype=np.float32)[rng.permutation(6)]
    q = np.eye(7, dtype=np.float32)[rng.permutation(7)]
    base = impl(a, b)
    assert np.array_equal(impl(p @ a, b), p.astype(np.float64) @ base)
    assert np.array_equal(impl(a, b @ q), base @ q.astype(np.float64))
    # permuting the contraction index changes the summation order only
    pk = np.eye(5, dtype=np.float32)[rng.permutation(5)]
    np.testing.assert_allclose(impl(a @ pk, pk.T @ b), base, rtol=1e-13, atol=1e-13)


def pin_positive_diagonal(impl):
    b = datagen.normal_f32(61, 5, 6)
    d = np.diag(np.array([0.5, 2.0, 4.0, 0.25, 1.0], np.float32))  # powers of two: exact
    assert np.array_equal(impl(d, b), d.astype(np.float64) @ np.maximum(b.astype(np.float64), 0))
    dn = -d
    assert np.all(impl(dn, np.abs(b)) == 0.0)


def pin_gram_diagonal(impl):
    a = datagen.small_int_f32(71, 6, 9)
    r = impl(a, np.ascontiguousarray(a.T))
    for i in range(6):
        nrm = int(sum(int(x) * int(x) for x in a[i]))
        assert r[i, i] == nrm
    assert np.array_equal(r, r.T)


def pin_rank_one(impl):
    u = datagen.normal_f32(81, 7, 1)
    v = datagen.normal_f32(82, 1, 6)
    want = np.maximum(u.astype(np.float64) @ v.astype(np.float64), 0)
    assert np.array_equal(impl(u, v), want)


def pin_relu_invariants(impl):
    """R >= 0; R = P where P > 0 and R = 0 where P < 0, P from float64 BLAS."""
    for (m, n, k, s) in [(37, 29, 53, 91), (64, 64, 64, 92), (5, 130, 257, 93)]:
        a = datagen.normal_f32(s, m, k, 1 / math.sqrt(k))
        b = datagen.normal_f32(s + 7, k, n, 1 / math.sqrt(k))
        p = np.matmul(a.astype(np.float64), b.astype(np.float64))
        tol = 1e-12 * k * float(np.abs(a).max() * np.abs(b).max())
        r = impl(a, b)
        assert r.shape == (m, n)
        assert np.all(r >= 0)
        pos, neg = p > tol, p < -tol
        assert np.all(np.abs(r[pos] - p[pos]) <= tol)
        assert np.all(r[neg] == 0)
        mid = ~(pos | neg)
        assert np.all(r[mid] <= tol)
        # both signs must actually occur, or the checks above say little
        assert pos.sum() > 0.3 * p.size and neg.sum() > 0.3 * p.size


def pin_exact_integers(impl):
    """Integer inputs with |sum| < 2^53: exact in any order; compare with int64 matmul."""
    a = datagen.small_int_f32(101, 33, 70)
    b = datagen.small_int_f32(102, 70, 45)
    want = np.maximum(a.astype(np.int64) @ b.astype(np.int64), 0).astype(np.float64)
    assert np.array_equal(impl(a, b), want)


def pin_zero_fraction(impl):
    """For N(0,1) inputs each sum is symmetric about 0, so half the outputs are 0.
    Signs of distinct outputs are pairwise uncorrelated, so the fraction has
    standard deviation 0.5/sqrt(MN)."""
    m = n = 96
    k = 64
    a = datagen.normal_f32(111, m, k, 1 / math.sqrt(k))
    b = datagen.normal_f32(112, k, n, 1 / math.sqrt(k))
    frac = float(np.mean(impl(a, b) == 0.0))
    assert abs(frac - 0.5) <= 5 * 0.5 / math.sqrt(m * n), frac


PINS = [pin_bruteforce_4x4x4, pin_bruteforce_ragged, pin_zero, pin_identity,
        pin_permutation, pin_positive_diagonal, pin_gram_diagonal, pin_rank_one,
        pin_relu_invariants, pin_exact_integers, pin_zero_fraction]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
@pytest.mark.parametrize("impl", [oracle_impl, oracle_at_impl], ids=["full", "at"])
def test_oracle_pin(pin, impl):
    pin(impl)


# ---------------------------------------------------------------------------
# The oracle's other entry points and edge cases.
# ---------------------------------------------------------------------------

def test_bf16_widening_matches_torch():
    """bf16 inputs: the oracle widens bit patterns exactly (checked via torch's
    own bf16 -> fp32 conversion, an implementation independent of both)."""
    a32 = datagen.normal_f32(121, 19, 23)
    b32 = datagen.normal_f32(122, 23, 17)
    ah, bh = datagen.f32_to_bf16_bits(a32), datagen.f32_to_bf16_bits(b32)
    at = torch.from_numpy(ah.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    bt = torch.from_numpy(bh.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    r = oracle.mmrelu(ah, bh)
    p = at @ bt
    tol = 1e-12 * 23
    assert np.all(np.abs(r - np.maximum(p, 0)) <= tol)
    ii = np.array([0, 18, 7]); jj = np.array([16, 0, 9])
    np.testing.assert_array_equal(oracle.mmrelu_at(ah, bh, ii, jj, 23, 23, 17), r[ii, jj])


def test_bf16_rounding_matches_torch():
    """The generator's fp32 -> bf16 rounding (nearest, ties to even) agrees with torch."""
    x = datagen.normal_f32(131, 64, 257)
    special = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 1.0 + 2 ** -8 + 2 ** -20,
                        3.0e38, -0.0, 1e-40], dtype=np.float32)
    for v in (x.ravel(), special):
        mine = datagen.f32_to_bf16_bits(v)
        theirs = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        np.testing.assert_array_equal(mine, theirs)


def test_leading_dimensions_ignore_padding():
    a = datagen.normal_f32(141, 7, 5)
    b = datagen.normal_f32(142, 5, 6)
    ap = datagen.pad_rows(a, 9, fill=np.nan)
    bp = datagen.pad_rows(b, 11, fill=np.nan)
    r = oracle.mmrelu(ap, bp, M=7, N=6, K=5, lda=9, ldb=11)
    np.testing.assert_array_equal(r, oracle.mmrelu(a, b))
    ii, jj = np.array([6, 0, 3]), np.array([5, 0, 2])
    np.testing.assert_array_equal(oracle.mmrelu_at(ap, bp, ii, jj, 5, 9, 11), r[ii, jj])


def test_empty_and_k0():
    a = np.zeros((0, 4), np.float32)
    assert oracle.mmrelu(a, np.ones((4, 3), np.float32)).shape == (0, 3)
    r = oracle.mmrelu(np.ones((3, 1), np.float32), np.ones((1, 2), np.float32), M=3, N=2, K=0, lda=1, ldb=2)
    assert r.shape == (3, 2) and np.all(r == 0)


def test_thread_count_independence(monkeypatch):
    """Rows are never split between threads, so the result is bit-identical for
    any thread count; compare against the single-dot-product entry point."""
    a = datagen.normal_f32(151, 40, 300)
    b = datagen.normal_f32(152, 300, 33)
    r = oracle.mmrelu(a, b)
    ii, jj = np.meshgrid(np.arange(40), np.arange(33), indexing="ij")
    np.testing.assert_array_equal(oracle.mmrelu_at(a, b, ii.ravel(), jj.ravel(), 300, 300, 33).reshape(40, 33), r)


def test_fp32_tolerance_is_attainable_and_discriminating():
    """The fp32 bound max|C - R| <= 1e-4*sqrt(K) at the 4096^3 U(-1,1) workload:
    an fp32-accumulated product (BLAS sgemm, a stand-in for any fp32 kernel)
    meets it on sampled rows, while the same product on bf16-rounded inputs
    (a reduced-precision shortcut) does not."""
    K = 4096
    a = datagen.uniform_pm1_f32(1003, 24, K)
    b = datagen.uniform_pm1_f32(2003, K, 512)
    r = oracle.mmrelu(a, b)
    bound = 1e-4 * math.sqrt(K)
    c32 = np.maximum(np.matmul(a, b), 0).astype(np.float64)
    assert np.abs(c32 - r).max() <= bound / 4
    ab = datagen.bf16_bits_to_f32(datagen.f32_to_bf16_bits(a))
    bb = datagen.bf16_bits_to_f32(datagen.f32_to_bf16_bits(b))
    cbf = np.maximum(np.matmul(ab, bb), 0).astype(np.float64)
    assert np.abs(cbf - r).max() > 10 * bound


# ---------------------------------------------------------------------------
# Planted mistakes: each variant of the oracle must fail at least one pin.
# ---------------------------------------------------------------------------

def _ref(a, b):
    return np.matmul(a.astype(np.float64), b.astype(np.float64))


MUTANTS = {
    "no_relu": lambda a, b: _ref(a, b),
    "relu_of_each_product": lambda a, b: np.maximum(
        a.astype(np.float64)[:, :, None] * b.astype(np.float64)[None, :, :], 0).sum(axis=1),
    "negated": lambda a, b: np.maximum(-_ref(a, b), 0),
    "dropped_last_k": lambda a, b: np.maximum(_ref(a[:, :-1], b[:-1, :]), 0),
    "dropped_first_k": lambda a, b: np.maximum(_ref(a[:, 1:], b[1:, :]), 0),
    "transposed_b": lambda a, b: np.maximum(_ref(a, b.T), 0) if a.shape[1] == b.shape[1] else
    np.maximum(_ref(a, b), 0)[:, ::-1],
    "rows_shifted": lambda a, b: np.maximum(_ref(np.roll(a, 1, axis=0), b), 0),
    "fp32_accumulate_then_bf16": lambda a, b: np.maximum(
        datagen.bf16_bits_to_f32(datagen.f32_to_bf16_bits(np.matmul(a, b))).astype(np.float64), 0),
    "relu_leaky": lambda a, b: np.where(_ref(a, b) > 0, _ref(a, b), 0.01 * _ref(a, b)),
    "abs_instead_of_relu": lambda a, b: np.abs(_ref(a, b)),
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
