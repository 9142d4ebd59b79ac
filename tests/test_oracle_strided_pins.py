"""Pins of the oracle's general-stride form to facts outside it (CPU only).

The lecture maps a (row, column) index to memory as row times the row stride
plus column times the column stride, and notes that a transpose is the same
data with the two strides exchanged ("Kernels, Triton, XLA", section
"Reductions and tiling", before the matmul kernel); the Chinese notes'
section 5.5 kernel takes one stride per dimension of each operand. The pins:
exact integer products of numpy-materialised views (transposed storage,
sub-sampled views, a zero stride that repeats one column), a closed form for
the zero-stride case, float64 BLAS within the rounding of K additions, and
the transpose identity relu(A·B)^T = relu(B^T·A^T) read through exchanged
strides. Deliberately broken stride handling at the bottom must each fail at
least one pin.
"""
import numpy as np
import pytest

import datagen
import oracle


def oracle_impl(act, a, b, bias, M, N, K, sam, sak, sbk, sbn):
    return oracle.strided(act, a, b, bias, M, N, K, sam, sak, sbk, sbn)


def oracle_at_impl(act, a, b, bias, M, N, K, sam, sak, sbk, sbn):
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    return oracle.strided_at(act, a, b, bias, ii.ravel(), jj.ravel(), M, N, K, sam, sak, sbk, sbn).reshape(M, N)


def _ints(seed, rows, cols):
    return datagen.small_int_f32(seed, rows, cols)


def _exact(a_log, b_log, bias=None, act="relu"):
    s = a_log.astype(np.int64) @ b_log.astype(np.int64)
    if bias is not None:
        s = s + bias.astype(np.int64)[None, :]
    return (np.maximum(s, 0) if act == "relu" else s).astype(np.float64)


def pin_transposed_storage(impl):
    """A stored as A^T (K x M row-major: sam = 1, sak = M) and B as B^T (N x K:
    sbk = 1, sbn = K), against the integer product of the logical matrices."""
    M, N, K = 13, 9, 11
    a_log, b_log = _ints(401, M, K), _ints(402, K, N)
    at, bt = np.ascontiguousarray(a_log.T), np.ascontiguousarray(b_log.T)
    assert np.array_equal(impl("relu", at.ravel(), bt.ravel(), None, M, N, K, 1, M, 1, K), _exact(a_log, b_log))
    assert np.array_equal(impl("none", at.ravel(), b_log.ravel(), None, M, N, K, 1, M, N, 1),
                          _exact(a_log, b_log, act="none"))
    assert np.array_equal(impl("none", a_log.ravel(), bt.ravel(), None, M, N, K, K, 1, 1, K),
                          _exact(a_log, b_log, act="none"))


def pin_subsampled_views(impl):
    """A = buf[::2, ::3] of a 2M x 3K buffer and B = buf[1::3, ::2] of a 3K x 2N
    buffer, with a bias: strides (6K, 3) and (6N, 2) from offsets 0 and 2N."""
    M, N, K = 7, 6, 10
    abuf, bbuf = _ints(411, 2 * M, 3 * K), _ints(412, 3 * K, 2 * N)
    bias = _ints(413, 1, N).ravel() * 4
    a_log, b_log = abuf[::2, ::3], bbuf[1::3, ::2]
    got = impl("none", abuf.ravel(), bbuf.ravel()[2 * N:].copy(), bias, M, N, K, 6 * K, 3, 6 * N, 2)
    assert np.array_equal(got, _exact(a_log, b_log, bias, act="none"))


def pin_zero_stride_closed_form(impl):
    """sak = 0 repeats A[i][0] along k: R[i][j] = A[i][0] * sum_k B[k][j]."""
    M, N, K = 5, 8, 12
    col = _ints(421, M, 1).ravel()
    b_log = _ints(422, K, N)
    expect = col.astype(np.int64)[:, None] * b_log.astype(np.int64).sum(axis=0)[None, :]
    got = impl("none", col, b_log.ravel(), None, M, N, K, 1, 0, N, 1)
    assert np.array_equal(got, expect.astype(np.float64))


def pin_float_against_blas(impl):
    """Random normal data in a transposed A and a padded B, against float64
    BLAS within 4 K eps |A||B|."""
    M, N, K = 17, 23, 129
    a_log = datagen.normal_f32(431, M, K, 1.0)
    b_pad = datagen.normal_f32(432, K, N + 5, 1.0)
    at = np.ascontiguousarray(a_log.T)
    ref = a_log.astype(np.float64) @ b_pad[:, :N].astype(np.float64)
    bound = 4 * K * np.finfo(np.float64).eps * (np.abs(a_log).astype(np.float64) @ np.abs(b_pad[:, :N]).astype(np.float64))
    got = impl("none", at.ravel(), b_pad.ravel(), None, M, N, K, 1, M, N + 5, 1)
    assert np.all(np.abs(got - ref) <= bound)
    assert (ref < 0).any()


def pin_transpose_identity(impl):
    """relu(A·B)^T = relu(B^T·A^T): the same buffers read with exchanged
    strides give the transposed result (bf16 inputs)."""
    M, N, K = 9, 14, 16
    a = datagen.f32_to_bf16_bits(_ints(441, M, K))
    b = datagen.f32_to_bf16_bits(_ints(442, K, N))
    r = impl("relu", a.ravel(), b.ravel(), None, M, N, K, K, 1, N, 1)
    rt = impl("relu", b.ravel(), a.ravel(), None, N, M, K, 1, N, 1, K)
    assert np.array_equal(r.T, rt)
    wide = datagen.bf16_bits_to_f32
    assert np.array_equal(r, _exact(wide(a), wide(b)))


PINS = [pin_transposed_storage, pin_subsampled_views, pin_zero_stride_closed_form, pin_float_against_blas,
        pin_transpose_identity]


@pytest.mark.parametrize("impl", [oracle_impl, oracle_at_impl], ids=["full", "at"])
@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_strided_pin(pin, impl):
    pin(impl)


def test_strided_arguments_are_checked():
    a, b = np.zeros(12, np.float32), np.zeros(12, np.float32)
    with pytest.raises(ValueError):
        oracle.strided("relu", a, b, None, 3, 4, 4, 4, 1, 4, 1)        # B needs 16 elements
    with pytest.raises(ValueError):
        oracle.strided("relu", a, b, None, 3, 3, 4, 4, 1, -1, 1)       # negative stride
    with pytest.raises(TypeError):
        oracle.strided("relu", a, b.astype(np.uint16), None, 3, 3, 4, 4, 1, 3, 1)


# ---------------------------------------------------------------------------
# Planted mistakes (numpy re-implementations on the CPU): each must fail a pin.
# ---------------------------------------------------------------------------

def _gather(buf, rows, cols, s_r, s_c):
    r = np.arange(rows)[:, None] * s_r + np.arange(cols)[None, :] * s_c
    return buf.ravel()[r]


def _mutant(a_idx, b_idx):
    def impl(act, a, b, bias, M, N, K, sam, sak, sbk, sbn):
        w = datagen.bf16_bits_to_f32 if a.dtype == np.uint16 else (lambda x: x)
        al = w(a_idx(a, M, K, sam, sak)).astype(np.float64)
        bl = w(b_idx(b, K, N, sbk, sbn)).astype(np.float64)
        s = al @ bl
        if bias is not None:
            s = s + w(bias).astype(np.float64)[None, :]
        return np.maximum(s, 0) if act == "relu" else s
    return impl


def _ok(buf, rows, cols, s_r, s_c):
    return _gather(buf, rows, cols, s_r, s_c)


def _clamped(buf, rows, cols, s_r, s_c):
    r = np.arange(rows)[:, None] * s_r + np.arange(cols)[None, :] * s_c
    return buf.ravel()[np.minimum(r, buf.size - 1)]


MUTANTS = {
    "a_strides_exchanged": _mutant(lambda a, M, K, s0, s1: _clamped(a, M, K, s1, s0), _ok),
    "b_strides_exchanged": _mutant(_ok, lambda b, K, N, s0, s1: _clamped(b, K, N, s1, s0)),
    "a_column_stride_taken_as_1": _mutant(lambda a, M, K, s0, s1: _clamped(a, M, K, s0, 1), _ok),
    "b_column_stride_taken_as_1": _mutant(_ok, lambda b, K, N, s0, s1: _clamped(b, K, N, s0, 1)),
    "b_row_stride_taken_as_n": _mutant(_ok, lambda b, K, N, s0, s1: _clamped(b, K, N, N, s1)),
    "a_row_stride_taken_as_k": _mutant(lambda a, M, K, s0, s1: _clamped(a, M, K, K, s1), _ok),
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


def test_correct_numpy_gather_passes_every_pin():
    """The mutants' harness itself is sound: with correct strides it passes."""
    impl = _mutant(_ok, _ok)
    for pin in PINS:
        pin(impl)
