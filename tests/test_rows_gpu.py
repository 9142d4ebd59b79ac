"""Parity of the row softmax and row sum with the fp64 oracle (needs the GPU;
every call goes through the C-ABI).

Tolerances, from the fp32 arithmetic of the kernels:
  * softmax, fp32 out: |Y - R| <= 2e-5 R + 1e-30. Each output is expf of a
    rounded difference (relative error about |x - m| 2^-24, a few 1e-6 for
    these inputs), times 1/s, where s is a sum of at most 64 terms per
    thread and a tree over the threads (relative error under 80 * 2^-24 =
    4.8e-6 for positive terms); the absolute term covers outputs that
    underflow fp32.
  * softmax, bf16 out: |Y - R| <= 2^-8 R + 1e-30 (one rounding to bf16 on
    top of the fp32 error).
  * row sum, fp32 accumulation: |out - R| <= (N/64 + 16) 2^-24 sum|x| (each
    element passes through at most N/64 additions per thread plus the tree);
    exact on small-integer inputs.
"""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
import tiled_matmul_relu_amd as mm

pytestmark = pytest.mark.gpu


def to_dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def logits(dtype, M, N, seed, scale=2.0, pad=0):
    x = datagen.normal_f32(seed, M, N, scale)
    if pad:
        x = datagen.pad_rows(x, N + pad, fill=np.nan)
    return datagen.f32_to_bf16_bits(x) if dtype == "bf16" else x


def run_softmax(x, M, N, ldx, ldy, variant=None, in_place=False, guard=16):
    dt = torch.float32 if x.dtype == np.float32 else torch.bfloat16
    dx = to_dev(x.ravel())
    if in_place:
        dy, yptr = dx, dx.data_ptr()
        total = dx.numel()
    else:
        total = M * ldy + 2 * guard
        dy = torch.full((total,), float("nan"), dtype=dt, device="cuda")
        yptr = dy.data_ptr() + guard * dy.element_size()
    s = torch.cuda.current_stream().cuda_stream
    if dt == torch.float32:
        rc = (mm.mmrelu_softmax_rows_f32(dx.data_ptr(), yptr, M, N, ldx, ldy, s) if variant is None else
              mm.mmrelu_softmax_rows_f32_variant(variant, dx.data_ptr(), yptr, M, N, ldx, ldy, s))
    else:
        rc = (mm.mmrelu_softmax_rows_bf16(dx.data_ptr(), yptr, M, N, ldx, ldy, s) if variant is None else
              mm.mmrelu_softmax_rows_bf16_variant(variant, dx.data_ptr(), yptr, M, N, ldx, ldy, s))
    assert rc == mm.MMRELU_OK, mm.status_string(rc)
    torch.cuda.synchronize()
    whole = to_host(dy)
    if in_place:
        return whole.reshape(M, ldx)[:, :N], None
    body = whole[guard:guard + M * ldy].reshape(M, ldy)
    outside = np.concatenate([whole[:guard], whole[guard + M * ldy:], body[:, N:].ravel()])
    return body[:, :N], outside


def check_softmax(y, r):
    if y.dtype == np.float32:
        assert np.all(np.isfinite(y))
        err = np.abs(y.astype(np.float64) - r)
        assert np.all(err <= 2e-5 * r + 1e-30), (err / np.maximum(r, 1e-300)).max()
        assert np.all(np.abs(y.astype(np.float64).sum(axis=1) - 1) <= 1e-4)
    else:
        yf = datagen.bf16_bits_to_f32(y).astype(np.float64)
        assert np.all(np.isfinite(yf))
        assert np.all(np.abs(yf - r) <= 2.0 ** -8 * r + 1e-30), np.abs(yf - r).max()


def nan_everywhere(outside):
    o = datagen.bf16_bits_to_f32(outside) if outside.dtype == np.uint16 else outside
    return np.all(np.isnan(o))


NS = {"f32": [1, 7, 64, 100, 1000, 1024, 1028, 3000, 4096, 4100, 10000, 16384, 16388, 40000],
      "bf16": [1, 9, 64, 100, 1000, 2048, 2056, 6000, 8192, 8200, 20000, 32768, 32776, 70000]}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ni", range(14))
def test_softmax_every_kernel(dtype, ni):
    N = NS[dtype][ni]
    kind = mm.DTYPE_F32 if dtype == "f32" else mm.DTYPE_BF16
    esize = 4 if dtype == "f32" else 2
    M = 37 if N <= 20000 else 9
    x = logits(dtype, M, N, 1400 + ni)
    r = oracle.softmax_rows(x)
    chosen = mm.mmrelu_softmax_rows_variant(kind, N, N, N)
    print(f"softmax {dtype} M={M} N={N} planner variant {chosen}", flush=True)
    y, outside = run_softmax(x, M, N, N, N)
    check_softmax(y, r)
    assert nan_everywhere(outside)
    caps = [64 * 4 * 16 // esize, 256 * 4 * 16 // esize, 256 * 16 * 16 // esize]
    for v in range(5):
        ok = v == 4 or (N % (16 // esize) == 0 and (v == 3 or N <= caps[v]))
        if not ok:
            continue
        print(f"softmax {dtype} M={M} N={N} variant {v}", flush=True)
        y, outside = run_softmax(x, M, N, N, N, variant=v)
        check_softmax(y, r)
        assert nan_everywhere(outside)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_softmax_padded_unaligned_and_in_place(dtype):
    for (M, N, pad) in [(33, 1000, 24), (17, 777, 5), (40, 4096, 8), (5, 20000, 3)]:
        x = logits(dtype, M, N, 1450 + N, pad=pad)
        ldx = N + pad
        r = oracle.softmax_rows(x, M=M, N=N, ldx=ldx)
        for ldy in (N, N + 16):
            print(f"softmax {dtype} M={M} N={N} ldx={ldx} ldy={ldy}", flush=True)
            y, outside = run_softmax(x, M, N, ldx, ldy)
            check_softmax(y, r)
            assert nan_everywhere(outside)
        y, _ = run_softmax(x, M, N, ldx, ldx, in_place=True)
        check_softmax(y, r)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_softmax_large_and_constant_rows(dtype):
    """Rows offset by +-1000 (finite only because the maximum is subtracted)
    and constant rows (exactly uniform)."""
    M, N = 8, 4096
    x = datagen.normal_f32(1461, M, N, 3.0)
    x[:3] += 1000.0
    x[3:5] -= 1000.0
    x[5] = 0.0
    x[6] = 7.5
    x = datagen.f32_to_bf16_bits(x) if dtype == "bf16" else x
    r = oracle.softmax_rows(x)
    for v in (None, 3, 4):
        y, _ = run_softmax(x, M, N, N, N, variant=v)
        check_softmax(y, r)
        yf = datagen.bf16_bits_to_f32(y) if y.dtype == np.uint16 else y
        if dtype == "f32":
            assert np.all(yf[5:7] == np.float32(1 / 4096))


def test_softmax_full_size_f32():
    """The 8192 x 8192 fp32 workload, compared on 64 sampled rows."""
    M = N = 8192
    x = datagen.normal_f32(1471, M, N, 2.0)
    y, _ = run_softmax(x, M, N, N, N, guard=0)
    rows = np.random.default_rng(1472).choice(M, 64, replace=False)
    check_softmax(y[rows], oracle.softmax_rows(np.ascontiguousarray(x[rows])))


def run_row_sum(x, M, N, ldx):
    dx = to_dev(x.ravel())
    out = torch.full((M + 32,), float("nan"), dtype=torch.float32, device="cuda")
    fn = mm.mmrelu_row_sum_f32 if x.dtype == np.float32 else mm.mmrelu_row_sum_bf16
    rc = fn(dx.data_ptr(), out.data_ptr() + 16 * 4, M, N, ldx, torch.cuda.current_stream().cuda_stream)
    assert rc == mm.MMRELU_OK, mm.status_string(rc)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(np.isnan(o[:16])) and np.all(np.isnan(o[16 + M:]))
    return o[16:16 + M]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_row_sum_shapes(dtype):
    for (M, N, pad) in [(1, 1, 0), (17, 5, 0), (300, 100, 0), (64, 1024, 0), (33, 1025, 3), (129, 4096, 0),
                        (7, 4099, 5), (5, 65536, 0), (40, 0, 0), (12, 3000, 8)]:
        x = datagen.normal_f32(1480 + N, M, max(N, 1), 1.0)[:, :N].copy()
        if pad:
            x = datagen.pad_rows(x, N + pad, fill=np.nan)
        x = datagen.f32_to_bf16_bits(x) if dtype == "bf16" else x
        ldx = max(N + pad, 1)
        print(f"row sum {dtype} M={M} N={N} ldx={ldx}", flush=True)
        o = run_row_sum(x if N else np.zeros(1, x.dtype), M, N, ldx)
        r = oracle.row_sum(x, M=M, N=N, ldx=ldx) if N else np.zeros(M)
        wide = datagen.bf16_bits_to_f32(x) if x.dtype == np.uint16 else x
        absum = np.nansum(np.abs(wide.reshape(M, -1)[:, :N].astype(np.float64)), axis=1) if N else np.zeros(M)
        assert np.all(np.abs(o - r) <= (N / 64 + 16) * 2.0 ** -24 * absum), np.abs(o - r).max()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_row_sum_exact_integers(dtype):
    M, N = 200, 4096
    x = datagen.small_int_f32(1491, M, N)
    x = datagen.f32_to_bf16_bits(x) if dtype == "bf16" else x
    assert np.array_equal(run_row_sum(x, M, N, N).astype(np.float64), oracle.row_sum(x))


def test_torch_wrappers():
    x = to_dev(datagen.normal_f32(1495, 64, 1000, 2.0))
    y = mm.softmax_rows(x)
    s = mm.row_sum(x)
    torch.cuda.synchronize()
    xh = x.cpu().numpy()
    check_softmax(y.cpu().numpy(), oracle.softmax_rows(xh))
    assert np.all(np.abs(s.cpu().numpy() - oracle.row_sum(xh)) <= 32 * 2.0 ** -24 * np.abs(xh).sum(axis=1))
    z = mm.softmax_rows(x, out=x)                      # in place
    torch.cuda.synchronize()
    assert z.data_ptr() == x.data_ptr()
    check_softmax(x.cpu().numpy(), oracle.softmax_rows(xh))
