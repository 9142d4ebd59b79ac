"""Parity at the size limits (needs the GPU).

The library accepts leading dimensions up to 2^21 elements: the tile and
skinny kernels address a tile with 32-bit byte offsets from a 64-bit tile
base, and at that limit the tallest tiles (256 bf16 rows, 128 fp32 rows)
reach offsets near 2^30. These tests run every kernel family at lda = ldb =
ldc = 2^21 (2^21 - 1 for the any-layout kernel) on operands whose padding
is filled with NaN, so a read past K or N would poison C, and with NaN
sentinels in C's padding and in guard rows around it, which must survive.
A very tall product (2^20 + a few rows) is checked on sampled rows, which
the oracle evaluates one dot product at a time, and on properties of the
whole output. Tolerances as in the parity tests: fp32 max |C - R| <= 1e-4
sqrt(K); bf16 relative Frobenius <= 1e-2 and elementwise 2^-8 |R| + 1e-6.
The padded buffers are built on the device, so host memory stays small.
"""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
import tiled_matmul_relu_amd as mm

pytestmark = pytest.mark.gpu

LD = 1 << 21


def dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def padded(x: np.ndarray, ld: int) -> torch.Tensor:
    """Device copy of the compact rows x cols matrix x with leading dimension
    ld; the padding columns hold NaN."""
    rows, cols = x.shape
    dt = torch.float32 if x.dtype == np.float32 else torch.bfloat16
    t = torch.full((rows, ld), float("nan"), dtype=dt, device="cuda")
    t[:, :cols] = dev(x)
    return t


def inputs(dtype, M, N, K, seed):
    a = datagen.normal_f32(seed, M, K, 1 / math.sqrt(K))
    b = datagen.normal_f32(seed + 1, K, N, 1 / math.sqrt(K))
    if dtype == "bf16":
        return datagen.f32_to_bf16_bits(a), datagen.f32_to_bf16_bits(b)
    return a, b


def check(c, r, K, dtype):
    if dtype == "f32":
        assert np.all(np.isfinite(c)) and np.all(c >= 0)
        assert np.abs(c.astype(np.float64) - r).max(initial=0) <= 1e-4 * math.sqrt(K)
    else:
        cf = datagen.bf16_bits_to_f32(c).astype(np.float64)
        assert np.all(np.isfinite(cf)) and np.all(cf >= 0)
        assert np.linalg.norm(cf - r) / np.linalg.norm(r) <= 1e-2
        assert np.all(np.abs(cf - r) <= 2.0 ** -8 * np.abs(r) + 1e-6)


def launch(dtype, variant, da, db, c_ptr, M, N, K, lda, ldb, ldc):
    args = (da.data_ptr(), db.data_ptr(), c_ptr, M, N, K, lda, ldb, ldc, torch.cuda.current_stream().cuda_stream)
    if dtype == "f32":
        rc = mm.mmrelu_f32(*args) if variant is None else mm.mmrelu_f32_variant(variant, *args)
    else:
        rc = mm.mmrelu_bf16(*args) if variant is None else mm.mmrelu_bf16_variant(variant, *args)
    assert rc == mm.MMRELU_OK, mm.status_string(rc)


# (dtype, M, N, K, ld, variants): None is the planner's choice. fp32: 1, 3
# the aligned 128/64 tiles, 2 the unaligned 128 tile, 12 the 64x64 skinny
# tile; bf16: 1 and 3 the ping-pong tiles (256 and 128 rows), 4 the 128
# tile, 12 the 64x64 skinny tile, 2/13/15 the any-layout tiles (128, 64, 256);
# N = 1 the matrix-vector kernel; M = 40 the few-rows skinny rule.
CASES = [
    ("f32", 300, 264, 136, LD, [None, 1, 2, 3, 12]),
    ("f32", 40, 264, 136, LD, [None]),
    ("f32", 300, 1, 136, LD, [None]),
    ("bf16", 300, 264, 136, LD, [None, 1, 3, 4, 12]),
    ("bf16", 40, 264, 136, LD, [None]),
    ("bf16", 300, 1, 136, LD, [None]),
    ("bf16", 300, 264, 136, LD - 1, [None, 2, 13, 15]),
]


@pytest.mark.parametrize("dtype,M,N,K,ld,vs", CASES,
                         ids=[f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-ld{c[4]}" for c in CASES])
def test_maximum_leading_dimensions(dtype, M, N, K, ld, vs):
    a, b = inputs(dtype, M, N, K, 1500 + M + N)
    r = oracle.mmrelu(a, b)
    da, db = padded(a, ld), padded(b, ld)
    dt = da.dtype
    guard = 2
    for v in vs:
        print(f"limits {dtype} {M}x{N}x{K} ld={ld} variant={v}", flush=True)
        buf = torch.full((M + 2 * guard, ld), float("nan"), dtype=dt, device="cuda")
        c_ptr = buf.data_ptr() + guard * ld * buf.element_size()
        launch(dtype, v, da, db, c_ptr, M, N, K, ld, ld, ld)
        torch.cuda.synchronize()
        check(host(buf[guard:guard + M, :N]), r, K, dtype)
        # nothing outside the M x N window was written
        assert bool(torch.isnan(buf[guard:guard + M, N:]).all()), f"variant {v} wrote into C's padding"
        assert bool(torch.isnan(buf[:guard]).all()) and bool(torch.isnan(buf[guard + M:]).all()), \
            f"variant {v} wrote outside C's rows"
        del buf
    del da, db
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,M,N,K", [("bf16", (1 << 20) + 5, 264, 40), ("f32", (1 << 20) + 3, 136, 40)])
def test_tall_product_sampled(dtype, M, N, K):
    """2^20 + a few rows through the planner's kernel; the oracle evaluates
    sampled rows (and the last rows, across a ragged tile) in full."""
    a, b = inputs(dtype, M, N, K, 1600)
    da, db = dev(a), dev(b)
    dt = da.dtype
    c = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
    print(f"tall {dtype} {M}x{N}x{K}", flush=True)
    launch(dtype, None, da, db, c.data_ptr(), M, N, K, K, N, N)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(c).all()) and bool((c >= 0).all())
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([rng.integers(0, M, 1500), np.arange(M - 8, M), np.arange(0, 8)]))
    ii = np.repeat(rows, N)
    jj = np.tile(np.arange(N), rows.size)
    r = oracle.mmrelu_at(a, b, ii, jj, K, K, N).reshape(rows.size, N)
    got = host(c[torch.from_numpy(rows).cuda()])
    check(got, r, K, dtype)
    del da, db, c
    torch.cuda.empty_cache()
