"""Parity of the skinny kernels (few rows: M <= 64, or few columns: N <= 64)
with the fp64 oracle (needs the GPU; every call goes through the C-ABI).

The skinny kernels split K over eight waves per workgroup and sum the eight
partial tiles at the end, so their summation order differs from the
large-tile kernels'; the tolerances are the same: fp32 max |C - R| <=
1e-4 * sqrt(K), bf16 relative Frobenius <= 1e-2 with the elementwise bound
2^-8 |R| + 1e-6, and exact results on small-integer inputs. Every skinny
variant tiles any shape, so each is also run on shapes many tiles wide and
tall.
"""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
import tiled_matmul_relu_amd as mm

pytestmark = pytest.mark.gpu

SKINNY = [5, 6, 7, 8, 9, 10, 12]  # tiles 16x32, 32x32, 64x32 (few rows), 32x16, 32x32, 32x64 (few columns), 64x64
SKINNY_F32 = SKINNY + [13, 14]    # fp32 also: 16x64 strips (few rows, many columns), 64x16 bands
SKINNY_BF16 = SKINNY + [14]       # the 16x64 strips in the bf16 table


def to_dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def run(a, b, M, N, K, lda, ldb, ldc=None, variant=None, act=mm.ACT_RELU, bias=None, guard=0):
    dt = torch.float32 if a.dtype == np.float32 else torch.bfloat16
    ldc = ldc or N
    da, db = to_dev(a), to_dev(b)
    dbias = to_dev(bias) if bias is not None else None
    buf = torch.full((M + 2 * guard, ldc), float("nan"), dtype=dt, device="cuda")
    c_ptr = buf.data_ptr() + guard * ldc * buf.element_size()
    args = (act, da.data_ptr(), db.data_ptr(), dbias.data_ptr() if dbias is not None else 0, c_ptr,
            M, N, K, lda, ldb, ldc, torch.cuda.current_stream().cuda_stream)
    if dt == torch.float32:
        rc = mm.mmrelu_fused_f32(*args) if variant is None else mm.mmrelu_fused_f32_variant(variant, *args)
    else:
        rc = mm.mmrelu_fused_bf16(*args) if variant is None else mm.mmrelu_fused_bf16_variant(variant, *args)
    assert rc == mm.MMRELU_OK, mm.status_string(rc)
    torch.cuda.synchronize()
    whole = to_host(buf)
    return whole[guard:guard + M, :N], whole


def check(c, r, K, dtype, relu=True):
    if dtype == "f32":
        assert np.all(np.isfinite(c))
        err = np.abs(c.astype(np.float64) - r)
        assert err.max(initial=0) <= 1e-4 * math.sqrt(max(K, 1)), err.max()
    else:
        cf = datagen.bf16_bits_to_f32(c).astype(np.float64)
        assert np.all(np.isfinite(cf))
        nr = np.linalg.norm(r)
        assert (np.linalg.norm(cf - r) / nr if nr > 0 else np.linalg.norm(cf)) <= 1e-2
        assert np.all(np.abs(cf - r) <= 2.0 ** -8 * np.abs(r) + 1e-6), np.abs(cf - r).max()
        c = cf
    if relu:
        assert np.all(c >= 0)


def inputs(dtype, M, N, K, seed):
    a = datagen.normal_f32(seed, M, K, 1 / math.sqrt(K))
    b = datagen.normal_f32(seed + 1, K, N, 1 / math.sqrt(K))
    if dtype == "bf16":
        return datagen.f32_to_bf16_bits(a), datagen.f32_to_bf16_bits(b)
    return a, b


MS = [1, 3, 16, 17, 32, 33, 64]
NK = [(32, 8), (264, 72), (1000, 1032), (520, 4096)]


def run_all_skinny(dtype, a, b, M, N, K, r):
    for v in (SKINNY_BF16 if dtype == "bf16" else SKINNY_F32):
        print(f"{dtype} {M}x{N}x{K} variant={v}", flush=True)
        check(run(a, b, M, N, K, K, N, variant=v)[0], r, K, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M", MS)
def test_skinny_rows_every_variant(dtype, M):
    kind = mm.DTYPE_F32 if dtype == "f32" else mm.DTYPE_BF16
    for si, (N, K) in enumerate(NK):
        a, b = inputs(dtype, M, N, K, 900 + 10 * M + si)
        r = oracle.mmrelu(a, b)
        plan = mm.mmrelu_plan(kind, M, N, K, K, N, N)
        assert "skinny" in plan["name"], plan["name"]
        print(f"{dtype} M={M} N={N} K={K} planner {plan['name']}", flush=True)
        check(run(a, b, M, N, K, K, N)[0], r, K, dtype)
        run_all_skinny(dtype, a, b, M, N, K, r)


NS = {"f32": [4, 12, 16, 24, 32, 40, 64], "bf16": [8, 16, 24, 32, 40, 64]}
MK = [(40, 8), (264, 72), (1000, 1032), (72, 4096)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ni", range(7))
def test_skinny_columns_every_variant(dtype, ni):
    if ni >= len(NS[dtype]):
        pytest.skip("fewer column counts for this dtype")
    N = NS[dtype][ni]
    kind = mm.DTYPE_F32 if dtype == "f32" else mm.DTYPE_BF16
    for si, (M, K) in enumerate(MK):
        a, b = inputs(dtype, M, N, K, 1900 + 10 * N + si)
        r = oracle.mmrelu(a, b)
        plan = mm.mmrelu_plan(kind, M, N, K, K, N, N)
        assert "skinny" in plan["name"], plan["name"]
        print(f"{dtype} M={M} N={N} K={K} planner {plan['name']}", flush=True)
        check(run(a, b, M, N, K, K, N)[0], r, K, dtype)
        run_all_skinny(dtype, a, b, M, N, K, r)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_skinny_variants_tile_large_shapes(dtype):
    """Every skinny variant on shapes many tiles tall and wide, with ragged
    edges in both directions."""
    for si, (M, N, K) in enumerate([(300, 200, 264), (129, 520, 1032)]):
        a, b = inputs(dtype, M, N, K, 961 + si)
        run_all_skinny(dtype, a, b, M, N, K, oracle.mmrelu(a, b))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_skinny_exact_integers(dtype):
    M, N, K = 33, 264, 520
    a, b = datagen.small_int_f32(921, M, K), datagen.small_int_f32(922, K, N)
    if dtype == "bf16":
        a, b = datagen.f32_to_bf16_bits(a), datagen.f32_to_bf16_bits(b)
    r = oracle.mmrelu(a, b)
    c, _ = run(a, b, M, N, K, K, N)
    if dtype == "f32":
        np.testing.assert_array_equal(c.astype(np.float64), r)
    else:
        ref = torch.from_numpy(r.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        np.testing.assert_array_equal(c, ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,N", [(40, 264), (264, 40)], ids=["rows", "columns"])
def test_skinny_guard_band_padded(dtype, M, N):
    """Padded lda/ldb/ldc (NaN padding in A and B must never be read) and rows
    around C: nothing outside the window is written."""
    K = 136
    lda, ldb, ldc = K + 8, N + 16, N + 24
    a32 = datagen.pad_rows(datagen.normal_f32(931, M, K, 1 / math.sqrt(K)), lda, fill=np.nan)
    b32 = datagen.pad_rows(datagen.normal_f32(932, K, N, 1 / math.sqrt(K)), ldb, fill=np.nan)
    a, b = (a32, b32) if dtype == "f32" else (datagen.f32_to_bf16_bits(a32), datagen.f32_to_bf16_bits(b32))
    r = oracle.mmrelu(a, b, M=M, N=N, K=K, lda=lda, ldb=ldb)
    kind = mm.DTYPE_F32 if dtype == "f32" else mm.DTYPE_BF16
    assert "skinny" in mm.mmrelu_plan(kind, M, N, K, lda, ldb, ldc)["name"]
    for v in [None] + (SKINNY_BF16 if dtype == "bf16" else SKINNY_F32):
        c, whole = run(a, b, M, N, K, lda, ldb, ldc=ldc, variant=v, guard=3)
        check(c, r, K, dtype)
        wf = whole.astype(np.float32) if dtype == "f32" else datagen.bf16_bits_to_f32(whole)
        outside = np.ones(wf.shape, bool)
        outside[3:3 + M, :N] = False
        assert np.all(np.isnan(wf[outside])), f"variant {v} wrote outside the window"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,N", [(24, 520), (520, 24)], ids=["rows", "columns"])
def test_skinny_fused_epilogue(dtype, M, N):
    K = 264
    a, b = inputs(dtype, M, N, K, 941)
    bias = datagen.normal_f32(943, 1, N, 0.5).ravel()
    if dtype == "bf16":
        bias = datagen.f32_to_bf16_bits(bias)
    for act_name, act in (("gelu_tanh", mm.ACT_GELU_TANH), ("none", mm.ACT_NONE), ("relu", mm.ACT_RELU)):
        r = oracle.fused(act_name, a, b, bias)
        c, _ = run(a, b, M, N, K, K, N, act=act, bias=bias)
        if dtype == "f32":
            slope = 1.13 if act_name == "gelu_tanh" else 1.0
            assert np.all(np.abs(c.astype(np.float64) - r) <= slope * 1e-4 * math.sqrt(K) + 2e-6 * (1 + np.abs(r)))
        else:
            cf = datagen.bf16_bits_to_f32(c).astype(np.float64)
            assert np.all(np.abs(cf - r) <= 2.0 ** -8 * np.abs(r) + 4e-6)


@pytest.mark.parametrize("dtype,M,N,K", [("bf16", 16, 8192, 8192), ("f32", 64, 4096, 4096),
                                         ("bf16", 8192, 16, 8192), ("f32", 4096, 64, 4096)])
def test_skinny_full_size(dtype, M, N, K):
    """Full compare at the sweep's skinny sizes (the oracle runs ~1e9 MACs)."""
    print(f"skinny full size {dtype} {M}x{N}x{K}", flush=True)
    a, b = inputs(dtype, M, N, K, 951)
    kind = mm.DTYPE_F32 if dtype == "f32" else mm.DTYPE_BF16
    assert "skinny" in mm.mmrelu_plan(kind, M, N, K, K, N, N)["name"]
    c, _ = run(a, b, M, N, K, K, N)
    check(c, oracle.mmrelu(a, b), K, dtype)
