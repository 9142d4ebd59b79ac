"""Parity of the matrix-vector kernel (one wave per output; the planner's
choice for N = 1) with the fp64 oracle (needs the GPU; every call goes
through the C-ABI). Tolerances as for the other kernels: fp32 max |C - R| <=
1e-4 sqrt(K) (L = 1.13 for GeLU, plus 2e-6 (1 + |R|) with a bias), bf16
2^-8 |R| + 1e-6 elementwise; exact on small-integer inputs.
"""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
import tiled_matmul_relu_amd as mm

pytestmark = pytest.mark.gpu

GEMV = 11


def to_dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def run(a, b, M, N, K, lda, ldb, ldc, variant=None, act=mm.ACT_RELU, bias=None, guard=8):
    dt = torch.float32 if a.dtype == np.float32 else torch.bfloat16
    da, db = to_dev(a), to_dev(b)
    dbias = to_dev(bias) if bias is not None else None
    buf = torch.full(((M - 1) * ldc + N + 2 * guard,), float("nan"), dtype=dt, device="cuda")
    cp = buf.data_ptr() + guard * buf.element_size()
    args = (act, da.data_ptr(), db.data_ptr(), dbias.data_ptr() if dbias is not None else 0, cp, M, N, K, lda, ldb,
            ldc, torch.cuda.current_stream().cuda_stream)
    if dt == torch.float32:
        rc = mm.mmrelu_fused_f32(*args) if variant is None else mm.mmrelu_fused_f32_variant(variant, *args)
    else:
        rc = mm.mmrelu_fused_bf16(*args) if variant is None else mm.mmrelu_fused_bf16_variant(variant, *args)
    assert rc == mm.MMRELU_OK, mm.status_string(rc)
    torch.cuda.synchronize()
    whole = to_host(buf)
    body = whole[guard:guard + (M - 1) * ldc + N]
    idx = np.arange(M)[:, None] * ldc + np.arange(N)[None, :]
    c = body[idx]
    untouched = np.ones(whole.size, bool)
    untouched[guard + idx.ravel()] = False
    rest = whole[untouched]
    rest = datagen.bf16_bits_to_f32(rest) if rest.dtype == np.uint16 else rest
    assert np.all(np.isnan(rest)), "wrote outside C"
    return c


def check(c, r, K, dtype, act="relu", bias=False):
    if dtype == "f32":
        slope = 1.13 if act == "gelu_tanh" else 1.0
        err = np.abs(c.astype(np.float64) - r)
        assert np.all(err <= slope * 1e-4 * math.sqrt(max(K, 1)) + (2e-6 * (1 + np.abs(r)) if bias else 0)), err.max()
    else:
        cf = datagen.bf16_bits_to_f32(c).astype(np.float64)
        assert np.all(np.abs(cf - r) <= 2.0 ** -8 * np.abs(r) + 4e-6), np.abs(cf - r).max()


def vec_inputs(dtype, M, K, lda, ldb, seed):
    a = datagen.pad_rows(datagen.normal_f32(seed, M, K, 1 / math.sqrt(K)), lda, fill=np.nan)
    bvals = datagen.normal_f32(seed + 1, K, 1, 1 / math.sqrt(K)).ravel()
    b = np.full((K - 1) * ldb + 1, np.nan, np.float32)
    b[::ldb] = bvals
    if dtype == "bf16":
        return datagen.f32_to_bf16_bits(a), datagen.f32_to_bf16_bits(b)
    return a, b


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gemv_shapes_and_layouts(dtype):
    kind = mm.DTYPE_F32 if dtype == "f32" else mm.DTYPE_BF16
    for (M, K, lda, ldb, ldc) in [(1, 1, 1, 1, 1), (5, 7, 7, 1, 1), (300, 1024, 1024, 1, 1), (257, 1000, 1008, 1, 3),
                                  (64, 4096, 4096, 2, 1), (1000, 77, 80, 1, 1), (33, 8200, 8200, 1, 2)]:
        a, b = vec_inputs(dtype, M, K, lda, ldb, 1500 + M)
        r = oracle.mmrelu(a, b, M=M, N=1, K=K, lda=lda, ldb=ldb)
        assert "gemv" in mm.mmrelu_plan(kind, M, 1, K, lda, ldb, ldc)["name"]
        print(f"gemv {dtype} M={M} K={K} lda={lda} ldb={ldb} ldc={ldc}", flush=True)
        check(run(a, b, M, 1, K, lda, ldb, ldc), r, K, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gemv_fused_epilogues_and_integers(dtype):
    M, K = 520, 264
    a, b = vec_inputs(dtype, M, K, K, 1, 1521)
    bias = datagen.normal_f32(1523, 1, 1, 0.5).ravel()
    bias = datagen.f32_to_bf16_bits(bias) if dtype == "bf16" else bias
    for act_name, act in (("gelu_tanh", mm.ACT_GELU_TANH), ("none", mm.ACT_NONE)):
        r = oracle.fused(act_name, a, b.reshape(K, 1), bias)
        check(run(a, b, M, 1, K, K, 1, 1, act=act, bias=bias), r, K, dtype, act_name, bias=True)
    ai, bi = datagen.small_int_f32(1524, M, K), datagen.small_int_f32(1525, K, 1)
    if dtype == "bf16":
        ai, bi = datagen.f32_to_bf16_bits(ai), datagen.f32_to_bf16_bits(bi)
    r = oracle.mmrelu(ai, bi)
    c = run(ai, bi.ravel(), M, 1, K, K, 1, 1)
    if dtype == "f32":
        assert np.array_equal(c.astype(np.float64), r)
    else:
        ref = torch.from_numpy(r.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(c, ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gemv_variant_on_wider_outputs(dtype):
    """The kernel covers any N (one wave per output), though the planner only
    uses it for N = 1."""
    M, N, K = 130, 9, 300
    a = datagen.normal_f32(1531, M, K, 1 / math.sqrt(K))
    b = datagen.normal_f32(1532, K, N, 1 / math.sqrt(K))
    if dtype == "bf16":
        a, b = datagen.f32_to_bf16_bits(a), datagen.f32_to_bf16_bits(b)
    check(run(a, b, M, N, K, K, N, N + 3, variant=GEMV), oracle.mmrelu(a, b), K, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gemv_full_size(dtype):
    """8192 x 1 x 8192 (the sweep's matrix-vector shape), all outputs."""
    M = K = 8192
    print(f"gemv full size {dtype}", flush=True)
    a, b = vec_inputs(dtype, M, K, K, 1, 1541)
    check(run(a, b, M, 1, K, K, 1, 1), oracle.mmrelu(a, b, M=M, N=1, K=K, lda=K, ldb=1), K, dtype)
