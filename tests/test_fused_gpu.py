"""Parity of the fused epilogues, act(A·B + bias), with the fp64 oracle
(needs the GPU; every call goes through the C-ABI).

Tolerances follow the ReLU path's, widened for the activation:
  * fp32: |C - R| <= L * 1e-4 * sqrt(K) + 2e-6 * (1 + |R|), with L = 1 for
    ReLU and none and L = 1.13 for GeLU (the largest slope of its tanh form
    is 1.129, at x = 1.42); the second term covers the fp32 bias add and the
    device tanhf (a few ulp of a value below 1, scaled by |x|/2);
  * bf16: ||C - R||_F / ||R||_F <= 1e-2, and elementwise |C - R| <= 2^-8 |R|
    + 4e-6 (one bf16 rounding, plus the fp32 terms above at these sizes);
  * exact: small-integer inputs and bias with ReLU or no activation make every
    partial sum an exact integer, so fp32 is bit-exact and bf16 is the
    round-to-nearest-even of the oracle.
"""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
import tiled_matmul_relu_amd as mm

pytestmark = pytest.mark.gpu

ACTS = {"relu": mm.ACT_RELU, "gelu_tanh": mm.ACT_GELU_TANH, "none": mm.ACT_NONE}


def to_dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def run_fused(act, a, b, bias, M, N, K, lda, ldb, ldc=None, variant=None, guard=0):
    """Launch through the fused C entry point into a NaN-filled buffer with
    `guard` rows above and below and ldc - N padding columns."""
    dt = torch.float32 if a.dtype == np.float32 else torch.bfloat16
    ldc = ldc or N
    da, db = to_dev(a), to_dev(b)
    dbias = to_dev(bias) if bias is not None else None
    buf = torch.full((M + 2 * guard, ldc), float("nan"), dtype=dt, device="cuda")
    c_ptr = buf.data_ptr() + guard * ldc * buf.element_size()
    bp = dbias.data_ptr() if dbias is not None else 0
    args = (ACTS[act], da.data_ptr(), db.data_ptr(), bp, c_ptr, M, N, K, lda, ldb, ldc,
            torch.cuda.current_stream().cuda_stream)
    if dt == torch.float32:
        rc = mm.mmrelu_fused_f32(*args) if variant is None else mm.mmrelu_fused_f32_variant(variant, *args)
    else:
        rc = mm.mmrelu_fused_bf16(*args) if variant is None else mm.mmrelu_fused_bf16_variant(variant, *args)
    assert rc == mm.MMRELU_OK, mm.status_string(rc)
    torch.cuda.synchronize()
    whole = to_host(buf)
    return whole[guard:guard + M, :N], whole


def check_f32(c, r, K, act):
    assert np.all(np.isfinite(c))
    slope = 1.13 if act == "gelu_tanh" else 1.0
    tol = slope * 1e-4 * math.sqrt(max(K, 1)) + 2e-6 * (1 + np.abs(r))
    err = np.abs(c.astype(np.float64) - r)
    assert np.all(err <= tol), f"max err {err.max()}"
    if act == "relu":
        assert np.all(c >= 0)


def check_bf16(c_bits, r, act):
    c = datagen.bf16_bits_to_f32(c_bits).astype(np.float64)
    assert np.all(np.isfinite(c))
    nr = np.linalg.norm(r)
    rel = np.linalg.norm(c - r) / nr if nr > 0 else np.linalg.norm(c)
    assert rel <= 1e-2, f"relative Frobenius error {rel}"
    assert np.all(np.abs(c - r) <= 2.0 ** -8 * np.abs(r) + 4e-6), np.abs(c - r).max()
    if act == "relu":
        assert np.all(c >= 0)


def variants(dtype):
    return list(range(mm.mmrelu_num_variants(dtype)))


def accepts(dtype, v, N, K, lda, ldb, ldc, M=1):
    plan = mm.mmrelu_plan_variant(dtype, v, 8, 8, 8, 8, 8, 8)
    name = plan["name"]
    if "simple" in name or "unaligned" in name or "gemv" in name or "_any<" in name or "_realign<" in name:
        return True
    q = 4 if dtype == mm.DTYPE_F32 else 8
    return all(x % q == 0 for x in (N, K, lda, ldb, ldc))


def inputs(dtype, M, N, K, seed, scale=None):
    s = scale if scale is not None else 1 / math.sqrt(K)
    a = datagen.normal_f32(seed, M, K, s)
    b = datagen.normal_f32(seed + 1, K, N, s)
    bias = datagen.normal_f32(seed + 2, 1, N, 0.5).ravel()
    if dtype == "bf16":
        return datagen.f32_to_bf16_bits(a), datagen.f32_to_bf16_bits(b), datagen.f32_to_bf16_bits(bias)
    return a, b, bias


SHAPES = {"f32": [(257, 131, 67), (264, 520, 136), (70, 64, 200)],
          # K = 104: the last 64-deep pair of the ping-pong kernel is partly past K
          "bf16": [(264, 520, 136), (300, 264, 72), (257, 131, 67), (136, 264, 104)]}


@pytest.mark.parametrize("act", sorted(ACTS))
@pytest.mark.parametrize("with_bias", [False, True], ids=["nobias", "bias"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_every_variant(dtype, with_bias, act):
    kind = mm.DTYPE_F32 if dtype == "f32" else mm.DTYPE_BF16
    for si, (M, N, K) in enumerate(SHAPES[dtype]):
        a, b, bias = inputs(dtype, M, N, K, 500 + 10 * si)
        bias = bias if with_bias else None
        r = oracle.fused(act, a, b, bias)
        for v in variants(kind):
            if not accepts(kind, v, N, K, K, N, N, M=M):
                continue
            print(f"{dtype} {act} bias={with_bias} shape={M}x{N}x{K} variant={v}", flush=True)
            c, _ = run_fused(act, a, b, bias, M, N, K, K, N, variant=v)
            (check_f32(c, r, K, act) if dtype == "f32" else check_bf16(c, r, act))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_exact_integers(dtype):
    """Integer inputs and bias: ReLU and identity outputs are exact."""
    kind = mm.DTYPE_F32 if dtype == "f32" else mm.DTYPE_BF16
    M, N, K = 136, 264, 96
    a, b = datagen.small_int_f32(611, M, K), datagen.small_int_f32(612, K, N)
    bias = datagen.small_int_f32(613, 1, N).ravel() * 8
    if dtype == "bf16":
        a, b, bias = (datagen.f32_to_bf16_bits(x) for x in (a, b, bias))
    for act in ("relu", "none"):
        r = oracle.fused(act, a, b, bias)
        for v in variants(kind):
            if not accepts(kind, v, N, K, K, N, N, M=M):
                continue
            c, _ = run_fused(act, a, b, bias, M, N, K, K, N, variant=v)
            if dtype == "f32":
                assert np.array_equal(c.astype(np.float64), r), (act, v)
            else:
                ref = torch.from_numpy(r.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
                assert np.array_equal(c, ref.view(np.uint16)), (act, v)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_guard_band(dtype):
    """Nothing outside the M x N window is written, whatever the epilogue."""
    M, N, K = 131, 264, 72
    a, b, bias = inputs(dtype, M, N, K, 700)
    ldc = N + 24
    kind = mm.DTYPE_F32 if dtype == "f32" else mm.DTYPE_BF16
    for v in variants(kind):
        if not accepts(kind, v, N, K, K, N, ldc, M=M):
            continue
        c, whole = run_fused("gelu_tanh", a, b, bias, M, N, K, K, N, ldc=ldc, variant=v, guard=3)
        wf = whole.astype(np.float32) if dtype == "f32" else datagen.bf16_bits_to_f32(whole)
        outside = np.ones(wf.shape, bool)
        outside[3:3 + M, :N] = False
        assert np.all(np.isnan(wf[outside])), f"variant {v} wrote outside the window"
        assert np.all(np.isfinite(wf[~outside]))


def test_fused_full_size_bf16_gelu_bias():
    """The 8192^3 bf16 workload with GeLU and a bias through the planner's
    kernel, on sampled rows, columns and entries."""
    cfg = datagen.CONFIGS[5]
    a, b = datagen.make_inputs(cfg)
    bias = datagen.f32_to_bf16_bits(datagen.normal_f32(801, 1, cfg.N, 0.5).ravel())
    c, _ = run_fused("gelu_tanh", a, b, bias, cfg.M, cfg.N, cfg.K, cfg.lda, cfg.ldb, ldc=cfg.ldc)
    rng = np.random.default_rng(802)
    rsel = np.array([0, cfg.M - 1, int(rng.integers(0, cfg.M))])
    ii = np.concatenate([np.repeat(rsel, cfg.N), rng.integers(0, cfg.M, 3000)])
    jj = np.concatenate([np.tile(np.arange(cfg.N), rsel.size), rng.integers(0, cfg.N, 3000)])
    r = oracle.fused_at("gelu_tanh", a, b, bias, ii, jj, cfg.K, cfg.lda, cfg.ldb)
    check_bf16(c[ii, jj], r, "gelu_tanh")
    cf = datagen.bf16_bits_to_f32(c)
    assert np.all(np.isfinite(cf)) and cf.min() >= -0.18   # GeLU's minimum is -0.170


def test_torch_wrapper_bias_and_gelu():
    M, N, K = 200, 136, 96
    a, b, bias = inputs("f32", M, N, K, 900)
    out = mm.mmrelu(to_dev(a), to_dev(b), bias=to_dev(bias), act="gelu_tanh")
    torch.cuda.synchronize()
    check_f32(out.cpu().numpy(), oracle.fused("gelu_tanh", a, b, bias), K, "gelu_tanh")
    with pytest.raises(ValueError):
        mm.mmrelu(to_dev(a), to_dev(b), act="tanh")
    with pytest.raises(ValueError):
        mm.mmrelu(to_dev(a), to_dev(b), bias=to_dev(bias[:-1]))
