"""The general-stride call without allocation, mmrelu_strided_static, against
mmrelu_strided_f32 / _bf16 with a caller workspace (needs the GPU; every
call goes through the C-ABI).

Both run the same copy and product kernels on the same plan, so their
outputs must agree bit for bit; both are also held to the oracle's
general-stride form at the fused-epilogue tolerances. Two calls in a row,
the second smaller, share the library's fixed array: the second must not
see the first's contents."""
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


def problem(dtype, M, N, K, seed):
    """A stored transposed (column-major), B transposed, C column-major with
    a bias: both operands are copied and C goes through a row-major
    temporary, so the call uses all three parts of the workspace."""
    a = datagen.normal_f32(seed, K, M, 1 / math.sqrt(K))         # A^T, row-major: A[i][k] = a[k*M + i]
    b = datagen.normal_f32(seed + 1, N, K, 1 / math.sqrt(K))     # B^T, row-major: B[k][j] = b[j*K + k]
    bias = datagen.normal_f32(seed + 2, 1, N, 0.5).ravel()
    if dtype == "bf16":
        a, b, bias = datagen.f32_to_bf16_bits(a), datagen.f32_to_bf16_bits(b), datagen.f32_to_bf16_bits(bias)
    strides = (1, M, 1, K, 1, M)            # sam, sak, sbk, sbn, scm, scn
    return a, b, bias, strides


def check(c, r, K, dtype):
    if dtype == "f32":
        err = np.abs(c.astype(np.float64) - r)
        assert np.all(err <= 1.13 * 1e-4 * math.sqrt(K) + 2e-6 * (1 + np.abs(r))), err.max()
    else:
        cf = datagen.bf16_bits_to_f32(c).astype(np.float64)
        assert np.linalg.norm(cf - r) / np.linalg.norm(r) <= 1e-2
        assert np.all(np.abs(cf - r) <= 2.0 ** -8 * np.abs(r) + 4e-6), np.abs(cf - r).max()


@pytest.mark.parametrize("act", ["relu", "gelu_tanh"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_static_workspace_matches_caller_workspace(dtype, act):
    kind = mm.DTYPE_F32 if dtype == "f32" else mm.DTYPE_BF16
    code = {"relu": mm.ACT_RELU, "gelu_tanh": mm.ACT_GELU_TANH}[act]
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    s = torch.cuda.current_stream().cuda_stream
    for M, N, K, seed in ((1000, 520, 264, 4100), (131, 72, 40, 4200)):
        print(f"no-alloc {dtype} {act} {M}x{N}x{K}", flush=True)
        a, b, bias, st = problem(dtype, M, N, K, seed)
        da, db, dbias = to_dev(a), to_dev(b), to_dev(bias)
        # C column-major (N rows of M), inside NaN-filled guard columns
        buf_ref = torch.full((N + 2, M), float("nan"), dtype=tdt, device="cuda")
        buf_st = torch.full((N + 2, M), float("nan"), dtype=tdt, device="cuda")
        c_ref = buf_ref.data_ptr() + M * buf_ref.element_size()
        c_st = buf_st.data_ptr() + M * buf_st.element_size()
        need = mm.mmrelu_strided_workspace_size(kind, code, da.data_ptr(), db.data_ptr(), dbias.data_ptr(), c_ref,
                                                M, N, K, *st)
        assert 0 < need <= mm.STATIC_WORKSPACE_BYTES
        ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
        wp = (ws.data_ptr() + 255) // 256 * 256
        fn = mm.mmrelu_strided_f32 if dtype == "f32" else mm.mmrelu_strided_bf16
        rc = fn(code, da.data_ptr(), db.data_ptr(), dbias.data_ptr(), c_ref, M, N, K, *st, wp, need, s)
        assert rc == mm.MMRELU_OK, mm.status_string(rc)
        rc = mm.mmrelu_strided_static(kind, code, da.data_ptr(), db.data_ptr(), dbias.data_ptr(), c_st,
                                      M, N, K, *st, s)
        assert rc == mm.MMRELU_OK, mm.status_string(rc)
        torch.cuda.synchronize()
        assert torch.equal(buf_st[1:N + 1], buf_ref[1:N + 1]), "static and caller workspaces differ"
        assert bool(torch.isnan(buf_st[0]).all()) and bool(torch.isnan(buf_st[N + 1]).all()), "wrote outside C"
        c = to_host(buf_st[1:N + 1]).T                       # C[i][j] = c_colmajor[j][i]
        r = oracle.strided(act, a, b, bias, M, N, K, *st[:4])
        check(np.ascontiguousarray(c), r, K, dtype)
        del ws


def test_static_workspace_rejects_past_the_limit():
    """A transposed 8192 x 8192 bf16 operand needs 128 MiB of workspace: the
    call returns MMRELU_ERR_WORKSPACE_LIMIT and enqueues nothing."""
    M = N = K = 8192
    a = torch.zeros((K, M), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((K, N), dtype=torch.bfloat16, device="cuda")
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    need = mm.mmrelu_strided_workspace_size(mm.DTYPE_BF16, mm.ACT_RELU, a.data_ptr(), b.data_ptr(), 0,
                                            c.data_ptr(), M, N, K, 1, M, N, 1, N, 1)
    assert need > mm.STATIC_WORKSPACE_BYTES
    rc = mm.mmrelu_strided_static(mm.DTYPE_BF16, mm.ACT_RELU, a.data_ptr(), b.data_ptr(), 0, c.data_ptr(),
                                  M, N, K, 1, M, N, 1, N, 1, torch.cuda.current_stream().cuda_stream)
    assert rc == mm.MMRELU_ERR_WORKSPACE_LIMIT
    torch.cuda.synchronize()
    assert bool(torch.isnan(c).all())
