"""Parity of the general-stride entry points with the fp64 oracle (needs the
GPU; every call goes through the C-ABI).

A and B are stored in a buffer and read through strides: row-major (with
padding), column-major (the transpose's storage) and sub-sampled views.
C is written through strides: row-major, column-major (the exchanged-operand
route, or a temporary when there is a bias) and padded. Buffers are filled
with NaN wherever nothing should be read or written, so a read outside the
strided elements shows up in the result and a stray write shows up in the
buffer. Tolerances are the row-major ones: fp32 max |C - R| <= L * 1e-4 *
sqrt(K) + 2e-6 (1 + |R|) (L = 1.13 for GeLU, else 1), bf16 elementwise
2^-8 |R| + 4e-6 with relative Frobenius <= 1e-2; integer inputs are exact.
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


def nan_of(dtype):
    return np.uint16(0x7FC0) if dtype == np.uint16 else np.float32(np.nan)


def store(logical: np.ndarray, layout: str):
    """A flat buffer holding `logical` (rows x cols) under `layout`, NaN
    elsewhere, and its (row stride, column stride)."""
    rows, cols = logical.shape
    if layout == "row":
        s_r, s_c, size = cols, 1, rows * cols
    elif layout == "row_pad":
        s_r, s_c, size = cols + 24, 1, rows * (cols + 24)
    elif layout == "col":
        s_r, s_c, size = 1, rows, rows * cols
    elif layout == "col_pad":
        s_r, s_c, size = 1, rows + 8, (rows + 8) * cols
    elif layout == "slice":                     # buf[::2, ::3] of a (2 rows) x (3 cols) buffer
        s_r, s_c, size = 6 * cols, 3, 6 * rows * cols
    else:
        raise ValueError(layout)
    buf = np.full(size, nan_of(logical.dtype), dtype=logical.dtype)
    idx = np.arange(rows)[:, None] * s_r + np.arange(cols)[None, :] * s_c
    buf[idx] = logical
    return buf, s_r, s_c


def out_layout(M, N, layout):
    if layout == "row":
        return N, 1, M * N
    if layout == "row_pad":
        return N + 16, 1, M * (N + 16)
    if layout == "col":
        return 1, M, M * N
    if layout == "col_pad":
        return 1, M + 8, (M + 8) * N
    raise ValueError(layout)


def run_strided(act, a_buf, sa, b_buf, sb, bias, M, N, K, c_layout):
    dt = torch.float32 if a_buf.dtype == np.float32 else torch.bfloat16
    kind = mm.DTYPE_F32 if dt == torch.float32 else mm.DTYPE_BF16
    scm, scn, size = out_layout(M, N, c_layout)
    guard = 64
    da, db = to_dev(a_buf), to_dev(b_buf)
    dbias = to_dev(bias) if bias is not None else None
    cbuf = torch.full((size + 2 * guard,), float("nan"), dtype=dt, device="cuda")
    cptr = cbuf.data_ptr() + guard * cbuf.element_size()
    bp = dbias.data_ptr() if dbias is not None else 0
    need = mm.mmrelu_strided_workspace_size(kind, ACTS[act], da.data_ptr(), db.data_ptr(), bp, cptr, M, N, K,
                                            sa[0], sa[1], sb[0], sb[1], scm, scn)
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    wp = (ws.data_ptr() + 255) // 256 * 256
    fn = mm.mmrelu_strided_f32 if kind == mm.DTYPE_F32 else mm.mmrelu_strided_bf16
    rc = fn(ACTS[act], da.data_ptr(), db.data_ptr(), bp, cptr, M, N, K, sa[0], sa[1], sb[0], sb[1], scm, scn,
            wp if need else 0, need, torch.cuda.current_stream().cuda_stream)
    assert rc == mm.MMRELU_OK, mm.status_string(rc)
    torch.cuda.synchronize()
    whole = to_host(cbuf)
    body = whole[guard:guard + size]
    idx = np.arange(M)[:, None] * scm + np.arange(N)[None, :] * scn
    c = body[idx]
    untouched = np.ones(whole.size, bool)
    untouched[guard + idx.ravel()] = False
    rest = whole[untouched]
    rest_f = datagen.bf16_bits_to_f32(rest) if rest.dtype == np.uint16 else rest
    assert np.all(np.isnan(rest_f)), "wrote outside the strided C"
    return c, need


def check(c, r, K, act, dtype):
    if dtype == np.float32:
        assert np.all(np.isfinite(c))
        slope = 1.13 if act == "gelu_tanh" else 1.0
        err = np.abs(c.astype(np.float64) - r)
        assert np.all(err <= slope * 1e-4 * math.sqrt(max(K, 1)) + 2e-6 * (1 + np.abs(r))), err.max()
    else:
        cf = datagen.bf16_bits_to_f32(c).astype(np.float64)
        assert np.all(np.isfinite(cf))
        nr = np.linalg.norm(r)
        assert (np.linalg.norm(cf - r) / nr if nr > 0 else np.linalg.norm(cf)) <= 1e-2
        assert np.all(np.abs(cf - r) <= 2.0 ** -8 * np.abs(r) + 4e-6), np.abs(cf - r).max()


def logical_inputs(dtype, M, N, K, seed):
    a = datagen.normal_f32(seed, M, K, 1 / math.sqrt(max(K, 1)))
    b = datagen.normal_f32(seed + 1, K, N, 1 / math.sqrt(max(K, 1)))
    bias = datagen.normal_f32(seed + 2, 1, N, 0.5).ravel()
    if dtype == "bf16":
        return datagen.f32_to_bf16_bits(a), datagen.f32_to_bf16_bits(b), datagen.f32_to_bf16_bits(bias)
    return a, b, bias


IN_LAYOUTS = ["row", "row_pad", "col", "slice"]
OUT_LAYOUTS = ["row", "row_pad", "col", "col_pad"]
SHAPES = [(264, 136, 72), (257, 131, 67), (40, 520, 264)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("a_layout", IN_LAYOUTS)
@pytest.mark.parametrize("b_layout", IN_LAYOUTS)
def test_strided_layouts(dtype, a_layout, b_layout):
    for si, (M, N, K) in enumerate(SHAPES):
        a, b, bias = logical_inputs(dtype, M, N, K, 1200 + si)
        a_buf, sam, sak = store(a, a_layout)
        b_buf, sbk, sbn = store(b, b_layout)
        for c_layout in OUT_LAYOUTS:
            for with_bias in (False, True):
                bv = bias if with_bias else None
                act = "gelu_tanh" if with_bias else "relu"
                r = oracle.strided(act, a_buf, b_buf, bv, M, N, K, sam, sak, sbk, sbn)
                print(f"{dtype} {M}x{N}x{K} A={a_layout} B={b_layout} C={c_layout} bias={with_bias}", flush=True)
                c, _ = run_strided(act, a_buf, (sam, sak), b_buf, (sbk, sbn), bv, M, N, K, c_layout)
                check(c, r, K, act, a_buf.dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_strided_exact_integers(dtype):
    """Integer inputs: every layout gives the exact (fp32) or correctly
    rounded (bf16) result, with and without the exchanged-operand route."""
    M, N, K = 136, 264, 96
    a, b = datagen.small_int_f32(1301, M, K), datagen.small_int_f32(1302, K, N)
    if dtype == "bf16":
        a, b = datagen.f32_to_bf16_bits(a), datagen.f32_to_bf16_bits(b)
    for a_layout, b_layout, c_layout in [("col", "col", "col"), ("row", "row", "col"), ("col", "row", "row"),
                                         ("slice", "col", "col_pad")]:
        a_buf, sam, sak = store(a, a_layout)
        b_buf, sbk, sbn = store(b, b_layout)
        r = oracle.strided("none", a_buf, b_buf, None, M, N, K, sam, sak, sbk, sbn)
        c, _ = run_strided("none", a_buf, (sam, sak), b_buf, (sbk, sbn), None, M, N, K, c_layout)
        if dtype == "f32":
            assert np.array_equal(c.astype(np.float64), r), (a_layout, b_layout, c_layout)
        else:
            ref = torch.from_numpy(r.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(c, ref), (a_layout, b_layout, c_layout)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_strided_zero_copy_routes_need_no_workspace(dtype):
    """Row-major in place, and A^T B^T into a column-major C through the
    exchanged operands, both with a zero workspace."""
    M, N, K = 264, 136, 72
    a, b, _ = logical_inputs(dtype, M, N, K, 1311)
    for a_layout, b_layout, c_layout in [("row", "row", "row"), ("col", "col", "col")]:
        a_buf, sam, sak = store(a, a_layout)
        b_buf, sbk, sbn = store(b, b_layout)
        r = oracle.strided("relu", a_buf, b_buf, None, M, N, K, sam, sak, sbk, sbn)
        c, need = run_strided("relu", a_buf, (sam, sak), b_buf, (sbk, sbn), None, M, N, K, c_layout)
        assert need == 0
        check(c, r, K, "relu", a_buf.dtype)


def test_strided_zero_strides_broadcast():
    """A zero stride repeats an element: A's rows all equal row 0 of the
    buffer, B's columns all equal column 0."""
    M, N, K = 96, 40, 64
    a_row = datagen.normal_f32(1321, 1, K, 0.2).ravel()
    b_col = datagen.normal_f32(1322, K, 1, 0.2).ravel()
    r = oracle.strided("none", a_row, b_col, None, M, N, K, 0, 1, 1, 0)
    c, _ = run_strided("none", a_row, (0, 1), b_col, (1, 0), None, M, N, K, "row")
    check(c, r, K, "none", np.float32)
    assert np.allclose(r, r[0:1, 0:1])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_strided_k0_and_edges(dtype):
    """K = 0 gives act(bias) in every output layout; one-row and one-column
    products with transposed operands."""
    for (M, N, K) in [(37, 24, 0), (1, 264, 136), (264, 1, 136), (1, 1, 9)]:
        a, b, bias = logical_inputs(dtype, M, N, max(K, 1), 1331)
        a, b = a[:, :K], b[:K, :]
        a_buf, sam, sak = store(np.ascontiguousarray(a), "col")
        b_buf, sbk, sbn = store(np.ascontiguousarray(b), "col")
        if K == 0:                              # nothing is read: one-element buffers
            a_buf, b_buf = np.zeros(1, a.dtype), np.zeros(1, b.dtype)
            sam = sak = sbk = sbn = 0
        for c_layout in ("row", "col"):
            r = oracle.strided("gelu_tanh", a_buf, b_buf, bias, M, N, K, sam, sak, sbk, sbn)
            c, _ = run_strided("gelu_tanh", a_buf, (sam, sak), b_buf, (sbk, sbn), bias, M, N, K, c_layout)
            check(c, r, max(K, 1), "gelu_tanh", a_buf.dtype)


def test_torch_wrapper_transposed_views():
    M, N, K = 200, 136, 96
    a, b, bias = logical_inputs("f32", M, N, K, 1341)
    da = to_dev(np.ascontiguousarray(a.T)).t()          # (M, K) view of a K x M buffer
    db = to_dev(np.ascontiguousarray(b.T)).t()
    out = torch.empty((N, M), dtype=torch.float32, device="cuda").t()    # column-major (M, N)
    res = mm.mmrelu(da, db, out=out, bias=to_dev(bias), act="gelu_tanh")
    torch.cuda.synchronize()
    assert res.data_ptr() == out.data_ptr()
    r = oracle.fused("gelu_tanh", a, b, bias)
    c = res.cpu().numpy()
    assert np.all(np.abs(c - r) <= 1.13e-4 * math.sqrt(K) + 2e-6 * (1 + np.abs(r)))
    sliced = to_dev(datagen.normal_f32(1344, 2 * M, 3 * K, 0.1))[::2, ::3]
    r2 = oracle.mmrelu(np.ascontiguousarray(sliced.cpu().numpy()), b)
    c2 = mm.mmrelu(sliced, to_dev(b))
    torch.cuda.synchronize()
    assert np.all(np.abs(c2.cpu().numpy() - r2) <= 1e-4 * math.sqrt(K))


@pytest.mark.parametrize("layout", ["TN", "NT"])
def test_strided_full_size_bf16(layout):
    """The 8192^3 bf16 workload with A or B stored transposed, through the
    copy and the planner's kernel, on sampled rows, columns and entries."""
    cfg = datagen.CONFIGS[5]
    a, b = datagen.make_inputs(cfg)
    M, N, K = cfg.M, cfg.N, cfg.K
    print(f"strided full size bf16 {layout}", flush=True)
    if layout == "TN":
        a_buf, sa = np.ascontiguousarray(a.T).ravel(), (1, M)
        b_buf, sb = b.ravel(), (N, 1)
    else:
        a_buf, sa = a.ravel(), (K, 1)
        b_buf, sb = np.ascontiguousarray(b.T).ravel(), (1, K)
    da, db = to_dev(a_buf), to_dev(b_buf)
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    need = mm.mmrelu_strided_workspace_size(mm.DTYPE_BF16, mm.ACT_RELU, da.data_ptr(), db.data_ptr(), 0,
                                            c.data_ptr(), M, N, K, *sa, *sb, N, 1)
    assert need == M * K * 2
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    rc = mm.mmrelu_strided_bf16(mm.ACT_RELU, da.data_ptr(), db.data_ptr(), 0, c.data_ptr(), M, N, K, *sa, *sb,
                                N, 1, ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
    assert rc == mm.MMRELU_OK
    torch.cuda.synchronize()
    ch = to_host(c)
    rng = np.random.default_rng(1351)
    rsel = np.array([0, M - 1, int(rng.integers(0, M))])
    ii = np.concatenate([np.repeat(rsel, N), rng.integers(0, M, 3000)])
    jj = np.concatenate([np.tile(np.arange(N), rsel.size), rng.integers(0, N, 3000)])
    r = oracle.strided_at("relu", a_buf, b_buf, None, ii, jj, M, N, K, *sa, *sb)
    cf = datagen.bf16_bits_to_f32(ch[ii, jj]).astype(np.float64)
    assert np.all(np.abs(cf - r) <= 2.0 ** -8 * np.abs(r) + 1e-6)
    assert np.linalg.norm(cf - r) / np.linalg.norm(r) <= 1e-2
