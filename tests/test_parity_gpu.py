"""Parity of the gfx950 library with the fp64 oracle (needs the GPU).

Every test generates seeded inputs on the host (``datagen``), runs the HIP
path through the C-ABI, and compares with the oracle on the same inputs:
  * fp32: max |C - R| <= 1e-4 * sqrt(K), and bit-exact on small-integer
    inputs (every partial sum is an integer below 2^24, so any summation
    order is exact).
  * bf16: ||C - R||_F / ||R||_F <= 1e-2, plus an element-wise bound
    |C - R| <= 2^-8 |R| + 1e-6 (one bf16 rounding is at most 2^-9 relative;
    the fp32 accumulation error is orders of magnitude below 1e-6 at these
    magnitudes), and exact equality with round-to-nearest-even of the oracle
    on small-integer inputs.
Small shapes span several tiles with ragged tails and are compared element
by element. The five full-size workloads run in the configuration the
benchmark times and every element of C is compared with the oracle, which
is evaluated one block of rows at a time; their shapes and leading
dimensions are also run on small-integer inputs, compared bit for bit. The
planner's tile kernels run multi-band ragged grids (the per-XCD regroup and
several bands of tile rows) element by element, and repeat bit for bit.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
import tiled_matmul_relu_amd as mm

pytestmark = pytest.mark.gpu

F32_TOL = lambda K: 1e-4 * math.sqrt(max(K, 1))


def to_dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_round_ref(r: np.ndarray) -> np.ndarray:
    """RNE of fp64 values to bf16 via torch on the CPU (values exactly
    representable in fp32 here, so fp64 -> fp32 is exact)."""
    return torch.from_numpy(r.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def run(a: np.ndarray, b: np.ndarray, M, N, K, lda, ldb, ldc=None, variant=None, guard=0):
    """Launch on device copies of a/b; C gets `guard` extra rows before and
    after and ldc - N padding columns, all pre-filled with a NaN sentinel.
    Returns (C window, whole C buffer, window row offset)."""
    dt = torch.float32 if a.dtype == np.float32 else torch.bfloat16
    ldc = ldc or N
    da, db = to_dev(a), to_dev(b)
    rows = M + 2 * guard
    buf = torch.full((max(rows, 1), max(ldc, 1)), float("nan"), dtype=dt, device="cuda")
    c_ptr = buf.data_ptr() + guard * ldc * buf.element_size()
    args = (da.data_ptr(), db.data_ptr(), c_ptr, M, N, K, lda, ldb, ldc, torch.cuda.current_stream().cuda_stream)
    if dt == torch.float32:
        rc = mm.mmrelu_f32(*args) if variant is None else mm.mmrelu_f32_variant(variant, *args)
    else:
        rc = mm.mmrelu_bf16(*args) if variant is None else mm.mmrelu_bf16_variant(variant, *args)
    assert rc == mm.MMRELU_OK, mm.status_string(rc)
    torch.cuda.synchronize()
    whole = to_host(buf)
    win = whole[guard:guard + M, :N] if M > 0 else whole[:0, :N]
    return win, whole


def check_f32(c, r, K):
    assert np.all(np.isfinite(c))
    err = np.abs(c.astype(np.float64) - r)
    assert err.max(initial=0) <= F32_TOL(K), f"max err {err.max()} > {F32_TOL(K)}"
    assert np.all(c >= 0)


def check_bf16(c_bits, r):
    c = datagen.bf16_bits_to_f32(c_bits).astype(np.float64)
    assert np.all(np.isfinite(c)) and np.all(c >= 0)
    nr = np.linalg.norm(r)
    rel = np.linalg.norm(c - r) / nr if nr > 0 else np.linalg.norm(c)
    assert rel <= 1e-2, f"relative Frobenius error {rel}"
    assert np.all(np.abs(c - r) <= 2.0 ** -8 * np.abs(r) + 1e-6)


def variants(dtype):
    return list(range(mm.mmrelu_num_variants(dtype)))


def accepts(dtype, v, N, K, lda, ldb, ldc, M=1):
    plan = mm.mmrelu_plan_variant(dtype, v, 8, 8, 8, 8, 8, 8)
    name = plan["name"]
    if "simple" in name or "unaligned" in name or "gemv" in name or "_any<" in name or "_realign<" in name:
        return True
    q = 4 if dtype == mm.DTYPE_F32 else 8
    return all(x % q == 0 for x in (N, K, lda, ldb, ldc))


F32_SHAPES = [  # (M, N, K) spanning several tiles with ragged tails, plus degenerate ones
    (1, 1, 1), (3, 5, 7), (17, 33, 65), (129, 131, 67), (257, 260, 132), (300, 264, 516),
    (64, 64, 64), (128, 256, 96), (260, 4, 12), (4, 260, 8), (513, 129, 33),
]
BF16_SHAPES = [
    (8, 8, 8), (1, 8, 8), (264, 520, 136), (256, 256, 64), (300, 264, 72), (520, 8, 200),
    (16, 512, 1032), (3, 5, 7), (257, 131, 67),
    # K mod 64 = 24 and 40: the last 64-deep pair of slabs is partly past K
    (136, 512, 88), (264, 256, 104), (256, 512, 1000),
]


@pytest.mark.parametrize("shape", F32_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("variant", variants(mm.DTYPE_F32))
def test_f32_variants_small(variant, shape):
    M, N, K = shape
    if not accepts(mm.DTYPE_F32, variant, N, K, K, N, N, M=M):
        pytest.skip("variant needs 16-byte rows")
    a = datagen.normal_f32(10 + M, M, K, 1 / math.sqrt(K))
    b = datagen.normal_f32(20 + N, K, N, 1 / math.sqrt(K))
    c, _ = run(a, b, M, N, K, K, N, variant=variant)
    check_f32(c, oracle.mmrelu(a, b), K)


@pytest.mark.parametrize("shape", BF16_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("variant", variants(mm.DTYPE_BF16))
def test_bf16_variants_small(variant, shape):
    M, N, K = shape
    if not accepts(mm.DTYPE_BF16, variant, N, K, K, N, N, M=M):
        pytest.skip("variant needs 16-byte rows")
    a = datagen.f32_to_bf16_bits(datagen.normal_f32(30 + M, M, K, 1 / math.sqrt(K)))
    b = datagen.f32_to_bf16_bits(datagen.normal_f32(40 + N, K, N, 1 / math.sqrt(K)))
    c, _ = run(a, b, M, N, K, K, N, variant=variant)
    check_bf16(c, oracle.mmrelu(a, b))


@pytest.mark.parametrize("variant", variants(mm.DTYPE_F32))
def test_f32_exact_integers_bit_exact(variant):
    M, N, K = 200, 132, 300
    if not accepts(mm.DTYPE_F32, variant, N, K, K, N, N, M=M):
        pytest.skip("variant needs 16-byte rows")
    a = datagen.small_int_f32(51, M, K)
    b = datagen.small_int_f32(52, K, N)
    c, _ = run(a, b, M, N, K, K, N, variant=variant)
    np.testing.assert_array_equal(c.astype(np.float64), oracle.mmrelu(a, b))


@pytest.mark.parametrize("variant", variants(mm.DTYPE_BF16))
def test_bf16_exact_integers_round_to_nearest_even(variant):
    """Integer inputs: fp32 accumulation is exact, so C must equal the oracle
    rounded to bf16 (nearest, ties to even) bit for bit: pins the epilogue
    rounding mode."""
    M, N, K = 136, 264, 520
    if not accepts(mm.DTYPE_BF16, variant, N, K, K, N, N, M=M):
        pytest.skip("variant needs 16-byte rows")
    a = datagen.f32_to_bf16_bits(datagen.small_int_f32(61, M, K))
    b = datagen.f32_to_bf16_bits(datagen.small_int_f32(62, K, N))
    r = oracle.mmrelu(a, b)
    assert np.abs(r).max() > 256          # results need more than bf16's 8 bits
    c, _ = run(a, b, M, N, K, K, N, variant=variant)
    np.testing.assert_array_equal(c, bf16_round_ref(r))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_guard_band_and_padded_leading_dimensions(dtype):
    """Masked store: nothing outside the M x N window is written, with padded
    lda/ldb/ldc (multiples of 8 so every variant applies) and rows around C."""
    M, N, K = 131, 264, 72
    lda, ldb, ldc = K + 8, N + 16, N + 24
    a32 = datagen.pad_rows(datagen.normal_f32(71, M, K, 1 / math.sqrt(K)), lda, fill=np.nan)
    b32 = datagen.pad_rows(datagen.normal_f32(72, K, N, 1 / math.sqrt(K)), ldb, fill=np.nan)
    if dtype == "bf16":
        a, b = datagen.f32_to_bf16_bits(a32), datagen.f32_to_bf16_bits(b32)
        dt = mm.DTYPE_BF16
    else:
        a, b, dt = a32, b32, mm.DTYPE_F32
    r = oracle.mmrelu(a, b, M=M, N=N, K=K, lda=lda, ldb=ldb)
    for v in variants(dt):
        if not accepts(dt, v, N, K, lda, ldb, ldc, M=M):
            continue
        c, whole = run(a, b, M, N, K, lda, ldb, ldc=ldc, variant=v, guard=3)
        if dtype == "bf16":
            check_bf16(c, r)
            wf = datagen.bf16_bits_to_f32(whole)
        else:
            check_f32(c, r, K)
            wf = whole
        outside = np.ones(wf.shape, bool)
        outside[3:3 + M, :N] = False
        assert np.all(np.isnan(wf[outside])), f"variant {v} wrote outside the window"


def placed(x: np.ndarray, off: int, ld: int):
    """A device buffer holding the compact matrix x with leading dimension ld,
    starting `off` elements past a 16-byte boundary; NaN everywhere else (a
    read outside x would poison the product). Returns (buffer, address)."""
    rows, cols = x.shape
    dt = torch.float32 if x.dtype == np.float32 else torch.bfloat16
    flat = torch.full((off + rows * ld + 16,), float("nan"), dtype=dt, device="cuda")
    flat[off:off + rows * ld].view(rows, ld)[:, :cols] = to_dev(x)
    return flat, flat.data_ptr() + off * flat.element_size()


# (dtype, element offsets of A, B, C, variants). Only element alignment is
# required of pointers; these start A, B and C 1..7 elements past a 16-byte
# boundary, through the planner (None) and the kernels that accept such
# layouts: bf16 2/13/15-18 (any layout) and 0 (plain); fp32 2/4 (unaligned tiles),
# 11 (matrix-vector) and 0.
MISALIGNED = [("bf16", (1, 3, 5), [None, 2, 13, 15, 16, 17, 18, 0]), ("bf16", (7, 2, 0), [None, 2, 13, 15, 18]),
              ("bf16", (0, 0, 3), [None, 13, 15]), ("f32", (1, 2, 3), [None, 2, 4, 0]), ("f32", (3, 0, 1), [None, 2, 4])]


@pytest.mark.parametrize("dtype,offs,vs", MISALIGNED, ids=[f"{m[0]}-{m[1]}" for m in MISALIGNED])
@pytest.mark.parametrize("M,N,K", [(300, 264, 136), (131, 97, 77)], ids=["even", "odd"])
def test_element_aligned_pointers(dtype, offs, vs, M, N, K):
    a = datagen.normal_f32(1700 + M, M, K, 1 / math.sqrt(K))
    b = datagen.normal_f32(1800 + N, K, N, 1 / math.sqrt(K))
    if dtype == "bf16":
        a, b = datagen.f32_to_bf16_bits(a), datagen.f32_to_bf16_bits(b)
    r = oracle.mmrelu(a, b)
    lda, ldb, ldc = K + 5, N + 3, N + 1
    fa, pa = placed(a, offs[0], lda)
    fb, pb = placed(b, offs[1], ldb)
    for v in vs:
        print(f"misaligned {dtype} offs={offs} {M}x{N}x{K} variant={v}", flush=True)
        fc, pc = placed(np.zeros((M, 0), a.dtype), offs[2], ldc)   # all NaN
        args = (pa, pb, pc, M, N, K, lda, ldb, ldc, torch.cuda.current_stream().cuda_stream)
        if dtype == "f32":
            rc = mm.mmrelu_f32(*args) if v is None else mm.mmrelu_f32_variant(v, *args)
        else:
            rc = mm.mmrelu_bf16(*args) if v is None else mm.mmrelu_bf16_variant(v, *args)
        assert rc == mm.MMRELU_OK, mm.status_string(rc)
        torch.cuda.synchronize()
        whole = to_host(fc)
        c = whole[offs[2]:offs[2] + M * ldc].reshape(M, ldc)
        if dtype == "f32":
            check_f32(c[:, :N], r, K)
            pad = c[:, N:].astype(np.float64)
        else:
            check_bf16(c[:, :N], r)
            pad = datagen.bf16_bits_to_f32(c[:, N:]).astype(np.float64)
        outside = np.concatenate([whole[:offs[2]], whole[offs[2] + M * ldc:]])
        outside = outside.astype(np.float64) if dtype == "f32" else datagen.bf16_bits_to_f32(outside)
        assert np.all(np.isnan(pad)) and np.all(np.isnan(outside)), f"variant {v} wrote outside C"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_k_zero_writes_zeros(dtype):
    M, N = 70, 136
    a = np.zeros((M, 1), np.float32 if dtype == "f32" else np.uint16)
    b = np.zeros((1, N), a.dtype)
    c, _ = run(a, b, M, N, 0, 1, N)
    assert np.all(c == 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_k_zero_every_variant_writes_zeros(dtype):
    """K = 0: the loop over K runs zero times and every kernel stores
    relu(0) = 0 over a C filled with NaN beforehand (the empty sum)."""
    M, N = 264, 520
    kind = mm.DTYPE_F32 if dtype == "f32" else mm.DTYPE_BF16
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    # A is M x 1 and B 1 x N (lda = 1, ldb = N), as the operands of a K = 1
    # product: any range a kernel derives from M, N and the leading
    # dimensions stays inside them.
    a = torch.zeros((M, 1), dtype=tdt, device="cuda")
    b = torch.zeros((1, N), dtype=tdt, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    for v in variants(kind):
        c = torch.full((M, N), float("nan"), dtype=tdt, device="cuda")
        fn = mm.mmrelu_f32_variant if dtype == "f32" else mm.mmrelu_bf16_variant
        print(f"k=0 {dtype} variant={v}", flush=True)
        rc = fn(v, a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, 0, 1, N, N, s)
        assert rc == mm.MMRELU_OK, (v, mm.status_string(rc))
        torch.cuda.synchronize()
        assert bool((c == 0).all()), f"variant {v}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_inputs_give_zero_outputs(dtype):
    """All-zero A and B (the inputs of bench.py's power check): every variant
    writes +0 or -0 everywhere, over several tiles and a ragged tail."""
    M, N, K = 520, 264, 200
    kind = mm.DTYPE_F32 if dtype == "f32" else mm.DTYPE_BF16
    a = np.zeros((M, K), np.float32 if dtype == "f32" else np.uint16)
    b = np.zeros((K, N), a.dtype)
    for v in variants(kind):
        if not accepts(kind, v, N, K, K, N, N, M=M):
            continue
        c, _ = run(a, b, M, N, K, K, N, variant=v)
        vals = c if dtype == "f32" else datagen.bf16_bits_to_f32(c)
        assert np.all(vals == 0), f"variant {v}"


def test_empty_outputs_launch_nothing():
    t = torch.zeros(4, 4, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert mm.mmrelu_f32(t.data_ptr(), t.data_ptr(), t.data_ptr(), 0, 4, 4, 4, 4, 4, s) == 0
    assert mm.mmrelu_f32(t.data_ptr(), t.data_ptr(), t.data_ptr(), 4, 0, 4, 4, 4, 4, s) == 0
    torch.cuda.synchronize()
    assert torch.all(t == 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_deterministic_repeats(dtype):
    """No atomics: 20 runs must agree bit for bit (a proxy for LDS races);
    this shape runs a skinny kernel, whose eight waves sum their partial
    tiles through LDS."""
    M, N, K = 512, 512, 1024
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    a = to_dev(datagen.normal_f32(81, M, K, 1 / math.sqrt(K))).to(tdt)
    b = to_dev(datagen.normal_f32(82, K, N, 1 / math.sqrt(K))).to(tdt)
    first = mm.mmrelu(a, b).clone()
    for _ in range(19):
        assert torch.equal(mm.mmrelu(a, b), first)


# (dtype, variant, shape): the tile kernels on grids of several waves. bf16 1
# and 3 are the ping-pong tiles (an LDS ring per operand, the two wave
# groups swapping roles at every barrier), 4 the 128 x 128 tile, 15 and 18
# the any-layout 256 x 256 and 160 x 256 tiles; fp32 1 the aligned 128 x 128
# tile, 4 the unaligned 64 x 64 tile.
DETERMINISM = [("bf16", 1, (4352, 4352, 520)), ("bf16", 3, (4352, 4352, 520)), ("bf16", 4, (4352, 4352, 520)),
               ("bf16", 15, (4352, 4352, 520)), ("bf16", 18, (4352, 4352, 520)),
               ("f32", 1, (4352, 4352, 264)), ("f32", 4, (4352, 4352, 264))]


@pytest.mark.parametrize("dtype,variant,shape", DETERMINISM, ids=[f"{d}-v{v}" for d, v, _ in DETERMINISM])
def test_tile_kernels_deterministic_repeats(dtype, variant, shape):
    M, N, K = shape
    kind = mm.DTYPE_F32 if dtype == "f32" else mm.DTYPE_BF16
    plan = mm.mmrelu_plan_variant(kind, variant, M, N, K, K, N, N)
    assert plan["waves"] >= 2, plan                 # more tiles than one round of the CUs holds
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    a = to_dev(datagen.normal_f32(83, M, K, 1 / math.sqrt(K))).to(tdt)
    b = to_dev(datagen.normal_f32(84, K, N, 1 / math.sqrt(K))).to(tdt)
    print(f"determinism {dtype} variant={variant} {M}x{N}x{K}", flush=True)
    first = mm.mmrelu(a, b, variant=variant).clone()
    for _ in range(19):
        assert torch.equal(mm.mmrelu(a, b, variant=variant), first)


def test_torch_wrapper_row_strided_out():
    M, N, K = 96, 136, 40
    a = datagen.normal_f32(91, M, K)
    b = datagen.normal_f32(92, K, N)
    big = torch.full((M, N + 8), -1.0, device="cuda")
    out = big[:, :N]
    mm.mmrelu(to_dev(a), to_dev(b), out=out)
    torch.cuda.synchronize()
    check_f32(out.cpu().numpy(), oracle.mmrelu(a, b), K)
    assert torch.all(big[:, N:] == -1.0)


def test_torch_wrapper_single_column_of_any_stride():
    """A (K, 1) view of a (1, K) tensor has column stride K, which a single
    column never uses: the wrapper takes it as row-major with ld 1."""
    M, K = 200, 136
    a = datagen.normal_f32(93, M, K)
    b = datagen.normal_f32(94, 1, K)
    col = to_dev(b).t()
    assert col.shape == (K, 1) and col.stride() == (1, K)
    c = mm.mmrelu(to_dev(a), col)
    torch.cuda.synchronize()
    check_f32(c.cpu().numpy(), oracle.mmrelu(a, np.ascontiguousarray(b.T)), K)


# --- the five workloads at full size -----------------------------------------

def oracle_row_blocks(a, b, M, N, K, lda, ldb, rows=512):
    """The oracle over the whole M x N output, one block of rows at a time
    (the 8192 x 8192 result in fp64 would take 512 MB): yields (i0, i1,
    R[i0:i1])."""
    for i0 in range(0, M, rows):
        i1 = min(M, i0 + rows)
        yield i0, i1, oracle.mmrelu(a[i0:i1], b, M=i1 - i0, N=N, K=K, lda=lda, ldb=ldb)


@pytest.mark.parametrize("ident", [1, 2, 3, 4, 5])
def test_workload_full_size(ident):
    """The workload as the benchmark runs it (planner's kernel, the config's
    leading dimensions), into a NaN-filled C with guard rows; every element
    is compared with the oracle: fp32 max |C - R| <= 1e-4 sqrt(K), bf16
    ||C - R||_F / ||R||_F <= 1e-2 over the whole output plus the element-wise
    bound."""
    cfg = datagen.CONFIGS[ident]
    print(f"workload {cfg.name}", flush=True)
    a, b = datagen.make_inputs(cfg)
    c, whole = run(a, b, cfg.M, cfg.N, cfg.K, cfg.lda, cfg.ldb, ldc=cfg.ldc, guard=2)
    num = den = worst = 0.0
    zeros = 0
    for i0, i1, r in oracle_row_blocks(a, b, cfg.M, cfg.N, cfg.K, cfg.lda, cfg.ldb):
        if cfg.dtype == "f32":
            blk = c[i0:i1]
            check_f32(blk, r, cfg.K)
            worst = max(worst, float(np.abs(blk.astype(np.float64) - r).max()))
        else:
            blk = datagen.bf16_bits_to_f32(c[i0:i1])
            cb = blk.astype(np.float64)
            assert np.all(np.isfinite(cb)) and np.all(cb >= 0)
            d = cb - r
            num += float(np.sum(d * d))
            den += float(np.sum(r * r))
            assert np.all(np.abs(d) <= 2.0 ** -8 * np.abs(r) + 1e-6), f"rows {i0}..{i1}: {np.abs(d).max()}"
        zeros += int(np.count_nonzero(blk == 0))
    if cfg.dtype == "bf16":
        worst = math.sqrt(num / den)
        assert worst <= 1e-2, f"relative Frobenius error {worst}"
    print(f"workload {cfg.name}: {'max abs' if cfg.dtype == 'f32' else 'rel Frobenius'} error {worst:.3g}", flush=True)
    # nothing outside C's rows was written
    rest = np.concatenate([whole[:2], whole[2 + cfg.M:]])
    rest = rest if cfg.dtype == "f32" else datagen.bf16_bits_to_f32(rest)
    assert np.all(np.isnan(rest))
    # inputs symmetric about 0: about half the outputs are exactly zero
    frac = zeros / (cfg.M * cfg.N)
    assert abs(frac - 0.5) < 0.01, frac


def small_int_inputs(cfg, seed):
    """Integers in [-4, 4] of the config's shape and leading dimensions, in
    its dtype: every partial sum is an integer below 16 K <= 2^17, exact in
    fp32 in any order."""
    a = datagen.small_int_f32(seed, cfg.M, cfg.K)
    b = datagen.small_int_f32(seed + 1, cfg.K, cfg.N)
    if cfg.dtype == "bf16":
        a, b = datagen.f32_to_bf16_bits(a), datagen.f32_to_bf16_bits(b)
    return datagen.pad_rows(a, cfg.lda), datagen.pad_rows(b, cfg.ldb)


# (config, dtype, variant): the workloads' shapes and leading dimensions on
# small-integer inputs, through the planner (None) and, for the ragged shape
# with odd leading dimensions, every kernel that accepts that layout: fp32 2
# and 4 (unaligned 128 and 64 tiles), bf16 2, 13 and 15 (any-layout 128, 64
# and 256 tiles), and the plain kernel 0.
EXACT = [(1, "f32", None), (2, "f32", None), (3, "f32", None), (4, "f32", None), (4, "f32", 2), (4, "f32", 4),
         (4, "f32", 0), (4, "bf16", None), (4, "bf16", 2), (4, "bf16", 13), (4, "bf16", 15), (4, "bf16", 0),
         (5, "bf16", None)]


@pytest.mark.parametrize("ident,dtype,variant", EXACT, ids=[f"C{i}-{d}-v{v}" for i, d, v in EXACT])
def test_workload_shapes_exact_integers(ident, dtype, variant):
    """Bit-exact parity at the workload shapes: fp32 C equals the oracle, bf16
    C equals its round-to-nearest-even (C4: lda 2049 and ldb = ldc = 3001,
    rows on every 4- or 2-byte boundary; C5: 8192^3 with results up to 2^17,
    which need bf16 rounding)."""
    cfg = dataclasses.replace(datagen.CONFIGS[ident], dtype=dtype)
    print(f"exact {cfg.name} as {dtype} variant={variant}", flush=True)
    a, b = small_int_inputs(cfg, 3000 + 10 * ident)
    c, whole = run(a, b, cfg.M, cfg.N, cfg.K, cfg.lda, cfg.ldb, ldc=cfg.ldc, variant=variant, guard=2)
    big = 0.0
    for i0, i1, r in oracle_row_blocks(a, b, cfg.M, cfg.N, cfg.K, cfg.lda, cfg.ldb):
        if dtype == "f32":
            np.testing.assert_array_equal(c[i0:i1].astype(np.float64), r, err_msg=f"rows {i0}..{i1}")
        else:
            np.testing.assert_array_equal(c[i0:i1], bf16_round_ref(r), err_msg=f"rows {i0}..{i1}")
        big = max(big, float(r.max()))
    if dtype == "bf16":
        assert big > 256                          # the results need bf16 rounding
    rest = np.concatenate([whole[:2], whole[2 + cfg.M:]])
    rest = rest if dtype == "f32" else datagen.bf16_bits_to_f32(rest)
    assert np.all(np.isnan(rest))


# --- the tile kernels' grid mapping, element by element ------------------------

def run_fused(act, a, b, bias, M, N, K, variant):
    """act(A·B + bias) through the fused C entry point with an explicit
    variant, into a NaN-filled C."""
    dt = torch.float32 if a.dtype == np.float32 else torch.bfloat16
    da, db = to_dev(a), to_dev(b)
    dbias = to_dev(bias) if bias is not None else None
    c = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
    code = {"relu": mm.ACT_RELU, "gelu_tanh": mm.ACT_GELU_TANH, "none": mm.ACT_NONE}[act]
    args = (variant, code, da.data_ptr(), db.data_ptr(), dbias.data_ptr() if dbias is not None else 0,
            c.data_ptr(), M, N, K, K, N, N, torch.cuda.current_stream().cuda_stream)
    fn = mm.mmrelu_fused_f32_variant if dt == torch.float32 else mm.mmrelu_fused_bf16_variant
    rc = fn(*args)
    assert rc == mm.MMRELU_OK, mm.status_string(rc)
    torch.cuda.synchronize()
    return to_host(c)


# 2312 x 2320 x 200: ragged in all three dimensions (the last tile row holds
# 8 rows, the last tile column 16 columns, the last 64-deep pair of slabs 8 k)
# and a grid of several bands of tile rows, with more tiles than XCDs and a
# tile count that is not a multiple of eight (so both the regrouped ids and
# the tail walk their bands). bf16: 1, 3 ping-pong tiles, 4 the 128 x 128
# tile, 2 and 13 the any-layout 128 x 128 and 64 x 64 tiles, 15 - 18 the
# any-layout BM x 256 tiles; fp32: 1, 2 the 128 x 128 tiles, 3, 4 the 64 x 64
# tiles.
MULTIBAND = (2312, 2320, 200)
TILE_KERNELS = [("bf16", 1), ("bf16", 3), ("bf16", 4), ("bf16", 2), ("bf16", 13), ("bf16", 15), ("bf16", 16),
                ("bf16", 17), ("bf16", 18), ("f32", 1), ("f32", 2), ("f32", 3), ("f32", 4)]
EPILOGUES = [("relu", False), ("gelu_tanh", True), ("none", True)]


@pytest.mark.parametrize("act,with_bias", EPILOGUES, ids=[f"{a}-{'bias' if b else 'nobias'}" for a, b in EPILOGUES])
@pytest.mark.parametrize("dtype,variant", TILE_KERNELS, ids=[f"{d}-v{v}" for d, v in TILE_KERNELS])
def test_tile_kernels_multiband_ragged(dtype, variant, act, with_bias):
    """Every element of a multi-band ragged product through one tile kernel,
    against the oracle's fused form (tolerances of the fused-epilogue tests:
    fp32 |C - R| <= L 1e-4 sqrt(K) + 2e-6 (1 + |R|), L = 1.13 for GeLU;
    bf16 relative Frobenius 1e-2 and |C - R| <= 2^-8 |R| + 4e-6)."""
    M, N, K = MULTIBAND
    kind = mm.DTYPE_F32 if dtype == "f32" else mm.DTYPE_BF16
    plan = mm.mmrelu_plan_variant(kind, variant, M, N, K, K, N, N)
    assert plan["tiles_m"] > 8 and plan["grid"] >= 16 and plan["grid"] % 8 != 0, plan
    a = datagen.normal_f32(3100 + variant, M, K, 1 / math.sqrt(K))
    b = datagen.normal_f32(3200 + variant, K, N, 1 / math.sqrt(K))
    bias = datagen.normal_f32(3300 + variant, 1, N, 0.5).ravel() if with_bias else None
    if dtype == "bf16":
        a, b = datagen.f32_to_bf16_bits(a), datagen.f32_to_bf16_bits(b)
        bias = datagen.f32_to_bf16_bits(bias) if bias is not None else None
    print(f"multiband {dtype} variant={variant} act={act} bias={with_bias}", flush=True)
    c = run_fused(act, a, b, bias, M, N, K, variant)
    r = oracle.fused(act, a, b, bias)
    if dtype == "f32":
        assert np.all(np.isfinite(c))
        slope = 1.13 if act == "gelu_tanh" else 1.0
        err = np.abs(c.astype(np.float64) - r)
        assert np.all(err <= slope * 1e-4 * math.sqrt(K) + 2e-6 * (1 + np.abs(r))), err.max()
    else:
        cf = datagen.bf16_bits_to_f32(c).astype(np.float64)
        assert np.all(np.isfinite(cf))
        assert np.linalg.norm(cf - r) / np.linalg.norm(r) <= 1e-2
        assert np.all(np.abs(cf - r) <= 2.0 ** -8 * np.abs(r) + 4e-6), np.abs(cf - r).max()


@pytest.mark.parametrize("dtype,variant", TILE_KERNELS, ids=[f"{d}-v{v}" for d, v in TILE_KERNELS])
def test_tile_kernels_multiband_exact_integers(dtype, variant):
    """The same grids on small-integer inputs: bit-exact (bf16: the oracle
    rounded to nearest-even), so a tile written to the wrong place, or a
    wrong slab summed into a right one, cannot hide under a tolerance."""
    M, N, K = MULTIBAND
    a = datagen.small_int_f32(3400 + variant, M, K)
    b = datagen.small_int_f32(3500 + variant, K, N)
    if dtype == "bf16":
        a, b = datagen.f32_to_bf16_bits(a), datagen.f32_to_bf16_bits(b)
    print(f"multiband exact {dtype} variant={variant}", flush=True)
    c = run_fused("relu", a, b, None, M, N, K, variant)
    r = oracle.mmrelu(a, b)
    if dtype == "f32":
        np.testing.assert_array_equal(c.astype(np.float64), r)
    else:
        np.testing.assert_array_equal(c, bf16_round_ref(r))


# --- the any-layout bf16 kernels on odd layouts over several bands ------------

# 2313 x 2317 x 233 with lda = 235, ldb = 2319, ldc = 2321 (all odd) and A, B,
# C starting 1, 2, 3 elements past a 16-byte boundary: rows of A and B start
# on alternate halves of 4-byte words, the last slab holds 9 k, and the grid
# has several bands of tiles. bf16 15 - 18 copy 4-byte words and realign the
# late rows in LDS (tiles of 256, 224, 192, 160 rows); 2 and 13 realign in
# registers.
ODD_SHAPE, ODD_LD, ODD_OFFS = (2313, 2317, 233), (235, 2319, 2321), (1, 2, 3)


def run_odd_layout(act, a, b, bias, variant):
    M, N, K = ODD_SHAPE
    lda, ldb, ldc = ODD_LD
    fa, pa = placed(a, ODD_OFFS[0], lda)
    fb, pb = placed(b, ODD_OFFS[1], ldb)
    fc, pc = placed(np.zeros((M, 0), np.uint16), ODD_OFFS[2], ldc)       # all NaN
    dbias = to_dev(bias) if bias is not None else None
    code = {"relu": mm.ACT_RELU, "gelu_tanh": mm.ACT_GELU_TANH, "none": mm.ACT_NONE}[act]
    rc = mm.mmrelu_fused_bf16_variant(variant, code, pa, pb, dbias.data_ptr() if dbias is not None else 0, pc,
                                      M, N, K, lda, ldb, ldc, torch.cuda.current_stream().cuda_stream)
    assert rc == mm.MMRELU_OK, mm.status_string(rc)
    torch.cuda.synchronize()
    whole = to_host(fc)
    c = whole[ODD_OFFS[2]:ODD_OFFS[2] + M * ldc].reshape(M, ldc)
    pad = np.concatenate([c[:, N:].ravel(), whole[:ODD_OFFS[2]], whole[ODD_OFFS[2] + M * ldc:]])
    assert np.all(np.isnan(datagen.bf16_bits_to_f32(pad))), "wrote outside C"
    return c[:, :N]


@pytest.mark.parametrize("variant", [15, 16, 17, 18, 2, 13])
def test_any_layout_odd_multiband_exact_integers(variant):
    """Small integers and an integer bias on the odd layout: bit-exact against
    the oracle rounded to nearest-even."""
    M, N, K = ODD_SHAPE
    a = datagen.f32_to_bf16_bits(datagen.small_int_f32(3600 + variant, M, K))
    b = datagen.f32_to_bf16_bits(datagen.small_int_f32(3700 + variant, K, N))
    bias = datagen.f32_to_bf16_bits(datagen.small_int_f32(3800 + variant, 1, N).ravel())
    print(f"odd layout exact variant={variant}", flush=True)
    c = run_odd_layout("none", a, b, bias, variant)
    np.testing.assert_array_equal(c, bf16_round_ref(oracle.fused("none", a, b, bias)))


@pytest.mark.parametrize("variant", [15, 16, 17, 18, 2])
@pytest.mark.parametrize("act", ["relu", "gelu_tanh"])
def test_any_layout_odd_multiband_normal(variant, act):
    """Normal inputs with a bias on the odd layout, every element against the
    oracle's fused form (bf16 tolerances of the fused tests)."""
    M, N, K = ODD_SHAPE
    a = datagen.f32_to_bf16_bits(datagen.normal_f32(3900 + variant, M, K, 1 / math.sqrt(K)))
    b = datagen.f32_to_bf16_bits(datagen.normal_f32(4000 + variant, K, N, 1 / math.sqrt(K)))
    bias = datagen.f32_to_bf16_bits(datagen.normal_f32(4100 + variant, 1, N, 0.5).ravel())
    print(f"odd layout normal variant={variant} act={act}", flush=True)
    c = datagen.bf16_bits_to_f32(run_odd_layout(act, a, b, bias, variant)).astype(np.float64)
    r = oracle.fused(act, a, b, bias)
    assert np.all(np.isfinite(c))
    assert np.linalg.norm(c - r) / np.linalg.norm(r) <= 1e-2
    assert np.all(np.abs(c - r) <= 2.0 ** -8 * np.abs(r) + 4e-6), np.abs(c - r).max()


# Even leading dimensions with operands that start one element past a 4-byte
# boundary: every row of A and B lands one element late in the 256 x 256
# any-layout kernel's copies (variant 15), and none does with an even start;
# through the planner, the register-shift kernel 2 and the plain kernel 0.
@pytest.mark.parametrize("offs", [(1, 1, 1), (2, 2, 2), (3, 2, 1)], ids=["all-late", "none-late", "A-late"])
@pytest.mark.parametrize("variant", [None, 15, 2, 0])
def test_any_layout_even_leading_dims(offs, variant):
    M, N, K = 520, 600, 166                              # K: the last slab holds 6 k
    lda, ldb, ldc = K + 2, N + 2, N + 6                  # even, not multiples of 8
    a = datagen.f32_to_bf16_bits(datagen.small_int_f32(4200, M, K))
    b = datagen.f32_to_bf16_bits(datagen.small_int_f32(4201, K, N))
    fa, pa = placed(a, offs[0], lda)
    fb, pb = placed(b, offs[1], ldb)
    fc, pc = placed(np.zeros((M, 0), np.uint16), offs[2], ldc)
    print(f"even ld offs={offs} variant={variant}", flush=True)
    args = (pa, pb, pc, M, N, K, lda, ldb, ldc, torch.cuda.current_stream().cuda_stream)
    rc = mm.mmrelu_bf16(*args) if variant is None else mm.mmrelu_bf16_variant(variant, *args)
    assert rc == mm.MMRELU_OK, mm.status_string(rc)
    torch.cuda.synchronize()
    whole = to_host(fc)
    c = whole[offs[2]:offs[2] + M * ldc].reshape(M, ldc)
    np.testing.assert_array_equal(c[:, :N], bf16_round_ref(oracle.mmrelu(a, b)))
    pad = np.concatenate([c[:, N:].ravel(), whole[:offs[2]], whole[offs[2] + M * ldc:]])
    assert np.all(np.isnan(datagen.bf16_bits_to_f32(pad))), "wrote outside C"


# The any-layout BM x 256 kernels (variants 15 - 18, BM = 256, 224, 192, 160)
# copy a slab without edge tests when every row of it lies inside K and none
# of its 16-byte copies can reach the end of an operand's range; the last
# slabs take the tested path. A tile shorter than 256 rows still stages 256
# rows, the rest belonging to the next tile (or past M).
# Where a tile's columns end within 256 of N, B's last rows can reach the end
# of B's range from several slabs before K's end (more of them the smaller
# ldb is), so those slabs are tested too. Odd leading dimensions, operands one
# element past a 16-byte boundary, NaN around and between the rows.
EDGE_SLABS = [(300, 40, 500, 501, 41, 43), (260, 300, 400, 401, 301, 300), (70, 3, 700, 703, 3, 5),
              (257, 259, 1000, 1001, 259, 261), (513, 600, 97, 99, 601, 603)]


@pytest.mark.parametrize("variant", [15, 16, 17, 18])     # 256, 224, 192, 160 tile rows
@pytest.mark.parametrize("M,N,K,lda,ldb,ldc", EDGE_SLABS, ids=[f"{s[0]}x{s[1]}x{s[2]}" for s in EDGE_SLABS])
def test_any_layout_realign_inner_and_edge_slabs(M, N, K, lda, ldb, ldc, variant):
    a = datagen.f32_to_bf16_bits(datagen.small_int_f32(4300 + M, M, K))
    b = datagen.f32_to_bf16_bits(datagen.small_int_f32(4400 + N, K, N))
    fa, pa = placed(a, 1, lda)
    fb, pb = placed(b, 1, ldb)
    fc, pc = placed(np.zeros((M, 0), np.uint16), 1, ldc)
    print(f"inner/edge slabs variant {variant} {M}x{N}x{K} ld {lda},{ldb},{ldc}", flush=True)
    rc = mm.mmrelu_bf16_variant(variant, pa, pb, pc, M, N, K, lda, ldb, ldc, torch.cuda.current_stream().cuda_stream)
    assert rc == mm.MMRELU_OK, mm.status_string(rc)
    torch.cuda.synchronize()
    whole = to_host(fc)
    c = whole[1:1 + M * ldc].reshape(M, ldc)
    np.testing.assert_array_equal(c[:, :N], bf16_round_ref(oracle.mmrelu(a, b)))
    pad = np.concatenate([c[:, N:].ravel(), whole[:1], whole[1 + M * ldc:]])
    assert np.all(np.isnan(datagen.bf16_bits_to_f32(pad))), "wrote outside C"


# The planner's tile height on odd-layout bf16 shapes, through the default
# entry point (odd N and K keep the 16-byte kernels out): bit-exact against
# the oracle on small integers, every element. On a 256-CU device the
# planner gives these 224-, 160- and 192-row tiles.
PLANNER_ODD = [((4097, 3001, 2049), "mmrelu_bf16_realign<224,256,32>"),
               ((3001, 3001, 3001), "mmrelu_bf16_realign<160,256,32>"),
               ((4607, 4607, 999), "mmrelu_bf16_realign<192,256,32>")]


@pytest.mark.parametrize("shape,kernel", PLANNER_ODD, ids=[f"{s[0]}x{s[1]}x{s[2]}" for s, _ in PLANNER_ODD])
def test_any_layout_planner_tile_heights_exact(shape, kernel):
    M, N, K = shape
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert mm.mmrelu_plan(mm.DTYPE_BF16, M, N, K, K, N, N, cus=256)["name"] == kernel
    a = datagen.f32_to_bf16_bits(datagen.small_int_f32(3900 + M, M, K))
    b = datagen.f32_to_bf16_bits(datagen.small_int_f32(3950 + N, K, N))
    print(f"planner tile height {M}x{N}x{K}", flush=True)
    c, _ = run(a, b, M, N, K, K, N)
    np.testing.assert_array_equal(c, bf16_round_ref(oracle.mmrelu(a, b)))


# Seeded random shapes, leading dimensions and element offsets through the
# planner in both dtypes: whatever kernel it picks (tile, skinny, any-layout,
# matrix-vector) must reproduce the oracle bit for bit on small integers, and
# write nothing outside C.
RANDOM_CASES = 36


@pytest.mark.parametrize("case", range(RANDOM_CASES))
def test_planner_random_layouts_exact(case):
    rng = np.random.default_rng(7000 + case)
    dtype = "f32" if case % 2 == 0 else "bf16"
    M, N, K = (int(rng.integers(1, 700)) for _ in range(3))
    if case % 3 == 0:
        # every third case meets the 16-byte kernels' contract (sizes, leading
        # dimensions and 16-byte aligned pointers), half of those with few
        # rows, so the tile and skinny kernels are reached too
        q = 4 if dtype == "f32" else 8
        M = int(rng.integers(1, 65)) if case % 6 == 0 else M
        N, K = -(-N // q) * q, -(-K // q) * q
        lda, ldb, ldc = (x + q * int(rng.integers(0, 3)) for x in (K, N, N))
        offs = [0, 0, 0]
    else:
        lda, ldb, ldc = K + int(rng.integers(0, 9)), N + int(rng.integers(0, 9)), N + int(rng.integers(0, 9))
        offs = [int(rng.integers(0, 8)) for _ in range(3)]
    a = datagen.small_int_f32(7100 + case, M, K)
    b = datagen.small_int_f32(7200 + case, K, N)
    if dtype == "bf16":
        a, b = datagen.f32_to_bf16_bits(a), datagen.f32_to_bf16_bits(b)
    fa, pa = placed(a, offs[0], lda)
    fb, pb = placed(b, offs[1], ldb)
    fc, pc = placed(np.zeros((M, 0), a.dtype), offs[2], ldc)
    kind = mm.DTYPE_F32 if dtype == "f32" else mm.DTYPE_BF16
    name = mm.mmrelu_plan(kind, M, N, K, lda, ldb, ldc)["name"]
    print(f"random layout case {case}: {dtype} {M}x{N}x{K} ld {lda},{ldb},{ldc} offs {offs} ({name})", flush=True)
    args = (pa, pb, pc, M, N, K, lda, ldb, ldc, torch.cuda.current_stream().cuda_stream)
    rc = mm.mmrelu_f32(*args) if dtype == "f32" else mm.mmrelu_bf16(*args)
    assert rc == mm.MMRELU_OK, mm.status_string(rc)
    torch.cuda.synchronize()
    whole = to_host(fc)
    c = whole[offs[2]:offs[2] + M * ldc].reshape(M, ldc)
    r = oracle.mmrelu(a, b)
    if dtype == "f32":
        np.testing.assert_array_equal(c[:, :N].astype(np.float64), r)
        pad = np.concatenate([c[:, N:].ravel(), whole[:offs[2]], whole[offs[2] + M * ldc:]])
        assert np.all(np.isnan(pad)), "wrote outside C"
    else:
        np.testing.assert_array_equal(c[:, :N], bf16_round_ref(r))
        pad = np.concatenate([c[:, N:].ravel(), whole[:offs[2]], whole[offs[2] + M * ldc:]])
        assert np.all(np.isnan(datagen.bf16_bits_to_f32(pad))), "wrote outside C"
