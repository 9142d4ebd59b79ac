"""The C-ABI library on the CPU: it loads, exports every declared symbol,
validates arguments before touching the GPU, and plans grids (no kernel is
launched here)."""
import json
import os
import re

import numpy as np
import pytest

import tiled_matmul_relu_amd as mm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mmrelu.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mmrelu_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = mm.load_library()
    names = declared_functions()
    assert "mmrelu_f32" in names and "mmrelu_bf16" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(mm.EXPORTED)


def test_status_strings_and_version():
    assert mm.status_string(0) == "ok"
    for s in range(1, 5):
        assert mm.status_string(s) not in ("ok", "unknown status")
    assert mm.status_string(99) == "unknown status"
    assert "gfx950" in mm.version()


A, B, C = 0x100000, 0x200000, 0x300000     # aligned fake device addresses (never dereferenced)


@pytest.mark.parametrize("fn", [mm.mmrelu_f32, mm.mmrelu_bf16])
def test_argument_validation_before_launch(fn):
    E = mm
    # negative sizes
    assert fn(A, B, C, -1, 4, 4, 4, 4, 4) == E.MMRELU_ERR_INVALID_VALUE
    assert fn(A, B, C, 4, -1, 4, 4, 4, 4) == E.MMRELU_ERR_INVALID_VALUE
    assert fn(A, B, C, 4, 4, -1, 4, 4, 4) == E.MMRELU_ERR_INVALID_VALUE
    # leading dimensions too small / too large
    assert fn(A, B, C, 4, 4, 8, 7, 4, 4) == E.MMRELU_ERR_INVALID_VALUE
    assert fn(A, B, C, 4, 8, 4, 4, 7, 8) == E.MMRELU_ERR_INVALID_VALUE
    assert fn(A, B, C, 4, 8, 4, 4, 8, 7) == E.MMRELU_ERR_INVALID_VALUE
    assert fn(A, B, C, 4, 4, 4, 0, 4, 4) == E.MMRELU_ERR_INVALID_VALUE
    assert fn(A, B, C, 4, 4, 4, (1 << 21) + 1, 4, 4) == E.MMRELU_ERR_INVALID_VALUE
    assert fn(A, B, C, 1 << 31, 4, 4, 4, 4, 4) == E.MMRELU_ERR_INVALID_VALUE
    # null pointers
    assert fn(A, B, 0, 4, 4, 4, 4, 4, 4) == E.MMRELU_ERR_NULL_POINTER
    assert fn(0, B, C, 4, 4, 4, 4, 4, 4) == E.MMRELU_ERR_NULL_POINTER
    assert fn(A, 0, C, 4, 4, 4, 4, 4, 4) == E.MMRELU_ERR_NULL_POINTER
    # misaligned to the element size
    assert fn(A + 1, B, C, 4, 4, 4, 4, 4, 4) == E.MMRELU_ERR_MISALIGNED
    assert fn(A, B, C + 1, 4, 4, 4, 4, 4, 4) == E.MMRELU_ERR_MISALIGNED
    # empty outputs: OK without a launch, even with null pointers
    assert fn(0, 0, 0, 0, 4, 4, 4, 4, 4) == E.MMRELU_OK
    assert fn(0, 0, 0, 4, 0, 4, 4, 1, 1) == E.MMRELU_OK


def test_fp32_alignment_only_needs_4_bytes_bf16_2_bytes():
    # misaligned by 2 bytes: fine for bf16 validation (fails only later for
    # lack of a GPU, so test with an empty output), not for fp32
    assert mm.mmrelu_f32(A + 2, B, C, 4, 4, 4, 4, 4, 4) == mm.MMRELU_ERR_MISALIGNED
    assert mm.mmrelu_bf16(A + 2, B, C, 4, 0, 4, 4, 1, 1) == mm.MMRELU_OK


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_entry_points_validate(dtype):
    E = mm
    fused = mm.mmrelu_fused_f32 if dtype == "f32" else mm.mmrelu_fused_bf16
    fused_v = mm.mmrelu_fused_f32_variant if dtype == "f32" else mm.mmrelu_fused_bf16_variant
    esize = 4 if dtype == "f32" else 2
    bias = 0x400000
    # unknown activation codes
    for act in (-1, 3, 99):
        assert fused(act, A, B, bias, C, 4, 4, 4, 4, 4, 4) == E.MMRELU_ERR_INVALID_VALUE
        assert fused_v(0, act, A, B, bias, C, 4, 4, 4, 4, 4, 4) == E.MMRELU_ERR_INVALID_VALUE
    # a bias not aligned to its element size
    assert fused(E.ACT_GELU_TANH, A, B, bias + esize // 2, C, 4, 4, 4, 4, 4, 4) == E.MMRELU_ERR_MISALIGNED
    # the shape checks apply as in the plain entry points
    assert fused(E.ACT_NONE, A, B, bias, C, -1, 4, 4, 4, 4, 4) == E.MMRELU_ERR_INVALID_VALUE
    assert fused(E.ACT_RELU, A, B, 0, 0, 4, 4, 4, 4, 4, 4) == E.MMRELU_ERR_NULL_POINTER
    assert fused_v(-1, E.ACT_RELU, A, B, bias, C, 4, 4, 4, 4, 4, 4) == E.MMRELU_ERR_INVALID_VALUE
    assert fused_v(99, E.ACT_RELU, A, B, bias, C, 4, 4, 4, 4, 4, 4) == E.MMRELU_ERR_INVALID_VALUE
    # empty outputs launch nothing, with or without a bias
    assert fused(E.ACT_GELU_TANH, A, B, bias, C, 0, 4, 4, 4, 4, 4) == E.MMRELU_OK
    assert fused(E.ACT_GELU_TANH, A, B, 0, C, 4, 0, 4, 4, 4, 4) == E.MMRELU_OK


def test_planner_picks_skinny_kernels_for_few_rows():
    for dt in (mm.DTYPE_F32, mm.DTYPE_BF16):
        for M, rows in ((1, 16), (16, 16), (17, 32), (32, 32), (33, 64), (64, 64)):
            p = mm.mmrelu_plan(dt, M, 8192, 8192, 8192, 8192, 8192, cus=256)
            assert "skinny" in p["name"] and p["block_m"] == rows and p["grid"] == 8192 // 32, (M, p["name"])
        # at most 16 rows and one 64-column strip per CU or more: 16 x 64 strips
        p = mm.mmrelu_plan(dt, 4, 16384, 4096, 4096, 16384, 16384, cus=256)
        want = 14 if dt == mm.DTYPE_BF16 else 13
        assert (p["variant"], p["block_m"], p["block_n"], p["grid"]) == (want, 16, 64, 256), p
        # ... but not at 8192 columns (128 strips of 64 for 256 CUs)
        assert mm.mmrelu_plan(dt, 4, 8192, 4096, 4096, 8192, 8192, cus=256)["variant"] == 5
        assert mm.mmrelu_plan(dt, 17, 16384, 4096, 4096, 16384, 16384, cus=256)["variant"] == 6
        # past 64 rows the cost model decides, not the few-rows rule's 64 x 32
        # strips (fp32: 32 x 32 tiles, three row tiles; bf16: 64 x 64 tiles)
        p = mm.mmrelu_plan(dt, 65, 8192, 8192, 8192, 8192, 8192, cus=256)
        assert p["variant"] != 7 and p["variant"] == (9 if dt == mm.DTYPE_F32 else 12), p["name"]
        # an odd leading dimension needs a kernel that accepts any layout
        p = mm.mmrelu_plan(dt, 16, 8191, 8192, 8192, 8191, 8191, cus=256)
        assert "skinny" not in p["name"]


def test_planner_picks_skinny_kernels_for_few_columns():
    q = {mm.DTYPE_F32: 4, mm.DTYPE_BF16: 8}
    for dt in (mm.DTYPE_F32, mm.DTYPE_BF16):
        for N, cols in ((q[dt], 16), (16, 16), (24, 32), (32, 32), (40, 64), (64, 64)):
            p = mm.mmrelu_plan(dt, 8192, N, 8192, 8192, N, N, cus=256)
            assert "skinny" in p["name"] and p["block_n"] == cols and p["block_m"] == 32, (N, p["name"])
            assert p["grid"] == 8192 // 32
        # past 64 columns the cost model decides among all candidates
        p = mm.mmrelu_plan(dt, 8192, 72, 8192, 8192, 72, 72, cus=256)
        assert p["grid"] == ((8192 + p["block_m"] - 1) // p["block_m"]) * ((72 + p["block_n"] - 1) // p["block_n"])
        # both small: the smaller dimension decides
        assert mm.mmrelu_plan(dt, 16, 64, 8192, 8192, 64, 64, cus=256)["block_m"] == 16
        p = mm.mmrelu_plan(dt, 64, 16, 8192, 8192, 16, 16, cus=256)
        assert (p["block_m"], p["block_n"]) == (32, 16)
        # fp32, at most 16 columns and one 64-row band per CU or more: 64 x 16 bands
        p = mm.mmrelu_plan(dt, 16384, 16, 8192, 8192, 16, 16, cus=256)
        if dt == mm.DTYPE_F32:
            assert (p["variant"], p["block_m"], p["block_n"], p["grid"]) == (14, 64, 16, 256), p
        else:
            assert (p["variant"], p["block_m"]) == (8, 32), p
        assert mm.mmrelu_plan(dt, 16384, 24, 8192, 8192, 24, 24, cus=256)["variant"] == 9


def test_skinny_variants_tile_any_shape():
    """A skinny variant covers a shape of any size with a grid of its tiles."""
    for dt in (mm.DTYPE_F32, mm.DTYPE_BF16):
        for v in range(mm.mmrelu_num_variants(dt)):
            p = mm.mmrelu_plan_variant(dt, v, 1000, 264, 512, 512, 264, 264, cus=256)
            if "skinny" not in p["name"]:
                continue
            tm = (1000 + p["block_m"] - 1) // p["block_m"]
            tn = (264 + p["block_n"] - 1) // p["block_n"]
            assert (p["tiles_m"], p["tiles_n"], p["grid"]) == (tm, tn, tm * tn), p["name"]


def test_variant_entry_points_validate():
    assert mm.mmrelu_f32_variant(-1, A, B, C, 4, 4, 4, 4, 4, 4) == mm.MMRELU_ERR_INVALID_VALUE
    assert mm.mmrelu_f32_variant(99, A, B, C, 4, 4, 4, 4, 4, 4) == mm.MMRELU_ERR_INVALID_VALUE
    assert mm.mmrelu_bf16_variant(99, A, B, C, 4, 4, 4, 4, 4, 4) == mm.MMRELU_ERR_INVALID_VALUE
    # a variant that needs 16-byte rows refuses an odd leading dimension
    nv = mm.mmrelu_num_variants(mm.DTYPE_F32)
    needs_align = [v for v in range(nv) if "unaligned" not in mm.mmrelu_plan_variant(0, v, 8, 8, 8, 8, 8, 8)["name"]
                   and "mfma" in mm.mmrelu_plan_variant(0, v, 8, 8, 8, 8, 8, 8)["name"]]
    assert needs_align
    for v in needs_align:
        assert mm.mmrelu_f32_variant(v, A, B, C, 5, 5, 5, 5, 5, 5) == mm.MMRELU_ERR_INVALID_VALUE


def test_wave_quantization_matches_lecture_arithmetic():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "wave_quantization.json")))
    for case in g["cases"]:
        assert mm.mmrelu_wave_quantization(case["blocks"], case["slots"]) == (case["waves"], case["idle_last"])
        if "tile" in case:
            assert (case["output"] // case["tile"]) ** 2 == case["blocks"]
    with pytest.raises(mm.MmreluError):
        mm.mmrelu_wave_quantization(5, 0)


def test_plans_for_the_workloads():
    # 4096^3 fp32: 128x128 tiles, 1024 workgroups, two resident per CU:
    # exactly two full waves over 256 CUs (no tail)
    p = mm.mmrelu_plan(mm.DTYPE_F32, 4096, 4096, 4096, 4096, 4096, 4096, cus=256)
    assert "mfma" in p["name"] and "unaligned" not in p["name"]
    assert p["grid"] == p["tiles_m"] * p["tiles_n"]
    assert p["idle_slots_last"] == 0
    # ragged 4097 x 3001 x 2049: odd leading dimensions need the dword path
    p = mm.mmrelu_plan(mm.DTYPE_F32, 4097, 3001, 2049, 2049, 3001, 3001, cus=256)
    assert "unaligned" in p["name"]
    assert p["tiles_m"] == -(-4097 // p["block_m"]) and p["tiles_n"] == -(-3001 // p["block_n"])
    # 8192^3 bf16: matrix-core kernel, whole waves
    p = mm.mmrelu_plan(mm.DTYPE_BF16, 8192, 8192, 8192, 8192, 8192, 8192, cus=256)
    assert p["name"] == "mmrelu_bf16_pingpong<256,256,64,A3B4>" and p["idle_slots_last"] == 0
    # bf16 with N, K or a leading dimension off the 8-element grid: the
    # any-layout matrix-core kernel
    p = mm.mmrelu_plan(mm.DTYPE_BF16, 100, 100, 100, 100, 100, 100, cus=256)
    assert "bf16_any" in p["name"] and p["grid"] == 4
    with pytest.raises(mm.MmreluError):
        mm.mmrelu_plan(mm.DTYPE_F32, -1, 4, 4, 4, 4, 4)
    with pytest.raises(mm.MmreluError):
        mm.mmrelu_plan(7, 4, 4, 4, 4, 4, 4)


def test_planner_tile_choice_by_wave_quantization():
    """Smaller tiles when the large tile's grid leaves CUs idle (the a7 rule:
    ceil(tiles / CUs) * tile outputs * measured relative cost)."""
    sq = lambda dt, n, cus=256: mm.mmrelu_plan(dt, n, n, n, n, n, n, cus=cus)
    # fp32: 2048^3 takes 64x64 tiles (four per CU: 4 * 4096 * 1.02 against one
    # 128x128 tile per CU at 16384 * 1.15); 4096^3 and up fill the CUs with 128x128
    for n, tile in ((2048, 64), (4096, 128), (8192, 128)):
        p = sq(mm.DTYPE_F32, n)
        assert (p["block_m"], p["block_n"]) == (tile, tile) and "mfma" in p["name"], (n, p["name"])
        assert "unaligned" not in p["name"]
    # the ragged shape: 792 tiles of 128x128 (4 on the busiest CU, 4 * 16384 outputs)
    # against 3055 of 64x64 (12 on the busiest CU, 12 * 4096 * 1.02)
    p = mm.mmrelu_plan(mm.DTYPE_F32, 4097, 3001, 2049, 2049, 3001, 3001, cus=256)
    assert "unaligned" in p["name"] and p["block_m"] == 64 and p["grid"] == 65 * 47
    # bf16: 128x128 at 2048^2 (one tile per CU on either grid); 256x256 from 3072^2 on
    for n, tile in ((2048, 128), (3072, 256), (4096, 256), (6144, 256), (8192, 256)):
        p = sq(mm.DTYPE_BF16, n)
        assert p["block_m"] == tile and "skinny" not in p["name"], (n, p["name"])
    assert "pingpong" in sq(mm.DTYPE_BF16, 8192)["name"]
    # fewer CUs shift the crossover: on 64 CUs 2048^2 bf16 has one 256x256 tile per CU
    assert sq(mm.DTYPE_BF16, 2048, cus=64)["block_m"] == 256
    # the plan's kernel is the one the launch uses: planning with any CU count
    # stays within the candidates that accept the layout
    p = mm.mmrelu_plan(mm.DTYPE_BF16, 1000, 1000, 1000, 1000, 1000, 1000, cus=256)
    assert "mfma" in p["name"] or "pingpong" in p["name"] or "skinny" in p["name"]
    p = mm.mmrelu_plan(mm.DTYPE_BF16, 1000, 1001, 1000, 1000, 1001, 1001, cus=256)
    assert "bf16_any" in p["name"]


def test_planner_square_skinny_tile():
    """The 64x64 skinny tile (variant 12) wins small squares and long-K
    products with 256 or fewer output tiles of 64x64; larger grids go back to
    the tile kernels, smaller ones to narrower skinny tiles."""
    plan = lambda dt, m, n, k: mm.mmrelu_plan(dt, m, n, k, k, n, n, cus=256)
    for dt in (mm.DTYPE_F32, mm.DTYPE_BF16):
        assert plan(dt, 1024, 1024, 1024)["variant"] == 12
        assert plan(dt, 1024, 1024, 8192)["variant"] == 12
        assert plan(dt, 2048, 2048, 2048)["variant"] in (3, 4)      # the 64x64 / 128x128 tile kernels
        assert plan(dt, 512, 512, 8192)["name"].startswith("mmrelu_skinny") and plan(dt, 512, 512, 8192)["block_m"] == 32
    assert plan(mm.DTYPE_F32, 768, 768, 768)["block_m"] == 32       # 576 tiles of 32x32
    p = mm.mmrelu_plan_variant(mm.DTYPE_F32, 12, 1000, 264, 512, 512, 264, 264, cus=256)
    assert (p["block_m"], p["block_n"], p["grid"]) == (64, 64, 16 * 5)


def test_planner_any_layout_tile():
    """Unaligned bf16: 64x64 tiles until the 128x128 grid gives three CUs in
    four a tile; then 128x128 tiles (two workgroups a CU) or BM x 256 tiles
    (one a CU, BM = 256, 224, 192, 160), whichever has the smallest busiest-
    CU tile count times a + b K, with the fitted a (us) and b (us per k):
    128x128 3.1 + 0.0165 K, 256 rows 17.2 + 0.0243 K, 224 rows 15.6 + 0.0236
    K, 192 rows 14.2 + 0.0225 K, 160 rows 12.3 + 0.0227 K."""
    plan = lambda m, n, k, cus=256: mm.mmrelu_plan(mm.DTYPE_BF16, m, n, k, k, n, n, cus=cus)
    # 4097 x 3001: 204 tiles of 256 rows (1 per CU: 67.0) against 228 of 224
    # rows (1: 64.0); 192 rows give 22 x 12 = 264 tiles, two on some CUs
    p = plan(4097, 3001, 2049)
    assert p["name"] == "mmrelu_bf16_realign<224,256,32>" and p["grid"] == 19 * 12
    odd = {(4095, 4095, 4095): 15,                     # 256 tiles of 256 rows: one each
           (8191, 8191, 8191): 15,                     # 4 per CU against 5, 6 and 7
           (5000, 5000, 999): 16,                      # 2 per CU: 2 x 39.2 against 2 x 41.5
           (4607, 4607, 999): 17,                      # 432 tiles of 192 rows: 2 x 36.7
           (3001, 3001, 3001): 18,                     # 228 tiles of 160 rows, one each
           (4097, 4097, 767): 18,                      # 442 of 160 rows: 2 x 29.7
           (2561, 2561, 1023): 18,                     # 187 of 160 rows: 35.5 against 2 x 20.0
           (1793, 1793, 1023): 2,                      # 196 tiles of 128x128, one each: 20.0
           (2049, 2049, 255): 2,
           (1537, 1537, 1537): 13}                     # 169 tiles of 128x128, under 192
    for (M, N, K), want in odd.items():
        assert plan(M, N, K)["variant"] == want, (M, N, K)
    # 2047^2: 16 * 16 = 256 tiles of 128x128, one per CU: 36.9 against 58.8
    # on 160 rows
    p = plan(2047, 2047, 2047)
    assert p["name"] == "mmrelu_bf16_any<128,128,32>" and p["grid"] == 16 * 16
    p = plan(1001, 1001, 1001)
    assert p["name"] == "mmrelu_bf16_any<64,64,32>" and p["grid"] == 16 * 16
    # the threshold moves with the CU count: 1001^2 on 64 CUs takes 128x128
    assert plan(1001, 1001, 1001, cus=64)["name"] == "mmrelu_bf16_any<128,128,32>"
    # just at the threshold: 12 x 16 = 192 tiles, and one tile row fewer
    assert plan(1536, 2047, 1001)["name"] == "mmrelu_bf16_any<128,128,32>"
    assert plan(1536 - 128, 2047, 1001)["name"] == "mmrelu_bf16_any<64,64,32>"


def test_every_variant_plans():
    for dt in (mm.DTYPE_F32, mm.DTYPE_BF16):
        n = mm.mmrelu_num_variants(dt)
        assert n >= 2
        names = set()
        for v in range(n):
            p = mm.mmrelu_plan_variant(dt, v, 1000, 1000, 1000, 1000, 1000, 1000, cus=256)
            assert p["variant"] == v and p["grid"] == p["tiles_m"] * p["tiles_n"] > 0
            names.add(p["name"])
        assert len(names) == n


def test_planner_picks_a_kernel_that_accepts_the_layout():
    """Seeded random shapes and leading dimensions, both dtypes, several CU
    counts: the planned kernel is one whose layout contract the arguments
    meet (16-byte-vector kernels need N, K and every leading dimension to be
    multiples of 16 bytes; any-layout, matrix-vector and plain kernels take
    anything), skinny tiles cover every row or column they are given, and
    the plan's grid covers the output exactly once."""
    rng = np.random.default_rng(20261202)
    any_layout = ("simple", "unaligned", "gemv", "_any<", "_realign<")
    for _ in range(3000):
        dt = int(rng.integers(0, 2))
        q = 4 if dt == mm.DTYPE_F32 else 8
        aligned = rng.random() < 0.5
        dims = []
        for _d in range(3):
            x = int(rng.choice([rng.integers(1, 65), rng.integers(1, 3000), rng.integers(1, 9000)]))
            dims.append((x + q - 1) // q * q if aligned else x)
        M, N, K = dims
        pad = lambda v: v + (int(rng.integers(0, 3)) * q if aligned else int(rng.integers(0, 5)))
        lda, ldb, ldc = pad(K), pad(N), pad(N)
        cus = int(rng.choice([64, 80, 256, 304]))
        p = mm.mmrelu_plan(dt, M, N, K, lda, ldb, ldc, cus=cus)
        name = p["name"]
        if not any(t in name for t in any_layout):
            assert all(x % q == 0 for x in (N, K, lda, ldb, ldc)), (dt, M, N, K, lda, ldb, ldc, name)
        assert p["tiles_m"] == -(-M // p["block_m"]) and p["tiles_n"] == -(-N // p["block_n"]), (M, N, p)
        assert p["grid"] == p["tiles_m"] * p["tiles_n"]
        assert p["variant"] != 0, "the plain kernel is only reached through the _variant entry points"


def test_python_wrapper_rejects_bad_tensors():
    import torch
    with pytest.raises(TypeError):
        mm.mmrelu(torch.zeros(2, 2), torch.zeros(2, 2, dtype=torch.float64))
    with pytest.raises(ValueError):
        mm.mmrelu(torch.zeros(2, 2), torch.zeros(2, 2))   # host tensors


# --- general strides: host-side planning and validation (no launch) ---------

_P = 1 << 20          # 16-byte aligned stand-in addresses; nothing is launched


def _ws(dt, M, N, K, sam, sak, sbk, sbn, scm, scn, bias=0, act=mm.ACT_RELU, a=_P, b=2 * _P, c=3 * _P):
    return mm.mmrelu_strided_workspace_size(dt, act, a, b, bias, c, M, N, K, sam, sak, sbk, sbn, scm, scn)


def _rup(x, q):
    return (x + q - 1) // q * q


def test_strided_workspace_plans():
    M, N, K = 512, 256, 128
    for dt, es in ((mm.DTYPE_F32, 4), (mm.DTYPE_BF16, 2)):
        assert _ws(dt, M, N, K, K, 1, N, 1, N, 1) == 0                       # row-major: in place
        assert _ws(dt, M, N, K, K + 64, 1, N + 32, 1, N + 16, 1) == 0        # padded rows: in place
        assert _ws(dt, M, N, K, 1, M, N, 1, N, 1) == M * K * es              # A^T: A packed
        assert _ws(dt, M, N, K, K, 1, 1, K, N, 1) == K * N * es              # B^T: B packed
        assert _ws(dt, M, N, K, 1, M, 1, K, N, 1) == (M * K + K * N) * es    # both
        assert _ws(dt, M, N, K, 1, M, 1, K, 1, M) == 0                       # TT into column-major C: swap
        # NN into column-major C: swap packs both operands (K*(M+N)) < temporary C (M*N)
        assert _ws(dt, M, N, K, K, 1, N, 1, 1, M) == (M * K + K * N) * es
        # a bias rules the swap out: row-major temporary C
        assert _ws(dt, M, N, K, 1, M, 1, K, 1, M, bias=4 * _P) == (M * K + K * N + M * N) * es
        # long K: the temporary C is smaller than packing both operands
        assert _ws(dt, 128, 128, 4096, 4096, 1, 128, 1, 1, 128) == 128 * 128 * es
        # sub-sampled views are packed
        assert _ws(dt, M, N, K, 6 * K, 3, 2 * N, 2, N, 1) == (M * K + K * N) * es
        # empty outputs need nothing
        assert _ws(dt, 0, N, K, 1, 1, 1, 1, 1, 1) == 0
    # bf16 shape that allows 16-byte vectors: a row-major A with an odd ld is packed
    assert _ws(mm.DTYPE_BF16, M, N, K, K + 1, 1, N, 1, N, 1) == M * K * 2
    # ... a misaligned pointer too, and the packed ld is rounded up to 8 elements
    assert _ws(mm.DTYPE_BF16, M, N, 120, 120, 1, N, 1, N, 1, a=_P + 2) == M * 120 * 2
    # a shape that rules the vector kernels out anyway keeps row-major operands in place
    assert _ws(mm.DTYPE_BF16, M, 100, K, K + 1, 1, 100, 1, 100, 1) == 0
    # packed operands get 256-byte aligned slots
    assert _ws(mm.DTYPE_F32, 3, 4, 5, 1, 3, 1, 5, 4, 1) == _rup(3 * 8 * 4, 256) + _rup(5 * 4 * 4, 256)


def test_strided_validation():
    M, N, K = 64, 32, 16
    bad = [
        (M, N, K, -1, 1, N, 1, N, 1),        # negative stride
        (M, N, K, K, 1, N, 1, N, 0),         # zero output stride
        (M, N, K, K, 1, N, 1, 1, 1),         # outputs overlap
        (M, N, K, K, 1, N, 1, N - 1, 1),     # rows of C overlap
        (M, N, K, 1 << 59, 1 << 59, N, 1, N, 1),    # offset past 2^60
        (-1, N, K, K, 1, N, 1, N, 1),
    ]
    for args in bad:
        with pytest.raises(mm.MmreluError) as e:
            _ws(mm.DTYPE_F32, *args)
        assert e.value.status == mm.MMRELU_ERR_INVALID_VALUE, args
    with pytest.raises(mm.MmreluError) as e:
        _ws(mm.DTYPE_F32, M, N, K, K, 1, N, 1, N, 1, act=7)
    assert e.value.status == mm.MMRELU_ERR_INVALID_VALUE
    with pytest.raises(mm.MmreluError) as e:
        _ws(mm.DTYPE_F32, M, N, K, K, 1, N, 1, N, 1, a=_P + 2)
    assert e.value.status == mm.MMRELU_ERR_MISALIGNED
    with pytest.raises(mm.MmreluError) as e:
        _ws(mm.DTYPE_F32, M, N, K, K, 1, N, 1, N, 1, c=0)
    assert e.value.status == mm.MMRELU_ERR_NULL_POINTER
    # zero strides in A and B (repeated elements) are allowed
    assert _ws(mm.DTYPE_F32, M, N, K, 0, 1, N, 0, N, 1) >= 0


def test_strided_entry_points_check_workspace_before_launch():
    M, N, K = 64, 32, 16
    need = _ws(mm.DTYPE_F32, M, N, K, 1, M, N, 1, N, 1)
    assert need == M * K * 4
    args = (mm.ACT_RELU, _P, 2 * _P, 0, 3 * _P, M, N, K, 1, M, N, 1, N, 1)
    assert mm.mmrelu_strided_f32(*args, 0, need) == mm.MMRELU_ERR_NULL_POINTER
    assert mm.mmrelu_strided_f32(*args, 4 * _P, need - 1) == mm.MMRELU_ERR_INVALID_VALUE
    assert mm.mmrelu_strided_f32(*args, 4 * _P + 16, need) == mm.MMRELU_ERR_MISALIGNED
    assert mm.mmrelu_strided_bf16(*args, 0, need) == mm.MMRELU_ERR_NULL_POINTER
    # invalid strides come back before the workspace is looked at
    assert mm.mmrelu_strided_f32(mm.ACT_RELU, _P, 2 * _P, 0, 3 * _P, M, N, K, 1, M, N, 1, 1, 1, 0, 0) == \
        mm.MMRELU_ERR_INVALID_VALUE
    # empty outputs: nothing to do, no workspace
    assert mm.mmrelu_strided_f32(mm.ACT_RELU, _P, 2 * _P, 0, 3 * _P, 0, N, K, 1, 1, 1, 1, 1, 1, 0, 0) == mm.MMRELU_OK


def test_strided_static_checks_before_any_hip_call():
    """mmrelu_strided_static validates like the strided entry points and
    refuses a call needing more than its fixed workspace before anything
    touches the device (these stand-in pointers are never dereferenced)."""
    M = N = K = 8192
    need = _ws(mm.DTYPE_BF16, M, N, K, 1, M, N, 1, N, 1)            # A^T: 128 MiB
    assert need == M * K * 2 > mm.STATIC_WORKSPACE_BYTES
    st = mm.mmrelu_strided_static
    assert st(mm.DTYPE_BF16, mm.ACT_RELU, _P, 2 * _P, 0, 3 * _P, M, N, K, 1, M, N, 1, N, 1) == \
        mm.MMRELU_ERR_WORKSPACE_LIMIT
    assert "MMRELU_STATIC_WORKSPACE_BYTES" in mm.status_string(mm.MMRELU_ERR_WORKSPACE_LIMIT)
    # just under the limit is planned, just over is refused: 4096 x 4096 bf16 A^T is 32 MiB
    assert _ws(mm.DTYPE_BF16, 4096, 4096, 4096, 1, 4096, 4096, 1, 4096, 1) <= mm.STATIC_WORKSPACE_BYTES
    assert _ws(mm.DTYPE_F32, 4096, 4096, 4096, 1, 4096, 1, 4096, 4096, 1) > mm.STATIC_WORKSPACE_BYTES
    assert st(mm.DTYPE_F32, mm.ACT_RELU, _P, 2 * _P, 0, 3 * _P, 4096, 4096, 4096, 1, 4096, 1, 4096, 4096, 1) == \
        mm.MMRELU_ERR_WORKSPACE_LIMIT
    # the strided entry points' own checks come first
    assert st(7, mm.ACT_RELU, _P, 2 * _P, 0, 3 * _P, 64, 32, 16, 16, 1, 32, 1, 32, 1) == mm.MMRELU_ERR_INVALID_VALUE
    assert st(mm.DTYPE_F32, 9, _P, 2 * _P, 0, 3 * _P, 64, 32, 16, 16, 1, 32, 1, 32, 1) == \
        mm.MMRELU_ERR_INVALID_VALUE
    assert st(mm.DTYPE_F32, mm.ACT_RELU, _P, 2 * _P, 0, 3 * _P, 64, 32, 16, 16, 1, 32, 1, 1, 1) == \
        mm.MMRELU_ERR_INVALID_VALUE
    assert st(mm.DTYPE_F32, mm.ACT_RELU, _P + 2, 2 * _P, 0, 3 * _P, 64, 32, 16, 16, 1, 32, 1, 32, 1) == \
        mm.MMRELU_ERR_MISALIGNED
    assert st(mm.DTYPE_F32, mm.ACT_RELU, _P, 2 * _P, 0, 0, 64, 32, 16, 16, 1, 32, 1, 32, 1) == \
        mm.MMRELU_ERR_NULL_POINTER
    # empty outputs: nothing to do
    assert st(mm.DTYPE_F32, mm.ACT_RELU, _P, 2 * _P, 0, 3 * _P, 0, 32, 16, 1, 1, 1, 1, 1, 1) == mm.MMRELU_OK


# --- row softmax and row sum: validation and kernel choice (no launch) -------

def test_softmax_variant_choice():
    F, B = mm.DTYPE_F32, mm.DTYPE_BF16
    assert [mm.mmrelu_softmax_rows_variant(F, n, n, n) for n in (4, 1024, 1028, 4096, 4100, 16384, 16388)] == \
        [0, 0, 1, 1, 2, 2, 3]
    assert [mm.mmrelu_softmax_rows_variant(B, n, n, n) for n in (8, 2048, 2056, 8192, 8200, 32768, 32776)] == \
        [0, 0, 1, 1, 2, 2, 3]
    assert mm.mmrelu_softmax_rows_variant(F, 1001, 1001, 1001) == 4       # N not a multiple of 4
    assert mm.mmrelu_softmax_rows_variant(F, 1000, 1001, 1000) == 4       # ldx not a multiple of 4
    assert mm.mmrelu_softmax_rows_variant(B, 1004, 1004, 1004) == 4       # bf16 N not a multiple of 8
    with pytest.raises(mm.MmreluError):
        mm.mmrelu_softmax_rows_variant(F, 100, 99, 100)


def test_row_ops_validate_before_launch():
    s = mm.mmrelu_softmax_rows_f32
    assert s(_P, 2 * _P, -1, 4, 4, 4) == mm.MMRELU_ERR_INVALID_VALUE
    assert s(_P, 2 * _P, 4, 8, 4, 8) == mm.MMRELU_ERR_INVALID_VALUE        # ldx < N
    assert s(_P, 2 * _P, 4, 8, 8, 4) == mm.MMRELU_ERR_INVALID_VALUE        # ldy < N
    assert s(_P, _P, 4, 8, 8, 16) == mm.MMRELU_ERR_INVALID_VALUE           # in place with another ld
    assert s(0, 2 * _P, 4, 8, 8, 8) == mm.MMRELU_ERR_NULL_POINTER
    assert s(_P, 0, 4, 8, 8, 8) == mm.MMRELU_ERR_NULL_POINTER
    assert s(_P + 2, 2 * _P, 4, 8, 8, 8) == mm.MMRELU_ERR_MISALIGNED
    assert s(_P, 2 * _P, 4, 8, 1 << 59, 8) == mm.MMRELU_ERR_INVALID_VALUE  # offset past 2^60
    assert s(_P, 2 * _P, 0, 8, 8, 8) == mm.MMRELU_OK                        # empty: nothing launched
    assert s(_P, 2 * _P, 5, 0, 1, 1) == mm.MMRELU_OK
    assert mm.mmrelu_softmax_rows_bf16(_P + 1, 2 * _P, 4, 8, 8, 8) == mm.MMRELU_ERR_MISALIGNED
    v = mm.mmrelu_softmax_rows_f32_variant
    assert v(9, _P, 2 * _P, 4, 8, 8, 8) == mm.MMRELU_ERR_INVALID_VALUE     # no such kernel
    assert v(0, _P, 2 * _P, 4, 7, 7, 7) == mm.MMRELU_ERR_INVALID_VALUE     # vector kernel, N % 4 != 0
    assert v(0, _P, 2 * _P, 4, 2048, 2048, 2048) == mm.MMRELU_ERR_INVALID_VALUE   # row too long for it
    assert v(-1, _P, 2 * _P, 4, 8, 8, 8) == mm.MMRELU_ERR_INVALID_VALUE
    r = mm.mmrelu_row_sum_f32
    assert r(_P, 2 * _P, -1, 4, 4) == mm.MMRELU_ERR_INVALID_VALUE
    assert r(_P, 2 * _P, 4, 8, 4) == mm.MMRELU_ERR_INVALID_VALUE
    assert r(_P, 0, 4, 8, 8) == mm.MMRELU_ERR_NULL_POINTER
    assert r(0, 2 * _P, 4, 8, 8) == mm.MMRELU_ERR_NULL_POINTER
    assert r(_P, 2 * _P + 2, 4, 8, 8) == mm.MMRELU_ERR_MISALIGNED          # out is fp32
    assert mm.mmrelu_row_sum_bf16(_P + 1, 2 * _P, 4, 8, 8) == mm.MMRELU_ERR_MISALIGNED
    assert r(_P, 2 * _P, 0, 8, 8) == mm.MMRELU_OK


def test_planner_picks_gemv_for_one_column():
    for dt in (mm.DTYPE_F32, mm.DTYPE_BF16):
        for (M, K, lda) in ((8192, 8192, 8192), (1000, 77, 80), (1, 5, 5), (4097, 2049, 2049)):
            p = mm.mmrelu_plan(dt, M, 1, K, lda, 1, 1, cus=256)
            assert "gemv" in p["name"] and p["block_m"] == 4 and p["grid"] == (M + 3) // 4, p
        # two columns or more: not the gemv
        assert "gemv" not in mm.mmrelu_plan(dt, 8192, 2, 8192, 8192, 2, 2, cus=256)["name"]


def test_planner_cost_model_uses_skinny_tiles_where_large_tiles_idle_cus():
    """The K-split skinny tiles enter the cost model (relative costs fitted
    to measured times): small squares and long-K products with few output
    tiles take them, large squares keep the tile kernels."""
    plan = lambda dt, M, N, K: mm.mmrelu_plan(dt, M, N, K, K, N, N, cus=256)
    F, B = mm.DTYPE_F32, mm.DTYPE_BF16
    expect = {
        (F, 256, 256, 256): "skinny", (F, 512, 512, 8192): "skinny<float,32x32,ks2>",
        (F, 1024, 1024, 8192): "skinny<float,64x64,ks2>", (F, 128, 4096, 4096): "skinny<float,32x64,ks2>",
        (F, 256, 8192, 1024): "f32_mfma<64,64", (F, 4096, 4096, 4096): "f32_mfma<128,128",
        (B, 256, 256, 256): "skinny", (B, 512, 512, 8192): "skinny<bf16,32x32,ks2>",
        (B, 1024, 1024, 1024): "skinny<bf16,64x64,ks2>", (B, 4096, 128, 4096): "skinny<bf16,32x64,ks2>",
        (B, 128, 8192, 8192): "skinny<bf16,64x64,ks2>", (B, 256, 4096, 4096): "skinny<bf16,64x64,ks2>",
        (B, 256, 8192, 1024): "bf16_mfma<128,128", (B, 2048, 2048, 2048): "bf16_mfma<128,128",
        (B, 4096, 4096, 4096): "pingpong<256,256,64", (B, 8192, 8192, 8192): "pingpong<256,256,64",
        # the 256 x 256 grid would fill half the CUs: 128 x 256 ping-pong tiles
        (B, 1024, 8192, 8192): "pingpong<128,256,64", (B, 2048, 4096, 4096): "pingpong<128,256,64",
        (B, 4096, 2048, 4096): "pingpong<128,256,64", (B, 3072, 3072, 3072): "pingpong<256,256,64",
    }
    for (dt, M, N, K), want in expect.items():
        name = plan(dt, M, N, K)["name"]
        assert want in name, ((M, N, K), name)
    # unaligned layouts keep the tile kernels (the skinny ones need 16-byte rows)
    p = mm.mmrelu_plan(F, 512, 511, 8192, 8192, 511, 511, cus=256)
    assert "unaligned" in p["name"]

