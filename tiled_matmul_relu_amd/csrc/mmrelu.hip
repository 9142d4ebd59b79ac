// C-ABI layer of libmmrelu: argument checks, the planner (kernel variant,
// grid, wave quantisation over the compute units) and the launch on the
// caller's stream. Declarations and the full contract are in mmrelu.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/mmrelu.h"
#include "kernels.hpp"

namespace mmrelu {
namespace {

// Kernel tables in a fixed order (the variant index of the C-ABI).
constexpr int kNumF32 = 15;
constexpr int kNumBf16 = 19;
// Both tables: 0 the plain kernel; 1 the large aligned tile and 2 the large
// tile for any layout; 3 and 4 smaller tiles; 5 - 10 and 12 the skinny
// tiles; 11 the matrix-vector kernel; 13 and 14 the rest; bf16 15 - 18 the
// BM x 256 tiles for any layout (BM = 256, 224, 192, 160).
const Variant *const *f32_table()
{
    static const Variant *const t[kNumF32] = {variant_f32_simple(), variant_f32_mfma128(),
                                              variant_f32_mfma128_unaligned(), variant_f32_mfma64(),
                                              variant_f32_mfma64_unaligned(), variant_f32_skinny(1, 2, 1),
                                              variant_f32_skinny(2, 2, 1), variant_f32_skinny(4, 2, 2),
                                              variant_f32_skinny(2, 1, 2), variant_f32_skinny(2, 2, 2),
                                              variant_f32_skinny(2, 4, 2), variant_f32_gemv(),
                                              variant_f32_skinny(4, 4, 2), variant_f32_skinny(1, 4, 1),
                                              variant_f32_skinny(4, 1, 2)};
    return t;
}
const Variant *const *bf16_table()
{
    static const Variant *const t[kNumBf16] = {variant_bf16_simple(), variant_bf16_pingpong256(),
                                               variant_bf16_any(128), variant_bf16_pingpong128(),
                                               variant_bf16_mfma128(), variant_bf16_skinny(1, 2, 1),
                                               variant_bf16_skinny(2, 2, 1), variant_bf16_skinny(4, 2, 1),
                                               variant_bf16_skinny(2, 1, 2), variant_bf16_skinny(2, 2, 2),
                                               variant_bf16_skinny(2, 4, 2), variant_bf16_gemv(),
                                               variant_bf16_skinny(4, 4, 2), variant_bf16_any(64),
                                               variant_bf16_skinny(1, 4, 1), variant_bf16_realign(256),
                                               variant_bf16_realign(224), variant_bf16_realign(192),
                                               variant_bf16_realign(160)};
    return t;
}

constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1;
constexpr int64_t kMaxLd = int64_t{1} << 21;
constexpr int kDefaultCus = 256;

const Variant *variant_at(int dtype, int32_t v)
{
    if (dtype == MMRELU_DTYPE_F32 && v >= 0 && v < kNumF32) return f32_table()[v];
    if (dtype == MMRELU_DTYPE_BF16 && v >= 0 && v < kNumBf16) return bf16_table()[v];
    return nullptr;
}

int check_shape(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc)
{
    if (M < 0 || N < 0 || K < 0) return MMRELU_ERR_INVALID_VALUE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return MMRELU_ERR_INVALID_VALUE;
    if (lda < std::max<int64_t>(1, K) || ldb < std::max<int64_t>(1, N) || ldc < std::max<int64_t>(1, N))
        return MMRELU_ERR_INVALID_VALUE;
    if (lda > kMaxLd || ldb > kMaxLd || ldc > kMaxLd) return MMRELU_ERR_INVALID_VALUE;
    return MMRELU_OK;
}

int check_pointers(const void *A, const void *B, const void *C, int64_t M, int64_t N, int64_t K, size_t esize)
{
    if (M == 0 || N == 0) return MMRELU_OK;
    if (C == nullptr) return MMRELU_ERR_NULL_POINTER;
    if (K > 0 && (A == nullptr || B == nullptr)) return MMRELU_ERR_NULL_POINTER;
    auto misaligned = [esize](const void *p) { return (reinterpret_cast<uintptr_t>(p) % esize) != 0; };
    if (misaligned(C) || (K > 0 && (misaligned(A) || misaligned(B)))) return MMRELU_ERR_MISALIGNED;
    return MMRELU_OK;
}

// Compute-unit count of the current device, cached per device id.
int device_cus()
{
    static std::atomic<int> cache[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return kDefaultCus;
    }
    if (dev < 64) {
        int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
        (void)hipGetLastError();
        cus = kDefaultCus;
    }
    if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

bool layout_fits(const Variant *v, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                 const void *A, const void *B, const void *C)
{
    if (v->align_elems == 0) return true;
    const int64_t q = v->align_elems;
    if (N % q || K % q || lda % q || ldb % q || ldc % q) return false;
    auto al16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    return al16(A) && al16(B) && al16(C);
}

// Planner: the default variant for a dtype and shape. Candidates are the
// dtype's matrix-core kernels at two tile sizes that accept the layout; the
// pick minimises the estimated time of the busiest CU, ceil(tiles / CUs)
// full tiles of block_m x block_n outputs at the variant's measured relative
// cost per output (wave quantisation of the grid over the CUs). bf16
// layouts the 16-byte-vector kernels do not accept go to the any-layout
// matrix-core kernels (variants 2, 13 and 15 - 18); the plain tiled kernel
// (variant 0) is only reached through the _variant entry points.
// Pointers are taken as 16-byte aligned when null (planning without buffers).
int32_t choose_variant(int dtype, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                       const void *A, const void *B, const void *C, int32_t cus)
{
    static const int32_t f32_aligned[] = {1, 3}, f32_any[] = {2, 4}, bf16_aligned[] = {1, 4};
    const Variant *const *table = dtype == MMRELU_DTYPE_F32 ? f32_table() : bf16_table();
    // A single output column is a matrix-vector product: one read of A, one
    // wave per output (variant 11), whatever the layout.
    if (N == 1) return 11;
    const bool fits = layout_fits(table[1], N, K, lda, ldb, ldc, A, B, C);
    // Skinny M or N (<= 64): the product is bound by reading the large
    // operand once, and the skinny kernels spread that read over one
    // workgroup per 32 columns of B (skinny M: variants 5, 6, 7 for up to 16,
    // 32, 64 rows) or per 32 rows of A (skinny N: variants 8, 9, 10 for up to
    // 16, 32, 64 columns), with K split across eight waves. When both are
    // small, the smaller one decides.
    // At most 16 rows and a 64-column strip for every CU: 64-column strips
    // (fp32 variant 13, bf16 variant 14), which read whole lines of B per
    // row (bf16) and keep the strip count at or under twice the CUs.
    if (fits && (M <= 64 || N <= 64)) {
        int32_t v;
        if (M <= 64 && M <= N) v = M <= 16 ? 5 : M <= 32 ? 6 : 7;
        else v = N <= 16 ? 8 : N <= 32 ? 9 : 10;
        if (v == 5 && (N + 63) / 64 >= cus) v = dtype == MMRELU_DTYPE_BF16 ? 14 : 13;
        // fp32, at most 16 columns and a 64-row band for every CU: 64-row
        // bands (variant 14).
        if (v == 8 && dtype == MMRELU_DTYPE_F32 && (M + 63) / 64 >= cus) v = 14;
        if (layout_fits(table[v], N, K, lda, ldb, ldc, A, B, C)) return v;
    }
    const int32_t *cand = nullptr;
    if (dtype == MMRELU_DTYPE_F32) cand = fits ? f32_aligned : f32_any;
    else if (fits) cand = bf16_aligned;
    else {
        // bf16, any layout, on the matrix cores: 64 x 64 tiles (variant 13)
        // until the 128 x 128 grid gives three CUs in four a tile (more CUs
        // busy; measured: 1001^3 20.8 against 32.0 us on 128 x 128 tiles,
        // 1537^3 43.2 against 45.9, 1281^2 x 4097 87.4 against 107.9). Then
        // the candidate with the shortest estimate: 128 x 128 tiles (variant
        // 2, two workgroups per CU) or BM x 256 tiles (variants 15 - 18, BM =
        // 256, 224, 192, 160 rows, one workgroup per CU), estimated as the
        // busiest CU's tile count times a + b K (us). a and b were fitted to
        // back-to-back times of all six any-layout kernels on 30 shapes from
        // 1001^3 to 8191^3 on one MI355X: a tile costs a fixed part (its
        // start-up and epilogue) and a part per k, both smaller for fewer rows.
        // The rule takes 1.4% more time than the best kernel of each shape
        // summed over the 30 (the 256-row tiles alone: 5.4%); its worst picks
        // are 2049^2 x 255 (128 x 128 tiles, 17.6 us, where 64 x 64 ones take
        // 16.0), 1999^2 x 8191 (128 x 128, 206.7 against 188.3 on 192 rows)
        // and 3001^3 (160 rows, 88.1 against 80.6 on 192). Shorter tiles win
        // where the 256-row grid leaves CUs idle or a round part-filled:
        // 4607^2 x 999 76.0 us on 192 rows against 87.2 on 256, 4097^2 x 767
        // 60.0 on 160 against 70.4; 8191^3 and 4095^3 keep 256 rows.
        const int64_t tiles128 = ((M + 127) / 128) * ((N + 127) / 128);
        if (4 * tiles128 < 3 * static_cast<int64_t>(cus)) return 13;
        struct Candidate { int32_t variant; int64_t rows; double a, b; };
        static const Candidate cands[] = {{2, 0, 3.1, 0.0165},    {15, 256, 17.2, 0.0243}, {16, 224, 15.6, 0.0236},
                                          {17, 192, 14.2, 0.0225}, {18, 160, 12.3, 0.0227}};
        int32_t pick = -1;
        double pick_cost = 0.0;
        for (const Candidate &c : cands) {
            const int64_t tiles = c.rows == 0 ? tiles128 : ((M + c.rows - 1) / c.rows) * ((N + 255) / 256);
            const double per_cu = static_cast<double>((tiles + cus - 1) / cus);
            const double cost = per_cu * (c.a + c.b * static_cast<double>(K));
            if (pick < 0 || cost < pick_cost) {
                pick = c.variant;
                pick_cost = cost;
            }
        }
        return pick;
    }
    // Candidates: the dtype's two tile kernels, and with an aligned layout the
    // seven skinny tiles (variants 5 - 10 and 12), which split K over eight
    // waves and so keep every CU busy when the large tiles would leave most
    // of them idle. A tile kernel
    // with a single tile per CU runs four waves per CU and is latency-bound:
    // its estimate carries a factor 1.15 (measured: 1024 x 1024 x 8192 fp32,
    // 185 us on 64x64 tiles against 159 us on 32x64 skinny tiles).
    int32_t best = -1;
    double best_cost = 0.0;
    auto consider = [&](int32_t index, bool tile_kernel) {
        const Variant *v = table[index];
        if (!layout_fits(v, N, K, lda, ldb, ldc, A, B, C)) return;
        const int64_t tiles = ((M + v->block_m - 1) / v->block_m) * ((N + v->block_n - 1) / v->block_n);
        const int64_t per_cu = (tiles + cus - 1) / cus;
        double cost = static_cast<double>(per_cu) * v->block_m * v->block_n * v->rel_cost;
        if (tile_kernel && per_cu == 1) cost *= 1.15;
        if (best < 0 || cost < best_cost) {
            best = index;
            best_cost = cost;
        }
    };
    consider(cand[0], true);
    consider(cand[1], true);
    if (fits && dtype == MMRELU_DTYPE_BF16) consider(3, true);    // the 128 x 256 ping-pong tile
    if (fits) {
        for (int32_t v = 5; v <= 10; ++v) consider(v, false);
        consider(12, false);
    }
    if (best < 0) best = cand[0];
    return best;
}

int fill_plan(const Variant *v, int32_t index, int64_t M, int64_t N, int32_t cus, mmrelu_plan_t *out)
{
    mmrelu_plan_t p;
    std::memset(&p, 0, sizeof p);
    p.variant = index;
    p.block_m = v->block_m;
    p.block_n = v->block_n;
    p.block_k = v->block_k;
    p.threads = v->threads;
    p.wg_per_cu = v->wg_per_cu;
    p.cus = cus;
    p.tiles_m = (M + v->block_m - 1) / v->block_m;
    p.tiles_n = (N + v->block_n - 1) / v->block_n;
    p.grid = p.tiles_m * p.tiles_n;
    // one launch holds fewer than 2^32 work-items
    if (p.grid * v->threads >= (int64_t{1} << 32)) return MMRELU_ERR_INVALID_VALUE;
    if (p.grid > 0) {
        int rc = mmrelu_wave_quantization(p.grid, int64_t{cus} * v->wg_per_cu, &p.waves, &p.idle_slots_last);
        if (rc != MMRELU_OK) return rc;
    }
    std::snprintf(p.name, sizeof p.name, "%s", v->name);
    *out = p;
    return MMRELU_OK;
}

int run(int dtype, int32_t variant, int act, const void *A, const void *B, const void *bias, void *C, int64_t M,
        int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, void *stream)
{
    const size_t esize = dtype == MMRELU_DTYPE_F32 ? 4 : 2;
    if (act != MMRELU_ACT_RELU && act != MMRELU_ACT_GELU_TANH && act != MMRELU_ACT_NONE) return MMRELU_ERR_INVALID_VALUE;
    int rc = check_shape(M, N, K, lda, ldb, ldc);
    if (rc != MMRELU_OK) return rc;
    rc = check_pointers(A, B, C, M, N, K, esize);
    if (rc != MMRELU_OK) return rc;
    if (bias != nullptr && reinterpret_cast<uintptr_t>(bias) % esize != 0) return MMRELU_ERR_MISALIGNED;
    if (variant < 0) variant = choose_variant(dtype, M, N, K, lda, ldb, ldc, A, B, C, device_cus());
    const Variant *v = variant_at(dtype, variant);
    if (v == nullptr) return MMRELU_ERR_INVALID_VALUE;
    if (K > 0 && !layout_fits(v, N, K, lda, ldb, ldc, A, B, C)) return MMRELU_ERR_INVALID_VALUE;
    if (M == 0 || N == 0) return MMRELU_OK;
    mmrelu_plan_t plan;
    rc = fill_plan(v, variant, M, N, kDefaultCus, &plan);
    if (rc != MMRELU_OK) return rc;
    Problem p{A, B, C, static_cast<int32_t>(M), static_cast<int32_t>(N), static_cast<int32_t>(K), lda, ldb, ldc,
              bias, act};
    hipError_t e = v->launch(p, plan.grid, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MMRELU_OK : MMRELU_ERR_LAUNCH;
}

// General strides: A[i][k] = A[i*sam + k*sak], B[k][j] = B[k*sbk + j*sbn],
// C[i][j] = C[i*scm + j*scn]. The product that runs is row-major; operands
// and outputs not already in that layout go through the caller's workspace.
struct StridedPlan {
    bool swap = false;                // run C^T = B^T·A^T (C column-major, no bias)
    int64_t M = 0, N = 0, K = 0;      // of the row-major product that runs
    const void *x = nullptr;          // its left operand in the caller's memory, strides (xr, xc)
    const void *y = nullptr;          // its right operand, strides (yr, yc)
    int64_t xr = 0, xc = 0, yr = 0, yc = 0;
    bool pack_x = false, pack_y = false, temp_out = false;
    int64_t ldx = 1, ldy = 1, ldz = 1;
    size_t off_x = 0, off_y = 0, off_z = 0, bytes = 0;
};

bool mul_ok(int64_t a, int64_t b, int64_t &out) { return !__builtin_mul_overflow(a, b, &out); }

// Largest element offset (rows-1)*s_r + (cols-1)*s_c, or -1 on overflow.
int64_t extent(int64_t rows, int64_t cols, int64_t s_r, int64_t s_c)
{
    int64_t a = 0, b = 0, sum = 0;
    if (rows <= 0 || cols <= 0) return 0;
    if (!mul_ok(rows - 1, s_r, a) || !mul_ok(cols - 1, s_c, b) || __builtin_add_overflow(a, b, &sum)) return -1;
    return sum < (int64_t{1} << 60) ? sum : -1;
}

size_t round_up(size_t x, size_t q) { return (x + q - 1) / q * q; }

int plan_strided(int dtype, int act, const void *A, const void *B, const void *bias, const void *C, int64_t M,
                 int64_t N, int64_t K, int64_t sam, int64_t sak, int64_t sbk, int64_t sbn, int64_t scm, int64_t scn,
                 StridedPlan &p)
{
    if (dtype != MMRELU_DTYPE_F32 && dtype != MMRELU_DTYPE_BF16) return MMRELU_ERR_INVALID_VALUE;
    if (act != MMRELU_ACT_RELU && act != MMRELU_ACT_GELU_TANH && act != MMRELU_ACT_NONE) return MMRELU_ERR_INVALID_VALUE;
    const int64_t esize = dtype == MMRELU_DTYPE_F32 ? 4 : 2, q = 16 / esize;
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return MMRELU_ERR_INVALID_VALUE;
    if (sam < 0 || sak < 0 || sbk < 0 || sbn < 0 || scm < 1 || scn < 1) return MMRELU_ERR_INVALID_VALUE;
    if (extent(M, K, sam, sak) < 0 || extent(K, N, sbk, sbn) < 0 || extent(M, N, scm, scn) < 0)
        return MMRELU_ERR_INVALID_VALUE;
    // Distinct outputs at distinct addresses: rows (or columns) of C occupy
    // disjoint ranges.
    if (M > 1 && N > 1) {
        int64_t span_row = 0, span_col = 0;
        const bool rows_apart = mul_ok(scn, N, span_row) && scm >= span_row;
        const bool cols_apart = mul_ok(scm, M, span_col) && scn >= span_col;
        if (!rows_apart && !cols_apart) return MMRELU_ERR_INVALID_VALUE;
    }
    int rc = check_pointers(A, B, C, M, N, K, static_cast<size_t>(esize));
    if (rc != MMRELU_OK) return rc;
    if (bias != nullptr && reinterpret_cast<uintptr_t>(bias) % esize != 0) return MMRELU_ERR_MISALIGNED;

    p = StridedPlan{};
    if (M == 0 || N == 0) return MMRELU_OK;
    auto al16 = [](const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; };
    // A matrix is taken as it is when it is row-major with a leading dimension
    // the kernels accept; when the product's K and N allow the 16-byte-vector
    // kernels, also only if it does not keep them out (ld and pointer aligned).
    auto usable = [&](const void *ptr, int64_t r, int64_t c, int64_t cols, bool dims_aligned) {
        if (c != 1 || r < std::max<int64_t>(1, cols) || r > kMaxLd) return false;
        return !dims_aligned || (r % q == 0 && al16(ptr));
    };
    const bool aligned_mn = K % q == 0 && N % q == 0, aligned_nm = K % q == 0 && M % q == 0;
    // One way of running the call (swap or not, C in place or through a
    // row-major temporary of leading dimension ldz) and its workspace layout.
    auto build = [&](bool swap, bool temp_out, int64_t ldz) {
        StridedPlan c;
        c.swap = swap;
        c.temp_out = temp_out;
        c.ldz = ldz;
        if (swap) {
            c.M = N; c.N = M; c.K = K;
            c.x = B; c.xr = sbn; c.xc = sbk;            // B^T[j][k] = B[k][j]
            c.y = A; c.yr = sak; c.yc = sam;            // A^T[k][i] = A[i][k]
        } else {
            c.M = M; c.N = N; c.K = K;
            c.x = A; c.xr = sam; c.xc = sak;
            c.y = B; c.yr = sbk; c.yc = sbn;
        }
        const bool dims_aligned = c.K % q == 0 && c.N % q == 0;
        if (c.K > 0) {
            if (usable(c.x, c.xr, c.xc, c.K, dims_aligned)) {
                c.ldx = c.xr;
            } else {
                c.pack_x = true;
                c.ldx = static_cast<int64_t>(round_up(static_cast<size_t>(c.K), static_cast<size_t>(q)));
            }
            if (usable(c.y, c.yr, c.yc, c.N, dims_aligned)) {
                c.ldy = c.yr;
            } else {
                c.pack_y = true;
                c.ldy = static_cast<int64_t>(round_up(static_cast<size_t>(c.N), static_cast<size_t>(q)));
            }
        } else {
            c.ldx = 1;
            c.ldy = std::max<int64_t>(1, c.N);
        }
        size_t off = 0;
        auto take = [&](bool used, int64_t rows, int64_t ld, size_t &at) {
            if (!used) return;
            at = off;
            off += round_up(static_cast<size_t>(rows) * static_cast<size_t>(ld) * static_cast<size_t>(esize), 256);
        };
        take(c.pack_x, c.M, c.ldx, c.off_x);
        take(c.pack_y, c.K, c.ldy, c.off_y);
        take(c.temp_out, c.M, c.ldz, c.off_z);
        c.bytes = off;
        return c;
    };
    const int64_t ld_temp = static_cast<int64_t>(round_up(static_cast<size_t>(N), static_cast<size_t>(q)));
    if (usable(C, scm, scn, N, aligned_mn)) {
        p = build(false, false, scm);
    } else {
        // C not row-major: through a row-major temporary, or (no bias, C
        // column-major) as C^T = B^T·A^T in place; the route that copies
        // fewer bytes through the workspace.
        p = build(false, true, ld_temp);
        if (bias == nullptr && usable(C, scn, scm, M, aligned_nm)) {
            const StridedPlan sw = build(true, false, scn);
            if (sw.bytes <= p.bytes) p = sw;
        }
    }
    if (p.ldx > kMaxLd || p.ldy > kMaxLd || p.ldz > kMaxLd) return MMRELU_ERR_INVALID_VALUE;
    return check_shape(p.M, p.N, p.K, p.ldx, p.ldy, p.ldz);
}

int run_strided(int dtype, int act, const void *A, const void *B, const void *bias, void *C, int64_t M, int64_t N,
                int64_t K, int64_t sam, int64_t sak, int64_t sbk, int64_t sbn, int64_t scm, int64_t scn,
                void *workspace, size_t workspace_bytes, void *stream)
{
    StridedPlan p;
    int rc = plan_strided(dtype, act, A, B, bias, C, M, N, K, sam, sak, sbk, sbn, scm, scn, p);
    if (rc != MMRELU_OK) return rc;
    if (M == 0 || N == 0) return MMRELU_OK;
    if (p.bytes > 0) {
        if (workspace == nullptr) return MMRELU_ERR_NULL_POINTER;
        if (workspace_bytes < p.bytes) return MMRELU_ERR_INVALID_VALUE;
        if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return MMRELU_ERR_MISALIGNED;
    }
    const int esize = dtype == MMRELU_DTYPE_F32 ? 4 : 2;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const void *x = p.pack_x ? ws + p.off_x : p.x;
    const void *y = p.pack_y ? ws + p.off_y : p.y;
    void *z = p.temp_out ? ws + p.off_z : C;
    if (p.pack_x && launch_pack(esize, p.x, ws + p.off_x, p.M, p.K, p.xr, p.xc, p.ldx, 1, s) != hipSuccess)
        return MMRELU_ERR_LAUNCH;
    if (p.pack_y && launch_pack(esize, p.y, ws + p.off_y, p.K, p.N, p.yr, p.yc, p.ldy, 1, s) != hipSuccess)
        return MMRELU_ERR_LAUNCH;
    rc = run(dtype, -1, act, x, y, bias, z, p.M, p.N, p.K, p.ldx, p.ldy, p.ldz, stream);
    if (rc != MMRELU_OK) return rc;
    if (p.temp_out && launch_pack(esize, ws + p.off_z, C, M, N, p.ldz, 1, scm, scn, s) != hipSuccess)
        return MMRELU_ERR_LAUNCH;
    return MMRELU_OK;
}

// Workspace of mmrelu_strided_static: a fixed array in device memory, one
// copy per device (created with the library's code object on that device and
// held until the process ends), so that the call allocates nothing. In host
// code `scratch` names a host-side stand-in: kernels and copies are given the
// device address that hipGetSymbolAddress returns for the current device.
constexpr size_t kStaticWorkspaceBytes = MMRELU_STATIC_WORKSPACE_BYTES;
static __device__ __align__(256) uint8_t scratch[kStaticWorkspaceBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_address[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of the current device's copy of `scratch`, looked up once
// per device (with that device current) and kept; null if HIP fails.
void *scratch_address()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    void *p = g_scratch_address[dev].load(std::memory_order_acquire);
    if (p != nullptr) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_address[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        void *q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_address[dev].store(q, std::memory_order_release);
        p = q;
    }
    return p;
}

// Row operations: shared argument checks. ld must cover the row and the
// largest offset must stay below 2^60.
int check_rows(const void *X, const void *Y, int64_t M, int64_t N, int64_t ldx, int64_t ldy, size_t esize_x,
               size_t esize_y)
{
    if (M < 0 || N < 0 || M > kMaxDim || N > kMaxDim) return MMRELU_ERR_INVALID_VALUE;
    if (ldx < std::max<int64_t>(1, N) || ldy < 1) return MMRELU_ERR_INVALID_VALUE;
    if (extent(M, N, ldx, 1) < 0 || extent(M, 1, ldy, 1) < 0) return MMRELU_ERR_INVALID_VALUE;
    if (M == 0) return MMRELU_OK;
    if (X == nullptr && N > 0) return MMRELU_ERR_NULL_POINTER;
    if (Y == nullptr) return MMRELU_ERR_NULL_POINTER;
    if (reinterpret_cast<uintptr_t>(X) % esize_x != 0 || reinterpret_cast<uintptr_t>(Y) % esize_y != 0)
        return MMRELU_ERR_MISALIGNED;
    return MMRELU_OK;
}

bool rows_vectorisable(const void *X, const void *Y, int64_t N, int64_t ldx, int64_t ldy, int64_t v)
{
    auto al16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    return N % v == 0 && ldx % v == 0 && ldy % v == 0 && al16(X) && al16(Y);
}

int softmax_rows(int esize, int variant, const void *X, void *Y, int64_t M, int64_t N, int64_t ldx, int64_t ldy,
                 void *stream)
{
    int rc = check_rows(X, Y, M, N, ldx, ldy, esize, esize);
    if (rc != MMRELU_OK) return rc;
    if (ldy < std::max<int64_t>(1, N) || extent(M, N, ldy, 1) < 0) return MMRELU_ERR_INVALID_VALUE;
    if (X == Y && ldx != ldy) return MMRELU_ERR_INVALID_VALUE;       // in place: the same layout
    const bool vec = rows_vectorisable(X, Y, N, ldx, ldy, 16 / esize);
    if (variant < 0) {
        variant = 4;
        if (vec) {
            variant = 3;
            for (int v = 2; v >= 0; --v)
                if (N <= softmax_capacity(v, esize)) variant = v;
        }
    } else if (variant >= kSoftmaxVariants || (variant < 4 && !vec) || N > softmax_capacity(variant, esize)) {
        return MMRELU_ERR_INVALID_VALUE;
    }
    if (M == 0 || N == 0) return MMRELU_OK;
    return launch_softmax(esize, variant, X, Y, M, N, ldx, ldy, static_cast<hipStream_t>(stream)) == hipSuccess
               ? MMRELU_OK
               : MMRELU_ERR_LAUNCH;
}

int row_sum_rows(int esize, const void *X, float *out, int64_t M, int64_t N, int64_t ldx, void *stream)
{
    int rc = check_rows(X, out, M, N, ldx, 1, esize, 4);
    if (rc != MMRELU_OK) return rc;
    if (M == 0) return MMRELU_OK;
    const int64_t v = 16 / esize;
    const bool vec = N % v == 0 && ldx % v == 0 && (reinterpret_cast<uintptr_t>(X) & 15) == 0;
    return launch_row_sum(esize, vec, N <= 1024, X, out, M, N, ldx, static_cast<hipStream_t>(stream)) == hipSuccess
               ? MMRELU_OK
               : MMRELU_ERR_LAUNCH;
}

}  // namespace
}  // namespace mmrelu

using namespace mmrelu;

extern "C" {

int mmrelu_f32(const float *A, const float *B, float *C, int64_t M, int64_t N, int64_t K,
               int64_t lda, int64_t ldb, int64_t ldc, void *stream)
{
    return run(MMRELU_DTYPE_F32, -1, MMRELU_ACT_RELU, A, B, nullptr, C, M, N, K, lda, ldb, ldc, stream);
}

int mmrelu_bf16(const uint16_t *A, const uint16_t *B, uint16_t *C, int64_t M, int64_t N, int64_t K,
                int64_t lda, int64_t ldb, int64_t ldc, void *stream)
{
    return run(MMRELU_DTYPE_BF16, -1, MMRELU_ACT_RELU, A, B, nullptr, C, M, N, K, lda, ldb, ldc, stream);
}

int mmrelu_f32_variant(int32_t variant, const float *A, const float *B, float *C, int64_t M, int64_t N,
                       int64_t K, int64_t lda, int64_t ldb, int64_t ldc, void *stream)
{
    if (variant < 0) return MMRELU_ERR_INVALID_VALUE;
    return run(MMRELU_DTYPE_F32, variant, MMRELU_ACT_RELU, A, B, nullptr, C, M, N, K, lda, ldb, ldc, stream);
}

int mmrelu_bf16_variant(int32_t variant, const uint16_t *A, const uint16_t *B, uint16_t *C, int64_t M,
                        int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, void *stream)
{
    if (variant < 0) return MMRELU_ERR_INVALID_VALUE;
    return run(MMRELU_DTYPE_BF16, variant, MMRELU_ACT_RELU, A, B, nullptr, C, M, N, K, lda, ldb, ldc, stream);
}

int mmrelu_fused_f32(int act, const float *A, const float *B, const float *bias, float *C, int64_t M, int64_t N,
                     int64_t K, int64_t lda, int64_t ldb, int64_t ldc, void *stream)
{
    return run(MMRELU_DTYPE_F32, -1, act, A, B, bias, C, M, N, K, lda, ldb, ldc, stream);
}

int mmrelu_fused_bf16(int act, const uint16_t *A, const uint16_t *B, const uint16_t *bias, uint16_t *C, int64_t M,
                      int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, void *stream)
{
    return run(MMRELU_DTYPE_BF16, -1, act, A, B, bias, C, M, N, K, lda, ldb, ldc, stream);
}

int mmrelu_fused_f32_variant(int32_t variant, int act, const float *A, const float *B, const float *bias, float *C,
                             int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, void *stream)
{
    if (variant < 0) return MMRELU_ERR_INVALID_VALUE;
    return run(MMRELU_DTYPE_F32, variant, act, A, B, bias, C, M, N, K, lda, ldb, ldc, stream);
}

int mmrelu_fused_bf16_variant(int32_t variant, int act, const uint16_t *A, const uint16_t *B, const uint16_t *bias,
                              uint16_t *C, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                              void *stream)
{
    if (variant < 0) return MMRELU_ERR_INVALID_VALUE;
    return run(MMRELU_DTYPE_BF16, variant, act, A, B, bias, C, M, N, K, lda, ldb, ldc, stream);
}

int mmrelu_strided_workspace_size(int dtype, int act, const void *A, const void *B, const void *bias, const void *C,
                                  int64_t M, int64_t N, int64_t K, int64_t sam, int64_t sak, int64_t sbk,
                                  int64_t sbn, int64_t scm, int64_t scn, size_t *bytes)
{
    if (bytes == nullptr) return MMRELU_ERR_NULL_POINTER;
    StridedPlan p;
    const int rc = plan_strided(dtype, act, A, B, bias, C, M, N, K, sam, sak, sbk, sbn, scm, scn, p);
    *bytes = rc == MMRELU_OK ? p.bytes : 0;
    return rc;
}

int mmrelu_strided_f32(int act, const float *A, const float *B, const float *bias, float *C, int64_t M, int64_t N,
                       int64_t K, int64_t sam, int64_t sak, int64_t sbk, int64_t sbn, int64_t scm, int64_t scn,
                       void *workspace, size_t workspace_bytes, void *stream)
{
    return run_strided(MMRELU_DTYPE_F32, act, A, B, bias, C, M, N, K, sam, sak, sbk, sbn, scm, scn, workspace,
                       workspace_bytes, stream);
}

int mmrelu_strided_bf16(int act, const uint16_t *A, const uint16_t *B, const uint16_t *bias, uint16_t *C, int64_t M,
                        int64_t N, int64_t K, int64_t sam, int64_t sak, int64_t sbk, int64_t sbn, int64_t scm,
                        int64_t scn, void *workspace, size_t workspace_bytes, void *stream)
{
    return run_strided(MMRELU_DTYPE_BF16, act, A, B, bias, C, M, N, K, sam, sak, sbk, sbn, scm, scn, workspace,
                       workspace_bytes, stream);
}

int mmrelu_strided_static(int dtype, int act, const void *A, const void *B, const void *bias, void *C, int64_t M,
                          int64_t N, int64_t K, int64_t sam, int64_t sak, int64_t sbk, int64_t sbn, int64_t scm,
                          int64_t scn, void *stream)
{
    StridedPlan p;
    const int rc = plan_strided(dtype, act, A, B, bias, C, M, N, K, sam, sak, sbk, sbn, scm, scn, p);
    if (rc != MMRELU_OK) return rc;
    if (p.bytes > kStaticWorkspaceBytes) return MMRELU_ERR_WORKSPACE_LIMIT;
    void *ws = nullptr;
    if (p.bytes > 0 && M > 0 && N > 0) {
        ws = scratch_address();
        if (ws == nullptr) return MMRELU_ERR_LAUNCH;
    }
    return run_strided(dtype, act, A, B, bias, C, M, N, K, sam, sak, sbk, sbn, scm, scn, ws, kStaticWorkspaceBytes,
                       stream);
}

int mmrelu_softmax_rows_f32(const float *X, float *Y, int64_t M, int64_t N, int64_t ldx, int64_t ldy, void *stream)
{
    return softmax_rows(4, -1, X, Y, M, N, ldx, ldy, stream);
}

int mmrelu_softmax_rows_bf16(const uint16_t *X, uint16_t *Y, int64_t M, int64_t N, int64_t ldx, int64_t ldy,
                             void *stream)
{
    return softmax_rows(2, -1, X, Y, M, N, ldx, ldy, stream);
}

int mmrelu_softmax_rows_f32_variant(int32_t variant, const float *X, float *Y, int64_t M, int64_t N, int64_t ldx,
                                    int64_t ldy, void *stream)
{
    if (variant < 0) return MMRELU_ERR_INVALID_VALUE;
    return softmax_rows(4, variant, X, Y, M, N, ldx, ldy, stream);
}

int mmrelu_softmax_rows_bf16_variant(int32_t variant, const uint16_t *X, uint16_t *Y, int64_t M, int64_t N,
                                     int64_t ldx, int64_t ldy, void *stream)
{
    if (variant < 0) return MMRELU_ERR_INVALID_VALUE;
    return softmax_rows(2, variant, X, Y, M, N, ldx, ldy, stream);
}

int mmrelu_softmax_rows_variant(int dtype, int64_t N, int64_t ldx, int64_t ldy, int32_t *variant)
{
    if (variant == nullptr) return MMRELU_ERR_NULL_POINTER;
    if ((dtype != MMRELU_DTYPE_F32 && dtype != MMRELU_DTYPE_BF16) || N < 0 || ldx < std::max<int64_t>(1, N) ||
        ldy < std::max<int64_t>(1, N))
        return MMRELU_ERR_INVALID_VALUE;
    const int esize = dtype == MMRELU_DTYPE_F32 ? 4 : 2;
    const int64_t v = 16 / esize;
    int32_t choice = 4;
    if (N % v == 0 && ldx % v == 0 && ldy % v == 0) {
        choice = 3;
        for (int c = 2; c >= 0; --c)
            if (N <= softmax_capacity(c, esize)) choice = c;
    }
    *variant = choice;
    return MMRELU_OK;
}

int mmrelu_row_sum_f32(const float *X, float *out, int64_t M, int64_t N, int64_t ldx, void *stream)
{
    return row_sum_rows(4, X, out, M, N, ldx, stream);
}

int mmrelu_row_sum_bf16(const uint16_t *X, float *out, int64_t M, int64_t N, int64_t ldx, void *stream)
{
    return row_sum_rows(2, X, out, M, N, ldx, stream);
}

const char *mmrelu_status_string(int status)
{
    switch (status) {
    case MMRELU_OK: return "ok";
    case MMRELU_ERR_INVALID_VALUE: return "invalid value (size, leading dimension, variant or activation)";
    case MMRELU_ERR_NULL_POINTER: return "null pointer";
    case MMRELU_ERR_MISALIGNED: return "pointer not aligned to its element size";
    case MMRELU_ERR_LAUNCH: return "kernel launch failed";
    case MMRELU_ERR_WORKSPACE_LIMIT:
        return "the call needs more workspace than the library's fixed buffer (MMRELU_STATIC_WORKSPACE_BYTES) holds";
    default: return "unknown status";
    }
}

const char *mmrelu_version(void) { return "mmrelu 0.1 (gfx950)"; }

int mmrelu_num_variants(int dtype)
{
    if (dtype == MMRELU_DTYPE_F32) return kNumF32;
    if (dtype == MMRELU_DTYPE_BF16) return kNumBf16;
    return 0;
}

int mmrelu_wave_quantization(int64_t blocks, int64_t slots, int64_t *waves, int64_t *idle_last)
{
    if (blocks < 0 || slots < 1 || waves == nullptr || idle_last == nullptr) return MMRELU_ERR_INVALID_VALUE;
    const int64_t w = (blocks + slots - 1) / slots;
    *waves = w;
    *idle_last = w * slots - blocks;
    return MMRELU_OK;
}

int mmrelu_plan_variant(int dtype, int32_t variant, int64_t M, int64_t N, int64_t K, int64_t lda,
                        int64_t ldb, int64_t ldc, int32_t cus, mmrelu_plan_t *out)
{
    if (out == nullptr) return MMRELU_ERR_NULL_POINTER;
    int rc = check_shape(M, N, K, lda, ldb, ldc);
    if (rc != MMRELU_OK) return rc;
    const Variant *v = variant_at(dtype, variant);
    if (v == nullptr || cus < 0) return MMRELU_ERR_INVALID_VALUE;
    return fill_plan(v, variant, M, N, cus > 0 ? cus : device_cus(), out);
}

int mmrelu_plan(int dtype, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                int32_t cus, mmrelu_plan_t *out)
{
    if (dtype != MMRELU_DTYPE_F32 && dtype != MMRELU_DTYPE_BF16) return MMRELU_ERR_INVALID_VALUE;
    int rc = check_shape(M, N, K, lda, ldb, ldc);
    if (rc != MMRELU_OK) return rc;
    if (cus < 0) return MMRELU_ERR_INVALID_VALUE;
    const int32_t n_cus = cus > 0 ? cus : device_cus();
    return mmrelu_plan_variant(dtype, choose_variant(dtype, M, N, K, lda, ldb, ldc, nullptr, nullptr, nullptr, n_cus),
                               M, N, K, lda, ldb, ldc, n_cus, out);
}

}  // extern "C"
