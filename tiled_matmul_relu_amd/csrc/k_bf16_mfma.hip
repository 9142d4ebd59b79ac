// bf16 relu(A·B) on the gfx950 matrix cores (v_mfma_f32_16x16x32_bf16),
// fp32 accumulation, ReLU on the fp32 sum, then one rounding to bf16 (nearest,
// ties to even) in the store epilogue.
//
// The lecture's tiled recipe (one workgroup per output tile; K swept in slabs
// staged in on-chip memory; fp32 accumulator; ReLU on the accumulator right
// before the single, masked store), laid out for CDNA4:
//  * 256 x 256 output tile per workgroup of 4 wave64s (2 x 2); each wave owns
//    a 128 x 128 sub-tile: 64 16x16 MFMA blocks, 256 fp32 accumulators per
//    lane held in AGPRs (one wave per SIMD).
//  * K slabs of 64 are copied global -> LDS by the buffer unit directly (no
//    VGPR round trip), double-buffered, so slab k+1 is in flight while slab k
//    is multiplied. Lanes outside M, N or K get an out-of-range offset and the
//    hardware writes zeros into LDS (the lecture's masked load with other=0).
//  * A (M x K, K contiguous) is read as the second MFMA operand with one
//    ds_read_b128 per lane: 8 consecutive k of one row. A rows are XOR
//    swizzled in 16-byte chunks so 16 rows read at one chunk hit all banks.
//  * B (K x N, N contiguous) must reach each lane as 8 consecutive k of one
//    column. It stays row-major in LDS and is read with ds_read_b64_tr_b16,
//    which transposes 16-bit elements across each 16-lane group: lane t of a
//    group receives element t%4 of the 8-byte rows addressed by lanes
//    4e + t/4, e = 0..3. Lane s therefore addresses row k0 + s/4, columns
//    4*(s%4) .. +3, and two such reads give the 8 k values of column t. B rows
//    are XOR swizzled so the 16 rows touched by one such read spread over
//    the banks.
//  * With B as the first MFMA operand, a lane's four accumulators are four
//    consecutive columns of one row of C: the epilogue writes 8 bytes a lane.
// Requires lda, ldb, ldc, K and N to be multiples of 8 and 16-byte aligned
// pointers (rows start on 16-byte boundaries).
#include "kernels.hpp"
#include "device_common.hpp"
#include "../../include/mmrelu.h"

namespace mmrelu {
namespace {

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N>
struct Bf16Tile {
    static constexpr int kWaves = WAVES_M * WAVES_N;
    static constexpr int kThreads = kWaves * 64;
    static constexpr int WTM = BM / WAVES_M;
    static constexpr int WTN = BN / WAVES_N;
    static constexpr int MB = WTM / 16;
    static constexpr int NB = WTN / 16;
    static constexpr int CA = BK / 8;   // 16-byte chunks per A row
    static constexpr int CB = BN / 8;   // 16-byte chunks per B row
    static constexpr int kStageA = BM * BK;          // elements
    static constexpr int kStage = BM * BK + BK * BN; // elements per stage
    static_assert(CA == 8, "A rows are 128 bytes: 8 chunks");
    static_assert(CB >= 16 && (CB & (CB - 1)) == 0, "B row chunk count");
    static_assert(BK % 32 == 0 && WTM % 16 == 0 && WTN % 16 == 0, "tile shape");
    static_assert((BM * CA) % (64 * kWaves) == 0 && (BK * CB) % (64 * kWaves) == 0, "load split");
    static constexpr int kLoadsA = (BM * CA) / (64 * kWaves);
    static constexpr int kLoadsB = (BK * CB) / (64 * kWaves);
};

// A: 16 consecutive rows read at one logical chunk hit distinct banks.
__device__ inline int swz_a(int r) { return (r & 7) ^ ((r >> 3) & 1); }
// B: the transposed reads of one wave touch rows k0 + {0..3} (+8, +16, +24)
// in 32-byte segments; XOR moves the four rows of a 16-lane group to distinct
// 32-byte segments and the next group's rows 128 bytes further.
__device__ inline int swz_b(int k) { return ((k & 3) << 1) | (((k >> 3) & 1) << 3); }

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64, 1) void mmrelu_bf16_mfma(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, uint16_t *__restrict__ C,
    int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc, int tiles_m, int tiles_n, int group_m)
{
    using T = Bf16Tile<BM, BN, BK, WAVES_M, WAVES_N>;
    __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * T::kStage];

    const int lane = threadIdx.x & 63;
    // wave index as a scalar, so LDS destinations of the copies are uniform
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int g = lane >> 4, t = lane & 15;

    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const rsrc_t ra = make_rsrc(A + static_cast<int64_t>(m0) * lda, ((static_cast<int64_t>(M) - 1 - m0) * lda + K) * 2);
    const bool full_mn = (m0 + BM <= M) && (n0 + BN <= N);
    const uint32_t lds0 = lds_address(lds);

    // Global -> LDS copy plan. Copy q of this wave fills the 1 KB LDS block
    // blk = q * waves + wave of the A (or B) part of a stage; lane l of it
    // holds one 16-byte chunk. Per-lane byte offsets exclude the K position
    // (A: added as a uniform offset; B: the resource is rebased every slab).
    uint32_t a_voff[T::kLoadsA], b_voff[T::kLoadsB];
    int a_row[T::kLoadsA], a_col[T::kLoadsA], b_row[T::kLoadsB], b_col[T::kLoadsB];
#pragma unroll
    for (int q = 0; q < T::kLoadsA; ++q) {
        const int blk = q * T::kWaves + wave;
        const int row = blk * (64 / T::CA) + lane / T::CA;
        a_row[q] = row;
        a_col[q] = ((lane % T::CA) ^ swz_a(row)) * 8;
        a_voff[q] = static_cast<uint32_t>((row * lda + a_col[q]) * 2);
    }
#pragma unroll
    for (int q = 0; q < T::kLoadsB; ++q) {
        const int blk = q * T::kWaves + wave;
        const int row = blk * (64 / T::CB) + lane / T::CB;
        b_row[q] = row;
        b_col[q] = ((lane % T::CB) ^ swz_b(row)) * 8;
        b_voff[q] = static_cast<uint32_t>((row * ldb + b_col[q]) * 2);
    }

    auto issue_loads = [&](int stage, int k0) {
        const rsrc_t rb = make_rsrc(B + static_cast<int64_t>(k0) * ldb + n0,
                                    ((static_cast<int64_t>(K) - 1 - k0) * ldb + N - n0) * 2);
        const uint32_t a_soff = static_cast<uint32_t>(k0) * 2;
        const uint32_t la = lds0 + stage * (T::kStage * 2);
        const uint32_t lb = la + T::kStageA * 2;
        if (full_mn && k0 + BK <= K) {
#pragma unroll
            for (int q = 0; q < T::kLoadsA; ++q)
                load_to_lds<16>(ra, la + (q * T::kWaves + wave) * 1024, a_voff[q], a_soff);
#pragma unroll
            for (int q = 0; q < T::kLoadsB; ++q)
                load_to_lds<16>(rb, lb + (q * T::kWaves + wave) * 1024, b_voff[q]);
        } else {
#pragma unroll
            for (int q = 0; q < T::kLoadsA; ++q) {
                const bool ok = (m0 + a_row[q] < M) && (k0 + a_col[q] < K);
                load_to_lds<16>(ra, la + (q * T::kWaves + wave) * 1024, ok ? a_voff[q] : kOutOfRange, a_soff);
            }
#pragma unroll
            for (int q = 0; q < T::kLoadsB; ++q) {
                const bool ok = (k0 + b_row[q] < K) && (n0 + b_col[q] < N);
                load_to_lds<16>(rb, lb + (q * T::kWaves + wave) * 1024, ok ? b_voff[q] : kOutOfRange);
            }
        }
    };

    // Fragment read plan (element offsets into a stage). A: the row of block
    // i is wm*WTM + 16i + t, so its swizzle depends on t only and block i is a
    // constant 16*BK further; the two 32-wide k halves differ in chunk bit 2.
    // B: lane t of group g addresses row 8g + t/4 (+32ks + 4h, constants; the
    // swizzle depends on the row only through t/4 and g) and columns
    // wn*WTN + 16j + 4(t%4) .. +3; one base per block j.
    int a_off[BK / 32], b_off[T::NB];
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks)
        a_off[ks] = (wm * T::WTM + t) * BK + (((ks * 4 + g) ^ swz_a(t)) << 3);
    {
        const int k_lane = 8 * g + (t >> 2);
#pragma unroll
        for (int j = 0; j < T::NB; ++j) {
            const int n = wn * T::WTN + j * 16 + 4 * (t & 3);
            b_off[j] = T::kStageA + k_lane * BN + (((n >> 3) ^ swz_b(k_lane)) << 3) + (n & 7);
        }
    }

    f32x4 acc[T::MB][T::NB];
#pragma unroll
    for (int i = 0; i < T::MB; ++i)
#pragma unroll
        for (int j = 0; j < T::NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (K + BK - 1) / BK;
    if (nk > 0) {
        issue_loads(0, 0);
        wait_vmcnt<0>();
        __syncthreads();
    }
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) issue_loads(cur ^ 1, (kt + 1) * BK);
        const uint16_t *st = lds + cur * T::kStage;
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            bf16x8 bv[T::NB];
#pragma unroll
            for (int j = 0; j < T::NB; ++j) {
                i16x4 half[2];
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    half[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (MMRELU_LDS i16x4 *)(st + b_off[j] + (ks * 32 + 4 * h) * BN));
                bv[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
            }
#pragma unroll
            for (int i = 0; i < T::MB; ++i) {
                const bf16x8 av = *reinterpret_cast<const bf16x8 *>(st + a_off[ks] + i * 16 * BK);
#pragma unroll
                for (int j = 0; j < T::NB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv[j], av, acc[i][j], 0, 0, 0);
            }
        }
        wait_vmcnt<0>();
        __syncthreads();
    }

    // Epilogue: lane (g, t) of block (i, j) holds C[row][col .. col+3]; ReLU
    // on fp32, round to bf16, one 8-byte masked store.
    const __amdgpu_buffer_rsrc_t rc = make_store_rsrc(C + static_cast<int64_t>(m0) * ldc + n0,
                                                      ((static_cast<int64_t>(M) - 1 - m0) * ldc + N - n0) * 2);
#pragma unroll
    for (int i = 0; i < T::MB; ++i) {
        const int row = wm * T::WTM + i * 16 + t;
#pragma unroll
        for (int j = 0; j < T::NB; ++j) {
            const int col = wn * T::WTN + j * 16 + 4 * g;
            const f32x4 v = acc[i][j];
            bf16x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = static_cast<__bf16>(__builtin_fmaxf(v[r], 0.0f));
            const uint32_t off =
                (m0 + row < M && n0 + col < N) ? static_cast<uint32_t>((row * ldc + col) * 2) : kOutOfRange;
            store_b64(rc, off, __builtin_bit_cast(u32x2, o));
        }
    }
}

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int GROUP_M>
hipError_t launch_bf16(const Problem &p, int64_t grid, hipStream_t stream)
{
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    hipLaunchKernelGGL((mmrelu_bf16_mfma<BM, BN, BK, WAVES_M, WAVES_N>), dim3(static_cast<uint32_t>(grid)),
                       dim3(WAVES_M * WAVES_N * 64), 0, stream, static_cast<const uint16_t *>(p.A),
                       static_cast<const uint16_t *>(p.B), static_cast<uint16_t *>(p.C), p.M, p.N, p.K, p.lda,
                       p.ldb, p.ldc, tiles_m, tiles_n, GROUP_M);
    return hipGetLastError();
}

}  // namespace

const Variant *variant_bf16_mfma256()
{
    static const Variant v = {"mmrelu_bf16_mfma<256,256,64,2,2>", MMRELU_DTYPE_BF16, 256, 256, 64, 256, 1, 8,
                              launch_bf16<256, 256, 64, 2, 2, 4>};
    return &v;
}

}  // namespace mmrelu
