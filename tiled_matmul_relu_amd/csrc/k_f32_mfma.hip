// fp32 relu(A·B) on the gfx950 matrix cores (v_mfma_f32_16x16x4_f32): fp32
// products accumulated in fp32 (no reduced-precision inputs). The epilogue
// adds the optional per-column bias and applies the activation (ReLU by
// default, GeLU's tanh form, or none) before the one store.
//
// The lecture's tiled recipe (one workgroup per output tile; K swept in slabs
// staged in on-chip memory; fp32 accumulator; the activation on the
// accumulator right before the single, masked store), laid out for CDNA4:
//  * A BM x BN tile per workgroup of WAVES_M x WAVES_N wave64s; each wave owns
//    a (BM/WAVES_M) x (BN/WAVES_N) sub-tile held in MFMA accumulators.
//  * K slabs are copied global -> LDS by the buffer unit directly (no VGPR
//    round trip), double-buffered: slab k+1 is in flight while slab k is
//    multiplied. Lanes outside M, N or K are given an out-of-range offset and
//    the hardware writes zeros into LDS (the lecture's masked load with
//    other=0), so the interior needs no branches.
//  * Within one 16-wide k step a lane of group g (lanes 16g..16g+15) takes
//    k = 4g + s in its s-th MFMA (any assignment works if both operands use
//    it), so its A operand for four MFMAs is one ds_read_b128 of 4
//    consecutive k of one row; the B operand is one dword per MFMA from a
//    row of B. LDS rows are XOR-swizzled in 16-byte chunks so both reads
//    spread over all banks.
//  * The MFMA operands are swapped (B slab as the first operand), so each
//    lane's four accumulators are four consecutive columns of one row of C
//    and the epilogue stores 16 bytes per lane.
// ALIGNED requires 16-byte aligned rows (lda, ldb, ldc, K, N multiples of 4
// and 16-byte aligned pointers). The unaligned instances take any shape and
// leading dimension: they copy 4 bytes a lane with every element masked and
// store element by element, except that the 64 x 64 one (kStaged) copies a
// slab of a tile wholly inside M, N and K 16 bytes a lane (a buffer load of a
// dword or more needs only 4-byte alignment, and no such copy can reach the
// end of its operand) and stages its output tile in LDS to store whole rows
// with the widest stores each row's alignment allows. Measured against the
// plain form, same process, bit-identical: 64 x 64 tiles 4097x3001x2049
// 439 -> 431 us, 2049^3 207 -> 204.5, 1025^3 57.3 -> 54.2; 128 x 128 tiles
// 4097x3001x2049 600 -> 590 but 4095^3 1261 -> 1291 and 3001^3 672 -> 705,
// so those keep the plain form.
#include "kernels.hpp"
#include "device_common.hpp"
#include "../../include/mmrelu.h"

namespace mmrelu {
namespace {

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, bool ALIGNED>
struct F32Tile {
    static constexpr int kWaves = WAVES_M * WAVES_N;
    static constexpr int kThreads = kWaves * 64;
    static constexpr int WTM = BM / WAVES_M;   // wave sub-tile rows
    static constexpr int WTN = BN / WAVES_N;   // wave sub-tile cols
    static constexpr int MB = WTM / 16;        // 16x16 MFMA blocks per wave, along m
    static constexpr int NB = WTN / 16;        // ... along n
    static constexpr int CA = BK / 4;          // 16-byte chunks per A row in LDS
    static constexpr int CB = BN / 4;          // 16-byte chunks per B row in LDS
    static constexpr int kStageA = BM * BK;    // floats
    static constexpr int kStage = BM * BK + BK * BN;
    // bytes one lane copies per load, and loads per wave per slab
    static constexpr int kLaneBytes = ALIGNED ? 16 : 4;
    static constexpr int kLoadsA = (BM * BK * 4) / (kLaneBytes * 64 * kWaves);
    static constexpr int kLoadsB = (BK * BN * 4) / (kLaneBytes * 64 * kWaves);
    // 16-byte copies per wave per slab (the aligned plan), which the
    // unaligned instance also uses for slabs of whole tiles inside K
    static constexpr int kLoadsAW = (BM * BK * 4) / (16 * 64 * kWaves);
    static constexpr int kLoadsBW = (BK * BN * 4) / (16 * 64 * kWaves);
    static constexpr bool kStaged = !ALIGNED && BM == 64;
    static_assert(CA == 8, "A rows are 128 bytes: 8 chunks");
    static_assert(CB >= 16 && (CB & (CB - 1)) == 0, "B row chunk count");
    static_assert(BK % 16 == 0 && WTM % 16 == 0 && WTN % 16 == 0, "tile shape");
    static_assert(kLoadsA * kLaneBytes * 64 * kWaves == BM * BK * 4, "A load split");
    static_assert(kLoadsB * kLaneBytes * 64 * kWaves == BK * BN * 4, "B load split");
};

// A: row r's chunk c sits at c ^ (r % 8); the 16 lanes of a ds_read_b128
// that read one logical chunk of 16 consecutive rows then run at the full
// LDS rate (measured on gfx950).
__device__ inline int swz_a(int r) { return r & 7; }
// B: row k's chunk c sits at c ^ swz_b(k); the four rows k, k+4, k+8, k+12
// read together by one ds_read_b32 land in different 64-byte quarters.
__device__ inline int swz_b(int k) { return ((k >> 2) & 3) << 2; }

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, bool ALIGNED>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64, 2) void mmrelu_f32_mfma(
    const float *__restrict__ A, const float *__restrict__ B, float *__restrict__ C,
    int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc, int tiles_m, int tiles_n, int group_m,
    const float *__restrict__ bias, int act)
{
    using T = F32Tile<BM, BN, BK, WAVES_M, WAVES_N, ALIGNED>;
    __shared__ __attribute__((aligned(1024))) float lds[2 * T::kStage];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int g = lane >> 4, t = lane & 15;

    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const rsrc_t ra = make_rsrc(A + static_cast<int64_t>(m0) * lda, ((static_cast<int64_t>(M) - 1 - m0) * lda + K) * 4);
    const bool full_mn = (m0 + BM <= M) && (n0 + BN <= N);
    const uint32_t lds0 = lds_address(lds);

    // Copy plan. Copy q of this wave fills LDS block blk = q * waves + wave
    // (64 lanes x kLaneBytes) of the A (or B) part of a stage. Each lane's
    // destination is fixed by its position, so the swizzle is applied to the
    // source: the lane fetches the element whose swizzled home is its slot.
    uint32_t a_voff[T::kLoadsA], b_voff[T::kLoadsB];
    int a_row[T::kLoadsA], a_col[T::kLoadsA], b_row[T::kLoadsB], b_col[T::kLoadsB];
#pragma unroll
    for (int q = 0; q < T::kLoadsA; ++q) {
        const int blk = q * T::kWaves + wave;
        int row, col;
        if (ALIGNED) {
            row = blk * (64 / T::CA) + lane / T::CA;
            col = ((lane % T::CA) ^ swz_a(row)) * 4;
        } else {
            const int d = blk * 64 + lane;  // float index within the A part of a stage
            row = d / BK;
            const int pd = d % BK;
            col = (((pd >> 2) ^ swz_a(row)) << 2) | (pd & 3);
        }
        a_row[q] = row;
        a_col[q] = col;
        a_voff[q] = static_cast<uint32_t>((row * lda + col) * 4);
    }
#pragma unroll
    for (int q = 0; q < T::kLoadsB; ++q) {
        const int blk = q * T::kWaves + wave;
        int row, col;
        if (ALIGNED) {
            row = blk * (64 / T::CB) + lane / T::CB;
            col = ((lane % T::CB) ^ swz_b(row)) * 4;
        } else {
            const int d = blk * 64 + lane;
            row = d / BN;
            const int pd = d % BN;
            col = (((pd >> 2) ^ swz_b(row)) << 2) | (pd & 3);
        }
        b_row[q] = row;
        b_col[q] = col;
        b_voff[q] = static_cast<uint32_t>((row * ldb + col) * 4);
    }

    // The staged instance's 16-byte plan: the aligned plan's offsets.
    uint32_t a_voffw[T::kLoadsAW], b_voffw[T::kLoadsBW];
    if constexpr (T::kStaged) {
#pragma unroll
        for (int q = 0; q < T::kLoadsAW; ++q) {
            const int row = (q * T::kWaves + wave) * (64 / T::CA) + lane / T::CA;
            a_voffw[q] = static_cast<uint32_t>((row * lda + ((lane % T::CA) ^ swz_a(row)) * 4) * 4);
        }
#pragma unroll
        for (int q = 0; q < T::kLoadsBW; ++q) {
            const int row = (q * T::kWaves + wave) * (64 / T::CB) + lane / T::CB;
            b_voffw[q] = static_cast<uint32_t>((row * ldb + ((lane % T::CB) ^ swz_b(row)) * 4) * 4);
        }
    }

    auto issue_loads = [&](int stage, int k0) {
        const rsrc_t rb = make_rsrc(B + static_cast<int64_t>(k0) * ldb + n0,
                                    ((static_cast<int64_t>(K) - 1 - k0) * ldb + N - n0) * 4);
        const uint32_t a_soff = static_cast<uint32_t>(k0) * 4;
        const uint32_t la = lds0 + stage * (T::kStage * 4);
        const uint32_t lb = la + T::kStageA * 4;
        constexpr int kBlk = 64 * T::kLaneBytes;
        if (ALIGNED && full_mn && k0 + BK <= K) {
#pragma unroll
            for (int q = 0; q < T::kLoadsA; ++q)
                load_to_lds<T::kLaneBytes>(ra, la + (q * T::kWaves + wave) * kBlk, a_voff[q], a_soff);
#pragma unroll
            for (int q = 0; q < T::kLoadsB; ++q)
                load_to_lds<T::kLaneBytes>(rb, lb + (q * T::kWaves + wave) * kBlk, b_voff[q]);
        } else if (T::kStaged && full_mn && k0 + BK <= K) {
            // Every row of the slab lies inside M (A) or K (B) and every
            // column inside K (A) or N (B), so each 16-byte copy ends at or
            // before its row's last element, inside its resource.
#pragma unroll
            for (int q = 0; q < T::kLoadsAW; ++q)
                load_to_lds<16>(ra, la + (q * T::kWaves + wave) * 1024, a_voffw[q], a_soff);
#pragma unroll
            for (int q = 0; q < T::kLoadsBW; ++q)
                load_to_lds<16>(rb, lb + (q * T::kWaves + wave) * 1024, b_voffw[q]);
        } else {
#pragma unroll
            for (int q = 0; q < T::kLoadsA; ++q) {
                const bool ok = (m0 + a_row[q] < M) && (k0 + a_col[q] < K);
                load_to_lds<T::kLaneBytes>(ra, la + (q * T::kWaves + wave) * kBlk, ok ? a_voff[q] : kOutOfRange,
                                           a_soff);
            }
#pragma unroll
            for (int q = 0; q < T::kLoadsB; ++q) {
                const bool ok = (k0 + b_row[q] < K) && (n0 + b_col[q] < N);
                load_to_lds<T::kLaneBytes>(rb, lb + (q * T::kWaves + wave) * kBlk, ok ? b_voff[q] : kOutOfRange);
            }
        }
    };

    // Fragment read plan (float offsets into a stage). A: block i's row is
    // wm*WTM + 16i + t, so the swizzle depends on t only and block i is a
    // constant 16*BK further; k steps ks differ in chunk bit 2. B: lane of
    // group g reads row ks*16 + 4g + s (the swizzle depends on g only) at
    // column wn*WTN + 16j + t; one base per block j, constants for ks and s.
    int a_off[BK / 16], b_off[T::NB];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks)
        a_off[ks] = (wm * T::WTM + t) * BK + (((ks * 4 + g) ^ swz_a(t)) << 2);
#pragma unroll
    for (int j = 0; j < T::NB; ++j) {
        const int n = wn * T::WTN + j * 16 + t;
        b_off[j] = T::kStageA + 4 * g * BN + (((n >> 2) ^ swz_b(4 * g)) << 2) + (n & 3);
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
        const float *st = lds + cur * T::kStage;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            float bv[T::NB][4];
#pragma unroll
            for (int j = 0; j < T::NB; ++j)
#pragma unroll
                for (int s = 0; s < 4; ++s) bv[j][s] = st[b_off[j] + (ks * 16 + s) * BN];
#pragma unroll
            for (int i = 0; i < T::MB; ++i) {
                const f32x4 av = *reinterpret_cast<const f32x4 *>(st + a_off[ks] + i * 16 * BK);
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int j = 0; j < T::NB; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(bv[j][s], av[s], acc[i][j], 0, 0, 0);
            }
        }
        wait_vmcnt<0>();
        __syncthreads();
    }

    // Epilogue: lane (g, t) of block (i, j) holds C[row][col .. col+3]; bias
    // and activation on the fp32 accumulators, one masked store.
    const __amdgpu_buffer_rsrc_t rc = make_store_rsrc(C + static_cast<int64_t>(m0) * ldc + n0,
                                                      ((static_cast<int64_t>(M) - 1 - m0) * ldc + N - n0) * 4);
    float bj[T::NB][4];   // the bias of the lane's columns, loaded once, only when there is one
    if (bias != nullptr) {
        const __amdgpu_buffer_rsrc_t rb = make_bias_rsrc(bias, n0, N, 4);
#pragma unroll
        for (int j = 0; j < T::NB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) bj[j][r] = bias_f32(rb, wn * T::WTN + j * 16 + 4 * g + r);
    } else {
#pragma unroll
        for (int j = 0; j < T::NB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) bj[j][r] = 0.0f;
    }
    if constexpr (!T::kStaged) {
        with_activation(act, [&](auto act_c) __attribute__((always_inline)) {
            constexpr int ACT = decltype(act_c)::value;
#pragma unroll
            for (int i = 0; i < T::MB; ++i) {
                const int row = wm * T::WTM + i * 16 + t;
                const bool row_ok = m0 + row < M;
#pragma unroll
                for (int j = 0; j < T::NB; ++j) {
                    const int col = wn * T::WTN + j * 16 + 4 * g;
                    f32x4 v = acc[i][j];
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = activate<ACT>(v[r] + bj[j][r]);
                    if (ALIGNED) {
                        const uint32_t off =
                            (row_ok && n0 + col < N) ? static_cast<uint32_t>((row * ldc + col) * 4) : kOutOfRange;
                        store_b128(rc, off, __builtin_bit_cast(u32x4, v));
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const uint32_t off = (row_ok && n0 + col + r < N)
                                                     ? static_cast<uint32_t>((row * ldc + col + r) * 4)
                                                     : kOutOfRange;
                            store_b32(rc, off, __float_as_uint(v[r]));
                        }
                    }
                }
            }
        });
    } else {
        // Staged: the tile goes to LDS (both stages are free after the
        // loop's last barrier), row r's 16-byte unit u (columns 4u .. 4u+3)
        // at float r BN + 4 ((u + r) % (BN/4)), and each wave stores whole
        // rows of it, BN/4 lanes a row: a row starting a (mod 4) floats past
        // a 16-byte boundary takes one 16-byte store per lane (a = 0), two
        // 8-byte ones (a = 2) or a 4-, an 8- and a 4-byte one (a odd). Stores
        // of single elements scattered over sixteen rows cost far more.
        // Lanes with columns past N store element by element, rows past M
        // nothing (kOutOfRange plus a few bytes is still past every range).
        constexpr int kUnits = BN / 4;
        constexpr int kRowsPerPass = 64 / kUnits;
        constexpr int kRowsPerWave = BM / T::kWaves;
        static_assert(BM * BN <= 2 * T::kStage, "the output tile fits in the stages");
        static_assert(kRowsPerWave % kRowsPerPass == 0, "whole passes");
        with_activation(act, [&](auto act_c) __attribute__((always_inline)) {
            constexpr int ACT = decltype(act_c)::value;
#pragma unroll
            for (int i = 0; i < T::MB; ++i) {
                const int row = wm * T::WTM + i * 16 + t;
#pragma unroll
                for (int j = 0; j < T::NB; ++j) {
                    const int u = wn * (T::WTN / 4) + j * 4 + g;
                    f32x4 v = acc[i][j];
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = activate<ACT>(v[r] + bj[j][r]);
                    *reinterpret_cast<f32x4 *>(lds + row * BN + 4 * ((u + row) & (kUnits - 1))) = v;
                }
            }
        });
        __syncthreads();
        const int rows = M - m0 < BM ? M - m0 : BM;
        const int ncols = N - n0;
        const int cu = lane & (kUnits - 1);
        const bool full_lane = 4 * cu + 3 < ncols;
        const int a0 = static_cast<int>(((reinterpret_cast<uintptr_t>(C) >> 2) + static_cast<uint64_t>(m0) * ldc + n0) & 3);
        const int ld3 = static_cast<int>(ldc & 3);
#pragma unroll 1
        for (int pass = 0; pass < kRowsPerWave / kRowsPerPass; ++pass) {
            const int first = wave * kRowsPerWave + pass * kRowsPerPass;
            if (first >= rows) break;
            const int row = first + lane / kUnits;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(lds + row * BN + 4 * ((cu + row) & (kUnits - 1)));
            const uint32_t off = row < rows ? static_cast<uint32_t>((row * ldc + 4 * cu) * 4) : kOutOfRange;
            const int a = (a0 + row * ld3) & 3;
            if (full_lane) {
                if (a == 0) {
                    store_b128(rc, off, v);
                } else if (a == 2) {
                    store_b64(rc, off, u32x2{v[0], v[1]});
                    store_b64(rc, off + 8, u32x2{v[2], v[3]});
                } else {
                    store_b32(rc, off, v[0]);
                    store_b64(rc, off + 4, u32x2{v[1], v[2]});
                    store_b32(rc, off + 12, v[3]);
                }
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    store_b32(rc, row < rows && 4 * cu + k < ncols ? off + 4 * k : kOutOfRange, v[k]);
            }
        }
    }
}

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, bool ALIGNED, int GROUP_M>
hipError_t launch_f32(const Problem &p, int64_t grid, hipStream_t stream)
{
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    hipLaunchKernelGGL((mmrelu_f32_mfma<BM, BN, BK, WAVES_M, WAVES_N, ALIGNED>), dim3(static_cast<uint32_t>(grid)),
                       dim3(WAVES_M * WAVES_N * 64), 0, stream, static_cast<const float *>(p.A),
                       static_cast<const float *>(p.B), static_cast<float *>(p.C), p.M, p.N, p.K, p.lda, p.ldb,
                       p.ldc, tiles_m, tiles_n, GROUP_M, static_cast<const float *>(p.bias), p.act);
    return hipGetLastError();
}

}  // namespace

const Variant *variant_f32_mfma128()
{
    static const Variant v = {"mmrelu_f32_mfma<128,128,32,2,2,aligned>", MMRELU_DTYPE_F32, 128, 128, 32, 256, 2, 4,
                              launch_f32<128, 128, 32, 2, 2, true, 8>};
    return &v;
}
const Variant *variant_f32_mfma128_unaligned()
{
    static const Variant v = {"mmrelu_f32_mfma<128,128,32,2,2,unaligned>", MMRELU_DTYPE_F32, 128, 128, 32, 256, 2, 0,
                              launch_f32<128, 128, 32, 2, 2, false, 8>};
    return &v;
}

// 64 x 64 tiles (2 x 2 waves of 32 x 32): four times the workgroups of the
// 128 x 128 tile, for shapes whose 128 x 128 grid leaves most CUs idle.
const Variant *variant_f32_mfma64()
{
    static const Variant v = {"mmrelu_f32_mfma<64,64,32,2,2,aligned>", MMRELU_DTYPE_F32, 64, 64, 32, 256, 5, 4,
                              launch_f32<64, 64, 32, 2, 2, true, 8>, 1.02f};
    return &v;
}
const Variant *variant_f32_mfma64_unaligned()
{
    static const Variant v = {"mmrelu_f32_mfma<64,64,32,2,2,unaligned>", MMRELU_DTYPE_F32, 64, 64, 32, 256, 5, 0,
                              launch_f32<64, 64, 32, 2, 2, false, 8>, 1.02f};
    return &v;
}

}  // namespace mmrelu
