// bf16 relu(A·B) on the gfx950 matrix cores (v_mfma_f32_16x16x32_bf16),
// fp32 accumulation, the fused epilogue on the fp32 sum (optional per-column
// bias, then ReLU by default, or GeLU's tanh form, or nothing), then one
// rounding to bf16 (nearest, ties to even) in the store epilogue.
//
// The lecture's tiled recipe (one workgroup per output tile; K swept in slabs
// staged in on-chip memory; fp32 accumulator; the activation on the
// accumulator right before the single, masked store), laid out for CDNA4:
//  * 128 x 128 output tile per workgroup of 4 wave64s (2 x 2); each wave owns
//    a 64 x 64 sub-tile: 16 16x16 MFMA blocks, 64 fp32 accumulators per
//    lane; two workgroups per CU.
//  * K slabs of 32 are copied global -> LDS by the buffer unit directly (no
//    VGPR round trip) into a ring of STAGES buffers, STAGES-1 slabs ahead of
//    the multiply, which hides the latency of copies that miss L2. Lanes
//    outside M, N or K get an out-of-range offset and the hardware writes
//    zeros into LDS (the lecture's masked load with other=0).
//  * A (M x K, K contiguous) is read as the second MFMA operand with one
//    ds_read_b128 per lane: 8 consecutive k of one row. In LDS, A is stored
//    chunk-major per 16-row block ([block][k chunk][row] in 16-byte units),
//    so the 16 lanes reading one chunk of 16 rows touch 256 contiguous bytes
//    (the full-rate LDS pattern on gfx950, with no swizzle).
//  * B (K x N, N contiguous) must reach each lane as 8 consecutive k of one
//    column. It stays row-major in LDS and is read with ds_read_b64_tr_b16,
//    which transposes 16-bit elements across each 16-lane group: lane t of a
//    group receives element t%4 of the 8-byte rows addressed by lanes
//    4e + t/4, e = 0..3. Lane s therefore addresses row k0 + s/4, columns
//    4*(s%4) .. +3, and two such reads give the 8 k values of column t. B rows
//    are XOR swizzled so the 16 rows touched by one such read spread over
//    the banks.
//  * Fragments are double-buffered in registers: while the MFMAs of slab kt
//    run, the fragments of slab kt+1 are read from LDS.
//  * With B as the first MFMA operand, a lane's four accumulators are four
//    consecutive columns of one row of C: the epilogue writes 8 bytes a lane.
// Requires lda, ldb, ldc, K and N to be multiples of 8 and 16-byte aligned
// pointers (rows start on 16-byte boundaries).
#include "kernels.hpp"
#include "device_common.hpp"
#include "../../include/mmrelu.h"

namespace mmrelu {
namespace {

template <int BM, int BN, int BK, int STAGES, int WAVES_M, int WAVES_N>
struct Bf16Tile {
    static constexpr int kWaves = WAVES_M * WAVES_N;
    static constexpr int kThreads = kWaves * 64;
    static constexpr int WTM = BM / WAVES_M;
    static constexpr int WTN = BN / WAVES_N;
    static constexpr int MB = WTM / 16;
    static constexpr int NB = WTN / 16;
    static constexpr int CA = BK / 8;   // 16-byte k chunks per A row
    static constexpr int CB = BN / 8;   // 16-byte chunks per B row
    static constexpr int kStageA = BM * BK;          // elements
    static constexpr int kStage = BM * BK + BK * BN; // elements per stage
    static_assert(BK == 32, "one 32-wide MFMA k step per slab");
    static_assert(CB >= 16 && (CB & (CB - 1)) == 0, "B row chunk count");
    static_assert(BM % 16 == 0 && WTM % 16 == 0 && WTN % 16 == 0, "tile shape");
    static_assert((STAGES & (STAGES - 1)) == 0 && STAGES >= 2, "power-of-two ring of stages");
    static_assert((BM * CA) % (64 * kWaves) == 0 && (BK * CB) % (64 * kWaves) == 0, "load split");
    static constexpr int kLoadsA = (BM * CA) / (64 * kWaves);   // 1 KB copies per wave per slab
    static constexpr int kLoadsB = (BK * CB) / (64 * kWaves);
    static constexpr int kLoads = kLoadsA + kLoadsB;
    static_assert(kLoads * STAGES <= 63, "copies in flight must fit the vmcnt counter");
};

// B: the transposed reads of one wave touch rows k0 + {0..3} (+8, +16, +24)
// in 32-byte segments; XOR moves the four rows of a 16-lane group to distinct
// 32-byte segments and the next group's rows 128 bytes further (measured
// full rate on gfx950).
__device__ inline int swz_b(int k) { return ((k & 3) << 1) | (((k >> 3) & 1) << 3); }

template <int BM, int BN, int BK, int STAGES, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64, 1) void mmrelu_bf16_mfma(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, uint16_t *__restrict__ C,
    int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc, int tiles_m, int tiles_n, int group_m,
    const uint16_t *__restrict__ bias, int act)
{
    using T = Bf16Tile<BM, BN, BK, STAGES, WAVES_M, WAVES_N>;
    __shared__ __attribute__((aligned(1024))) uint16_t lds[STAGES * T::kStage];

    const int lane = threadIdx.x & 63;
    // wave index as a scalar, so LDS destinations of the copies are uniform
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int g = lane >> 4, t = lane & 15;

    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const rsrc_t ra = make_rsrc(A + static_cast<int64_t>(m0) * lda, ((static_cast<int64_t>(M) - 1 - m0) * lda + K) * 2);
    const uint32_t lds0 = lds_address(lds);

    // Global -> LDS copy plan: copy q of this wave fills the 1 KB LDS block
    // blk = q * waves + wave of the A (or B) part of a stage; lane l of it
    // holds one 16-byte chunk. A block = 16 rows x 4 k chunks (chunk-major);
    // B block = two 512-byte rows. Per-lane byte offsets exclude the K
    // position (A: added as a uniform offset; B: the resource is rebased per
    // slab). The M and N edges are folded into the offsets once per tile
    // (out-of-range offset for lanes past the edge); B rows past K fall
    // outside the rebased resource's byte range and read as zeros, so only
    // A needs a per-slab test (k chunk past K).
    uint32_t a_voff[T::kLoadsA], b_voff[T::kLoadsB];
    int a_col[T::kLoadsA];
#pragma unroll
    for (int q = 0; q < T::kLoadsA; ++q) {
        const int blk = q * T::kWaves + wave;
        const int row = (blk / (T::CA / 4)) * 16 + (lane & 15);
        const int col = ((blk % (T::CA / 4)) * 4 + (lane >> 4)) * 8;
        a_col[q] = col;
        a_voff[q] = (m0 + row < M) ? static_cast<uint32_t>((row * lda + col) * 2) : kOutOfRange;
    }
#pragma unroll
    for (int q = 0; q < T::kLoadsB; ++q) {
        const int blk = q * T::kWaves + wave;
        const int row = blk * (64 / T::CB) + lane / T::CB;
        const int col = ((lane % T::CB) ^ swz_b(row)) * 8;
        b_voff[q] = (n0 + col < N) ? static_cast<uint32_t>((row * ldb + col) * 2) : kOutOfRange;
    }

    // Copy q (A copies first, then B) of the slab at k0 into a stage, with
    // the B resource of that slab. Every lane is masked (a slab at or past K
    // only zero-fills a stage that is never read), so the main loop has no
    // branches and every slab costs the same vmcnt count.
    auto b_rsrc = [&](int k0) __attribute__((always_inline)) {
        return make_rsrc(B + static_cast<int64_t>(k0) * ldb + n0,
                         ((static_cast<int64_t>(K) - 1 - k0) * ldb + N - n0) * 2);
    };
    auto issue_copy = [&](int q, int stage, int k0, const rsrc_t &rb) __attribute__((always_inline)) {
        const uint32_t la = lds0 + stage * (T::kStage * 2);
        if (q < T::kLoadsA) {
            const uint32_t off = (a_col[q] < K - k0) ? a_voff[q] : kOutOfRange;
            load_to_lds<16>(ra, la + (q * T::kWaves + wave) * 1024, off, static_cast<uint32_t>(k0) * 2);
        } else {
            const int qb = q - T::kLoadsA;
            load_to_lds<16>(rb, la + T::kStageA * 2 + (qb * T::kWaves + wave) * 1024, b_voff[qb]);
        }
    };
    auto issue_loads = [&](int stage, int k0) __attribute__((always_inline)) {
        const rsrc_t rb = b_rsrc(k0);
#pragma unroll
        for (int q = 0; q < T::kLoads; ++q) issue_copy(q, stage, k0, rb);
    };

    // Fragment read plan (element offsets into a stage). A, block i: rows
    // wm*WTM + 16i + t, chunk g -> ((16-row block)*CA + g)*16 + t in 16-byte
    // units, so block i is a constant 16*BK further. B: lane t of group g
    // addresses row 8g + t/4 (+4h, a constant; the swizzle depends on the row
    // only through t/4 and g) and columns wn*WTN + 16j + 4(t%4) .. +3.
    const int a_off = (((wm * T::MB) * T::CA + g) * 16 + t) * 8;
    int b_off[T::NB];
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

    // Two register sets of MFMA operands: while the MFMAs of slab kt run, the
    // fragments of slab kt+1 are read from LDS.
    bf16x8 fa[2][T::MB], fb[2][T::NB];
    // Fragment reads of one 16-row A block (c < MB) or one 16-column B block
    // (c < NB) of a stage into register set `set`.
    auto load_frag_a = [&](int set, int stage, int c) __attribute__((always_inline)) {
        const uint16_t *st = lds + stage * T::kStage;
        fa[set][c] = *reinterpret_cast<const bf16x8 *>(st + a_off + c * 16 * BK);
    };
    auto load_frag_b = [&](int set, int stage, int c) __attribute__((always_inline)) {
        const uint16_t *st = lds + stage * T::kStage;
        i16x4 half[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
            half[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MMRELU_LDS i16x4 *)(st + b_off[c] + 4 * h * BN));
        fb[set][c] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto load_frags = [&](int set, int stage) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < T::NB; ++c) load_frag_b(set, stage, c);
#pragma unroll
        for (int c = 0; c < T::MB; ++c) load_frag_a(set, stage, c);
    };
    auto mfmas = [&](int set) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < T::MB; ++i)
#pragma unroll
            for (int j = 0; j < T::NB; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[set][j], fa[set][i], acc[i][j], 0, 0, 0);
    };
    // One pipeline step while slab kt+1 exists: wait for slab kt+1's copy
    // (slabs kt+2 .. kt+STAGES-1 may stay in flight), barrier (every wave
    // has slab kt's fragments in registers, so its stage is free), then run
    // slab kt's MFMAs while refilling that stage with slab kt+STAGES and
    // reading slab kt+1's fragments.
    //
    // Issue order matters with one wave per SIMD: copies and LDS reads are
    // spread between MFMAs (a burst of either stalls the wave's issue while
    // the matrix core idles). The scheduling fences keep each step's MFMAs
    // inside the step; MFMAs touch no memory, so the compiler would otherwise
    // move the next step's MFMAs above the barrier, right behind the reads
    // that feed them.
    constexpr int kChunks = (T::MB > T::NB ? T::MB : T::NB) > T::kLoads ? (T::MB > T::NB ? T::MB : T::NB) : T::kLoads;
    auto step = [&](int kt, int set) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<(STAGES - 2) * T::kLoads>();
        __syncthreads();
        const int fill = kt & (STAGES - 1), next = (kt + 1) & (STAGES - 1);
        const int kfill = (kt + STAGES) * BK;
        const rsrc_t rb = b_rsrc(kfill);
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            if (c < T::kLoads) issue_copy(c, fill, kfill, rb);
            if (c < T::NB) load_frag_b(set ^ 1, next, c);
            if (c < T::MB) load_frag_a(set ^ 1, next, c);
        }
        mfmas(set);
        // Issue order per chunk of MFMAs: [M R M R M R M M M M M]. The copy of
        // chunk c precedes its reads in program order (copies are ordered
        // against LDS accesses), so copies and reads are spread evenly over
        // the whole step: bursts stall the wave (a 64-lane copy occupies the
        // CU's address unit for ~16 cycles, and 32 queued copies per CU
        // otherwise block MFMA issue for hundreds of cycles).
        constexpr int kReadsPerChunk = 3;
        constexpr int kMfmaPerChunk = (T::MB * T::NB) / kChunks;
        static_assert(kMfmaPerChunk >= kReadsPerChunk, "chunk too small");
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
#pragma unroll
            for (int r = 0; r < kReadsPerChunk; ++r) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
            }
            __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPerChunk - kReadsPerChunk, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    const int nk = (K + BK - 1) / BK;
    if (nk > 0) {
#pragma unroll
        for (int s = 0; s < STAGES; ++s) issue_loads(s, s * BK);
        wait_vmcnt<(STAGES - 1) * T::kLoads>();
        __syncthreads();
        load_frags(0, 0);
        int kt = 0;
        for (; kt + 2 < nk; kt += 2) {
            step(kt, 0);
            step(kt + 1, 1);
        }
        if (kt + 1 < nk) {
            step(kt, 0);
            mfmas(1);
        } else {
            mfmas(0);
        }
    }

    // Epilogue: lane (g, t) of block (i, j) holds C[row][col .. col+3]; bias
    // and activation on fp32, round to bf16, one 8-byte masked store. The
    // bias values of the lane's columns are loaded once, up front, and only
    // when there is a bias; stores go row block by row block, so the four
    // column blocks of a row complete its lines back to back.
    const __amdgpu_buffer_rsrc_t rc = make_store_rsrc(C + static_cast<int64_t>(m0) * ldc + n0,
                                                      ((static_cast<int64_t>(M) - 1 - m0) * ldc + N - n0) * 2);
    float bj[T::NB][4];
    if (bias != nullptr) {
        const __amdgpu_buffer_rsrc_t rb = make_bias_rsrc(bias, n0, N, 2);
#pragma unroll
        for (int j = 0; j < T::NB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) bj[j][r] = bias_bf16(rb, wn * T::WTN + j * 16 + 4 * g + r);
    } else {
#pragma unroll
        for (int j = 0; j < T::NB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) bj[j][r] = 0.0f;
    }
    with_activation(act, [&](auto act_c) __attribute__((always_inline)) {
        constexpr int ACT = decltype(act_c)::value;
#pragma unroll
        for (int i = 0; i < T::MB; ++i) {
            const int row = wm * T::WTM + i * 16 + t;
#pragma unroll
            for (int j = 0; j < T::NB; ++j) {
                const int col = wn * T::WTN + j * 16 + 4 * g;
                const f32x4 v = acc[i][j];
                bf16x4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = static_cast<__bf16>(activate<ACT>(v[r] + bj[j][r]));
                const uint32_t off =
                    (m0 + row < M && n0 + col < N) ? static_cast<uint32_t>((row * ldc + col) * 2) : kOutOfRange;
                store_b64(rc, off, __builtin_bit_cast(u32x2, o));
            }
        }
    });
}

template <int BM, int BN, int BK, int STAGES, int WAVES_M, int WAVES_N, int GROUP_M>
hipError_t launch_bf16(const Problem &p, int64_t grid, hipStream_t stream)
{
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    hipLaunchKernelGGL((mmrelu_bf16_mfma<BM, BN, BK, STAGES, WAVES_M, WAVES_N>), dim3(static_cast<uint32_t>(grid)),
                       dim3(WAVES_M * WAVES_N * 64), 0, stream, static_cast<const uint16_t *>(p.A),
                       static_cast<const uint16_t *>(p.B), static_cast<uint16_t *>(p.C), p.M, p.N, p.K, p.lda,
                       p.ldb, p.ldc, tiles_m, tiles_n, GROUP_M, static_cast<const uint16_t *>(p.bias), p.act);
    return hipGetLastError();
}

}  // namespace

// 128 x 128 tiles (2 x 2 waves of 64 x 64): four times the workgroups of the
// 256 x 256 tile, for shapes whose 256 x 256 grid leaves most CUs idle.
// Relative cost per output 1.66 against the 256 x 256 ping-pong tile.
const Variant *variant_bf16_mfma128()
{
    static const Variant v = {"mmrelu_bf16_mfma<128,128,32,4,2,2>", MMRELU_DTYPE_BF16, 128, 128, 32, 256, 2, 8,
                              launch_bf16<128, 128, 32, 4, 2, 2, 8>, 1.66f};
    return &v;
}

}  // namespace mmrelu
