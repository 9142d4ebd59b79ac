// relu(A·B) (and the fused epilogues) for skinny products, where the work is
// bound by reading the large operand from HBM once, not by the matrix cores:
//  * skinny M (M <= 64): a 64 x 8192 x 8192 bf16 product is 8.6 GFLOP (3.4 us
//    of MFMA at peak) but 128 MB of B (16.8 us at 8 TB/s);
//  * skinny N (N <= 64): the mirror image, 128 MB of A for an 8192 x 64 C.
//
// The arithmetic is the same tiled product with the activation fused into
// the one store ("Kernels, Triton, XLA", section "Reductions and tiling"); the
// tile is shaped for a memory-bound product:
//  * One workgroup per (16 MB) x (16 NB) tile of C: MB = 1, 2, 4 row blocks
//    by NB = 2 column blocks for skinny M (a 32-column strip of B per
//    workgroup, 256 workgroups at N = 8192), MB = 2 by NB = 1, 2, 4 for
//    skinny N (a 32-row band of A per workgroup). The small operand is read
//    by every workgroup and stays in L2. A 64 x 64 tile (MB = NB = 4) serves
//    small squares and long-K products with few output tiles, where it
//    halves the operand bytes per output of the 32 x 64 tile.
//  * Its eight waves (four for the 16 x 64 few-rows strips) split K into as
//    many contiguous ranges of slabs and run independently, with no barrier
//    inside the loop; the partial tiles are summed through LDS at the end
//    (fixed order: deterministic results), one 16 x 16 block per wave (two
//    at 64 x 64).
//  * Both operands are issued kDepth slabs ahead of the slab being
//    multiplied: A fragments straight into registers (each lane's 8 bf16 /
//    4 fp32 of a row are contiguous), rotating through kDepth + 1 register
//    sets, and B slabs into a private ring of kDepth + 1 LDS stages per wave
//    (buffer -> LDS DMA). The memory counter retires loads in issue order, so
//    the two operands run at the same distance: a wait for a nearer A load
//    would also wait for every B copy issued before it. One slab in flight
//    per wave (eight per CU) reads HBM fastest here; deeper rings were
//    measured slower.
//  * A slab holds KS k blocks of 32 (bf16) or 16 (fp32) k. With KS = 2 a
//    step reads 128 bytes of each A row, a whole line, instead of half of
//    one (HBM reads in 64-byte pieces of lines ran at about half the rate of
//    whole lines in a read-only probe).
//  * A and B are loaded with inline assembly and waited for with explicit
//    vmcnt counts (a compiler-visible load would make the compiler's own wait
//    count drain the copies in flight every slab).
//  * B fragments are read from the stage with ds_read_b64_tr_b16 (bf16: each
//    lane gets 8 consecutive k of one column) or ds_read_b32 (fp32), as in the
//    large-tile kernels; MFMA 16x16x32 bf16 / 16x16x4 f32 with the operands
//    swapped so a lane's four accumulators are four consecutive columns.
//  * Epilogue: bias, activation and one masked store, as in the other kernels.
// Requires lda, ldb, ldc, K and N to be multiples of 8 (bf16) or 4 (fp32)
// and 16-byte aligned pointers.
#include <type_traits>

#include "kernels.hpp"
#include "device_common.hpp"
#include "../../include/mmrelu.h"

namespace mmrelu {
namespace {

// Waves per workgroup: eight, or four for the 16 x 64 few-rows strips (see
// their variants).
constexpr int kWaves = 8, kThreads = kWaves * 64;

template <typename T>
struct KBlock;
template <>
struct KBlock<uint16_t> {                          // bf16: 32 k per MFMA
    static constexpr int kK = 32;
};
template <>
struct KBlock<float> {                             // fp32: 16 k per four MFMAs
    static constexpr int kK = 16;
};

// buffer_load_dwordx4 into registers, not visible to the compiler's wait
// counting (see the file comment); the caller waits explicitly.
__device__ inline u32x4 load_b128_async(rsrc_t r, uint32_t voffset)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_readfirstlane(r[i]);
    asm("" : "+s"(r));
    u32x4 v;
    asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(v) : "v"(voffset), "s"(r) : "memory");
    return v;
}

// KS k blocks per slab (KS = 2: a row of A read in a step covers a whole
// 128-byte line); kStages slabs in the ring, kStages - 1 of them in flight.
template <typename T, int MB, int NB, int KS, int STAGES, int W>
struct SkinnyShape {
    static constexpr int kBlkK = KBlock<T>::kK;
    static constexpr int kSlabK = KS * kBlkK;
    static constexpr int kEsize = sizeof(T);
    static constexpr int kRowBytes = 16 * NB * kEsize;             // one k row of the B slab
    static constexpr int kStageBytes = kSlabK * kRowBytes;         // KS * NB KB
    static constexpr int kStages = STAGES;
    static constexpr int kDepth = kStages - 1;                     // slabs in flight ahead
    static constexpr int kRingBytes = W * kStages * kStageBytes;
    static constexpr int kRedBytes = W * MB * NB * 64 * 16;        // partial tiles
    static constexpr int kLdsBytes = kRingBytes > kRedBytes ? kRingBytes : kRedBytes;
    static_assert(kBlkK * kRowBytes == NB * 1024, "one 1 KB copy per 16 columns and k block");
    static_assert(kStages >= 2, "ring depth");
    static_assert(MB * NB <= W || (MB * NB) % W == 0, "whole blocks per reducing wave");
    static_assert(kDepth * KS * (NB + MB) <= 63, "vmcnt range");
    static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
};

template <typename T, int MB, int NB, int KS, int STAGES, int W>
__global__ __launch_bounds__(W * 64, 1) void mmrelu_skinny(
    const T *__restrict__ A, const T *__restrict__ B, T *__restrict__ C, int M, int N, int K,
    int64_t lda, int64_t ldb, int64_t ldc, const T *__restrict__ bias, int act)
{
    using S = SkinnyShape<T, MB, NB, KS, STAGES, W>;
    constexpr int kSlabK = S::kSlabK, kBlkK = S::kBlkK, kEsize = S::kEsize, kRowBytes = S::kRowBytes;
    constexpr int kStageBytes = S::kStageBytes, kStages = S::kStages, kDepth = S::kDepth;
    constexpr int kSets = kDepth + 1;                  // A register sets = ring stages
    constexpr int kNBlk = MB * NB;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[S::kLdsBytes];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, t = lane & 15;

    // Tile of this workgroup. bf16: each XCD takes a contiguous range of
    // tiles, walked in bands of up to eight tile rows, column by column, so
    // the tiles that share a strip of B (or a band of A) run on one XCD and
    // its L2 serves the operand once (measured: 128 x 8192 x 8192, 53.4 ->
    // 47.1 us; 256 x 4096 x 4096, 30.4 -> 26.6; 8192 x 64 x 8192, 31.1 ->
    // 28.8). A bf16 32-column strip row is also only 64 bytes, half of a
    // 128-byte line, and the neighbouring strip reads the other half; on the
    // same XCD the two share one L2 fill. fp32 keeps the dispatch order,
    // which spreads the tiles that run together over more HBM channels
    // (measured: fp32 8192 x 8192 B at M <= 16 reads 10% faster that way, and
    // the grouped order gained nothing on the shapes above).
    const int tiles_n = (N + 16 * NB - 1) / (16 * NB);
    int tm, tn;
    if (sizeof(T) == 2) {
        tile_of(blockIdx.x, gridDim.x, (M + 16 * MB - 1) / (16 * MB), tiles_n, 8, tm, tn);
    } else {
        tm = blockIdx.x / tiles_n;
        tn = blockIdx.x % tiles_n;
    }
    const int m0 = tm * 16 * MB, n0 = tn * 16 * NB;
    const uint32_t ring = lds_address(lds) + wave * (kStages * kStageBytes);

    // This wave's slabs: a contiguous, balanced share of ceil(K / kSlabK).
    const int nk = (K + kSlabK - 1) / kSlabK;
    const int s_begin = (nk * wave) / W, s_end = (nk * (wave + 1)) / W;
    const int n_w = s_end - s_begin;

    // B copies: KS * NB 1 KB copies per slab; lane l of copy c fills LDS byte
    // c * 1024 + 16 l of the stage, i.e. row-major rows of kRowBytes.
    constexpr int kCopies = KS * NB;
    constexpr int kLanesPerRow = kRowBytes / 16;
    uint32_t b_voff[kCopies];
#pragma unroll
    for (int c = 0; c < kCopies; ++c) {
        const int row = c * (64 / kLanesPerRow) + lane / kLanesPerRow;
        const int col = (lane % kLanesPerRow) * (16 / kEsize);
        b_voff[c] = (n0 + col < N) ? static_cast<uint32_t>((row * ldb + col) * kEsize) : kOutOfRange;
    }
    auto copy_b = [&](int j, int stage) __attribute__((always_inline)) {   // slab j of this wave's range
        const int k0 = (s_begin + j) * kSlabK;
        const bool live = j < n_w;
        const rsrc_t rb = make_rsrc(B + static_cast<int64_t>(live ? k0 : 0) * ldb + n0,
                                    live ? ((static_cast<int64_t>(K) - 1 - k0) * ldb + N - n0) * kEsize : 0);
#pragma unroll
        for (int c = 0; c < kCopies; ++c) load_to_lds<16>(rb, ring + stage * kStageBytes + c * 1024, b_voff[c]);
    };

    // A loads: row block i and k block u of the slab; lane (g, t) takes row
    // m0 + 16 i + t and the lane group's k chunk of the block (bf16: k 8g..8g+7;
    // fp32: k 4g..4g+3). The resource is rebased on each slab so every
    // offset stays small.
    constexpr int kChunkK = 16 / kEsize;
    uint32_t a_voff[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
        a_voff[i] = (m0 + 16 * i + t < M) ? static_cast<uint32_t>(((16 * i + t) * lda + kChunkK * g) * kEsize)
                                          : kOutOfRange;
    auto load_a = [&](int j, u32x4 (&fa)[KS][MB]) __attribute__((always_inline)) {
        const int k0 = (s_begin + j) * kSlabK;
        const bool live = j < n_w;
        const rsrc_t ra = make_rsrc(A + static_cast<int64_t>(m0) * lda + (live ? k0 : 0),
                                    live ? ((static_cast<int64_t>(M) - 1 - m0) * lda + K - k0) * kEsize : 0);
#pragma unroll
        for (int u = 0; u < KS; ++u) {
            const bool in_k = k0 + u * kBlkK + kChunkK * g < K;   // past K the row's padding follows
#pragma unroll
            for (int i = 0; i < MB; ++i)
                fa[u][i] = load_b128_async(ra, in_k ? a_voff[i] + u * kBlkK * kEsize : kOutOfRange);
        }
    };

    f32x4 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One slab: B fragments from the stage, MFMAs with the A fragments.
    auto compute = [&](int stage, const u32x4 (&fa)[KS][MB]) __attribute__((always_inline)) {
        const uint8_t *st = lds + wave * (kStages * kStageBytes) + stage * kStageBytes;
#pragma unroll
        for (int u = 0; u < KS; ++u) {
            const uint8_t *sb = st + u * kBlkK * kRowBytes;
            if constexpr (std::is_same_v<T, uint16_t>) {
#pragma unroll
                for (int jb = 0; jb < NB; ++jb) {
                    i16x4 half[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int row = 8 * g + 4 * h + (t >> 2);
                        const int col = 16 * jb + 4 * (t & 3);
                        half[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (MMRELU_LDS i16x4 *)(sb + row * kRowBytes + col * 2));
                    }
                    const bf16x8 fb = __builtin_bit_cast(bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                    for (int i = 0; i < MB; ++i)
                        acc[i][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb, __builtin_bit_cast(bf16x8, fa[u][i]), acc[i][jb], 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int jb = 0; jb < NB; ++jb) {
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const float b = *reinterpret_cast<const float *>(sb + (4 * g + s) * kRowBytes + (16 * jb + t) * 4);
#pragma unroll
                        for (int i = 0; i < MB; ++i)
                            acc[i][jb] = __builtin_amdgcn_mfma_f32_16x16x4f32(b, __uint_as_float(fa[u][i][s]), acc[i][jb], 0, 0, 0);
                    }
                }
            }
        }
    };

    // Pipeline: slabs 0 .. kDepth-1 issued up front (B copy, then A load).
    // Step j issues slab j + kDepth into the ring stage and register set that
    // slab j - 1 used (read and consumed in step j - 1), then waits until
    // everything issued before slab j + 1 has landed, i.e. slab j itself, and
    // multiplies slab j. Slab j lives in stage and set j mod kSets; the loop
    // is unrolled by kSets so both are compile-time constants (a runtime
    // index would put the register sets in scratch), and no set is ever
    // copied into another: a copy of a register whose load is still in flight
    // would read stale data. Copies and loads past the wave's range are fully
    // masked, so every step issues the same count.
    u32x4 fa[kSets][KS][MB];
    auto step = [&](int j, int q) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        copy_b(j + kDepth, (q + kDepth) % kSets);
        load_a(j + kDepth, fa[(q + kDepth) % kSets]);
        asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kDepth * KS * (NB + MB)) : "memory");
#pragma unroll
        for (int u = 0; u < KS; ++u)
#pragma unroll
            for (int i = 0; i < MB; ++i) asm volatile("" : "+v"(fa[q][u][i]));
        __builtin_amdgcn_sched_barrier(0);
        compute(q, fa[q]);
        __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int q = 0; q < kDepth; ++q) {
        copy_b(q, q);
        load_a(q, fa[q]);
    }
    for (int j0 = 0; j0 < n_w; j0 += kSets) {
#pragma unroll
        for (int q = 0; q < kSets; ++q)
            if (j0 + q < n_w) step(j0 + q, q);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // Sum the eight waves' partial tiles: wave w writes block b of lane l at
    // ((w * kNBlk + b) * 64 + l) * 16 bytes; the reducing wave of block b
    // then adds them over the waves in order.
    f32x4 *red = reinterpret_cast<f32x4 *>(lds);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) red[(wave * kNBlk + i * NB + jb) * 64 + lane] = acc[i][jb];
    __syncthreads();
    // Wave w reduces blocks w, w + 8, ... (one block per wave up to 32 x 64
    // tiles, two at 64 x 64).
    const __amdgpu_buffer_rsrc_t rc =
        make_store_rsrc(C + static_cast<int64_t>(m0) * ldc + n0, ((static_cast<int64_t>(M) - 1 - m0) * ldc + N - n0) * kEsize);
    for (int b = wave; b < kNBlk; b += W) {
        f32x4 v = red[b * 64 + lane];
#pragma unroll
        for (int w = 1; w < W; ++w) v += red[(w * kNBlk + b) * 64 + lane];
        const int i = b / NB, jb = b % NB;
        const int row = 16 * i + t;                    // within the tile
        const int col = 16 * jb + 4 * g;

        // Epilogue: bias of the lane's four columns (only when there is one),
        // activation, one masked store of four consecutive columns.
        float bj[4];
        if (bias != nullptr) {
            const __amdgpu_buffer_rsrc_t rbias = make_bias_rsrc(bias, n0, N, kEsize);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                bj[r] = std::is_same_v<T, uint16_t> ? bias_bf16(rbias, col + r) : bias_f32(rbias, col + r);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) bj[r] = 0.0f;
        }
        const uint32_t off =
            (m0 + row < M && n0 + col < N) ? static_cast<uint32_t>((row * ldc + col) * kEsize) : kOutOfRange;
        with_activation(act, [&](auto act_c) __attribute__((always_inline)) {
            constexpr int ACT = decltype(act_c)::value;
            if constexpr (std::is_same_v<T, uint16_t>) {
                bf16x4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = static_cast<__bf16>(activate<ACT>(v[r] + bj[r]));
                store_b64(rc, off, __builtin_bit_cast(u32x2, o));
            } else {
                f32x4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = activate<ACT>(v[r] + bj[r]);
                store_b128(rc, off, __builtin_bit_cast(u32x4, o));
            }
        });
    }
}

template <typename T, int MB, int NB, int KS, int STAGES, int W = kWaves>
hipError_t launch_skinny(const Problem &p, int64_t grid, hipStream_t stream)
{
    hipLaunchKernelGGL((mmrelu_skinny<T, MB, NB, KS, STAGES, W>), dim3(static_cast<uint32_t>(grid)), dim3(W * 64), 0, stream,
                       static_cast<const T *>(p.A), static_cast<const T *>(p.B), static_cast<T *>(p.C), p.M, p.N,
                       p.K, p.lda, p.ldb, p.ldc, static_cast<const T *>(p.bias), p.act);
    return hipGetLastError();
}

}  // namespace

// Skinny-M tiles (16, 32 or 64 rows by 32 columns), skinny-N tiles (32
// rows by 16, 32 or 64 columns) and the 64 x 64 tile (relative cost 1.03
// fp32, 4.8 bf16: measured 1024^3 fp32 25.7 against 27.5 us on 32 x 64
// tiles, bf16 10.0 against 12.7; 1024 x 1024 x 8192 bf16 48.6 against 65).
// Any shape is covered by a grid of tiles;
// the planner uses them where one dimension is small, and through its cost
// model where the large tiles would leave CUs idle. Their relative cost per
// output (against the dtype's fastest tile kernel at full occupancy) was
// fitted on 256^3 .. 2048^3, 512 x 512 x 8192, 1024 x 1024 x 8192 and
// 128 / 4096-row products: about 1.04 - 1.1 in fp32, 5.3 - 9.5 in bf16 (the
// bf16 ping-pong kernel does far more per output at full occupancy), the
// bf16 figures then scaled by 1.067 when the 64-deep ping-pong schedule
// became the reference (8192^3: 753 against 804 us); the
// 16-wide tiles, slower per output, are priced up so that the planner uses
// them only through the few-rows and few-columns rules. Each uses the k depth
// per slab (KS) and ring depth measured fastest for its role at 8192 x 8192:
// two stages (one slab in flight) throughout, since deeper rings read HBM
// more slowly here (fp32 1 x 8192 x 8192: 39 us with two stages, 48 us with
// eight); KS = 2 where the rows of the streamed operand would otherwise be
// read as half lines (skinny N, and fp32 at 64 rows). wg_per_cu 1.
const Variant *variant_f32_skinny(int mb, int nb, int ks)
{
    static const Variant m1 = {"mmrelu_skinny<float,16x32,ks1>", MMRELU_DTYPE_F32, 16, 32, 16, kThreads, 1, 4,
                               launch_skinny<float, 1, 2, 1, 2>, 2.3f};
    static const Variant m2 = {"mmrelu_skinny<float,32x32,ks1>", MMRELU_DTYPE_F32, 32, 32, 16, kThreads, 1, 4,
                               launch_skinny<float, 2, 2, 1, 2>, 1.1f};
    static const Variant m4 = {"mmrelu_skinny<float,64x32,ks2>", MMRELU_DTYPE_F32, 64, 32, 32, kThreads, 1, 4,
                               launch_skinny<float, 4, 2, 2, 2>, 1.05f};
    static const Variant n1 = {"mmrelu_skinny<float,32x16,ks2>", MMRELU_DTYPE_F32, 32, 16, 32, kThreads, 1, 4,
                               launch_skinny<float, 2, 1, 2, 2>, 2.3f};
    static const Variant n2 = {"mmrelu_skinny<float,32x32,ks2>", MMRELU_DTYPE_F32, 32, 32, 32, kThreads, 1, 4,
                               launch_skinny<float, 2, 2, 2, 2>, 1.08f};
    static const Variant n4 = {"mmrelu_skinny<float,32x64,ks2>", MMRELU_DTYPE_F32, 32, 64, 32, kThreads, 1, 4,
                               launch_skinny<float, 2, 4, 2, 2>, 1.04f};
    static const Variant sq = {"mmrelu_skinny<float,64x64,ks2>", MMRELU_DTYPE_F32, 64, 64, 32, kThreads, 1, 4,
                               launch_skinny<float, 4, 4, 2, 2>, 1.03f};
    // 64-column strips (256-byte rows of B) for M <= 16 when N is large:
    // more 32-column strips than CUs read HBM more slowly (1 x 16384 x 8192:
    // 4.8 TB/s, against 6.9 at 8192 columns); measured 1 x 16384 x 16384,
    // 188.7 against 221.1 us; 16 x 16384 x 8192, 97.8 against 118.2. Four
    // waves, four streams of B rows per CU instead of eight, read these deep
    // products faster (1 x 16384 x 16384: 167.7 against 190.1 us; 1 x 16384
    // x 32768: 326.1 against 380.7; 16 x 16384 x 4096: 38.4 against 41.4;
    // equal at 1 x 32768 x 8192 and 8 x 65536 x 4096).
    static const Variant w1 = {"mmrelu_skinny<float,16x64,ks1,w4>", MMRELU_DTYPE_F32, 16, 64, 16, 4 * 64, 1, 4,
                               launch_skinny<float, 1, 4, 1, 2, 4>, 2.3f};
    // 64-row bands of A for N <= 16 when M is large, for the same reason
    // (measured: 16384 x 16 x 8192, 122.6 against 150.4 us on 32-row bands;
    // 32768 x 16 x 4096, 110.9 against 117.0). bf16 gains nothing from it.
    static const Variant h1 = {"mmrelu_skinny<float,64x16,ks2>", MMRELU_DTYPE_F32, 64, 16, 32, kThreads, 1, 4,
                               launch_skinny<float, 4, 1, 2, 2>, 2.3f};
    if (nb == 1 && mb == 4) return &h1;
    if (nb == 4 && mb == 1) return &w1;
    if (nb == 4 && mb == 4) return &sq;
    if (nb == 2 && ks == 1) return mb == 1 ? &m1 : &m2;
    if (nb == 2 && mb == 4) return &m4;
    return nb == 1 ? &n1 : nb == 2 ? &n2 : &n4;
}
const Variant *variant_bf16_skinny(int mb, int nb, int ks)
{
    static const Variant m1 = {"mmrelu_skinny<bf16,16x32,ks1>", MMRELU_DTYPE_BF16, 16, 32, 32, kThreads, 1, 8,
                               launch_skinny<uint16_t, 1, 2, 1, 2>, 10.1f};
    static const Variant m2 = {"mmrelu_skinny<bf16,32x32,ks1>", MMRELU_DTYPE_BF16, 32, 32, 32, kThreads, 1, 8,
                               launch_skinny<uint16_t, 2, 2, 1, 2>, 10.1f};
    static const Variant m4 = {"mmrelu_skinny<bf16,64x32,ks1>", MMRELU_DTYPE_BF16, 64, 32, 32, kThreads, 1, 8,
                               launch_skinny<uint16_t, 4, 2, 1, 2>, 6.4f};
    static const Variant n1 = {"mmrelu_skinny<bf16,32x16,ks2>", MMRELU_DTYPE_BF16, 32, 16, 64, kThreads, 1, 8,
                               launch_skinny<uint16_t, 2, 1, 2, 2>, 10.1f};
    static const Variant n2 = {"mmrelu_skinny<bf16,32x32,ks2>", MMRELU_DTYPE_BF16, 32, 32, 64, kThreads, 1, 8,
                               launch_skinny<uint16_t, 2, 2, 2, 2>, 9.6f};
    static const Variant n4 = {"mmrelu_skinny<bf16,32x64,ks2>", MMRELU_DTYPE_BF16, 32, 64, 64, kThreads, 1, 8,
                               launch_skinny<uint16_t, 2, 4, 2, 2>, 5.7f};
    static const Variant sq = {"mmrelu_skinny<bf16,64x64,ks2>", MMRELU_DTYPE_BF16, 64, 64, 64, kThreads, 1, 8,
                               launch_skinny<uint16_t, 4, 4, 2, 2>, 4.8f};
    // 64-column strips for M <= 16 when N is large: whole 128-byte lines of B
    // per row (measured: 1 x 16384 x 16384, 120.5 against 136.1 us on 32-column
    // strips; 4 x 32768 x 4096, 44.5 against 49.5). At N = 8192 they leave
    // half the CUs idle and tie with the 32-column strips. Four waves, four
    // streams of B rows per CU instead of eight (1 x 16384 x 16384: 96.9
    // against 120.2 us; 1 x 16384 x 32768: 189.9 against 223.0; 16 x 16384 x
    // 16384: 106.5 against 114.0; within 2% elsewhere).
    static const Variant w1 = {"mmrelu_skinny<bf16,16x64,ks1,w4>", MMRELU_DTYPE_BF16, 16, 64, 32, 4 * 64, 1, 8,
                               launch_skinny<uint16_t, 1, 4, 1, 2, 4>, 10.1f};
    if (nb == 4 && mb == 4) return &sq;
    if (nb == 4 && mb == 1) return &w1;
    if (nb == 2 && ks == 1) return mb == 1 ? &m1 : mb == 2 ? &m2 : &m4;
    return nb == 1 ? &n1 : nb == 2 ? &n2 : &n4;
}

}  // namespace mmrelu
