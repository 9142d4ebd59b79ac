// relu(A·B) (and the fused epilogues) for skinny M (M <= 64), where the work
// is bound by reading B from HBM once, not by the matrix cores: a 64 x 8192 x
// 8192 bf16 product is 8.6 GFLOP (3.4 us of MFMA at peak) but 128 MB of B
// (16.8 us at 8 TB/s).
//
// The arithmetic is the same tiled product with the activation fused into
// the one store ("Kernels, Triton, XLA", section "Reductions and tiling"); the
// tile is shaped for a memory-bound product:
//  * One workgroup per 32-column strip of B and C (N = 8192 gives 256
//    workgroups, one per CU), covering all M <= 16 * MB rows. Every workgroup
//    reads all of A, which is small and stays in L2.
//  * Its eight waves split K into eight contiguous ranges of slabs and run
//    independently: each wave streams its range of the B strip through a
//    private ring of eight 2 KB LDS stages (buffer -> LDS DMA, seven slabs
//    ahead), so a CU keeps ~112 KB of B in flight, enough to cover HBM latency
//    at its 1/256 share of the bandwidth, with no barrier inside the loop.
//  * A fragments come straight from global memory into registers (each lane's
//    8 bf16 / 4 fp32 of a row are contiguous), one slab ahead. A and B are
//    both loaded with inline assembly and waited for with explicit vmcnt
//    counts (a compiler-visible load would make the compiler's own wait
//    count drain the B copies in flight every iteration).
//  * B fragments are read from the stage with ds_read_b64_tr_b16 (bf16: each
//    lane gets 8 consecutive k of one column) or ds_read_b32 (fp32), as in the
//    large-tile kernels; MFMA 16x16x32 bf16 / 16x16x4 f32 with the operands
//    swapped so a lane's four accumulators are four consecutive columns.
//  * At the end the eight waves' partial tiles are summed through LDS
//    (fixed order, so results are deterministic), then bias, activation and
//    one masked store, as in the other kernels.
// Requires lda, ldb, ldc, K and N to be multiples of 8 (bf16) or 4 (fp32)
// and 16-byte aligned pointers.
#include <type_traits>

#include "kernels.hpp"
#include "device_common.hpp"
#include "../../include/mmrelu.h"

namespace mmrelu {
namespace {

constexpr int kWaves = 8, kThreads = kWaves * 64;
constexpr int kBN = 32, kNB = 2;                  // strip width, 16-column blocks per strip
constexpr int kStages = 8;                         // per-wave ring
constexpr int kStageBytes = 2048;
constexpr int kRingBytes = kWaves * kStages * kStageBytes;   // 128 KB

template <typename T>
struct Skinny;
template <>
struct Skinny<uint16_t> {                          // bf16
    static constexpr int kSlabK = 32;              // k rows per stage (64-byte rows)
    static constexpr int kRowBytes = kBN * 2;
};
template <>
struct Skinny<float> {
    static constexpr int kSlabK = 16;              // k rows per stage (128-byte rows)
    static constexpr int kRowBytes = kBN * 4;
};

// buffer_load_dwordx4 into registers, not visible to the compiler's wait
// counting (see the file comment); the caller waits explicitly.
__device__ inline u32x4 load_b128_async(rsrc_t r, uint32_t voffset, uint32_t soffset)
{
    soffset = __builtin_amdgcn_readfirstlane(soffset);
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_readfirstlane(r[i]);
    asm("" : "+s"(soffset), "+s"(r));
    u32x4 v;
    asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen" : "=v"(v) : "v"(voffset), "s"(r), "s"(soffset) : "memory");
    return v;
}

template <typename T, int MB>
__global__ __launch_bounds__(kThreads, 1) void mmrelu_skinny(
    const T *__restrict__ A, const T *__restrict__ B, T *__restrict__ C, int M, int N, int K,
    int64_t lda, int64_t ldb, int64_t ldc, const T *__restrict__ bias, int act)
{
    using S = Skinny<T>;
    constexpr int kSlabK = S::kSlabK;
    constexpr int kEsize = sizeof(T);
    constexpr int kNBlk = MB * kNB;
    static_assert(kWaves * kNBlk * 64 * 16 <= kRingBytes, "reduction buffer fits in the ring");
    static_assert(kSlabK * S::kRowBytes == kStageBytes, "stage size");
    constexpr int kInFlight = 2 + MB;               // copies and loads issued per iteration
    static_assert(2 * (kStages - 1) + MB <= 63, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kRingBytes];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, t = lane & 15;
    // bf16: consecutive strips on one XCD. A bf16 strip row is 64 bytes, half
    // of a 128-byte line, and the neighbouring strip reads the other half; on
    // the same XCD the two share one L2 fill instead of each fetching the
    // line. An fp32 strip row is a whole line and keeps the dispatch order,
    // which spreads the strips that run together over more HBM channels
    // (measured: 8192 x 8192 B at M <= 16 reads 10% faster that way).
    int n0 = blockIdx.x * kBN;
    if constexpr (sizeof(T) == 2) {
        int tm, tn;
        tile_of(blockIdx.x, gridDim.x, 1, gridDim.x, 1, tm, tn);
        n0 = tn * kBN;
    }
    const uint32_t lds0 = lds_address(lds);
    const uint32_t ring = lds0 + wave * (kStages * kStageBytes);

    // This wave's slabs: a contiguous, balanced share of ceil(K / kSlabK).
    const int nk = (K + kSlabK - 1) / kSlabK;
    const int s_begin = (nk * wave) / kWaves, s_end = (nk * (wave + 1)) / kWaves;
    const int n_w = s_end - s_begin;

    // B copies: two 1 KB copies per slab; lane l of copy c fills LDS byte
    // c*1024 + 16*l of the stage, i.e. row-major rows of kRowBytes.
    constexpr int kLanesPerRow = S::kRowBytes / 16;
    uint32_t b_voff[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int row = c * (64 / kLanesPerRow) + lane / kLanesPerRow;
        const int col = (lane % kLanesPerRow) * (16 / kEsize);
        b_voff[c] = (n0 + col < N) ? static_cast<uint32_t>((row * ldb + col) * kEsize) : kOutOfRange;
    }
    auto copy_b = [&](int j) __attribute__((always_inline)) {   // slab j of this wave's range
        const int k0 = (s_begin + j) * kSlabK;
        const bool live = j < n_w;
        const rsrc_t rb = make_rsrc(B + static_cast<int64_t>(live ? k0 : 0) * ldb + n0,
                                    live ? ((static_cast<int64_t>(K) - 1 - k0) * ldb + N - n0) * kEsize : 0);
        const uint32_t st = ring + (j % kStages) * kStageBytes;
#pragma unroll
        for (int c = 0; c < 2; ++c) load_to_lds<16>(rb, st + c * 1024, b_voff[c]);
    };

    // A loads: block i, lane (g, t) takes row 16i + t and the lane group's k
    // chunk (bf16: k 8g..8g+7; fp32: k 4g..4g+3) of the slab.
    constexpr int kChunkK = 16 / kEsize;
    const rsrc_t ra = make_rsrc(A, ((static_cast<int64_t>(M) - 1) * lda + K) * kEsize);
    uint32_t a_voff[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
        a_voff[i] = (16 * i + t < M) ? static_cast<uint32_t>(((16 * i + t) * lda + kChunkK * g) * kEsize) : kOutOfRange;
    auto load_a = [&](int j, u32x4 (&fa)[MB]) __attribute__((always_inline)) {
        const int k0 = (s_begin + j) * kSlabK;
        const bool live = j < n_w && k0 + kChunkK * g < K;
#pragma unroll
        for (int i = 0; i < MB; ++i) fa[i] = load_b128_async(ra, live ? a_voff[i] : kOutOfRange, live ? k0 * kEsize : 0);
    };

    f32x4 acc[MB][kNB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One slab: B fragments from the stage, MFMAs with the A fragments.
    auto compute = [&](int j, const u32x4 (&fa)[MB]) __attribute__((always_inline)) {
        const uint8_t *st = lds + wave * (kStages * kStageBytes) + (j % kStages) * kStageBytes;
        if constexpr (std::is_same_v<T, uint16_t>) {
#pragma unroll
            for (int jb = 0; jb < kNB; ++jb) {
                i16x4 half[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int row = 8 * g + 4 * h + (t >> 2);
                    const int col = 16 * jb + 4 * (t & 3);
                    half[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (MMRELU_LDS i16x4 *)(st + row * S::kRowBytes + col * 2));
                }
                const bf16x8 fb = __builtin_bit_cast(bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    acc[i][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb, __builtin_bit_cast(bf16x8, fa[i]), acc[i][jb], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int jb = 0; jb < kNB; ++jb) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const float b = *reinterpret_cast<const float *>(st + (4 * g + s) * S::kRowBytes + (16 * jb + t) * 4);
#pragma unroll
                    for (int i = 0; i < MB; ++i)
                        acc[i][jb] = __builtin_amdgcn_mfma_f32_16x16x4f32(b, __uint_as_float(fa[i][s]), acc[i][jb], 0, 0, 0);
                }
            }
        }
    };

    // Pipeline: slabs 0 .. kStages-2 copied and slab 0's A loaded up front.
    // Step j issues the copy of slab j+kStages-1 into the stage slab j-1 used
    // (read and consumed in step j-1), then A of slab j+1, then waits until
    // everything issued before this step has landed (slab j's A, and its B
    // copy, issued earlier), and multiplies slab j. Copies and loads past the
    // wave's range are fully masked, so every step issues the same count.
    // Two A register sets alternate (the loop is unrolled by two): a load
    // lands in the set the following step reads after its wait. Copying a
    // register whose load is still in flight would read stale data, so no
    // step moves one set into the other.
    u32x4 fa0[MB], fa1[MB];
    auto step = [&](int j, u32x4 (&cur)[MB], u32x4 (&next)[MB]) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        copy_b(j + kStages - 1);
        load_a(j + 1, next);
        asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kInFlight) : "memory");
#pragma unroll
        for (int i = 0; i < MB; ++i) asm volatile("" : "+v"(cur[i]));
        __builtin_amdgcn_sched_barrier(0);
        compute(j, cur);
        __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int j = 0; j + 1 < kStages; ++j) copy_b(j);
    load_a(0, fa0);
    for (int j = 0; j < n_w; j += 2) {
        step(j, fa0, fa1);
        if (j + 1 < n_w) step(j + 1, fa1, fa0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // Sum the eight waves' partial tiles: wave w writes block b of lane l at
    // ((w * kNBlk + b) * 64 + l) * 16 bytes; wave q < kNBlk then reduces
    // block q over the waves in order.
    f32x4 *red = reinterpret_cast<f32x4 *>(lds);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int jb = 0; jb < kNB; ++jb) red[(wave * kNBlk + i * kNB + jb) * 64 + lane] = acc[i][jb];
    __syncthreads();
    if (wave >= kNBlk) return;
    f32x4 v = red[wave * 64 + lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += red[(w * kNBlk + wave) * 64 + lane];
    const int i = wave / kNB, jb = wave % kNB;
    const int row = 16 * i + t;
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
    const __amdgpu_buffer_rsrc_t rc = make_store_rsrc(C + n0, ((static_cast<int64_t>(M) - 1) * ldc + N - n0) * kEsize);
    const uint32_t off = (row < M && n0 + col < N) ? static_cast<uint32_t>((row * ldc + col) * kEsize) : kOutOfRange;
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

template <typename T, int MB>
hipError_t launch_skinny(const Problem &p, int64_t grid, hipStream_t stream)
{
    hipLaunchKernelGGL((mmrelu_skinny<T, MB>), dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0, stream,
                       static_cast<const T *>(p.A), static_cast<const T *>(p.B), static_cast<T *>(p.C), p.M, p.N,
                       p.K, p.lda, p.ldb, p.ldc, static_cast<const T *>(p.bias), p.act);
    return hipGetLastError();
}

}  // namespace

// block_m is the most rows a variant covers; the planner picks the smallest
// that holds M. wg_per_cu 1 (128 KB of LDS per workgroup).
const Variant *variant_f32_skinny(int mb)
{
    static const Variant v1 = {"mmrelu_skinny<float,16x32>", MMRELU_DTYPE_F32, 16, kBN, 16, kThreads, 1, 4,
                               launch_skinny<float, 1>, 1.0f, 16};
    static const Variant v2 = {"mmrelu_skinny<float,32x32>", MMRELU_DTYPE_F32, 32, kBN, 16, kThreads, 1, 4,
                               launch_skinny<float, 2>, 1.0f, 32};
    static const Variant v4 = {"mmrelu_skinny<float,64x32>", MMRELU_DTYPE_F32, 64, kBN, 16, kThreads, 1, 4,
                               launch_skinny<float, 4>, 1.0f, 64};
    return mb == 1 ? &v1 : mb == 2 ? &v2 : &v4;
}
const Variant *variant_bf16_skinny(int mb)
{
    static const Variant v1 = {"mmrelu_skinny<bf16,16x32>", MMRELU_DTYPE_BF16, 16, kBN, 32, kThreads, 1, 8,
                               launch_skinny<uint16_t, 1>, 1.0f, 16};
    static const Variant v2 = {"mmrelu_skinny<bf16,32x32>", MMRELU_DTYPE_BF16, 32, kBN, 32, kThreads, 1, 8,
                               launch_skinny<uint16_t, 2>, 1.0f, 32};
    static const Variant v4 = {"mmrelu_skinny<bf16,64x32>", MMRELU_DTYPE_BF16, 64, kBN, 32, kThreads, 1, 8,
                               launch_skinny<uint16_t, 4>, 1.0f, 64};
    return mb == 1 ? &v1 : mb == 2 ? &v2 : &v4;
}

}  // namespace mmrelu
