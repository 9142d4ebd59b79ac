// bf16 relu(A·B) on the gfx950 matrix cores, "ping-pong" schedule: eight
// wave64s per 256 x 256 output tile, two on each SIMD, split into two groups
// of four. Between two consecutive barriers one group only runs MFMAs while
// the other only reads operand fragments from LDS and issues global->LDS
// copies; at the barrier the roles swap. Each SIMD therefore always has one
// wave feeding its matrix core and one wave doing memory work, and the
// hardware issues both streams side by side.
//
// The arithmetic is the lecture's tiled matmul with the fused activation
// ("Kernels, Triton, XLA", section "Reductions and tiling", and the Chinese
// notes' section 5.5): per output tile, K is swept in slabs staged in LDS,
// fp32 accumulation (v_mfma_f32_16x16x32_bf16), ReLU on the accumulator, one
// rounding to bf16 (nearest, ties to even), one masked store.
//
// Layout: wave w belongs to group w / 4; within a group, waves (wm, wn') =
// ((w%4)/2, (w%4)%2) and the wave owns rows 128*wm .. +128 and columns
// 64*(wn' + 2*group) .. +64 of the tile (8 x 4 MFMA blocks, 128 fp32
// accumulators per lane). LDS stages, fragment reads, the transposed B reads
// (ds_read_b64_tr_b16) and the copy layout are those of the four-wave kernel
// in k_bf16_mfma.hip. Group 0 copies the B half of every slab, group 1 the
// A half.
//
// Schedule (S stages, slabs of 32 along K; interval I_t ends at a barrier):
//   prologue: every wave copies its half of slabs 0 .. S-2; wait; barrier;
//             I_-1: group 0 reads slab 0, copies its half of slab S-1.
//   I_2k:   group 0 multiplies slab k;
//           group 1 reads slab k, copies its half of slab k+S-1.
//           Both then wait until slab k+1 has landed (slabs up to k+S-2 may
//           stay in flight: vmcnt((S-2) * 4)).
//   I_2k+1: group 0 reads slab k+1, copies its half of slab k+S;
//           group 1 multiplies slab k.
// Slab j's stage is refilled (with slab j+S) from I_2j+1 on: by then group 0
// read it in I_2j-1 and group 1 in I_2j. Copies past K are fully masked and
// only zero-fill a stage that is never read, so every slab costs the same
// vmcnt count and the loop has no data-dependent branches.
//
// Requires lda, ldb, ldc, K and N to be multiples of 8 and 16-byte aligned
// pointers.
#include <type_traits>

#include "kernels.hpp"
#include "device_common.hpp"
#include "../../include/mmrelu.h"

namespace mmrelu {
namespace {

constexpr int kBM = 256, kBN = 256, kBK = 32;
constexpr int kThreads = 512;
constexpr int kMB = 8, kNB = 4;                 // MFMA blocks per wave: 128 x 64
constexpr int kCA = kBK / 8;                    // 16-byte k chunks per A row
constexpr int kCB = kBN / 8;                    // 16-byte chunks per B row
constexpr int kStageA = kBM * kBK;              // elements
constexpr int kStage = kBM * kBK + kBK * kBN;   // elements per stage
constexpr int kCopies = 4;                      // 1 KB copies per wave per slab

__device__ inline int swz_b(int k) { return ((k & 3) << 1) | (((k >> 3) & 1) << 3); }

template <int STAGES>
__global__ __launch_bounds__(kThreads, 1) void mmrelu_bf16_pingpong(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, uint16_t *__restrict__ C,
    int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc, int tiles_m, int tiles_n, int group_m)
{
    static_assert((STAGES & (STAGES - 1)) == 0 && STAGES >= 3, "power-of-two ring of at least three stages");
    static_assert(kCopies * STAGES <= 63, "copies in flight must fit the vmcnt counter");
    __shared__ __attribute__((aligned(1024))) uint16_t lds[STAGES * kStage];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave >> 2, wl = wave & 3;
    const int wm = wl >> 1, wn = (wl & 1) + 2 * grp;
    const int g = lane >> 4, t = lane & 15;

    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * kBM, n0 = tn * kBN;
    const uint32_t lds0 = lds_address(lds);

    // Copy plan: copy q of wave wl of a group fills 1 KB block 4q + wl of the
    // group's half of a stage (group 1: A, 16 rows x 4 k chunks, chunk-major;
    // group 0: B, two 512-byte rows). Edges in M and N are folded into the
    // offsets once; B rows past K fall outside the rebased B resource; A
    // chunks past K are tested per slab.
    const rsrc_t ra = make_rsrc(A + static_cast<int64_t>(m0) * lda, ((static_cast<int64_t>(M) - 1 - m0) * lda + K) * 2);
    uint32_t voff[kCopies];
    int a_col[kCopies];
#pragma unroll
    for (int q = 0; q < kCopies; ++q) {
        const int blk = 4 * q + wl;
        if (grp == 1) {
            const int row = blk * 16 + (lane & 15);
            const int col = (lane >> 4) * 8;
            a_col[q] = col;
            voff[q] = (m0 + row < M) ? static_cast<uint32_t>((row * lda + col) * 2) : kOutOfRange;
        } else {
            const int row = blk * 2 + (lane >> 5);
            const int col = ((lane & 31) ^ swz_b(row)) * 8;
            a_col[q] = 0;
            voff[q] = (n0 + col < N) ? static_cast<uint32_t>((row * ldb + col) * 2) : kOutOfRange;
        }
    }
    // This wave's half of slab `slab` into its stage.
    auto copy_half = [&](int slab) __attribute__((always_inline)) {
        const int k0 = slab * kBK;
        const uint32_t st = lds0 + (slab & (STAGES - 1)) * (kStage * 2);
        if (grp == 1) {
#pragma unroll
            for (int q = 0; q < kCopies; ++q) {
                const uint32_t off = (a_col[q] < K - k0) ? voff[q] : kOutOfRange;
                load_to_lds<16>(ra, st + (4 * q + wl) * 1024, off, static_cast<uint32_t>(k0) * 2);
            }
        } else {
            const rsrc_t rb = make_rsrc(B + static_cast<int64_t>(k0) * ldb + n0,
                                        ((static_cast<int64_t>(K) - 1 - k0) * ldb + N - n0) * 2);
#pragma unroll
            for (int q = 0; q < kCopies; ++q)
                load_to_lds<16>(rb, st + kStageA * 2 + (4 * q + wl) * 1024, voff[q]);
        }
    };

    // Fragment read plan (element offsets into a stage), as in the four-wave
    // kernel: A block i at rows wm*128 + 16i + t, chunk g; B block j at
    // columns wn*64 + 16j + 4(t%4), rows 8g + t/4 (+4h).
    const int a_off = ((wm * kMB * kCA + g) * 16 + t) * 8;
    int b_off[kNB];
    {
        const int k_lane = 8 * g + (t >> 2);
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
            const int n = wn * 64 + j * 16 + 4 * (t & 3);
            b_off[j] = kStageA + k_lane * kBN + (((n >> 3) ^ swz_b(k_lane)) << 3) + (n & 7);
        }
    }

    bf16x8 fa[kMB], fb[kNB];
    auto read_frags = [&](int slab) __attribute__((always_inline)) {
        const uint16_t *st = lds + (slab & (STAGES - 1)) * kStage;
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
            i16x4 half[2];
#pragma unroll
            for (int h = 0; h < 2; ++h)
                half[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MMRELU_LDS i16x4 *)(st + b_off[j] + 4 * h * kBN));
            fb[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int i = 0; i < kMB; ++i) fa[i] = *reinterpret_cast<const bf16x8 *>(st + a_off + i * 16 * kBK);
    };

    f32x4 acc[kMB][kNB];
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto mfmas = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kMB; ++i)
#pragma unroll
            for (int j = 0; j < kNB; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
    };
    // End of an interval. The fences keep each interval's work between its
    // barriers (MFMAs touch no memory and would otherwise be moved across).
    auto interval_end = [&](bool wait_copies) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        if (wait_copies) wait_vmcnt<(STAGES - 2) * kCopies>();
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    };

    // Each group runs its own loop (one copy of the fragment registers and
    // the MFMA chain per code path); both execute the same barriers.
    const int nk = (K + kBK - 1) / kBK;
    if (nk > 0) {
#pragma unroll
        for (int s = 0; s + 1 < STAGES; ++s) copy_half(s);
        interval_end(true);                          // slab 0 has landed
        if (grp == 0) {
            read_frags(0);                           // I_-1
            copy_half(STAGES - 1);
            interval_end(false);
            for (int k = 0; k < nk; ++k) {
                mfmas();                             // I_2k
                interval_end(true);                  // slab k+1 has landed
                if (k + 1 < nk) read_frags(k + 1);   // I_2k+1
                copy_half(k + STAGES);
                interval_end(false);
            }
        } else {
            interval_end(false);                     // I_-1
            for (int k = 0; k < nk; ++k) {
                read_frags(k);                       // I_2k
                copy_half(k + STAGES - 1);
                interval_end(true);                  // slab k+1 has landed
                mfmas();                             // I_2k+1
                interval_end(false);
            }
        }
    }

    // Epilogue: lane (g, t) of block (i, j) holds C[row][col .. col+3]; ReLU
    // on fp32, round to bf16, one 8-byte masked store.
    const __amdgpu_buffer_rsrc_t rc = make_store_rsrc(C + static_cast<int64_t>(m0) * ldc + n0,
                                                      ((static_cast<int64_t>(M) - 1 - m0) * ldc + N - n0) * 2);
#pragma unroll
    for (int i = 0; i < kMB; ++i) {
        const int row = wm * 128 + i * 16 + t;
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
            const int col = wn * 64 + j * 16 + 4 * g;
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

template <int STAGES, int GROUP_M>
hipError_t launch_pingpong(const Problem &p, int64_t grid, hipStream_t stream)
{
    const int tiles_m = (p.M + kBM - 1) / kBM, tiles_n = (p.N + kBN - 1) / kBN;
    hipLaunchKernelGGL((mmrelu_bf16_pingpong<STAGES>), dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t *>(p.A), static_cast<const uint16_t *>(p.B),
                       static_cast<uint16_t *>(p.C), p.M, p.N, p.K, p.lda, p.ldb, p.ldc, tiles_m, tiles_n, GROUP_M);
    return hipGetLastError();
}

}  // namespace

const Variant *variant_bf16_pingpong256()
{
    static const Variant v = {"mmrelu_bf16_pingpong<256,256,32,4>", MMRELU_DTYPE_BF16, 256, 256, 32, 512, 1, 8,
                              launch_pingpong<4, 4>};
    return &v;
}

}  // namespace mmrelu
