// bf16 act(A·B + bias) on the matrix cores for any layout: leading
// dimensions, N and K need not be multiples of 8 nor rows 16-byte aligned,
// which every other bf16 matrix-core kernel here requires. The lecture's
// tiled recipe ("Kernels, Triton, XLA", section "Reductions and tiling") with
// masked element loads:
//  * BT x BT output tile (BT = 64 or 128) per workgroup of four waves
//    (2 x 2), each wave a BT/2 x BT/2 sub-tile as blocks of
//    v_mfma_f32_16x16x32_bf16; K in slabs of 32.
//  * Each thread loads BT/8 elements of the A slab and as many of the B slab with
//    bounds checks (zero outside M, N, K: the masked load with other = 0),
//    one slab ahead in registers, and writes them to the other half of a
//    double-buffered LDS. B is written transposed (column n holds its 32 k
//    contiguously), so both operands' fragments (8 consecutive k of one row
//    of A or one column of B) are single 16-byte LDS reads.
//  * Epilogue as in the other kernels (bias, activation, one rounding to
//    bf16), with a store per element so that any ldc works.
// The element loads bound it well below the aligned kernels; it exists so
// that no bf16 shape falls back to the plain (non-matrix-core) kernel.
#include <type_traits>

#include "kernels.hpp"
#include "device_common.hpp"
#include "../../include/mmrelu.h"

namespace mmrelu {
namespace {

constexpr int kAnyBK = 32, kAnyThreads = 256;
constexpr int kPitch = kAnyBK + 8;             // LDS row pitch in elements (80 bytes, 16-byte aligned)

__device__ inline float bf16f(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }

// BT x BT output tile; four waves of (BT/2) x (BT/2), each NBLK x NBLK blocks.
template <int BT>
__global__ __launch_bounds__(kAnyThreads, 2) void mmrelu_bf16_any(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, uint16_t *__restrict__ C, int M, int N, int K,
    int64_t lda, int64_t ldb, int64_t ldc, int tiles_m, int tiles_n, int group_m, const uint16_t *__restrict__ bias,
    int act)
{
    constexpr int kAnyBM = BT, kAnyBN = BT, NBLK = BT / 32;
    constexpr int kPer = kAnyBM * kAnyBK / kAnyThreads;   // elements of A (and of B) per thread per slab
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kAnyBM * kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t Bt[2][kAnyBN * kPitch];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int g = lane >> 4, t = lane & 15;
    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * kAnyBM, n0 = tn * kAnyBN;

    // Slab loads: element e of this thread is A[m0 + r][k0 + k] with
    // (r, k) = divmod(e * 256 + tid, 32), and B[k0 + k][n0 + n] with
    // (k, n) = divmod(e * 256 + tid, BT): consecutive threads read
    // consecutive columns of a row.
    uint16_t ra[kPer], rb[kPer];
    auto load = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int idx = e * kAnyThreads + static_cast<int>(threadIdx.x);
            const int r = idx / kAnyBK, k = idx % kAnyBK;
            const int gm = m0 + r, gk = k0 + k;
            ra[e] = (gm < M && gk < K) ? A[static_cast<int64_t>(gm) * lda + gk] : uint16_t(0);
            const int kb = idx / kAnyBN, n = idx % kAnyBN;
            const int gkb = k0 + kb, gn = n0 + n;
            rb[e] = (gkb < K && gn < N) ? B[static_cast<int64_t>(gkb) * ldb + gn] : uint16_t(0);
        }
    };
    auto store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int idx = e * kAnyThreads + static_cast<int>(threadIdx.x);
            As[buf][(idx / kAnyBK) * kPitch + idx % kAnyBK] = ra[e];
            Bt[buf][(idx % kAnyBN) * kPitch + idx / kAnyBN] = rb[e];   // transposed: column n, row k
        }
    };

    f32x4 acc[NBLK][NBLK];
#pragma unroll
    for (int i = 0; i < NBLK; ++i)
#pragma unroll
        for (int j = 0; j < NBLK; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (K + kAnyBK - 1) / kAnyBK;
    load(0);
    store(0);
    __syncthreads();
    for (int s = 0; s < nk; ++s) {
        const int buf = s & 1;
        if (s + 1 < nk) load((s + 1) * kAnyBK);            // next slab in flight during the MFMAs
        bf16x8 fa[NBLK], fb[NBLK];
#pragma unroll
        for (int i = 0; i < NBLK; ++i)
            fa[i] = *reinterpret_cast<const bf16x8 *>(&As[buf][(wm * (BT / 2) + i * 16 + t) * kPitch + 8 * g]);
#pragma unroll
        for (int j = 0; j < NBLK; ++j)
            fb[j] = *reinterpret_cast<const bf16x8 *>(&Bt[buf][(wn * (BT / 2) + j * 16 + t) * kPitch + 8 * g]);
#pragma unroll
        for (int i = 0; i < NBLK; ++i)
#pragma unroll
            for (int j = 0; j < NBLK; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
        if (s + 1 < nk) store(buf ^ 1);                     // the other half: last read two slabs ago
        __syncthreads();
    }

    // Lane (g, t) of block (i, j) holds C[row t][cols 4g .. 4g+3] of the block.
    with_activation(act, [&](auto act_c) __attribute__((always_inline)) {
        constexpr int ACT = decltype(act_c)::value;
#pragma unroll
        for (int i = 0; i < NBLK; ++i) {
            const int row = m0 + wm * (BT / 2) + i * 16 + t;
            if (row >= M) continue;
#pragma unroll
            for (int j = 0; j < NBLK; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int col = n0 + wn * (BT / 2) + j * 16 + 4 * g + r;
                    if (col >= N) continue;
                    const float b = bias != nullptr ? bf16f(bias[col]) : 0.0f;
                    const float o = activate<ACT>(acc[i][j][r] + b);
                    C[static_cast<int64_t>(row) * ldc + col] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(o));
                }
        }
    });
}

template <int BT>
hipError_t launch_bf16_any(const Problem &p, int64_t grid, hipStream_t stream)
{
    const int tiles_m = (p.M + BT - 1) / BT, tiles_n = (p.N + BT - 1) / BT;
    hipLaunchKernelGGL(mmrelu_bf16_any<BT>, dim3(static_cast<uint32_t>(grid)), dim3(kAnyThreads), 0, stream,
                       static_cast<const uint16_t *>(p.A), static_cast<const uint16_t *>(p.B),
                       static_cast<uint16_t *>(p.C), p.M, p.N, p.K, p.lda, p.ldb, p.ldc, tiles_m, tiles_n, 8,
                       static_cast<const uint16_t *>(p.bias), p.act);
    return hipGetLastError();
}

}  // namespace

// 64x64 or 128x128 tiles, any layout.
const Variant *variant_bf16_any(int bt)
{
    static const Variant v64 = {"mmrelu_bf16_any<64,64,32>", MMRELU_DTYPE_BF16, 64, 64, kAnyBK, kAnyThreads, 2, 0,
                                launch_bf16_any<64>, 1.0f};
    static const Variant v128 = {"mmrelu_bf16_any<128,128,32>", MMRELU_DTYPE_BF16, 128, 128, kAnyBK, kAnyThreads, 2, 0,
                                 launch_bf16_any<128>, 1.0f};
    return bt == 64 ? &v64 : &v128;
}

}  // namespace mmrelu
