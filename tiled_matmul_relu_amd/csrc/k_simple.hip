// Plain LDS-tiled kernel: 64x64 output tile per 256-thread workgroup, K swept
// in slabs of 16, each thread owning a 4x4 patch of the tile in registers
// (the lecture's tiled matmul with BLOCK_M = BLOCK_N = 64; fp32 multiply-add
// on the vector ALUs, no matrix cores). It accepts every shape and leading
// dimension the interface allows and serves as the reference layout for the
// matrix-core kernels. Edge tiles: loads outside M, N or K read 0 (the masked
// loads with other=0 of the lecture's listing), stores outside M x N are
// skipped, so C outside the window is never written. The epilogue adds the
// optional per-column bias to the fp32 accumulator and applies the
// activation (ReLU, GeLU's tanh form or none) before the store.
#include "kernels.hpp"
#include "device_common.hpp"
#include "../../include/mmrelu.h"

namespace mmrelu {
namespace {

constexpr int BM = 64, BN = 64, BK = 16, THREADS = 256;

template <typename T> __device__ inline float to_f32(T v);
template <> __device__ inline float to_f32<float>(float v) { return v; }
template <> __device__ inline float to_f32<uint16_t>(uint16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

template <typename T> __device__ inline T from_f32(float v);
template <> __device__ inline float from_f32<float>(float v) { return v; }
template <> __device__ inline uint16_t from_f32<uint16_t>(float v) {
    // v_cvt_pk_bf16_f32: round to nearest, ties to even
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

template <typename T>
__global__ __launch_bounds__(THREADS) void mmrelu_simple_64x64x16(
    const T *__restrict__ A, const T *__restrict__ B, T *__restrict__ C,
    int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc, int tiles_n, const T *__restrict__ bias, int act)
{
    __shared__ float As[BK][BM + 4];   // A slab stored k-major: As[k][m]
    __shared__ float Bs[BK][BN + 4];   // B slab as in memory:   Bs[k][n]

    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;
    const int64_t m0 = static_cast<int64_t>(blockIdx.x / tiles_n) * BM;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x % tiles_n) * BN;

    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
        for (int q = 0; q < (BM * BK) / THREADS; ++q) {
            const int idx = tid + q * THREADS;
            const int r = idx / BK, c = idx % BK;
            const int64_t m = m0 + r;
            const int k = k0 + c;
            As[c][r] = (m < M && k < K) ? to_f32(A[m * lda + k]) : 0.0f;
        }
#pragma unroll
        for (int q = 0; q < (BK * BN) / THREADS; ++q) {
            const int idx = tid + q * THREADS;
            const int r = idx / BN, c = idx % BN;
            const int k = k0 + r;
            const int64_t n = n0 + c;
            Bs[r][c] = (k < K && n < N) ? to_f32(B[static_cast<int64_t>(k) * ldb + n]) : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
    float bj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + tx * 4 + j;
        bj[j] = (bias != nullptr && n < N) ? to_f32(bias[n]) : 0.0f;
    }
    with_activation(act, [&](auto act_c) {
        constexpr int ACT = decltype(act_c)::value;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = m0 + ty * 4 + i;
            if (m >= M) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t n = n0 + tx * 4 + j;
                if (n < N) C[m * ldc + n] = from_f32<T>(activate<ACT>(acc[i][j] + bj[j]));
            }
        }
    });
}

template <typename T>
hipError_t launch_simple(const Problem &p, int64_t grid, hipStream_t stream)
{
    const int tiles_n = (p.N + BN - 1) / BN;
    hipLaunchKernelGGL(mmrelu_simple_64x64x16<T>, dim3(static_cast<uint32_t>(grid)), dim3(THREADS), 0, stream,
                       static_cast<const T *>(p.A), static_cast<const T *>(p.B), static_cast<T *>(p.C),
                       p.M, p.N, p.K, p.lda, p.ldb, p.ldc, tiles_n, static_cast<const T *>(p.bias), p.act);
    return hipGetLastError();
}

}  // namespace

const Variant *variant_f32_simple()
{
    static const Variant v = {"mmrelu_simple_64x64x16<float>", MMRELU_DTYPE_F32, BM, BN, BK, THREADS, 4, 0,
                            launch_simple<float>};
    return &v;
}
const Variant *variant_bf16_simple()
{
    static const Variant v = {"mmrelu_simple_64x64x16<bf16>", MMRELU_DTYPE_BF16, BM, BN, BK, THREADS, 4, 0,
                             launch_simple<uint16_t>};
    return &v;
}

}  // namespace mmrelu
