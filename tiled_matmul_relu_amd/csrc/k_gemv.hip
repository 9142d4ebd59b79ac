// act(A·B + bias) one output at a time, for products with a single (or very
// few) output columns: N = 1 is a matrix-vector product, C[i] =
// act(sum_k A[i][k] B[k] + bias), and B and C then have unit leading
// dimensions, which no 16-byte-vector tile kernel accepts. The work is one
// read of A (M x K) from HBM; the lecture's naive kernel, one output
// element per thread block reading its row and column ("Kernels, Triton,
// XLA", section "Reductions and tiling"), is here the efficient form because
// A is read once whatever the order.
//
// One wave per output: a workgroup of four waves covers four rows of one
// column of C, so the grid is ceil(M / 4) x N (block 4 x 1 in the planner's
// terms) and any shape is covered. A wave sweeps its row of A in 16-byte
// pieces (8 bf16 / 4 fp32 per lane, 64 lanes side by side, several pieces in
// flight) when rows are 16-byte aligned, else element by element; the
// matching B values come from L2 (B is K x N and small here), in the same
// 16-byte pieces when B is one contiguous column. fp32
// accumulation, a shuffle reduction, then bias, activation and one store.
#include <type_traits>

#include "kernels.hpp"
#include "device_common.hpp"
#include "../../include/mmrelu.h"

namespace mmrelu {
namespace {

constexpr int kGemvThreads = 256, kGemvRows = 4;

template <typename T>
__device__ inline float elem(const T *p)
{
    if constexpr (std::is_same_v<T, float>) return *p;
    else return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}

// 16 bytes of A (or B) widened to floats.
template <typename T>
__device__ inline void load16(const T *p, float (&f)[16 / sizeof(T)])
{
    const u32x4 raw = *reinterpret_cast<const u32x4 *>(p);
    if constexpr (std::is_same_v<T, float>) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(raw[i]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(raw[i] << 16);
            f[2 * i + 1] = __uint_as_float(raw[i] & 0xFFFF0000u);
        }
    }
}

// VEC: 16-byte loads of A (lda and K multiples of 16 / sizeof(T), A 16-byte
// aligned). BVEC (with VEC): B is a contiguous, 16-byte aligned column
// (ldb = 1, N = 1) and is read in the same 16-byte pieces; otherwise B is
// read element by element with stride ldb.
template <typename T, bool VEC, bool BVEC>
__global__ __launch_bounds__(kGemvThreads) void mmrelu_gemv(const T *__restrict__ A, const T *__restrict__ B,
                                                           T *__restrict__ C, int M, [[maybe_unused]] int N, int K,
                                                           int64_t lda,
                                                           int64_t ldb, int64_t ldc, const T *__restrict__ bias,
                                                           int act)
{
    constexpr int V = VEC ? 16 / static_cast<int>(sizeof(T)) : 1;
    constexpr int kUnroll = 4;                 // pieces in flight per lane
    const int lane = threadIdx.x & 63;
    const int64_t tiles_m = (static_cast<int64_t>(M) + kGemvRows - 1) / kGemvRows;
    const int64_t tm = blockIdx.x % tiles_m, col = blockIdx.x / tiles_m;
    const int64_t row = tm * kGemvRows + (threadIdx.x >> 6);
    if (row >= M) return;                      // whole wave; no barriers in this kernel
    const T *a = A + row * lda;
    const T *b = B + col;
    float acc = 0.0f;
    constexpr int64_t kStep = 64 * V;
    int64_t k0 = static_cast<int64_t>(lane) * V;
    for (; k0 + (kUnroll - 1) * kStep < K; k0 += kUnroll * kStep) {
        float av[kUnroll][V], bv[kUnroll][V];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t k = k0 + u * kStep;
            if constexpr (VEC) load16<T>(a + k, av[u]);
            else av[u][0] = elem(a + k);
            if constexpr (BVEC) {
                load16<T>(b + k, bv[u]);
            } else {
#pragma unroll
                for (int i = 0; i < V; ++i) bv[u][i] = elem(b + (k + i) * ldb);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int i = 0; i < V; ++i) acc += av[u][i] * bv[u][i];
    }
    for (; k0 < K; k0 += kStep) {              // the tail, one piece at a time
        if constexpr (VEC) {
#pragma unroll
            for (int i = 0; i < V; ++i) acc += elem(a + k0 + i) * elem(b + (k0 + i) * ldb);
        } else {
            acc += elem(a + k0) * elem(b + k0 * ldb);
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (lane != 0) return;
    if (bias != nullptr) acc += elem(bias + col);
    with_activation(act, [&](auto act_c) __attribute__((always_inline)) {
        constexpr int ACT = decltype(act_c)::value;
        const float o = activate<ACT>(acc);
        if constexpr (std::is_same_v<T, float>) C[row * ldc + col] = o;
        else C[row * ldc + col] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(o));
    });
}

template <typename T>
hipError_t launch_gemv(const Problem &p, int64_t grid, hipStream_t stream)
{
    constexpr int64_t V = 16 / sizeof(T);
    const bool vec = p.K % V == 0 && p.lda % V == 0 && (reinterpret_cast<uintptr_t>(p.A) & 15) == 0;
    auto args = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(grid)), dim3(kGemvThreads), 0, stream,
                           static_cast<const T *>(p.A), static_cast<const T *>(p.B), static_cast<T *>(p.C), p.M, p.N,
                           p.K, p.lda, p.ldb, p.ldc, static_cast<const T *>(p.bias), p.act);
    };
    const bool bvec = vec && p.N == 1 && p.ldb == 1 && (reinterpret_cast<uintptr_t>(p.B) & 15) == 0;
    if (bvec) args(mmrelu_gemv<T, true, true>);
    else if (vec) args(mmrelu_gemv<T, true, false>);
    else args(mmrelu_gemv<T, false, false>);
    return hipGetLastError();
}

}  // namespace

// Four rows by one column per workgroup; any layout.
const Variant *variant_f32_gemv()
{
    static const Variant v = {"mmrelu_gemv<float>", MMRELU_DTYPE_F32, kGemvRows, 1, 64, kGemvThreads, 8, 0,
                              launch_gemv<float>, 1.0f};
    return &v;
}
const Variant *variant_bf16_gemv()
{
    static const Variant v = {"mmrelu_gemv<bf16>", MMRELU_DTYPE_BF16, kGemvRows, 1, 64, kGemvThreads, 8, 0,
                              launch_gemv<uint16_t>, 1.0f};
    return &v;
}

}  // namespace mmrelu
