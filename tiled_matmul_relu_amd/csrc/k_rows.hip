// Row softmax and row sum: the two rungs before the matmul on the lecture's
// ladder ("Kernels, Triton, XLA", section "Reductions and tiling"; the
// Chinese notes' sections 5.3 and 5.4), on the same recipe of tiles held on
// chip. Both are HBM-bound: softmax needs one read and one write of X, the
// row sum one read.
//
// Softmax: y[i][j] = exp(x[i][j] - m_i) / sum_j exp(x[i][j] - m_i) with m_i the
// row maximum (which keeps exp finite; masked entries are -inf, the
// softmax's zero). Three kernels:
//  * softmax_regs<T, TPR, E>: the row lives in registers. TPR threads per
//    row (a wave, four rows per workgroup, or the whole 256-thread
//    workgroup), E 16-byte vectors per thread, so rows up to TPR * E * 16
//    bytes: one HBM read and one write. Max and sum are reduced with lane
//    shuffles in a wave and through LDS across waves.
//  * softmax_online<T, V>: any N. Pass 1 streams the row keeping a running
//    maximum and a sum rescaled whenever the maximum grows; the per-thread
//    pairs are merged the same way. Pass 2 reads the row again and writes.
//    V = 16 / sizeof(T) elements per access when the layout allows 16-byte
//    vectors, else V = 1.
// Row sum: row_sum<T, TPR>: the pages' tiled loop, a per-thread fp32
// accumulator over 16-byte vectors, then the wave and workgroup reduction.
// Output is fp32 for both input dtypes.
//
// The per-element exponential is the hardware one (__expf: exp2 of the
// argument times log2(e) on v_exp_f32, about 2 + 1.16 |x - m| ulp); the
// rescaling factors of the two-pass merge use the accurate expf. 1/s is
// computed once per row.
#include <cmath>
#include <type_traits>

#include "kernels.hpp"
#include "device_common.hpp"
#include "../../include/mmrelu.h"

namespace mmrelu {
namespace {

constexpr int kRowThreads = 256;

template <typename T>
__device__ inline float widen(T v)
{
    if constexpr (std::is_same_v<T, float>) return v;
    else return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

template <typename T>
__device__ inline T narrow(float f)
{
    if constexpr (std::is_same_v<T, float>) return f;
    else return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));   // nearest, ties to even
}

// Reductions over `width` consecutive lanes (a power of two up to 64).
template <int WIDTH>
__device__ inline float wave_max(float v)
{
#pragma unroll
    for (int o = WIDTH / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WIDTH));
    return v;
}
template <int WIDTH>
__device__ inline float wave_sum(float v)
{
#pragma unroll
    for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, WIDTH);
    return v;
}

// Max or sum over the TPR threads of a row (TPR 64: one wave; 256: the
// workgroup, through `red`, which holds 4 floats and is reused after a barrier).
template <int TPR, bool MAX>
__device__ inline float row_reduce(float v, float *red)
{
    v = MAX ? wave_max<64>(v) : wave_sum<64>(v);
    if constexpr (TPR == 64) {
        return v;
    } else {
        const int wave = threadIdx.x >> 6;
        __syncthreads();                       // red free (a previous reduction read it)
        if ((threadIdx.x & 63) == 0) red[wave] = v;
        __syncthreads();
        float r = red[0];
#pragma unroll
        for (int w = 1; w < 4; ++w) r = MAX ? fmaxf(r, red[w]) : r + red[w];
        return r;
    }
}

template <typename T>
struct Vec {
    static constexpr int kV = 16 / sizeof(T);
};

// 16-byte load of V elements widened to float; the caller masks columns >= N.
template <typename T>
__device__ inline void load_vec(const T *p, float (&f)[Vec<T>::kV])
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

template <typename T>
__device__ inline void store_vec(T *p, const float (&f)[Vec<T>::kV])
{
    u32x4 raw;
    if constexpr (std::is_same_v<T, float>) {
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[i] = __float_as_uint(f[i]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            raw[i] = static_cast<uint32_t>(narrow<T>(f[2 * i])) | (static_cast<uint32_t>(narrow<T>(f[2 * i + 1])) << 16);
    }
    *reinterpret_cast<u32x4 *>(p) = raw;
}

// Row in registers: TPR threads per row, E vectors of V elements each;
// vector e of thread t covers columns (e * TPR + t) * V .. + V - 1, so a
// wave's accesses are consecutive 16-byte pieces. N % V == 0 and 16-byte
// aligned rows (checked by the host).
template <typename T, int TPR, int E>
__global__ __launch_bounds__(kRowThreads) void softmax_regs(const T *__restrict__ X, T *Y, int64_t M, int64_t N,
                                                           int64_t ldx, int64_t ldy)
{
    constexpr int V = Vec<T>::kV;
    constexpr int kRowsPerGroup = kRowThreads / TPR;
    __shared__ float red[4];
    const int t = threadIdx.x % TPR;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerGroup + threadIdx.x / TPR;
    const bool live = row < M;                 // uniform per row group; every thread reaches the barriers
    const T *x = X + (live ? row : 0) * ldx;
    float v[E][V];
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int64_t c = (static_cast<int64_t>(e) * TPR + t) * V;
        if (live && c < N) {
            load_vec<T>(x + c, v[e]);
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) v[e][i] = -INFINITY;
        }
#pragma unroll
        for (int i = 0; i < V; ++i) m = fmaxf(m, v[e][i]);
    }
    m = row_reduce<TPR, true>(m, red);
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
        for (int i = 0; i < V; ++i) {
            v[e][i] = __expf(v[e][i] - m);     // exp(-inf) = 0 for the masked entries
            s += v[e][i];
        }
    s = row_reduce<TPR, false>(s, red);
    const float inv = 1.0f / s;
    if (!live) return;
    T *y = Y + row * ldy;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int64_t c = (static_cast<int64_t>(e) * TPR + t) * V;
        if (c < N) {
#pragma unroll
            for (int i = 0; i < V; ++i) v[e][i] *= inv;
            store_vec<T>(y + c, v[e]);
        }
    }
}

// Merge (m2, s2) into (m, s): the sums of exp(x - m) over two sets.
__device__ inline void merge(float &m, float &s, float m2, float s2)
{
    const float mm = fmaxf(m, m2);
    if (mm == -INFINITY) return;               // both empty
    s = s * expf(m - mm) + s2 * expf(m2 - mm);
    m = mm;
}

// Any N: two passes over the row, one workgroup per row. V = 1 takes any
// layout; V = 16 / sizeof(T) needs N % V == 0 and 16-byte aligned rows.
template <typename T, int V>
__global__ __launch_bounds__(kRowThreads) void softmax_online(const T *__restrict__ X, T *Y, [[maybe_unused]] int64_t M,
                                                             int64_t N,
                                                             int64_t ldx, int64_t ldy)
{
    __shared__ float red_m[4], red_s[4];
    const int64_t row = blockIdx.x;
    const T *x = X + row * ldx;
    constexpr int64_t kStep = static_cast<int64_t>(kRowThreads) * V;
    float m = -INFINITY, s = 0.0f;
    for (int64_t c0 = 0; c0 < N; c0 += kStep) {
        const int64_t c = c0 + static_cast<int64_t>(threadIdx.x) * V;
        if (c >= N) continue;
        float f[V];
        if constexpr (V == 1) f[0] = widen<T>(x[c]);
        else load_vec<T>(x + c, f);
        float lm = f[0];
#pragma unroll
        for (int i = 1; i < V; ++i) lm = fmaxf(lm, f[i]);
        float ls = 0.0f;
#pragma unroll
        for (int i = 0; i < V; ++i) ls += __expf(f[i] - lm);
        merge(m, s, lm, ls);
    }
    // Merge across the wave, then across the four waves.
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
        merge(m, s, m2, s2);
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red_m[wave] = m;
        red_s[wave] = s;
    }
    __syncthreads();
    m = red_m[0];
    s = red_s[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) merge(m, s, red_m[w], red_s[w]);
    const float inv = 1.0f / s;
    T *y = Y + row * ldy;
    for (int64_t c0 = 0; c0 < N; c0 += kStep) {
        const int64_t c = c0 + static_cast<int64_t>(threadIdx.x) * V;
        if (c >= N) continue;
        if constexpr (V == 1) {
            y[c] = narrow<T>(__expf(widen<T>(x[c]) - m) * inv);
        } else {
            float f[V];
            load_vec<T>(x + c, f);
#pragma unroll
            for (int i = 0; i < V; ++i) f[i] = __expf(f[i] - m) * inv;
            store_vec<T>(y + c, f);
        }
    }
}

// Row sum: TPR threads per row sweep the row in tiles of TPR * V elements
// (V = 16 / sizeof(T) with 16-byte aligned rows and N % V == 0, else 1), each
// into its own fp32 accumulator, then one reduction.
template <typename T, int TPR, int V>
__global__ __launch_bounds__(kRowThreads) void row_sum(const T *__restrict__ X, float *__restrict__ out, int64_t M,
                                                      int64_t N, int64_t ldx)
{
    constexpr int kRowsPerGroup = kRowThreads / TPR;
    __shared__ float red[4];
    const int t = threadIdx.x % TPR;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerGroup + threadIdx.x / TPR;
    const bool live = row < M;
    const T *x = X + (live ? row : 0) * ldx;
    float acc = 0.0f;
    if (live) {
        for (int64_t c = static_cast<int64_t>(t) * V; c < N; c += static_cast<int64_t>(TPR) * V) {
            if constexpr (V == 1) {
                acc += widen<T>(x[c]);
            } else {
                float f[V];
                load_vec<T>(x + c, f);
#pragma unroll
                for (int i = 0; i < V; ++i) acc += f[i];
            }
        }
    }
    acc = row_reduce<TPR, false>(acc, red);
    if (live && t == 0) out[row] = acc;
}

}  // namespace

// Softmax kernel table, in the order of the variant index of the C-ABI:
//   0  row in registers, a wave per row, 4 vectors per thread
//   1  row in registers, 256 threads per row, 4 vectors per thread
//   2  row in registers, 256 threads per row, 16 vectors per thread
//   3  two passes, 16-byte vectors
//   4  two passes, single elements (any layout)
int64_t softmax_capacity(int variant, int esize)
{
    const int64_t v = 16 / esize;
    switch (variant) {
    case 0: return 64 * 4 * v;
    case 1: return 256 * 4 * v;
    case 2: return 256 * 16 * v;
    default: return INT64_MAX;
    }
}

template <typename T>
static hipError_t launch_softmax_t(int variant, const T *X, T *Y, int64_t M, int64_t N, int64_t ldx, int64_t ldy,
                                   hipStream_t s)
{
    constexpr int V = Vec<T>::kV;
    switch (variant) {
    case 0:
        hipLaunchKernelGGL((softmax_regs<T, 64, 4>), dim3(static_cast<uint32_t>((M + 3) / 4)), dim3(kRowThreads), 0, s,
                           X, Y, M, N, ldx, ldy);
        break;
    case 1:
        hipLaunchKernelGGL((softmax_regs<T, 256, 4>), dim3(static_cast<uint32_t>(M)), dim3(kRowThreads), 0, s, X, Y, M,
                           N, ldx, ldy);
        break;
    case 2:
        hipLaunchKernelGGL((softmax_regs<T, 256, 16>), dim3(static_cast<uint32_t>(M)), dim3(kRowThreads), 0, s, X, Y,
                           M, N, ldx, ldy);
        break;
    case 3:
        hipLaunchKernelGGL((softmax_online<T, V>), dim3(static_cast<uint32_t>(M)), dim3(kRowThreads), 0, s, X, Y, M, N,
                           ldx, ldy);
        break;
    default:
        hipLaunchKernelGGL((softmax_online<T, 1>), dim3(static_cast<uint32_t>(M)), dim3(kRowThreads), 0, s, X, Y, M, N,
                           ldx, ldy);
        break;
    }
    return hipGetLastError();
}

hipError_t launch_softmax(int esize, int variant, const void *X, void *Y, int64_t M, int64_t N, int64_t ldx,
                          int64_t ldy, hipStream_t s)
{
    if (esize == 4)
        return launch_softmax_t<float>(variant, static_cast<const float *>(X), static_cast<float *>(Y), M, N, ldx, ldy, s);
    return launch_softmax_t<uint16_t>(variant, static_cast<const uint16_t *>(X), static_cast<uint16_t *>(Y), M, N, ldx,
                                      ldy, s);
}

// Row sum: vectors when `vec`, a wave per row when `short_rows`.
hipError_t launch_row_sum(int esize, bool vec, bool short_rows, const void *X, float *out, int64_t M, int64_t N,
                          int64_t ldx, hipStream_t s)
{
    const uint32_t g4 = static_cast<uint32_t>((M + 3) / 4), g1 = static_cast<uint32_t>(M);
    if (esize == 4) {
        const float *x = static_cast<const float *>(X);
        if (short_rows && vec) hipLaunchKernelGGL((row_sum<float, 64, 4>), dim3(g4), dim3(kRowThreads), 0, s, x, out, M, N, ldx);
        else if (short_rows) hipLaunchKernelGGL((row_sum<float, 64, 1>), dim3(g4), dim3(kRowThreads), 0, s, x, out, M, N, ldx);
        else if (vec) hipLaunchKernelGGL((row_sum<float, 256, 4>), dim3(g1), dim3(kRowThreads), 0, s, x, out, M, N, ldx);
        else hipLaunchKernelGGL((row_sum<float, 256, 1>), dim3(g1), dim3(kRowThreads), 0, s, x, out, M, N, ldx);
    } else {
        const uint16_t *x = static_cast<const uint16_t *>(X);
        if (short_rows && vec) hipLaunchKernelGGL((row_sum<uint16_t, 64, 8>), dim3(g4), dim3(kRowThreads), 0, s, x, out, M, N, ldx);
        else if (short_rows) hipLaunchKernelGGL((row_sum<uint16_t, 64, 1>), dim3(g4), dim3(kRowThreads), 0, s, x, out, M, N, ldx);
        else if (vec) hipLaunchKernelGGL((row_sum<uint16_t, 256, 8>), dim3(g1), dim3(kRowThreads), 0, s, x, out, M, N, ldx);
        else hipLaunchKernelGGL((row_sum<uint16_t, 256, 1>), dim3(g1), dim3(kRowThreads), 0, s, x, out, M, N, ldx);
    }
    return hipGetLastError();
}

}  // namespace mmrelu
