// Strided 2-D copy, dst[r][c] = src[r][c] with an element stride per
// dimension on each side. The general-stride entry points use it to bring an
// operand stored in any layout into the row-major layout the matrix-core
// kernels read, and to write a row-major product out to a strided C. The
// lecture describes a stored matrix by its two strides, a transpose being
// the same data with them exchanged ("Kernels, Triton, XLA", section
// "Reductions and tiling").
//
// The copy is HBM-bound (one read and one write per element). Each workgroup
// moves 64 x 64 tiles through LDS: the loads walk the source along its unit
// stride and the stores walk the destination along its own, so a transpose
// reads and writes whole lines on both sides. The general kernel moves single
// elements (a row padded to 65 keeps its column walk off a single LDS bank);
// a transpose between 16-byte aligned layouts moves 16-byte pieces.
#include "kernels.hpp"
#include "device_common.hpp"

namespace mmrelu {
namespace {

constexpr int kTile = 64, kPackThreads = 256, kPer = kTile * kTile / kPackThreads;   // 16 elements per thread

template <typename T>
__global__ __launch_bounds__(kPackThreads) void pack2d(const T *__restrict__ src, T *__restrict__ dst,
                                                       int64_t rows, int64_t cols, int64_t s_r, int64_t s_c,
                                                       int64_t d_r, int64_t d_c, int64_t tiles_c, int64_t tiles,
                                                       int src_cols_fast, int dst_cols_fast)
{
    __shared__ T tile[kTile][kTile + 1];
    for (int64_t id = blockIdx.x; id < tiles; id += gridDim.x) {   // uniform trip count per workgroup
        const int64_t r0 = (id / tiles_c) * kTile, c0 = (id % tiles_c) * kTile;
        T v[kPer];
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int idx = e * kPackThreads + static_cast<int>(threadIdx.x);
            const int fast = idx % kTile, slow = idx / kTile;
            const int rr = src_cols_fast ? slow : fast, cc = src_cols_fast ? fast : slow;
            const int64_t r = r0 + rr, c = c0 + cc;
            v[e] = (r < rows && c < cols) ? src[r * s_r + c * s_c] : T(0);
        }
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int idx = e * kPackThreads + static_cast<int>(threadIdx.x);
            const int fast = idx % kTile, slow = idx / kTile;
            const int rr = src_cols_fast ? slow : fast, cc = src_cols_fast ? fast : slow;
            tile[rr][cc] = v[e];
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int idx = e * kPackThreads + static_cast<int>(threadIdx.x);
            const int fast = idx % kTile, slow = idx / kTile;
            const int rr = dst_cols_fast ? slow : fast, cc = dst_cols_fast ? fast : slow;
            const int64_t r = r0 + rr, c = c0 + cc;
            if (r < rows && c < cols) dst[r * d_r + c * d_c] = tile[rr][cc];
        }
        __syncthreads();
    }
}

// Transpose with 16-byte accesses on both sides: the source is contiguous
// down its columns (s_r == 1) and the destination along its rows (d_c == 1),
// both 16-byte aligned (s_c and d_r multiples of V = 16 / sizeof(T)). Full
// 64 x 64 tiles go through LDS as vectors; edge tiles take the element path.
//
// LDS holds the tile in the source's orientation, one 64-element row per
// source column c, in 16-byte chunks of V rows. Chunk k of column c is stored
// at chunk k ^ (c / V) (mod 64 / V), so that the store phase, where a lane
// reads V consecutive columns of one row, finds the lanes of one instruction
// on distinct banks (the V columns of one lane group differ in c / V).
template <typename T>
__global__ __launch_bounds__(kPackThreads) void pack2d_t16(const T *__restrict__ src, T *__restrict__ dst,
                                                           int64_t rows, int64_t cols, int64_t s_c, int64_t d_r,
                                                           int64_t tiles_c, int64_t tiles)
{
    constexpr int V = 16 / sizeof(T), CH = kTile / V;        // elements per chunk, chunks per tile row
    constexpr int kVecs = kTile * CH / kPackThreads;          // 16-byte pieces per thread (2 bf16, 4 fp32)
    __shared__ __attribute__((aligned(16))) T tile[kTile * kTile];
    for (int64_t id = blockIdx.x; id < tiles; id += gridDim.x) {
        const int64_t r0 = (id / tiles_c) * kTile, c0 = (id % tiles_c) * kTile;
        if (r0 + kTile <= rows && c0 + kTile <= cols) {
            u32x4 v[kVecs];
#pragma unroll
            for (int e = 0; e < kVecs; ++e) {
                const int idx = e * kPackThreads + static_cast<int>(threadIdx.x);
                const int k = idx % CH, c = idx / CH;             // chunk k of rows, column c
                v[e] = *reinterpret_cast<const u32x4 *>(src + (r0 + k * V) + (c0 + c) * s_c);
            }
#pragma unroll
            for (int e = 0; e < kVecs; ++e) {
                const int idx = e * kPackThreads + static_cast<int>(threadIdx.x);
                const int k = idx % CH, c = idx / CH;
                *reinterpret_cast<u32x4 *>(tile + c * kTile + ((k ^ (c / V)) % CH) * V) = v[e];
            }
            __syncthreads();
#pragma unroll
            for (int e = 0; e < kVecs; ++e) {
                const int idx = e * kPackThreads + static_cast<int>(threadIdx.x);
                const int cg = idx % CH, r = idx / CH;            // columns cg*V .. +V-1 of row r
                T out[V];
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    const int c = cg * V + i;
                    out[i] = tile[c * kTile + (((r / V) ^ (c / V)) % CH) * V + r % V];
                }
                *reinterpret_cast<u32x4 *>(dst + (r0 + r) * d_r + c0 + cg * V) = __builtin_bit_cast(u32x4, out);
            }
            __syncthreads();
        } else {
            // Edge tile: element by element, both sides along their unit stride.
            T *t2 = tile;
#pragma unroll
            for (int e = 0; e < kPer; ++e) {
                const int idx = e * kPackThreads + static_cast<int>(threadIdx.x);
                const int rr = idx % kTile, cc = idx / kTile;
                const int64_t r = r0 + rr, c = c0 + cc;
                t2[cc * kTile + rr] = (r < rows && c < cols) ? src[r + c * s_c] : T(0);
            }
            __syncthreads();
#pragma unroll
            for (int e = 0; e < kPer; ++e) {
                const int idx = e * kPackThreads + static_cast<int>(threadIdx.x);
                const int cc = idx % kTile, rr = idx / kTile;
                const int64_t r = r0 + rr, c = c0 + cc;
                if (r < rows && c < cols) dst[r * d_r + c] = t2[cc * kTile + rr];
            }
            __syncthreads();
        }
    }
}

}  // namespace

hipError_t launch_pack(int esize, const void *src, void *dst, int64_t rows, int64_t cols, int64_t s_r,
                       int64_t s_c, int64_t d_r, int64_t d_c, hipStream_t stream)
{
    if (rows <= 0 || cols <= 0) return hipSuccess;
    const int64_t tiles_c = (cols + kTile - 1) / kTile;
    const int64_t tiles = ((rows + kTile - 1) / kTile) * tiles_c;
    const uint32_t grid = static_cast<uint32_t>(tiles < 65536 ? tiles : 65536);
    // A transpose between 16-byte aligned layouts takes the vector kernel; the
    // other direction (source along rows, destination down columns) is the
    // same copy with rows and columns exchanged.
    const int64_t v = 16 / esize;
    auto al16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    auto t16 = [&](const void *sp, void *dp, int64_t nr, int64_t nc, int64_t sc, int64_t dr) {
        const int64_t tc = (nc + kTile - 1) / kTile, tt = ((nr + kTile - 1) / kTile) * tc;
        const uint32_t g = static_cast<uint32_t>(tt < 65536 ? tt : 65536);
        if (esize == 4)
            hipLaunchKernelGGL(pack2d_t16<float>, dim3(g), dim3(kPackThreads), 0, stream, static_cast<const float *>(sp),
                               static_cast<float *>(dp), nr, nc, sc, dr, tc, tt);
        else
            hipLaunchKernelGGL(pack2d_t16<uint16_t>, dim3(g), dim3(kPackThreads), 0, stream,
                               static_cast<const uint16_t *>(sp), static_cast<uint16_t *>(dp), nr, nc, sc, dr, tc, tt);
        return hipGetLastError();
    };
    if (al16(src) && al16(dst)) {
        if (s_r == 1 && d_c == 1 && s_c % v == 0 && d_r % v == 0) return t16(src, dst, rows, cols, s_c, d_r);
        if (s_c == 1 && d_r == 1 && s_r % v == 0 && d_c % v == 0) return t16(src, dst, cols, rows, s_r, d_c);
    }
    // Walk each side along its unit stride; with neither stride 1, along columns.
    const int src_cols_fast = !(s_r == 1 && s_c != 1);
    const int dst_cols_fast = !(d_r == 1 && d_c != 1);
    if (esize == 4) {
        hipLaunchKernelGGL(pack2d<float>, dim3(grid), dim3(kPackThreads), 0, stream, static_cast<const float *>(src),
                           static_cast<float *>(dst), rows, cols, s_r, s_c, d_r, d_c, tiles_c, tiles, src_cols_fast,
                           dst_cols_fast);
    } else {
        hipLaunchKernelGGL(pack2d<uint16_t>, dim3(grid), dim3(kPackThreads), 0, stream,
                           static_cast<const uint16_t *>(src), static_cast<uint16_t *>(dst), rows, cols, s_r, s_c,
                           d_r, d_c, tiles_c, tiles, src_cols_fast, dst_cols_fast);
    }
    return hipGetLastError();
}

}  // namespace mmrelu
