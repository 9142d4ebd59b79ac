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
// reads and writes whole lines on both sides. A row padded to 65 elements
// keeps the column walk off a single LDS bank.
#include "kernels.hpp"

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

}  // namespace

hipError_t launch_pack(int esize, const void *src, void *dst, int64_t rows, int64_t cols, int64_t s_r,
                       int64_t s_c, int64_t d_r, int64_t d_c, hipStream_t stream)
{
    if (rows <= 0 || cols <= 0) return hipSuccess;
    const int64_t tiles_c = (cols + kTile - 1) / kTile;
    const int64_t tiles = ((rows + kTile - 1) / kTile) * tiles_c;
    const uint32_t grid = static_cast<uint32_t>(tiles < 65536 ? tiles : 65536);
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
