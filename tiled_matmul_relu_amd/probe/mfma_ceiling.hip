// Measurement probe, not part of libmmrelu: the sustained rate of the bf16
// matrix cores with nothing but MFMAs in flight, on operand values taken
// from the caller's own matrices.
//
// Each workgroup has the shape of one 256 x 256 output tile of the bf16
// product (eight wave64s, two per SIMD) and each wave issues, per 32-deep
// slab, the same multiply-accumulates that wave issues in the product: a
// 128 x 64 block of fp32 accumulators updated as 8 x 4 MFMAs of 16x16x32, or
// as 4 x 2 x 2 MFMAs of 32x32x16 (the same 524288 FLOPs). The operands are
// loaded once, before the loop, from A and B (each lane 12 runs of eight
// consecutive bf16 values), so the multipliers see the matrices' own bit
// patterns; no memory is touched inside the loop. `tiles` workgroups of
// `slabs` slabs do 2 * 256 * 256 * 32 * slabs * tiles FLOPs, the work of a
// (256 tiles_m) x (256 tiles_n) x (32 slabs) product.
//
// The board's power limit lowers the clock when the multipliers toggle, so
// this rate on the workload's values is a ceiling for any kernel of the
// product on those values: a real kernel adds copies and LDS reads.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 512;
constexpr int kFrags = 12;   // 8 fragments of A and 4 of B per lane

// Run r of lane-global thread index tid: eight consecutive elements starting
// at a multiple of 8 below n8 * 8 (n8 = number of whole runs in the matrix).
__device__ inline bf16x8 load_run(const uint16_t *p, int64_t n8, uint64_t tid, int r)
{
    const uint64_t idx = ((tid * kFrags + static_cast<uint64_t>(r)) * 2654435761ull) % static_cast<uint64_t>(n8);
    return *reinterpret_cast<const bf16x8 *>(p + idx * 8);
}

template <int SHAPE>
__global__ __launch_bounds__(kThreads, 1) void mfma_ceiling(const uint16_t *__restrict__ A,
                                                            const uint16_t *__restrict__ B, int64_t na8,
                                                            int64_t nb8, int slabs, float *__restrict__ out)
{
    const uint64_t tid = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x;
    bf16x8 fa[8], fb[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) fa[i] = load_run(A, na8, tid, i);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = load_run(B, nb8, tid, 8 + j);
    float s = 0.f;
    if constexpr (SHAPE == 16) {
        f32x4 acc[8][4];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int it = 0; it < slabs; ++it) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) s += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
    } else {
        f32x16 acc[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
        for (int it = 0; it < slabs; ++it) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[2 * ks + j], fa[4 * ks + i],
                                                                            acc[i][j], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) s += acc[i][j][r];
    }
    out[tid] = s;   // keeps the chain live; one float per thread
}

}  // namespace

// Launch `tiles` workgroups of the probe on `stream`. A holds na elements and
// B nb elements (bf16 bit patterns, 16-byte aligned, at least 8 each); out
// holds tiles * 512 floats. shape is 16 (v_mfma_f32_16x16x32_bf16) or 32
// (v_mfma_f32_32x32x16_bf16). Returns 0, 1 for invalid arguments (nothing is
// launched), or 4 if the launch failed.
extern "C" int mfma_ceiling_bf16(const uint16_t *A, const uint16_t *B, int64_t na, int64_t nb, int shape,
                                 int tiles, int slabs, float *out, hipStream_t stream)
{
    if (A == nullptr || B == nullptr || out == nullptr || na < 8 || nb < 8 || tiles <= 0 || slabs < 0 ||
        (shape != 16 && shape != 32) || (reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B)) % 16)
        return 1;
    if (shape == 16)
        hipLaunchKernelGGL(mfma_ceiling<16>, dim3(tiles), dim3(kThreads), 0, stream, A, B, na / 8, nb / 8, slabs, out);
    else
        hipLaunchKernelGGL(mfma_ceiling<32>, dim3(tiles), dim3(kThreads), 0, stream, A, B, na / 8, nb / 8, slabs, out);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}
