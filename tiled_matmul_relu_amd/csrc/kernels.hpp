// Launch interface shared by the kernel translation units and the C-ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace mmrelu {

// Validated problem description handed to every launcher. Sizes fit int32
// (checked by the C-ABI layer); leading dimensions are in elements.
struct Problem {
    const void *A;
    const void *B;
    void *C;
    int32_t M, N, K;
    int64_t lda, ldb, ldc;
    const void *bias;   // N elements of the input dtype, or null
    int32_t act;        // activation code of mmrelu.h (0 ReLU, 1 GeLU tanh, 2 none)
};

// Launches one variant over `grid` workgroups on `stream`; returns the launch
// status (hipGetLastError right after the launch).
using Launcher = hipError_t (*)(const Problem &, int64_t grid, hipStream_t stream);

struct Variant {
    const char *name;     // kernel symbol family, as a profiler shows it
    int dtype;            // MMRELU_DTYPE_*
    int block_m, block_n, block_k;
    int threads;
    int wg_per_cu;        // resident workgroups per CU (register / LDS bound)
    int align_elems;      // 0: any layout; else lda, ldb, ldc, K, N must be
                          // multiples of this and A, B, C 16-byte aligned
    Launcher launch;
    // Measured time per output element of a full tile, relative to the
    // dtype's fastest kernel (the planner's cost model).
    float rel_cost = 1.0f;
};

// Kernel variants, defined in the kernel translation units (host functions
// returning static descriptors).
const Variant *variant_f32_simple();
const Variant *variant_bf16_simple();
const Variant *variant_f32_mfma128();
const Variant *variant_f32_mfma128_unaligned();
const Variant *variant_f32_mfma64();
const Variant *variant_f32_mfma64_unaligned();
const Variant *variant_bf16_pingpong256();   // k_bf16_pingpong.hip
const Variant *variant_bf16_pingpong128();
const Variant *variant_bf16_mfma128();       // k_bf16_mfma.hip
// Skinny kernels (k_skinny.hip), tiles of 16 mb x 16 nb with K split over
// the eight waves and ks k blocks per slab: (mb, nb, ks) = (1, 2, 1),
// (2, 2, 1), (4, 2, 2 for fp32 / 1 for bf16) for skinny M, (2, 1, 2),
// (2, 2, 2), (2, 4, 2) for skinny N, and (4, 4, 2), a 64 x 64 tile for
// small squares and long-K products with few output tiles, (1, 4, 1),
// 16 x 64 strips for few rows and many columns, and (fp32) (4, 1, 2), 64 x 16
// bands for few columns and many rows.
const Variant *variant_f32_skinny(int mb, int nb, int ks);
const Variant *variant_bf16_skinny(int mb, int nb, int ks);
// bf16 matrix-core kernel for any layout (k_bf16_any.hip).
const Variant *variant_bf16_any(int bt);   // bt = 64 or 128
// bf16 matrix-core kernel for any layout fed by 4-byte copies to LDS
// (k_bf16_realign.hip): bm x 256 tiles, bm = 256, 224, 192 or 160.
const Variant *variant_bf16_realign(int bm);
// One wave per output (k_gemv.hip): matrix-vector products (N = 1), any layout.
const Variant *variant_f32_gemv();
const Variant *variant_bf16_gemv();

// Strided 2-D copy (k_pack.hip): dst[r][c] = src[r][c] for r < rows, c < cols,
// element strides (s_r, s_c) and (d_r, d_c); esize 4 or 2. Enqueues nothing
// for an empty copy.
hipError_t launch_pack(int esize, const void *src, void *dst, int64_t rows, int64_t cols, int64_t s_r,
                       int64_t s_c, int64_t d_r, int64_t d_c, hipStream_t stream);

// Row softmax and row sum (k_rows.hip). Softmax variants 0-2 keep a row in
// registers (up to softmax_capacity(variant, esize) columns; N % (16/esize)
// == 0 and 16-byte aligned rows), 3 is two passes with 16-byte vectors (same
// layout rule), 4 two passes over single elements (any layout).
constexpr int kSoftmaxVariants = 5;
int64_t softmax_capacity(int variant, int esize);
hipError_t launch_softmax(int esize, int variant, const void *X, void *Y, int64_t M, int64_t N, int64_t ldx,
                          int64_t ldy, hipStream_t stream);
hipError_t launch_row_sum(int esize, bool vec, bool short_rows, const void *X, float *out, int64_t M, int64_t N,
                          int64_t ldx, hipStream_t stream);

}  // namespace mmrelu
