/*
 * mmrelu: C = relu(A·B) on one AMD Instinct MI355X (gfx950).
 *
 * The operation is the lecture's matmul finale with the fused activation
 * ("Kernels, Triton, XLA" lecture notes, section "Reductions and tiling",
 * the matmul paragraph and its kernel sketch; the Chinese notes' section 5.5,
 * listing matmul_relu_kernel): A is M x K, B is K x N, C is M x N, each output
 * tile accumulates its K-term dot products in fp32, applies max(x, 0), and is
 * stored once, with loads and the store masked at the matrix edges.
 *
 * Layout: every matrix is row-major with a leading dimension in ELEMENTS:
 *     A[i][k] = A[i*lda + k],  B[k][j] = B[k*ldb + j],  C[i][j] = C[i*ldc + j]
 * and for 0 <= i < M, 0 <= j < N:
 *     C[i][j] = max(0, sum_{k<K} A[i][k] * B[k][j])
 * (the lecture's kernel takes a stride per dimension; this interface fixes the
 * column strides to 1, the row-major case).
 *
 * Ownership and execution: all pointers are DEVICE pointers owned by the
 * caller; the library never allocates, frees, or synchronises (the
 * general-stride calls below take a caller-provided workspace instead). The caller
 * allocates C (as on the pages, where the host allocates the output and the
 * kernel writes into it). Work is enqueued on `stream` (a hipStream_t; NULL
 * means the null stream) and the call returns right after the enqueue, so a
 * device-side fault is reported by the caller's next synchronisation. Calls
 * are thread-safe and reentrant (the library keeps no mutable state beyond a
 * per-device cache of the compute-unit count). Elements of C outside the
 * M x N window (row padding between N and ldc) are never written. C must not
 * overlap A or B (not checked).
 *
 * Errors: arguments are checked BEFORE anything is enqueued; on any non-zero
 * status nothing has been launched and C is untouched. This follows the host
 * wrapper of the diy-llm chapter ("Chapter 7: GPU High-Performance
 * Programming", section 7.4.3, writing kernels with the C++ API): before the
 * launch the wrapper checks that its input is device memory laid out the way
 * the kernel indexes it, the caller-side output is written without being
 * cleared first, and the launch itself is checked right after it is issued.
 * Here the layout check is the leading-dimension and alignment rules below,
 * and the launch check is hipGetLastError.
 *   MMRELU_ERR_INVALID_VALUE  M, N or K negative; lda < max(1,K), ldb < max(1,N),
 *                             ldc < max(1,N); or a size past the limits below.
 *   MMRELU_ERR_NULL_POINTER   C null (M, N > 0), or A/B null (M, N, K > 0).
 *   MMRELU_ERR_MISALIGNED     a pointer not aligned to its element size.
 *   MMRELU_ERR_LAUNCH         the HIP launch itself failed (hipGetLastError);
 *                             e.g. the current device is not a gfx950. The
 *                             check also returns (and clears) an error that
 *                             an earlier HIP call on the same thread left
 *                             pending, so callers should check their own HIP
 *                             calls before calling the library.
 * Empty outputs (M == 0 or N == 0) return MMRELU_OK without a launch; K == 0
 * writes C = 0 (the K loop runs zero times and relu(0) is stored).
 *
 * Limits: M, N, K <= 2^31 - 1 and lda, ldb, ldc <= 2^21 elements (the kernels
 * address each tile with 32-bit offsets from a 64-bit tile base), and one
 * launch holds fewer than 2^32 work-items: the planned grid times the
 * kernel's threads per workgroup (mmrelu_plan reports both) must stay below
 * 2^32, else MMRELU_ERR_INVALID_VALUE. That bounds only extreme shapes, e.g.
 * N = 1 runs one 256-thread workgroup per four rows, so M < 2^26 rows.
 */
#ifndef MMRELU_H
#define MMRELU_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MMRELU_OK = 0,
    MMRELU_ERR_INVALID_VALUE = 1,
    MMRELU_ERR_NULL_POINTER = 2,
    MMRELU_ERR_MISALIGNED = 3,
    MMRELU_ERR_LAUNCH = 4,
    MMRELU_ERR_WORKSPACE_LIMIT = 5   /* mmrelu_strided_static only */
};

enum { MMRELU_DTYPE_F32 = 0, MMRELU_DTYPE_BF16 = 1 };

/* fp32 inputs, fp32 products accumulated in fp32 on the matrix cores, fp32 output. */
int mmrelu_f32(const float *A, const float *B, float *C,
               int64_t M, int64_t N, int64_t K,
               int64_t lda, int64_t ldb, int64_t ldc, void *stream);

/* bf16 inputs and output, given as uint16_t bit patterns; bf16 products
 * accumulated in fp32; ReLU on the fp32 sum, then rounded to bf16 (nearest,
 * ties to even). */
int mmrelu_bf16(const uint16_t *A, const uint16_t *B, uint16_t *C,
                int64_t M, int64_t N, int64_t K,
                int64_t lda, int64_t ldb, int64_t ldc, void *stream);

/*
 * Fused epilogues (widening of the operation above). The lecture notes make
 * the point that, with the output tile already in registers before its one
 * store, any elementwise activation costs nothing extra (section "Reductions
 * and tiling", the matmul's fusion bonus), and open with GeLU in its tanh form
 * (section "GeLU three ways: the case for fusion"); a linear layer is a
 * matmul followed by an activation. For 0 <= i < M, 0 <= j < N:
 *     C[i][j] = act(sum_{k<K} A[i][k] * B[k][j] + bias[j])
 * with the sum and the bias added in fp32 and
 *     MMRELU_ACT_RELU       act(x) = max(x, 0)        (mmrelu_f32 / _bf16)
 *     MMRELU_ACT_GELU_TANH  act(x) = 0.5 x (1 + tanh(0.79788456 (x + 0.044715 x^3)))
 *     MMRELU_ACT_NONE       act(x) = x
 * bias: N elements of the input dtype (fp32, or bf16 bit patterns widened to
 * fp32), one per output column, or NULL for none; device pointer, caller-owned,
 * aligned to its element size. bf16 outputs are rounded once, after act.
 * Errors as above, plus MMRELU_ERR_INVALID_VALUE for an unknown act and
 * MMRELU_ERR_MISALIGNED for a misaligned bias.
 */
enum { MMRELU_ACT_RELU = 0, MMRELU_ACT_GELU_TANH = 1, MMRELU_ACT_NONE = 2 };

int mmrelu_fused_f32(int act, const float *A, const float *B, const float *bias, float *C,
                     int64_t M, int64_t N, int64_t K,
                     int64_t lda, int64_t ldb, int64_t ldc, void *stream);
int mmrelu_fused_bf16(int act, const uint16_t *A, const uint16_t *B, const uint16_t *bias, uint16_t *C,
                      int64_t M, int64_t N, int64_t K,
                      int64_t lda, int64_t ldb, int64_t ldc, void *stream);

/* Static text for a status code ("unknown status" for anything else). */
const char *mmrelu_status_string(int status);

/* Library version string. */
const char *mmrelu_version(void);

/*
 * General strides (widening of the interface above). The lecture describes a
 * stored matrix by two strides, the position of element (row, column) being
 * row * row_stride + column * column_stride, and a transpose as the same data
 * with the two strides exchanged ("Kernels, Triton, XLA", section "Reductions
 * and tiling"); the Chinese notes' section 5.5 kernel takes a stride for each
 * dimension of A, B and C. Here, in ELEMENTS:
 *     A[i][k] = A[i*sam + k*sak],  B[k][j] = B[k*sbk + j*sbn],  C[i][j] = C[i*scm + j*scn]
 * and C[i][j] = act(sum_{k<K} A[i][k] * B[k][j] + bias[j]) as for the fused
 * entry points (same act codes, bias of N elements or NULL).
 *   - sam, sak, sbk, sbn >= 0 (a zero stride repeats an element); scm, scn >= 1
 *     and the outputs must not overlap: scm >= N * scn or scn >= M * scm
 *     (when M > 1 and N > 1). Every largest offset must stay below 2^60.
 *   - Row-major operands and output (unit column stride, row stride within
 *     the leading-dimension limits) are used in place, as by mmrelu_fused_*.
 *     A column-major C (scm = 1) with no bias is computed as C^T = B^T A^T with
 *     the operands' roles exchanged, also in place; so are transposed operands
 *     that this exchange turns row-major (sam = 1 and sbk = 1 into scm = 1).
 *   - Any other operand is first copied into row-major form, and any other C
 *     is written from a row-major product, by a strided copy kernel through
 *     the caller's WORKSPACE (device memory, 256-byte aligned, caller-owned,
 *     not read before it is written; the library still allocates nothing).
 *     An operand whose leading dimension or address would keep a 16-byte-
 *     vector kernel out is also copied when the shape itself allows one.
 *   - mmrelu_strided_workspace_size writes the bytes a call with the same
 *     arguments needs (0 when everything is used in place). Pass the same
 *     pointers: their alignment is part of the decision.
 * Work (copies, product, copy-out) is enqueued in order on `stream`; the
 * workspace must stay allocated until it completes, and calls sharing one
 * workspace must be ordered (e.g. on one stream).
 * Errors: as for the fused entry points, checked before anything is
 * enqueued, plus MMRELU_ERR_INVALID_VALUE for a stride outside the rules above
 * or workspace_bytes below the size needed, MMRELU_ERR_NULL_POINTER for a
 * null workspace when one is needed, MMRELU_ERR_MISALIGNED for a workspace
 * not 256-byte aligned.
 */
int mmrelu_strided_workspace_size(int dtype, int act, const void *A, const void *B, const void *bias, const void *C,
                                  int64_t M, int64_t N, int64_t K, int64_t sam, int64_t sak, int64_t sbk,
                                  int64_t sbn, int64_t scm, int64_t scn, size_t *bytes);
int mmrelu_strided_f32(int act, const float *A, const float *B, const float *bias, float *C,
                       int64_t M, int64_t N, int64_t K, int64_t sam, int64_t sak, int64_t sbk, int64_t sbn,
                       int64_t scm, int64_t scn, void *workspace, size_t workspace_bytes, void *stream);
int mmrelu_strided_bf16(int act, const uint16_t *A, const uint16_t *B, const uint16_t *bias, uint16_t *C,
                        int64_t M, int64_t N, int64_t K, int64_t sam, int64_t sak, int64_t sbk, int64_t sbn,
                        int64_t scm, int64_t scn, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The general-stride call without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments, semantics and checks as
 * mmrelu_strided_f32 / _bf16 (dtype MMRELU_DTYPE_F32 or MMRELU_DTYPE_BF16
 * selects which; A, B, bias and C point to elements of that type), but the
 * operand copies and the row-major temporary of C go to a fixed device array
 * of MMRELU_STATIC_WORKSPACE_BYTES that the library holds on each device it
 * runs on, from that device's first such call until the process ends.
 * Nothing is allocated or freed and nothing is cleared (every byte the
 * kernels read from the array was written earlier in the same call).
 *   - A call whose mmrelu_strided_workspace_size exceeds the limit returns
 *     MMRELU_ERR_WORKSPACE_LIMIT before anything is enqueued; calls that
 *     need no workspace (row-major or in-place layouts) never touch it.
 *   - Every call on one device shares that device's array, which keeps the
 *     last call's contents: calls that may overlap on one device (different
 *     streams, or host threads without ordering) race and must not be mixed;
 *     calls ordered on one stream are safe.
 *   - MMRELU_ERR_LAUNCH if the device address of the array cannot be
 *     obtained (hipGetSymbolAddress, once per device), or a launch fails.
 */
#define MMRELU_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
int mmrelu_strided_static(int dtype, int act, const void *A, const void *B, const void *bias, void *C,
                          int64_t M, int64_t N, int64_t K, int64_t sam, int64_t sak, int64_t sbk, int64_t sbn,
                          int64_t scm, int64_t scn, void *stream);

/*
 * Row softmax and row sum: the two rungs before the matmul on the lecture's
 * ladder ("Kernels, Triton, XLA", section "Reductions and tiling", the softmax
 * and row-sum paragraphs; the Chinese notes' sections 5.3 and 5.4). X is
 * M x N, row-major with leading dimension ldx (elements), device memory.
 *
 *   softmax: Y[i][j] = exp(X[i][j] - m_i) / sum_j exp(X[i][j] - m_i),
 *            m_i = max_j X[i][j]; computed in fp32 (bf16 inputs widened, bf16
 *            outputs rounded once to nearest-even). Y is M x N with leading
 *            dimension ldy >= N; Y may be X itself (in place, ldy == ldx),
 *            otherwise the two must not overlap (not checked). Elements
 *            beyond column N are neither read nor written.
 *   row sum: out[i] = sum_j X[i][j], accumulated in fp32; out is M floats
 *            for both input dtypes. N == 0 writes zeros.
 *
 * X must be finite (infinities and NaN are outside the contract). Work is
 * enqueued on `stream`; arguments are checked first, and on any non-zero
 * status nothing is launched. Errors: MMRELU_ERR_INVALID_VALUE for negative
 * or too large sizes, ldx < max(1, N) (or ldy < max(1, N)), X == Y with
 * ldx != ldy, or an offset past 2^60; MMRELU_ERR_NULL_POINTER for a null
 * pointer that would be used; MMRELU_ERR_MISALIGNED for a pointer not aligned
 * to its element size. Empty outputs (M == 0, or N == 0 for softmax) launch
 * nothing.
 *
 * Softmax kernels (the _variant forms force one, for tests): 0, 1, 2 hold a
 * row in registers and need N, ldx and ldy multiples of 16 / sizeof(element)
 * with 16-byte aligned X and Y; they take rows of up to 1024, 4096 or 16384
 * fp32 (2048, 8192 or 32768 bf16) columns. 3 reads each row twice with
 * 16-byte vectors (same layout rule, any N); 4 reads single elements (any
 * layout). mmrelu_softmax_rows_variant reports the choice for a shape,
 * taking X and Y as 16-byte aligned.
 */
int mmrelu_softmax_rows_f32(const float *X, float *Y, int64_t M, int64_t N, int64_t ldx, int64_t ldy, void *stream);
int mmrelu_softmax_rows_bf16(const uint16_t *X, uint16_t *Y, int64_t M, int64_t N, int64_t ldx, int64_t ldy,
                             void *stream);
int mmrelu_softmax_rows_f32_variant(int32_t variant, const float *X, float *Y, int64_t M, int64_t N, int64_t ldx,
                                    int64_t ldy, void *stream);
int mmrelu_softmax_rows_bf16_variant(int32_t variant, const uint16_t *X, uint16_t *Y, int64_t M, int64_t N,
                                     int64_t ldx, int64_t ldy, void *stream);
int mmrelu_softmax_rows_variant(int dtype, int64_t N, int64_t ldx, int64_t ldy, int32_t *variant);
int mmrelu_row_sum_f32(const float *X, float *out, int64_t M, int64_t N, int64_t ldx, void *stream);
int mmrelu_row_sum_bf16(const uint16_t *X, float *out, int64_t M, int64_t N, int64_t ldx, void *stream);

/*
 * Host-only planning (no GPU needed): which kernel variant and grid a call
 * of this shape would use, and how its workgroups quantise into waves over
 * the compute units (the lecture's "wave quantization": a last, partial wave
 * leaves compute units idle).
 */
typedef struct {
    int32_t variant;          /* index in the library's kernel table */
    int32_t block_m, block_n, block_k;
    int32_t threads;          /* per workgroup */
    int32_t wg_per_cu;        /* workgroups resident per compute unit */
    int32_t cus;              /* compute units assumed */
    int32_t reserved;
    int64_t tiles_m, tiles_n, grid;
    int64_t waves;            /* ceil(grid / (cus * wg_per_cu)) */
    int64_t idle_slots_last;  /* workgroup slots left empty in the last wave */
    char name[64];            /* kernel name as a profiler shows it */
} mmrelu_plan_t;

/* Fill *out for a call of this dtype and shape. cus = 0 uses the current
 * device's compute-unit count when a device is present, else 256. Returns a
 * status as above (arguments are validated the same way, pointers aside).
 * The choice, in order:
 *   - N == 1 (a matrix-vector product): the one-wave-per-output kernel;
 *   - an aligned layout with M <= 64 and M <= N: the skinny-M kernel of the
 *     smallest row count that covers M (16, 32 or 64 rows; it splits K over
 *     the eight waves of a workgroup so a 32-column strip of B streams from
 *     memory once); M <= 16 with at least one 64-column strip per CU takes
 *     64-column strips (fp32 variant 13, bf16 variant 14);
 *   - an aligned layout with N <= 64: the skinny-N kernel of the smallest
 *     column count that covers N (16, 32 or 64), over 32-row bands of A;
 *     fp32 with N <= 16 and at least one 64-row band per CU takes 64-row
 *     bands (variant 14);
 *   - otherwise the candidate with the least estimated time on the busiest
 *     compute unit, ceil(tiles / cus) tiles times the tile's outputs times
 *     the kernel's measured relative cost per output (times 1.15 for a tile
 *     kernel left with one tile per CU, which then runs latency-bound).
 *     Candidates: the dtype's matrix-core kernels at a large and a small
 *     tile that accept the layout (aligned bf16: the 256 x 256 ping-pong
 *     tile, variant 1, the 128 x 256 ping-pong tile, variant 3, and the
 *     128 x 128 tile, variant 4) and, for aligned layouts, the seven
 *     skinny tiles (variants 5 - 10 and the 64 x 64 variant 12), which split
 *     K over eight waves and keep every CU busy when the large tiles cannot
 *     (small squares, long K with few output tiles); other layouts run the
 *     fp32 unaligned matrix-core kernels, or for bf16 the any-layout
 *     matrix-core kernels: 64 x 64 tiles (variant 13) until the 128 x 128
 *     grid gives three CUs in four a tile, then 128 x 128 tiles (variant 2,
 *     registers realign the operands) or BM x 256 tiles with BM = 256, 224,
 *     192 or 160 (variants 15 - 18, 4- and 16-byte copies to LDS realigned
 *     there), whichever has the smallest estimate: the busiest CU's tile
 *     count times a fixed plus a per-k cost measured for each kernel.
 * The launch entry points make the same choice with the device's count. */
int mmrelu_plan(int dtype, int64_t M, int64_t N, int64_t K,
                int64_t lda, int64_t ldb, int64_t ldc, int32_t cus, mmrelu_plan_t *out);

/* Number of kernel variants for a dtype, and the plan a given variant would
 * use for a shape (variant must be valid for that dtype). For tests and
 * tuning: it lets every variant be checked on every shape. */
int mmrelu_num_variants(int dtype);
int mmrelu_plan_variant(int dtype, int32_t variant, int64_t M, int64_t N, int64_t K,
                        int64_t lda, int64_t ldb, int64_t ldc, int32_t cus, mmrelu_plan_t *out);

/* Wave quantisation of `blocks` workgroups over `slots` concurrent slots:
 * *waves = ceil(blocks / slots), *idle_last = slots * waves - blocks.
 * Returns MMRELU_ERR_INVALID_VALUE for blocks < 0, slots < 1 or null outputs. */
int mmrelu_wave_quantization(int64_t blocks, int64_t slots, int64_t *waves, int64_t *idle_last);

/* As mmrelu_f32 / mmrelu_bf16 but with an explicit kernel variant instead of
 * the planner's choice (for tests and tuning). Same checks and semantics; a
 * skinny variant given more rows than it covers returns
 * MMRELU_ERR_INVALID_VALUE. */
int mmrelu_f32_variant(int32_t variant, const float *A, const float *B, float *C,
                       int64_t M, int64_t N, int64_t K,
                       int64_t lda, int64_t ldb, int64_t ldc, void *stream);
int mmrelu_bf16_variant(int32_t variant, const uint16_t *A, const uint16_t *B, uint16_t *C,
                        int64_t M, int64_t N, int64_t K,
                        int64_t lda, int64_t ldb, int64_t ldc, void *stream);

/* The fused entry points with an explicit kernel variant (every variant
 * applies every epilogue). */
int mmrelu_fused_f32_variant(int32_t variant, int act, const float *A, const float *B, const float *bias,
                             float *C, int64_t M, int64_t N, int64_t K,
                             int64_t lda, int64_t ldb, int64_t ldc, void *stream);
int mmrelu_fused_bf16_variant(int32_t variant, int act, const uint16_t *A, const uint16_t *B,
                              const uint16_t *bias, uint16_t *C, int64_t M, int64_t N, int64_t K,
                              int64_t lda, int64_t ldb, int64_t ldc, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MMRELU_H */
