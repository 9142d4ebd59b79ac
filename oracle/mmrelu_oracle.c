/*
 * Oracle for C = relu(A·B): TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library. It shares no code with the gfx950 library: no
 * headers, helpers, tables or pre/post-processing.
 *
 * What it computes (lecture notes "Kernels, Triton, XLA", section
 * "Reductions and tiling", matmul finale; and the Chinese notes' section 5.5
 * on matrix multiplication, the matmul_relu_kernel listing): A is M x K, B is
 * K x N, C is M x N, and every output element is the K-term dot product of a
 * row of A with a column of B, passed through ReLU (max with 0) before it is
 * stored. Tiling only changes the order in which the same products are
 * summed, so the oracle is the plain definition:
 *
 *     s      = sum over k = 0 .. K-1, in ascending k, of A[i][k] * B[k][j]
 *     R[i][j] = s > 0 ? s : 0
 *
 * evaluated in IEEE double precision. Inputs are fp32 (or bf16 widened to
 * fp32 by placing the 16 stored bits in the high half of a 32-bit word), and
 * every fp32 x fp32 product is exact in double (24 + 24 <= 53 significand
 * bits), so only the K-1 additions round. The result stays in double.
 *
 * Matrices are row-major with leading dimensions in elements:
 * A[i][k] = A[i*lda + k], B[k][j] = B[k*ldb + j], R[i][j] = R[i*ldr + j].
 *
 * The full-matrix routines loop i, then k, then j with one double
 * accumulator per output column. Each R[i][j] is still a single running sum
 * taken in ascending k, so the result is bit-identical to the i, j, k order
 * and does not depend on the number of threads (rows are split over OpenMP
 * threads; a row is never split). The "_at" routines evaluate single entries
 * with the i, j, k order directly, for sampled checks at large sizes.
 *
 * The sign of a zero result and NaN inputs are outside what the pages fix:
 * s <= 0 (including -0.0) gives +0.0, and a NaN sum gives 0 (parity
 * unpinned for NaN and infinities; the workloads never produce them).
 *
 * Fused epilogues (the "oracle_fused_*" routines; the relu routines are the
 * case act = ReLU without a bias). The lecture applies any elementwise
 * activation to the finished tile before its one store (section
 * "Reductions and tiling", the fusion bonus) and defines GeLU by its tanh
 * form (section "GeLU three ways: the case for fusion"):
 *
 *     s' = s + bias[j]           (bias optional, widened exactly to double)
 *     R  = act(s'), act one of   relu(x)  = x > 0 ? x : 0
 *                                gelu(x)  = 0.5 x (1 + tanh(0.79788456 (x + 0.044715 x^3)))
 *                                none(x)  = x
 *
 * with the pages' constants and libm's tanh, all in double.
 *
 * General strides (the "oracle_strided_*" routines; every other routine is
 * the case of unit column strides). The lecture reminds that a tensor is
 * linearised in memory and that its strides map a (row, column) index to a
 * position, row times the row stride plus column times the column stride,
 * a transpose being the same data with the two strides exchanged (section
 * "Reductions and tiling", before the matmul kernel); the Chinese notes'
 * section 5.5 kernel takes one stride per dimension of A, B and C. So
 *
 *     A[i][k] = A[i*sam + k*sak],   B[k][j] = B[k*sbk + j*sbn]
 *
 * with any non-negative strides (zero repeats an element), and the result is
 * the same act(sum + bias) as above, stored row-major in R (ld ldr): where C
 * lives is the library's concern, the values are the oracle's.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double relu(double s) { return s > 0.0 ? s : 0.0; }

static double gelu_tanh(double x)
{
    return 0.5 * x * (1.0 + tanh(0.79788456 * (x + 0.044715 * x * x * x)));
}

/* Activation codes: 0 ReLU, 1 GeLU (tanh form), 2 none. */
static double activate(int act, double s)
{
    if (act == 0) return relu(s);
    if (act == 1) return gelu_tanh(s);
    return s;
}

static double widen_bf16(uint16_t h)
{
    uint32_t w = (uint32_t)h << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Full act(A·B + bias) for fp32 inputs with general strides into a double
 * M x N matrix R (ld ldr); bias is N floats or NULL. Returns 0, or -1 if a row
 * accumulator could not be allocated. */
int oracle_strided_f32(int act, const float *A, const float *B, const float *bias, double *R,
                       int64_t M, int64_t N, int64_t K, int64_t sam, int64_t sak, int64_t sbk,
                       int64_t sbn, int64_t ldr)
{
    int failed = 0;
#pragma omp parallel
    {
        double *acc = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        if (!acc) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t i = 0; i < M; ++i) {
            if (!acc) continue;
            for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double a = (double)A[i * sam + k * sak];
                const float *brow = B + k * sbk;
                for (int64_t j = 0; j < N; ++j) acc[j] += a * (double)brow[j * sbn];
            }
            for (int64_t j = 0; j < N; ++j)
                R[i * ldr + j] = activate(act, acc[j] + (bias ? (double)bias[j] : 0.0));
        }
        free(acc);
    }
    return failed ? -1 : 0;
}

/* Same for bf16 inputs and bias given as uint16 bit patterns. */
int oracle_strided_bf16(int act, const uint16_t *A, const uint16_t *B, const uint16_t *bias, double *R,
                        int64_t M, int64_t N, int64_t K, int64_t sam, int64_t sak, int64_t sbk,
                        int64_t sbn, int64_t ldr)
{
    int failed = 0;
#pragma omp parallel
    {
        double *acc = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        if (!acc) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t i = 0; i < M; ++i) {
            if (!acc) continue;
            for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double a = widen_bf16(A[i * sam + k * sak]);
                const uint16_t *brow = B + k * sbk;
                for (int64_t j = 0; j < N; ++j) acc[j] += a * widen_bf16(brow[j * sbn]);
            }
            for (int64_t j = 0; j < N; ++j)
                R[i * ldr + j] = activate(act, acc[j] + (bias ? widen_bf16(bias[j]) : 0.0));
        }
        free(acc);
    }
    return failed ? -1 : 0;
}

/* Entries R[ii[t]][jj[t]] for t < n, each as one dot product in ascending k. */
void oracle_strided_f32_at(int act, const float *A, const float *B, const float *bias, int64_t K,
                           int64_t sam, int64_t sak, int64_t sbk, int64_t sbn,
                           const int64_t *ii, const int64_t *jj, int64_t n, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k)
            s += (double)A[ii[t] * sam + k * sak] * (double)B[k * sbk + jj[t] * sbn];
        out[t] = activate(act, s + (bias ? (double)bias[jj[t]] : 0.0));
    }
}

void oracle_strided_bf16_at(int act, const uint16_t *A, const uint16_t *B, const uint16_t *bias, int64_t K,
                            int64_t sam, int64_t sak, int64_t sbk, int64_t sbn,
                            const int64_t *ii, const int64_t *jj, int64_t n, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k)
            s += widen_bf16(A[ii[t] * sam + k * sak]) * widen_bf16(B[k * sbk + jj[t] * sbn]);
        out[t] = activate(act, s + (bias ? widen_bf16(bias[jj[t]]) : 0.0));
    }
}

/* Row-major operands with leading dimensions: unit column strides. */
int oracle_fused_f32(int act, const float *A, const float *B, const float *bias, double *R,
                     int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldr)
{
    return oracle_strided_f32(act, A, B, bias, R, M, N, K, lda, 1, ldb, 1, ldr);
}

int oracle_fused_bf16(int act, const uint16_t *A, const uint16_t *B, const uint16_t *bias, double *R,
                      int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldr)
{
    return oracle_strided_bf16(act, A, B, bias, R, M, N, K, lda, 1, ldb, 1, ldr);
}

void oracle_fused_f32_at(int act, const float *A, const float *B, const float *bias, int64_t K,
                         int64_t lda, int64_t ldb,
                         const int64_t *ii, const int64_t *jj, int64_t n, double *out)
{
    oracle_strided_f32_at(act, A, B, bias, K, lda, 1, ldb, 1, ii, jj, n, out);
}

void oracle_fused_bf16_at(int act, const uint16_t *A, const uint16_t *B, const uint16_t *bias, int64_t K,
                          int64_t lda, int64_t ldb,
                          const int64_t *ii, const int64_t *jj, int64_t n, double *out)
{
    oracle_strided_bf16_at(act, A, B, bias, K, lda, 1, ldb, 1, ii, jj, n, out);
}

/* relu(A·B): the fused routines with ReLU and no bias. */
int oracle_mmrelu_f32(const float *A, const float *B, double *R,
                      int64_t M, int64_t N, int64_t K,
                      int64_t lda, int64_t ldb, int64_t ldr)
{
    return oracle_fused_f32(0, A, B, NULL, R, M, N, K, lda, ldb, ldr);
}

int oracle_mmrelu_bf16(const uint16_t *A, const uint16_t *B, double *R,
                       int64_t M, int64_t N, int64_t K,
                       int64_t lda, int64_t ldb, int64_t ldr)
{
    return oracle_fused_bf16(0, A, B, NULL, R, M, N, K, lda, ldb, ldr);
}

void oracle_mmrelu_f32_at(const float *A, const float *B, int64_t K,
                          int64_t lda, int64_t ldb,
                          const int64_t *ii, const int64_t *jj, int64_t n, double *out)
{
    oracle_fused_f32_at(0, A, B, NULL, K, lda, ldb, ii, jj, n, out);
}

void oracle_mmrelu_bf16_at(const uint16_t *A, const uint16_t *B, int64_t K,
                           int64_t lda, int64_t ldb,
                           const int64_t *ii, const int64_t *jj, int64_t n, double *out)
{
    oracle_fused_bf16_at(0, A, B, NULL, K, lda, ldb, ii, jj, n, out);
}

/*
 * Row softmax and row sum (the rungs before the matmul on the lecture's
 * ladder: "Kernels, Triton, XLA", section "Reductions and tiling", the
 * softmax and row-sum paragraphs; the Chinese notes' sections 5.3 and 5.4).
 * X is M x N, row-major with leading dimension ldx; inputs are finite
 * (parity unpinned for infinities and NaN).
 *
 *   softmax: m = max_j X[i][j];  e_j = exp(X[i][j] - m);  s = sum_j e_j
 *            (ascending j);  R[i][j] = e_j / s
 *   row sum: R[i] = sum_j X[i][j] in ascending j
 *
 * all in double, with libm's exp; the result is row-major with ld N (softmax)
 * or a vector of M (row sum). Subtracting the row maximum is what keeps exp
 * finite for large inputs; mathematically it cancels in the quotient.
 */
static void softmax_row(const double *x, double *r, int64_t n)
{
    double m = x[0];
    for (int64_t j = 1; j < n; ++j) m = x[j] > m ? x[j] : m;
    double s = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        r[j] = exp(x[j] - m);
        s += r[j];
    }
    for (int64_t j = 0; j < n; ++j) r[j] = r[j] / s;
}

int oracle_softmax_rows_f32(const float *X, double *R, int64_t M, int64_t N, int64_t ldx)
{
    int failed = 0;
#pragma omp parallel
    {
        double *x = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        if (!x) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t i = 0; i < M; ++i) {
            if (!x || N == 0) continue;
            for (int64_t j = 0; j < N; ++j) x[j] = (double)X[i * ldx + j];
            softmax_row(x, R + i * N, N);
        }
        free(x);
    }
    return failed ? -1 : 0;
}

int oracle_softmax_rows_bf16(const uint16_t *X, double *R, int64_t M, int64_t N, int64_t ldx)
{
    int failed = 0;
#pragma omp parallel
    {
        double *x = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        if (!x) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t i = 0; i < M; ++i) {
            if (!x || N == 0) continue;
            for (int64_t j = 0; j < N; ++j) x[j] = widen_bf16(X[i * ldx + j]);
            softmax_row(x, R + i * N, N);
        }
        free(x);
    }
    return failed ? -1 : 0;
}

void oracle_row_sum_f32(const float *X, double *R, int64_t M, int64_t N, int64_t ldx)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double s = 0.0;
        for (int64_t j = 0; j < N; ++j) s += (double)X[i * ldx + j];
        R[i] = s;
    }
}

void oracle_row_sum_bf16(const uint16_t *X, double *R, int64_t M, int64_t N, int64_t ldx)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double s = 0.0;
        for (int64_t j = 0; j < N; ++j) s += widen_bf16(X[i * ldx + j]);
        R[i] = s;
    }
}
