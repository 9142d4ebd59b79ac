/* Using the library from C, without Python or torch: read A and B from
 * binary files, run C = relu(A·B) on the GPU through the C-ABI, write C.
 *
 *   mmrelu_run f32|bf16 M N K A.bin B.bin C.bin
 *
 * A.bin holds M*K and B.bin K*N row-major elements (fp32, or bf16 bit
 * patterns as uint16) with no padding; C.bin receives M*N elements of the
 * same type. Device memory, the stream and the copies are the caller's, as
 * the library's contract requires: the library itself allocates nothing.
 * Exit status 0 on success; otherwise a message on stderr and status 1. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "mmrelu.h"

static int fail(const char *what, const char *detail)
{
    fprintf(stderr, "mmrelu_run: %s: %s\n", what, detail);
    return 1;
}

static int read_file(const char *path, void *dst, size_t bytes)
{
    FILE *f = fopen(path, "rb");
    size_t got;
    if (f == NULL) return -1;
    got = fread(dst, 1, bytes, f);
    fclose(f);
    return got == bytes ? 0 : -1;
}

int main(int argc, char **argv)
{
    int bf16, rc;
    long long M, N, K;
    size_t es, a_bytes, b_bytes, c_bytes;
    void *ha = NULL, *hb = NULL, *hc = NULL, *da = NULL, *db = NULL, *dc = NULL;
    hipStream_t stream = NULL;
    hipError_t e;
    FILE *out;

    if (argc != 8) return fail("usage", "mmrelu_run f32|bf16 M N K A.bin B.bin C.bin");
    if (strcmp(argv[1], "f32") != 0 && strcmp(argv[1], "bf16") != 0) return fail("dtype", argv[1]);
    bf16 = strcmp(argv[1], "bf16") == 0;
    M = atoll(argv[2]);
    N = atoll(argv[3]);
    K = atoll(argv[4]);
    if (M < 1 || N < 1 || K < 1) return fail("sizes", "M, N and K must be positive");
    es = bf16 ? 2 : 4;
    a_bytes = (size_t)M * (size_t)K * es;
    b_bytes = (size_t)K * (size_t)N * es;
    c_bytes = (size_t)M * (size_t)N * es;

    ha = malloc(a_bytes);
    hb = malloc(b_bytes);
    hc = malloc(c_bytes);
    if (ha == NULL || hb == NULL || hc == NULL) return fail("host memory", "malloc failed");
    if (read_file(argv[5], ha, a_bytes) != 0) return fail("read", argv[5]);
    if (read_file(argv[6], hb, b_bytes) != 0) return fail("read", argv[6]);

    if ((e = hipMalloc(&da, a_bytes)) != hipSuccess || (e = hipMalloc(&db, b_bytes)) != hipSuccess ||
        (e = hipMalloc(&dc, c_bytes)) != hipSuccess)
        return fail("hipMalloc", hipGetErrorString(e));
    if ((e = hipStreamCreate(&stream)) != hipSuccess) return fail("hipStreamCreate", hipGetErrorString(e));
    if ((e = hipMemcpyAsync(da, ha, a_bytes, hipMemcpyHostToDevice, stream)) != hipSuccess ||
        (e = hipMemcpyAsync(db, hb, b_bytes, hipMemcpyHostToDevice, stream)) != hipSuccess)
        return fail("hipMemcpyAsync", hipGetErrorString(e));

    if (bf16)
        rc = mmrelu_bf16((const uint16_t *)da, (const uint16_t *)db, (uint16_t *)dc, M, N, K, K, N, N, stream);
    else
        rc = mmrelu_f32((const float *)da, (const float *)db, (float *)dc, M, N, K, K, N, N, stream);
    if (rc != MMRELU_OK) return fail("mmrelu", mmrelu_status_string(rc));

    if ((e = hipMemcpyAsync(hc, dc, c_bytes, hipMemcpyDeviceToHost, stream)) != hipSuccess)
        return fail("hipMemcpyAsync", hipGetErrorString(e));
    if ((e = hipStreamSynchronize(stream)) != hipSuccess) return fail("hipStreamSynchronize", hipGetErrorString(e));

    out = fopen(argv[7], "wb");
    if (out == NULL || fwrite(hc, 1, c_bytes, out) != c_bytes) return fail("write", argv[7]);
    fclose(out);

    hipStreamDestroy(stream);
    hipFree(da);
    hipFree(db);
    hipFree(dc);
    free(ha);
    free(hb);
    free(hc);
    return 0;
}
