/* A plain C99 client of the library: it includes only include/mmrelu.h and
 * calls the host-side entry points (planning, workspace sizing, status
 * strings, and argument checks that fail before anything touches a GPU).
 * tests/test_c_abi.py builds it with gcc and compares each printed line with
 * the same call made through the Python binding. One JSON object per line. */
#include <stdio.h>

#include "mmrelu.h"

static void plan_line(int dtype, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc)
{
    mmrelu_plan_t p;
    const int rc = mmrelu_plan(dtype, M, N, K, lda, ldb, ldc, 256, &p);
    if (rc != MMRELU_OK) {
        printf("{\"call\": \"plan\", \"shape\": [%lld, %lld, %lld], \"status\": %d}\n", (long long)M, (long long)N,
               (long long)K, rc);
        return;
    }
    printf("{\"call\": \"plan\", \"shape\": [%lld, %lld, %lld], \"status\": 0, \"variant\": %d, \"name\": \"%s\", "
           "\"grid\": %lld, \"waves\": %lld}\n",
           (long long)M, (long long)N, (long long)K, (int)p.variant, p.name, (long long)p.grid, (long long)p.waves);
}

int main(void)
{
    int64_t waves = 0, idle = 0;
    size_t ws = 0;
    int rc;

    printf("{\"call\": \"version\", \"value\": \"%s\"}\n", mmrelu_version());
    printf("{\"call\": \"status\", \"value\": [\"%s\", \"%s\", \"%s\"]}\n", mmrelu_status_string(MMRELU_OK),
           mmrelu_status_string(MMRELU_ERR_MISALIGNED), mmrelu_status_string(99));

    plan_line(MMRELU_DTYPE_F32, 256, 256, 256, 256, 256, 256);
    plan_line(MMRELU_DTYPE_F32, 1024, 1024, 1024, 1024, 1024, 1024);
    plan_line(MMRELU_DTYPE_F32, 4096, 4096, 4096, 4096, 4096, 4096);
    plan_line(MMRELU_DTYPE_F32, 4097, 3001, 2049, 2049, 3001, 3001);
    plan_line(MMRELU_DTYPE_BF16, 8192, 8192, 8192, 8192, 8192, 8192);
    plan_line(MMRELU_DTYPE_BF16, 4097, 3001, 2049, 2049, 3001, 3001);
    plan_line(MMRELU_DTYPE_F32, 8192, 1, 8192, 8192, 1, 1);
    plan_line(MMRELU_DTYPE_F32, -1, 4, 4, 4, 4, 4);

    rc = mmrelu_wave_quantization(3055, 1280, &waves, &idle);
    printf("{\"call\": \"waves\", \"status\": %d, \"value\": [%lld, %lld]}\n", rc, (long long)waves, (long long)idle);

    /* A^T stored row-major (sam = 1, sak = M): one operand copy. */
    rc = mmrelu_strided_workspace_size(MMRELU_DTYPE_BF16, MMRELU_ACT_RELU, (const void *)0x100000,
                                       (const void *)0x200000, NULL, (void *)0x300000, 1024, 512, 256, 1, 1024, 512,
                                       1, 512, 1, &ws);
    printf("{\"call\": \"workspace\", \"status\": %d, \"value\": %llu}\n", rc, (unsigned long long)ws);

    /* Checks that fail before any launch: a negative size, a null output, a
     * misaligned bf16 pointer, a leading dimension below K. */
    printf("{\"call\": \"checks\", \"value\": [%d, %d, %d, %d]}\n",
           mmrelu_f32((const float *)0x100000, (const float *)0x200000, (float *)0x300000, -1, 4, 4, 4, 4, 4, NULL),
           mmrelu_f32((const float *)0x100000, (const float *)0x200000, NULL, 4, 4, 4, 4, 4, 4, NULL),
           mmrelu_bf16((const uint16_t *)0x100001, (const uint16_t *)0x200000, (uint16_t *)0x300000, 4, 4, 4, 4, 4, 4,
                       NULL),
           mmrelu_f32((const float *)0x100000, (const float *)0x200000, (float *)0x300000, 4, 4, 8, 4, 4, 4, NULL));
    return 0;
}
