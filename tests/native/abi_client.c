/*
 * A plain C client of the library's C ABI (include/dmp_gemm.h), built with gcc
 * against the HIP runtime and libdmp_gemm.so -- no Python, no torch.  It checks
 * that the ABI is usable as declared:
 *   - gemm_create / gemm_destroy and gemm_status_string;
 *   - gemm_run on fp16 (row-major A, column-major B), int8 and fp64 products
 *     with small-integer inputs, where every sum is exact, compared with a
 *     triple loop here (exact equality);
 *   - gemm_run_ex with a bf16 D (values exactly representable);
 *   - gemm_prune24 + gemm_run_sparse24 on an A that already is 2:4;
 *   - rejected arguments return GEMM_ERR_INVALID_ARG and leave D untouched;
 *   - gemm_plan with a NULL handle.
 * Prints "abi_client: N checks, 0 failures" and exits 0 when all hold.
 * Run by tests/test_gpu_abi_client.py; built by __graft_entry__.build().
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/dmp_gemm.h"

static int checks = 0, failures = 0;
#define CHECK(cond, what)                                          \
    do {                                                           \
        ++checks;                                                  \
        if (!(cond)) {                                             \
            fprintf(stderr, "FAILED: %s (%s)\n", #cond, what);     \
            ++failures;                                            \
        }                                                          \
    } while (0)
#define HIPOK(x) CHECK((x) == hipSuccess, #x)

/* binary16 / bfloat16 patterns of small integers (exact) */
static uint16_t f16_of(int v) {
    if (v == 0) return 0;
    const uint16_t sign = v < 0 ? 0x8000 : 0;
    unsigned a = (unsigned)(v < 0 ? -v : v), e = 0;
    while ((a >> e) > 1) ++e;                        /* a in [2^e, 2^(e+1)) */
    const unsigned mant = (a << (10 - e)) & 0x3FF;   /* a < 2^11: exact */
    return (uint16_t)(sign | ((e + 15) << 10) | mant);
}
static float bf16_to_float(uint16_t b) {
    uint32_t w = (uint32_t)b << 16;
    float f;
    memcpy(&f, &w, 4);
    return f;
}

static void *dev_copy(const void *host, size_t bytes) {
    void *p = NULL;
    HIPOK(hipMalloc(&p, bytes));
    HIPOK(hipMemcpy(p, host, bytes, hipMemcpyHostToDevice));
    return p;
}

int main(void) {
    gemm_handle_t h = NULL;
    int rc = gemm_create(&h);
    CHECK(rc == GEMM_OK && h != NULL, "gemm_create");
    if (rc != GEMM_OK) {
        printf("abi_client: gemm_create failed: %s\n", gemm_status_string(rc));
        return 1;
    }
    CHECK(strcmp(gemm_status_string(GEMM_OK), "") != 0, "status string");
    hipStream_t s;
    HIPOK(hipStreamCreate(&s));
    srand(12345);

    /* fp16: A row-major M x K, B column-major (ldb = K), C, D fp32 */
    {
        const int64_t M = 70, N = 90, K = 136;
        uint16_t *A = malloc(2 * M * K), *B = malloc(2 * N * K);
        int *Ai = malloc(sizeof(int) * M * K), *Bi = malloc(sizeof(int) * N * K);
        float *C = malloc(4 * M * N), *D = malloc(4 * M * N);
        for (int64_t e = 0; e < M * K; ++e) { Ai[e] = rand() % 5 - 2; A[e] = f16_of(Ai[e]); }
        for (int64_t e = 0; e < N * K; ++e) { Bi[e] = rand() % 5 - 2; B[e] = f16_of(Bi[e]); }
        for (int64_t e = 0; e < M * N; ++e) C[e] = (float)(rand() % 17 - 8);
        void *dA = dev_copy(A, 2 * M * K), *dB = dev_copy(B, 2 * N * K), *dC = dev_copy(C, 4 * M * N);
        void *dD = NULL;
        HIPOK(hipMalloc(&dD, 4 * M * N));
        rc = gemm_run(h, dA, dB, dC, dD, M, N, K, K, K, N, GEMM_F16, GEMM_B_COLMAJOR, 1, s);
        CHECK(rc == GEMM_OK, "gemm_run f16");
        HIPOK(hipStreamSynchronize(s));
        HIPOK(hipMemcpy(D, dD, 4 * M * N, hipMemcpyDeviceToHost));
        int bad = 0;
        for (int64_t i = 0; i < M; ++i)
            for (int64_t j = 0; j < N; ++j) {
                long acc = (long)C[i * N + j];
                for (int64_t k = 0; k < K; ++k) acc += (long)Ai[i * K + k] * Bi[j * K + k];
                bad += D[i * N + j] != (float)acc;
            }
        CHECK(bad == 0, "fp16 product exact on small integers");

        /* the same product with a bf16 D: D = cvt_bf16(2 * AB + 1 * C); |values| < 256 are exact */
        void *dD16 = NULL;
        HIPOK(hipMalloc(&dD16, 2 * M * N));
        rc = gemm_run_ex(h, dA, dB, dC, dD16, M, N, K, K, K, N, GEMM_F16, GEMM_B_COLMAJOR, 1, 2.0f,
                         1.0f, GEMM_OUT_F32, GEMM_OUT_BF16, s);
        CHECK(rc == GEMM_OK, "gemm_run_ex bf16 D");
        HIPOK(hipStreamSynchronize(s));
        uint16_t *D16 = malloc(2 * M * N);
        HIPOK(hipMemcpy(D16, dD16, 2 * M * N, hipMemcpyDeviceToHost));
        bad = 0;
        for (int64_t i = 0; i < M; ++i)
            for (int64_t j = 0; j < N; ++j) {
                long acc = 0;
                for (int64_t k = 0; k < K; ++k) acc += (long)Ai[i * K + k] * Bi[j * K + k];
                const long want = 2 * acc + (long)C[i * N + j];
                if (want > -256 && want < 256) bad += bf16_to_float(D16[i * N + j]) != (float)want;
            }
        CHECK(bad == 0, "bf16 output stage exact on small values");

        /* rejected: lda < K for row-major A; D must stay as it is */
        HIPOK(hipMemset(dD, 0x7F, 4 * M * N));
        rc = gemm_run(h, dA, dB, dC, dD, M, N, K, K - 1, K, N, GEMM_F16, GEMM_B_COLMAJOR, 1, s);
        CHECK(rc == GEMM_ERR_INVALID_ARG, "lda < K rejected");
        rc = gemm_run(h, dA, dB, dC, dD, M, N, K, K, K, N, 9, 0, 1, s);
        CHECK(rc == GEMM_ERR_INVALID_ARG, "bad dtype rejected");
        rc = gemm_run(h, NULL, dB, dC, dD, M, N, K, K, K, N, GEMM_F16, 0, 1, s);
        CHECK(rc == GEMM_ERR_INVALID_ARG, "NULL A rejected");
        HIPOK(hipStreamSynchronize(s));
        HIPOK(hipMemcpy(D, dD, 4 * M * N, hipMemcpyDeviceToHost));
        uint32_t w;
        memcpy(&w, &D[0], 4);
        CHECK(w == 0x7F7F7F7Fu, "nothing enqueued on rejection");
        hipFree(dA); hipFree(dB); hipFree(dC); hipFree(dD); hipFree(dD16);
        free(A); free(B); free(Ai); free(Bi); free(C); free(D); free(D16);
    }

    /* int8 row-major A and B, int32 C and D, batch 2 */
    {
        const int64_t M = 33, N = 48, K = 80, batch = 2;
        int8_t *A = malloc(batch * M * K), *B = malloc(batch * K * N);
        int32_t *C = malloc(4 * batch * M * N), *D = malloc(4 * batch * M * N);
        for (int64_t e = 0; e < batch * M * K; ++e) A[e] = (int8_t)(rand() % 256 - 128);
        for (int64_t e = 0; e < batch * K * N; ++e) B[e] = (int8_t)(rand() % 256 - 128);
        for (int64_t e = 0; e < batch * M * N; ++e) C[e] = rand() % 2001 - 1000;
        void *dA = dev_copy(A, batch * M * K), *dB = dev_copy(B, batch * K * N);
        void *dC = dev_copy(C, 4 * batch * M * N), *dD = NULL;
        HIPOK(hipMalloc(&dD, 4 * batch * M * N));
        rc = gemm_run(h, dA, dB, dC, dD, M, N, K, K, N, N, GEMM_I8, 0, batch, s);
        CHECK(rc == GEMM_OK, "gemm_run int8");
        HIPOK(hipStreamSynchronize(s));
        HIPOK(hipMemcpy(D, dD, 4 * batch * M * N, hipMemcpyDeviceToHost));
        int bad = 0;
        for (int64_t b = 0; b < batch; ++b)
            for (int64_t i = 0; i < M; ++i)
                for (int64_t j = 0; j < N; ++j) {
                    long acc = C[(b * M + i) * N + j];
                    for (int64_t k = 0; k < K; ++k)
                        acc += (long)A[(b * M + i) * K + k] * B[(b * K + k) * N + j];
                    bad += D[(b * M + i) * N + j] != (int32_t)acc;
                }
        CHECK(bad == 0, "int8 product bit-exact");
        hipFree(dA); hipFree(dB); hipFree(dC); hipFree(dD);
        free(A); free(B); free(C); free(D);
    }

    /* fp64, column-major A, small integers: exact */
    {
        const int64_t M = 40, N = 24, K = 52;
        double *A = malloc(8 * M * K), *B = malloc(8 * K * N), *C = malloc(8 * M * N), *D = malloc(8 * M * N);
        for (int64_t e = 0; e < M * K; ++e) A[e] = rand() % 9 - 4;     /* A[i + k*M] */
        for (int64_t e = 0; e < K * N; ++e) B[e] = rand() % 9 - 4;
        for (int64_t e = 0; e < M * N; ++e) C[e] = rand() % 9 - 4;
        void *dA = dev_copy(A, 8 * M * K), *dB = dev_copy(B, 8 * K * N), *dC = dev_copy(C, 8 * M * N);
        void *dD = NULL;
        HIPOK(hipMalloc(&dD, 8 * M * N));
        rc = gemm_run(h, dA, dB, dC, dD, M, N, K, M, N, N, GEMM_F64, GEMM_A_COLMAJOR, 1, s);
        CHECK(rc == GEMM_OK, "gemm_run fp64");
        HIPOK(hipStreamSynchronize(s));
        HIPOK(hipMemcpy(D, dD, 8 * M * N, hipMemcpyDeviceToHost));
        int bad = 0;
        for (int64_t i = 0; i < M; ++i)
            for (int64_t j = 0; j < N; ++j) {
                double acc = C[i * N + j];
                for (int64_t k = 0; k < K; ++k) acc += A[i + k * M] * B[k * N + j];
                bad += D[i * N + j] != acc;
            }
        CHECK(bad == 0, "fp64 product exact on small integers");
        hipFree(dA); hipFree(dB); hipFree(dC); hipFree(dD);
        free(A); free(B); free(C); free(D);
    }

    /* 2:4 sparse fp16: an A whose every group of four holds two zeros */
    {
        const int64_t M = 32, N = 64, K = 128;
        uint16_t *A = malloc(2 * M * K), *B = malloc(2 * N * K);
        int *Ai = malloc(sizeof(int) * M * K), *Bi = malloc(sizeof(int) * N * K);
        float *C = malloc(4 * M * N), *D = malloc(4 * M * N);
        for (int64_t e = 0; e < M * K; ++e) {
            const int keep = (e % 4) == (e / 4) % 4 || (e % 4) == ((e / 4) + 1) % 4;
            Ai[e] = keep ? rand() % 7 - 3 : 0;
            A[e] = f16_of(Ai[e]);
        }
        for (int64_t e = 0; e < N * K; ++e) { Bi[e] = rand() % 5 - 2; B[e] = f16_of(Bi[e]); }
        for (int64_t e = 0; e < M * N; ++e) C[e] = (float)(rand() % 9 - 4);
        const int64_t kp = 64 * ((K + 63) / 64), mp = 16 * ((M + 15) / 16);
        void *dA = dev_copy(A, 2 * M * K), *dB = dev_copy(B, 2 * N * K), *dC = dev_copy(C, 4 * M * N);
        void *dAc = NULL, *dMeta = NULL, *dD = NULL;
        HIPOK(hipMalloc(&dAc, 2 * mp * kp / 2));
        HIPOK(hipMalloc(&dMeta, 2 * mp * kp / 16));
        HIPOK(hipMalloc(&dD, 4 * M * N));
        rc = gemm_prune24(h, dA, M, K, K, GEMM_F16, 1, dAc, dMeta, s);
        CHECK(rc == GEMM_OK, "gemm_prune24");
        rc = gemm_run_sparse24(h, dAc, dMeta, dB, dC, dD, M, N, K, K, N, GEMM_F16, GEMM_B_COLMAJOR, 1, s);
        CHECK(rc == GEMM_OK, "gemm_run_sparse24");
        HIPOK(hipStreamSynchronize(s));
        HIPOK(hipMemcpy(D, dD, 4 * M * N, hipMemcpyDeviceToHost));
        int bad = 0;
        for (int64_t i = 0; i < M; ++i)
            for (int64_t j = 0; j < N; ++j) {
                long acc = (long)C[i * N + j];
                for (int64_t k = 0; k < K; ++k) acc += (long)Ai[i * K + k] * Bi[j * K + k];
                bad += D[i * N + j] != (float)acc;
            }
        CHECK(bad == 0, "2:4 product of an already-sparse A exact");
        hipFree(dA); hipFree(dB); hipFree(dC); hipFree(dAc); hipFree(dMeta); hipFree(dD);
        free(A); free(B); free(Ai); free(Bi); free(C); free(D);
    }

    char label[128];
    rc = gemm_plan(NULL, 4096, 4096, 4096, 4096, 4096, 4096, GEMM_BF16, GEMM_B_COLMAJOR, 1, label,
                   sizeof label);
    CHECK(rc == GEMM_OK && strncmp(label, "tile256x256", 11) == 0, "gemm_plan without a handle");

    HIPOK(hipStreamDestroy(s));
    CHECK(gemm_destroy(h) == GEMM_OK, "gemm_destroy");
    printf("abi_client: %d checks, %d failures\n", checks, failures);
    return failures ? 1 : 0;
}
