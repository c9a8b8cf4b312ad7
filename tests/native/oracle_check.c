/*
 * Memory and undefined-behaviour check of the CPU oracle (oracle/oracle_gemm.c),
 * built with the address and undefined-behaviour sanitizers by
 * tests/test_sanitizers.py.  Every operand lives in a heap buffer of exactly
 * its extent (batch strides, leading dimensions, padding), so any read past it
 * is reported.  The full and the single-position entry points are run on random
 * small problems in every layout, single- and multi-threaded, and must agree;
 * an identity B must return A + C exactly.  Exit status 0: all checks held.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_gemm_float(int dtype, const uint16_t *A, const uint16_t *B, const uint32_t *C,
                      double *D, double *S, int64_t M, int64_t N, int64_t K, int64_t lda,
                      int64_t ldb, int64_t ldc, int a_col, int b_col, int64_t batch, int64_t sa,
                      int64_t sb, int64_t sc, int nthreads);
int oracle_gemm_int8(const int8_t *A, const int8_t *B, const int32_t *C, int64_t *D, int64_t M,
                     int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int a_col,
                     int b_col, int64_t batch, int64_t sa, int64_t sb, int64_t sc, int nthreads);
int oracle_gemm_points(int dtype, const void *A, const void *B, const void *C, const int64_t *pts,
                       int64_t npts, double *D, double *S, int64_t *Di, int64_t M, int64_t N,
                       int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int a_col, int b_col,
                       int64_t batch, int64_t sa, int64_t sb, int64_t sc);
int oracle_gemm_f64(const double *A, const double *B, const double *C, double *Dhi, double *Dlo,
                    double *S, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                    int64_t ldc, int a_col, int b_col, int64_t batch, int64_t sa, int64_t sb,
                    int64_t sc, int nthreads);
int oracle_gemm_f64_points(const double *A, const double *B, const double *C, const int64_t *pts,
                           int64_t npts, double *Dhi, double *Dlo, double *S, int64_t M, int64_t N,
                           int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int a_col, int b_col,
                           int64_t batch, int64_t sa, int64_t sb, int64_t sc);

static int failures = 0;
#define CHECK(cond, what)                                                  \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "FAILED %s (%s) at case %d\n", #cond, what, cs); \
            ++failures;                                                    \
        }                                                                  \
    } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 11);
}
static int64_t rint_in(int64_t lo, int64_t hi) { return lo + (int64_t)(rnd() % (uint32_t)(hi - lo + 1)); }

/* extent (elements) of `batch` blocks `stride` apart of `rows` rows `ld` apart, `cols` used */
static int64_t extent(int64_t batch, int64_t stride, int64_t rows, int64_t ld, int64_t cols) {
    if (batch == 0 || rows == 0 || cols == 0) return 1;
    return (batch - 1) * stride + (rows - 1) * ld + cols;
}

/* small exactly representable values: fp16 / bf16 patterns of integers in [-4, 4] */
static uint16_t f16_small(void) {
    static const uint16_t t[9] = {0xC400, 0xC200, 0xC000, 0xBC00, 0x0000,
                                  0x3C00, 0x4000, 0x4200, 0x4400};
    return t[rnd() % 9];
}
static uint16_t bf16_small(void) {
    static const uint16_t t[9] = {0xC080, 0xC040, 0xC000, 0xBF80, 0x0000,
                                  0x3F80, 0x4000, 0x4040, 0x4080};
    return t[rnd() % 9];
}

int main(void) {
    int cs = 0;
    for (cs = 0; cs < 400; ++cs) {
        const int dtype = cs % 4; /* 0 f16, 1 bf16, 2 int8, 3 fp64 */
        const int a_col = (cs >> 2) & 1, b_col = (cs >> 3) & 1;
        const int64_t M = rint_in(0, 9), N = rint_in(0, 9), K = rint_in(0, 13);
        const int64_t batch = rint_in(1, 3), pad = rint_in(0, 2);
        const int64_t lda = (a_col ? M : K) + pad + (a_col ? (M == 0) : (K == 0));
        const int64_t ldb = (b_col ? K : N) + pad + (b_col ? (K == 0) : (N == 0));
        const int64_t ldc = N + pad + (N == 0);
        const int64_t sa = (a_col ? K : M) * lda, sb = (b_col ? N : K) * ldb, sc = M * ldc;
        const int64_t nA = extent(batch, sa, a_col ? K : M, lda, a_col ? M : K);
        const int64_t nB = extent(batch, sb, b_col ? N : K, ldb, b_col ? K : N);
        const int64_t nC = extent(batch, sc, M, ldc, N);
        const int64_t nD = batch * M * N > 0 ? batch * M * N : 1;
        const int threads = (cs & 1) ? 4 : 1;
        int64_t *pts = malloc(sizeof(int64_t) * 3 * (size_t)nD);
        int64_t np = 0;
        for (int64_t b = 0; b < batch; ++b)
            for (int64_t i = 0; i < M; ++i)
                for (int64_t j = 0; j < N; ++j) {
                    pts[3 * np] = b; pts[3 * np + 1] = i; pts[3 * np + 2] = j; ++np;
                }
        if (dtype <= 1) {
            uint16_t *A = malloc(2 * (size_t)nA), *B = malloc(2 * (size_t)nB);
            uint32_t *C = malloc(4 * (size_t)nC);
            for (int64_t e = 0; e < nA; ++e) A[e] = dtype ? bf16_small() : f16_small();
            for (int64_t e = 0; e < nB; ++e) B[e] = dtype ? bf16_small() : f16_small();
            for (int64_t e = 0; e < nC; ++e) C[e] = (rnd() % 2) ? 0x3F800000u : 0xC0000000u;
            double *D = malloc(8 * (size_t)nD), *S = malloc(8 * (size_t)nD);
            double *Dp = malloc(8 * (size_t)nD), *Sp = malloc(8 * (size_t)nD);
            CHECK(oracle_gemm_float(dtype, A, B, C, D, S, M, N, K, lda, ldb, ldc, a_col, b_col,
                                    batch, sa, sb, sc, threads) == 0, "float full");
            CHECK(oracle_gemm_points(dtype, A, B, C, pts, np, Dp, Sp, NULL, M, N, K, lda, ldb, ldc,
                                     a_col, b_col, batch, sa, sb, sc) == 0, "float points");
            for (int64_t p = 0; p < np; ++p)  /* small integers: every sum is exact */
                CHECK(D[p] == Dp[p] && S[p] == Sp[p], "full == points");
            free(A); free(B); free(C); free(D); free(S); free(Dp); free(Sp);
        } else if (dtype == 2) {
            int8_t *A = malloc((size_t)nA), *B = malloc((size_t)nB);
            int32_t *C = malloc(4 * (size_t)nC);
            for (int64_t e = 0; e < nA; ++e) A[e] = (int8_t)(rnd() & 0xFF);
            for (int64_t e = 0; e < nB; ++e) B[e] = (int8_t)(rnd() & 0xFF);
            for (int64_t e = 0; e < nC; ++e) C[e] = (int32_t)(rnd() % 2000001) - 1000000;
            int64_t *D = malloc(8 * (size_t)nD), *Dp = malloc(8 * (size_t)nD);
            CHECK(oracle_gemm_int8(A, B, C, D, M, N, K, lda, ldb, ldc, a_col, b_col, batch, sa, sb,
                                   sc, threads) == 0, "int8 full");
            CHECK(oracle_gemm_points(2, A, B, C, pts, np, NULL, NULL, Dp, M, N, K, lda, ldb, ldc,
                                     a_col, b_col, batch, sa, sb, sc) == 0, "int8 points");
            for (int64_t p = 0; p < np; ++p) CHECK(D[p] == Dp[p], "int8 full == points");
            free(A); free(B); free(C); free(D); free(Dp);
        } else {
            double *A = malloc(8 * (size_t)nA), *B = malloc(8 * (size_t)nB);
            double *C = malloc(8 * (size_t)nC);
            for (int64_t e = 0; e < nA; ++e) A[e] = ldexp((double)(int32_t)rnd(), -31);
            for (int64_t e = 0; e < nB; ++e) B[e] = ldexp((double)(int32_t)rnd(), -31);
            for (int64_t e = 0; e < nC; ++e) C[e] = ldexp((double)(int32_t)rnd(), -20);
            double *Dh = malloc(8 * (size_t)nD), *Dl = malloc(8 * (size_t)nD), *S = malloc(8 * (size_t)nD);
            double *Ph = malloc(8 * (size_t)nD), *Pl = malloc(8 * (size_t)nD), *Ps = malloc(8 * (size_t)nD);
            CHECK(oracle_gemm_f64(A, B, C, Dh, Dl, S, M, N, K, lda, ldb, ldc, a_col, b_col, batch,
                                  sa, sb, sc, threads) == 0, "f64 full");
            CHECK(oracle_gemm_f64_points(A, B, C, pts, np, Ph, Pl, Ps, M, N, K, lda, ldb, ldc,
                                         a_col, b_col, batch, sa, sb, sc) == 0, "f64 points");
            for (int64_t p = 0; p < np; ++p)
                CHECK(Dh[p] == Ph[p] && Dl[p] == Pl[p] && S[p] == Ps[p], "f64 full == points");
            free(A); free(B); free(C); free(Dh); free(Dl); free(S); free(Ph); free(Pl); free(Ps);
        }
        free(pts);
    }
    /* identity: A (int8, row-major 5 x 7) times I_7 plus C equals A + C */
    {
        int8_t A[35], B[49];
        int32_t C[35];
        int64_t D[35];
        for (int e = 0; e < 35; ++e) { A[e] = (int8_t)(rnd() & 0xFF); C[e] = (int32_t)rnd() % 1000; }
        for (int e = 0; e < 49; ++e) B[e] = (int8_t)(e % 8 == 0);
        CHECK(oracle_gemm_int8(A, B, C, D, 5, 7, 7, 7, 7, 7, 0, 0, 1, 35, 49, 35, 2) == 0, "identity");
        for (int e = 0; e < 35; ++e) CHECK(D[e] == (int64_t)A[e] + C[e], "A * I + C");
    }
    printf("oracle_check: %d cases, %d failures\n", cs, failures);
    return failures ? 1 : 0;
}
