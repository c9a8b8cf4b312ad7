/*
 * oracle_gemm.c -- slow, plain CPU reference for the dense multiply-accumulate
 * D = A*B + C.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library; the GPU library never
 * does, and the two share no code.
 *
 * What it follows (pages: "CDNA2 dense MFMA builtins", section "Naming
 * convention"; "RDNA3 dense WMMA builtins", builtin reference, where each
 * builtin yields the new accumulator): one multiply-accumulate step multiplies a
 * slice of A (M rows, a few k) by the matching slice of B (same k, N columns)
 * and adds it into an M x N tile, so the full product is the sum over all k
 * slices, plus the accumulator input C.  The
 * oracle does not split K into panels at all: the plain definition
 *
 *     D[b][i][j] = x(C[b][i][j]) + sum_k x(A[b][i][k]) * x(B[b][k][j])
 *
 * is evaluated directly, where x() decodes every stored element exactly:
 *   - fp16 (1 sign, 5 exponent, 10 mantissa bits) and bf16 (the top 16 bits of
 *     an IEEE binary32) and fp32 are decoded to double from their bit fields;
 *     every such value is exactly representable in double;
 *   - int8 and int32 are widened to int64.
 * Products of two decoded fp16 (11 significant bits) or bf16 (8 bits) values
 * are exact in double (at most 22 of 53 bits), so the only rounding in the
 * float path is the fp64 summation, bounded by (K-1) * 2^-53 * S with
 * S = sum_k |x(a) x(b)|, far below the tolerance the GPU result is held to.
 * The integer path is exact (|D| < 2^63 for every K < 2^47).
 *
 * The i-k-j loop order keeps B accesses contiguous for row-major B; there is
 * no blocking or reordering beyond that.  Rows are split over threads.
 *
 * fp64 inputs (pages: "CDNA2 dense MFMA builtins", section "FP64-accumulate
 * builtins": one double per lane for A and B, a double accumulator) are not
 * exactly multipliable in double, so that path keeps every product and every
 * partial sum as an unevaluated pair hi + lo (double-double): the product's
 * rounding error is recovered exactly with a fused multiply-add and each
 * addition's with Knuth's two-sum, so the result carries about 106 significant
 * bits -- exact for practical purposes next to the fp64 tolerance.
 *
 * Layout of the inputs (same convention as the GPU library):
 *   A row-major: A[i][k] at A[i*lda + k]   col-major: A[i + k*lda]
 *   B row-major: B[k][j] at B[k*ldb + j]   col-major: B[k + j*ldb]
 *   C row-major: C[i][j] at C[i*ldc + j]
 *   batch b is offset by sa*b, sb*b, sc*b elements.
 * Outputs are dense: D[b][i][j] at D[(b*M + i)*N + j], same for S.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F16 = 0, OR_BF16 = 1, OR_I8 = 2 };

/* ---- exact decoders -------------------------------------------------- */

/* binary16: value = (-1)^s * 2^(e-15) * (1 + m/1024) for 0 < e < 31,
 * (-1)^s * 2^-14 * (m/1024) for e == 0, inf/nan for e == 31. */
double oracle_decode_f16(uint16_t h)
{
    const int s = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1f;
    const int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = (m == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return s ? -v : v;
}

/* binary32: value = (-1)^s * 2^(e-127) * (1 + m/2^23) for 0 < e < 255,
 * (-1)^s * 2^-126 * (m/2^23) for e == 0, inf/nan for e == 255. */
double oracle_decode_f32(uint32_t w)
{
    const int s = (int)(w >> 31);
    const int e = (int)((w >> 23) & 0xff);
    const uint32_t m = w & 0x7fffffu;
    double v;
    if (e == 0)
        v = ldexp((double)m, -149);
    else if (e == 255)
        v = (m == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(0x800000u + m), e - 150);
    return s ? -v : v;
}

/* bfloat16 is the upper half of a binary32. */
double oracle_decode_bf16(uint16_t h) { return oracle_decode_f32((uint32_t)h << 16); }

/* ---- full GEMM -------------------------------------------------------- */

typedef struct {
    int dtype;
    const void *A, *B, *C;
    double *D, *S;       /* float path */
    int64_t *Di;         /* int path */
    int64_t M, N, K, lda, ldb, ldc;
    int a_col, b_col;
    int64_t batch, sa, sb, sc;
    const double *tab;   /* 65536-entry decode table for the 16-bit input type */
    int64_t next_row;    /* work counter over batch*M rows */
    pthread_mutex_t lock;
} job_t;

static int64_t take_row(job_t *J)
{
    pthread_mutex_lock(&J->lock);
    int64_t r = J->next_row++;
    pthread_mutex_unlock(&J->lock);
    return r;
}

static void *float_worker(void *arg)
{
    job_t *J = (job_t *)arg;
    const int64_t N = J->N, K = J->K;
    double *acc = (double *)calloc((size_t)(N > 0 ? N : 1), sizeof(double));
    double *sab = (double *)calloc((size_t)(N > 0 ? N : 1), sizeof(double));
    const uint16_t *A = (const uint16_t *)J->A;
    const uint16_t *B = (const uint16_t *)J->B;
    const uint32_t *C = (const uint32_t *)J->C;
    for (;;) {
        const int64_t r = take_row(J);
        if (r >= J->batch * J->M) break;
        const int64_t b = r / J->M, i = r % J->M;
        const uint16_t *Ab = A + b * J->sa;
        const uint16_t *Bb = B + b * J->sb;
        for (int64_t j = 0; j < N; ++j) { acc[j] = 0.0; sab[j] = 0.0; }
        for (int64_t k = 0; k < K; ++k) {
            const double a = J->tab[J->a_col ? Ab[i + k * J->lda] : Ab[i * J->lda + k]];
            for (int64_t j = 0; j < N; ++j) {
                const double bv = J->tab[J->b_col ? Bb[k + j * J->ldb] : Bb[k * J->ldb + j]];
                const double p = a * bv;
                acc[j] += p;
                sab[j] += fabs(p);
            }
        }
        const uint32_t *Cb = C + b * J->sc;
        for (int64_t j = 0; j < N; ++j) {
            J->D[r * N + j] = oracle_decode_f32(Cb[i * J->ldc + j]) + acc[j];
            J->S[r * N + j] = sab[j];
        }
    }
    free(acc);
    free(sab);
    return NULL;
}

static void *int_worker(void *arg)
{
    job_t *J = (job_t *)arg;
    const int64_t N = J->N, K = J->K;
    int64_t *acc = (int64_t *)calloc((size_t)(N > 0 ? N : 1), sizeof(int64_t));
    const int8_t *A = (const int8_t *)J->A;
    const int8_t *B = (const int8_t *)J->B;
    const int32_t *C = (const int32_t *)J->C;
    for (;;) {
        const int64_t r = take_row(J);
        if (r >= J->batch * J->M) break;
        const int64_t b = r / J->M, i = r % J->M;
        const int8_t *Ab = A + b * J->sa;
        const int8_t *Bb = B + b * J->sb;
        for (int64_t j = 0; j < N; ++j) acc[j] = 0;
        for (int64_t k = 0; k < K; ++k) {
            const int64_t a = (int64_t)(J->a_col ? Ab[i + k * J->lda] : Ab[i * J->lda + k]);
            for (int64_t j = 0; j < N; ++j) {
                const int64_t bv = (int64_t)(J->b_col ? Bb[k + j * J->ldb] : Bb[k * J->ldb + j]);
                acc[j] += a * bv;
            }
        }
        const int32_t *Cb = C + b * J->sc;
        for (int64_t j = 0; j < N; ++j)
            J->Di[r * N + j] = (int64_t)Cb[i * J->ldc + j] + acc[j];
    }
    free(acc);
    return NULL;
}

static double *make_table(int dtype)
{
    double *t = (double *)malloc(65536 * sizeof(double));
    if (!t) return NULL;
    for (uint32_t h = 0; h < 65536; ++h)
        t[h] = (dtype == OR_F16) ? oracle_decode_f16((uint16_t)h) : oracle_decode_bf16((uint16_t)h);
    return t;
}

static int run_threads(job_t *J, void *(*fn)(void *), int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, fn, J) != 0) break;
        ++started;
    }
    if (started == 0) fn(J);
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    return 0;
}

/*
 * Float path: A, B hold fp16 (dtype 0) or bf16 (dtype 1) bit patterns, C holds
 * fp32 bit patterns.  Writes D_ref and S = sum_k |a*b| (both dense, double).
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_gemm_float(int dtype, const uint16_t *A, const uint16_t *B, const uint32_t *C,
                      double *D, double *S, int64_t M, int64_t N, int64_t K,
                      int64_t lda, int64_t ldb, int64_t ldc, int a_col, int b_col,
                      int64_t batch, int64_t sa, int64_t sb, int64_t sc, int nthreads)
{
    if ((dtype != OR_F16 && dtype != OR_BF16) || M < 0 || N < 0 || K < 0 || batch < 0)
        return -1;
    job_t J;
    memset(&J, 0, sizeof(J));
    J.dtype = dtype; J.A = A; J.B = B; J.C = C; J.D = D; J.S = S;
    J.M = M; J.N = N; J.K = K; J.lda = lda; J.ldb = ldb; J.ldc = ldc;
    J.a_col = a_col; J.b_col = b_col; J.batch = batch; J.sa = sa; J.sb = sb; J.sc = sc;
    double *tab = make_table(dtype);
    if (!tab) return -1;
    J.tab = tab;
    pthread_mutex_init(&J.lock, NULL);
    run_threads(&J, float_worker, nthreads);
    pthread_mutex_destroy(&J.lock);
    free(tab);
    return 0;
}

/* Integer path: int8 A and B, int32 C, exact int64 D_ref. */
int oracle_gemm_int8(const int8_t *A, const int8_t *B, const int32_t *C, int64_t *D,
                     int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                     int a_col, int b_col, int64_t batch, int64_t sa, int64_t sb, int64_t sc,
                     int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || batch < 0) return -1;
    job_t J;
    memset(&J, 0, sizeof(J));
    J.dtype = OR_I8; J.A = A; J.B = B; J.C = C; J.Di = D;
    J.M = M; J.N = N; J.K = K; J.lda = lda; J.ldb = ldb; J.ldc = ldc;
    J.a_col = a_col; J.b_col = b_col; J.batch = batch; J.sa = sa; J.sb = sb; J.sc = sc;
    pthread_mutex_init(&J.lock, NULL);
    run_threads(&J, int_worker, nthreads);
    pthread_mutex_destroy(&J.lock);
    return 0;
}

/* ---- fp64 inputs -------------------------------------------------------- */

/* a + b = *s + *e exactly (Knuth's two-sum; valid for any ordering of |a|, |b|). */
static void two_sum(double a, double b, double *s, double *e)
{
    const double x = a + b;
    const double bv = x - a;
    const double av = x - bv;
    *s = x;
    *e = (a - av) + (b - bv);
}

/* a * b = *p + *e exactly (fma rounds once, so it returns the exact residual). */
static void two_prod(double a, double b, double *p, double *e)
{
    const double x = a * b;
    *p = x;
    *e = fma(a, b, -x);
}

/* (hi, lo) += v + w, keeping the rounding error of the leading addition. */
static void dd_add(double *hi, double *lo, double v, double w)
{
    double s, e;
    two_sum(*hi, v, &s, &e);
    *hi = s;
    *lo += e + w;
}

typedef struct {
    const double *A, *B, *C;
    double *Dhi, *Dlo, *S;
    int64_t M, N, K, lda, ldb, ldc;
    int a_col, b_col;
    int64_t batch, sa, sb, sc;
    int64_t next_row;
    pthread_mutex_t lock;
} job64_t;

static void *f64_worker(void *arg)
{
    job64_t *J = (job64_t *)arg;
    const int64_t N = J->N, K = J->K;
    double *hi = (double *)calloc((size_t)(N > 0 ? N : 1), sizeof(double));
    double *lo = (double *)calloc((size_t)(N > 0 ? N : 1), sizeof(double));
    double *sab = (double *)calloc((size_t)(N > 0 ? N : 1), sizeof(double));
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int64_t r = J->next_row++;
        pthread_mutex_unlock(&J->lock);
        if (r >= J->batch * J->M) break;
        const int64_t b = r / J->M, i = r % J->M;
        const double *Ab = J->A + b * J->sa;
        const double *Bb = J->B + b * J->sb;
        for (int64_t j = 0; j < N; ++j) { hi[j] = 0.0; lo[j] = 0.0; sab[j] = 0.0; }
        for (int64_t k = 0; k < K; ++k) {
            const double a = J->a_col ? Ab[i + k * J->lda] : Ab[i * J->lda + k];
            for (int64_t j = 0; j < N; ++j) {
                const double bv = J->b_col ? Bb[k + j * J->ldb] : Bb[k * J->ldb + j];
                double p, pe;
                two_prod(a, bv, &p, &pe);
                dd_add(&hi[j], &lo[j], p, pe);
                sab[j] += fabs(p);
            }
        }
        const double *Cb = J->C + b * J->sc;
        for (int64_t j = 0; j < N; ++j) {
            dd_add(&hi[j], &lo[j], Cb[i * J->ldc + j], 0.0);
            two_sum(hi[j], lo[j], &J->Dhi[r * N + j], &J->Dlo[r * N + j]);
            J->S[r * N + j] = sab[j];
        }
    }
    free(hi);
    free(lo);
    free(sab);
    return NULL;
}

/*
 * fp64 path: D_ref = C + sum_k A B as the pair Dhi + Dlo (|Dlo| <= ulp(Dhi)/2),
 * and S = sum_k |a*b| (plain double).  Same layouts and outputs as the float path.
 */
int oracle_gemm_f64(const double *A, const double *B, const double *C, double *Dhi,
                    double *Dlo, double *S, int64_t M, int64_t N, int64_t K, int64_t lda,
                    int64_t ldb, int64_t ldc, int a_col, int b_col, int64_t batch, int64_t sa,
                    int64_t sb, int64_t sc, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || batch < 0) return -1;
    job64_t J;
    memset(&J, 0, sizeof(J));
    J.A = A; J.B = B; J.C = C; J.Dhi = Dhi; J.Dlo = Dlo; J.S = S;
    J.M = M; J.N = N; J.K = K; J.lda = lda; J.ldb = ldb; J.ldc = ldc;
    J.a_col = a_col; J.b_col = b_col; J.batch = batch; J.sa = sa; J.sb = sb; J.sc = sc;
    pthread_mutex_init(&J.lock, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, f64_worker, &J) != 0) break;
        ++started;
    }
    if (started == 0) f64_worker(&J);
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    pthread_mutex_destroy(&J.lock);
    return 0;
}

/* fp64 path at listed (b, i, j) positions only. */
int oracle_gemm_f64_points(const double *A, const double *B, const double *C,
                           const int64_t *pts, int64_t npts, double *Dhi, double *Dlo, double *S,
                           int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                           int64_t ldc, int a_col, int b_col, int64_t batch, int64_t sa,
                           int64_t sb, int64_t sc)
{
    if (K < 0) return -1;
    for (int64_t p = 0; p < npts; ++p) {
        const int64_t b = pts[3 * p], i = pts[3 * p + 1], j = pts[3 * p + 2];
        if (b < 0 || b >= batch || i < 0 || i >= M || j < 0 || j >= N) return -1;
    }
    for (int64_t p = 0; p < npts; ++p) {
        const int64_t b = pts[3 * p], i = pts[3 * p + 1], j = pts[3 * p + 2];
        const double *Ab = A + b * sa, *Bb = B + b * sb;
        double hi = 0.0, lo = 0.0, sab = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = a_col ? Ab[i + k * lda] : Ab[i * lda + k];
            const double bv = b_col ? Bb[k + j * ldb] : Bb[k * ldb + j];
            double q, qe;
            two_prod(a, bv, &q, &qe);
            dd_add(&hi, &lo, q, qe);
            sab += fabs(q);
        }
        dd_add(&hi, &lo, C[b * sc + i * ldc + j], 0.0);
        two_sum(hi, lo, &Dhi[p], &Dlo[p]);
        S[p] = sab;
    }
    return 0;
}

/* ---- selected elements ------------------------------------------------ */

/*
 * The same definition evaluated for a list of output positions only, one
 * K-long dot product each, so that samples of full-size problems can be
 * checked.  pts holds npts triples (b, i, j).  For dtype 0/1, D and S receive
 * doubles; for dtype 2 (int8), Di receives int64 and D/S are ignored.
 */
int oracle_gemm_points(int dtype, const void *A, const void *B, const void *C,
                       const int64_t *pts, int64_t npts, double *D, double *S, int64_t *Di,
                       int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                       int a_col, int b_col, int64_t batch, int64_t sa, int64_t sb, int64_t sc)
{
    if (dtype < 0 || dtype > 2 || K < 0) return -1;
    for (int64_t p = 0; p < npts; ++p) {
        const int64_t b = pts[3 * p], i = pts[3 * p + 1], j = pts[3 * p + 2];
        if (b < 0 || b >= batch || i < 0 || i >= M || j < 0 || j >= N) return -1;
    }
    if (dtype == OR_I8) {
        const int8_t *Ap = (const int8_t *)A, *Bp = (const int8_t *)B;
        const int32_t *Cp = (const int32_t *)C;
        for (int64_t p = 0; p < npts; ++p) {
            const int64_t b = pts[3 * p], i = pts[3 * p + 1], j = pts[3 * p + 2];
            const int8_t *Ab = Ap + b * sa, *Bb = Bp + b * sb;
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k) {
                const int64_t a = a_col ? Ab[i + k * lda] : Ab[i * lda + k];
                const int64_t bv = b_col ? Bb[k + j * ldb] : Bb[k * ldb + j];
                acc += a * bv;
            }
            Di[p] = (int64_t)Cp[b * sc + i * ldc + j] + acc;
        }
        return 0;
    }
    const uint16_t *Ap = (const uint16_t *)A, *Bp = (const uint16_t *)B;
    const uint32_t *Cp = (const uint32_t *)C;
    for (int64_t p = 0; p < npts; ++p) {
        const int64_t b = pts[3 * p], i = pts[3 * p + 1], j = pts[3 * p + 2];
        const uint16_t *Ab = Ap + b * sa, *Bb = Bp + b * sb;
        double acc = 0.0, sab = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const uint16_t ah = a_col ? Ab[i + k * lda] : Ab[i * lda + k];
            const uint16_t bh = b_col ? Bb[k + j * ldb] : Bb[k * ldb + j];
            const double a = dtype == OR_F16 ? oracle_decode_f16(ah) : oracle_decode_bf16(ah);
            const double bv = dtype == OR_F16 ? oracle_decode_f16(bh) : oracle_decode_bf16(bh);
            acc += a * bv;
            sab += fabs(a * bv);
        }
        D[p] = oracle_decode_f32(Cp[b * sc + i * ldc + j]) + acc;
        S[p] = sab;
    }
    return 0;
}
