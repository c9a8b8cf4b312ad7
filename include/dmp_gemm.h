/*
 * dmp_gemm.h -- C ABI of the gfx950 (MI355X) dense mixed-precision GEMM library.
 *
 * Operation (pages: "CDNA2 dense MFMA builtins", section "Naming convention",
 * and "RDNA3 dense WMMA builtins", builtin reference): one MFMA step multiplies
 * a slice of A (M rows, a few k) by the matching slice of B (same k, N columns)
 * and adds the result into an M x N accumulator tile, srcA x srcB + srcC; the
 * caller steps through all of K.  This library runs the whole loop on the GPU and computes,
 * for every batch index b < batch,
 *
 *         D_b = A_b * B_b + C_b
 *
 * with the input types and accumulators below.  C is added once, after the
 * whole K reduction (an fp32 round-to-nearest-even add, or an exact int32 add).
 *
 *   dtype      A, B elements         C and D elements    accumulation
 *   GEMM_F16   IEEE binary16         float (fp32)        fp32 (MFMA)
 *   GEMM_BF16  bfloat16              float (fp32)        fp32 (MFMA)
 *   GEMM_I8    int8 (signed)         int32               int32 (MFMA), exact
 *   GEMM_F64   IEEE binary64         double (fp64)       fp64 (MFMA), every step
 *                                                        rounded to nearest even
 *
 * int8 results are exact whenever the true result fits in int32 (the
 * accumulation wraps modulo 2^32, which is associative, so partial sums may
 * overflow as long as the final value fits).  fp16/bf16 results satisfy, per
 * element, |D - D_exact| <= 4*K*2^-24 * sum_k |a_ik b_kj| + 2^-24 * |c_ij|;
 * fp64 results satisfy |D - D_exact| <= (2K+2)*2^-53 * sum_k |a_ik b_kj| +
 * 2^-53 * |c_ij| (pages: "CDNA2 dense MFMA builtins", section "FP64-accumulate
 * builtins": the FP64 instructions round partial products to nearest even).
 *
 * Memory layout (element strides, not bytes):
 *   A row-major (default):        A[i][k] at A[i*lda + k], lda >= K
 *   A col-major (GEMM_A_COLMAJOR): A[i][k] at A[i + k*lda], lda >= M
 *   B row-major (default):        B[k][j] at B[k*ldb + j], ldb >= N
 *   B col-major (GEMM_B_COLMAJOR): B[k][j] at B[k + j*ldb], ldb >= K
 *   C and D are row-major and share ldc >= N: X[i][j] at X[i*ldc + j]
 *   Batches are contiguous: A_b = A + b*(row-major ? M : K)*lda,
 *   B_b = B + b*(row-major ? K : N)*ldb, C_b = C + b*M*ldc, D_b = D + b*M*ldc;
 *   with GEMM_A_SHARED (GEMM_B_SHARED) A_b = A (B_b = B) for every b.
 *
 * Products with M <= 16 and N <= 16 (fp16, bf16, int8) run on the multi-block
 * matrix instructions, several batch entries per instruction (pages: "CDNA2
 * dense MFMA builtins", section "Accumulator layout", 4x4 and 16x16 shapes);
 * a shared A or B is then loaded once and broadcast by the instruction's
 * cbsz/abid and blgp modifiers ("MFMA common parameters").
 *
 * Ownership: the caller allocates A, B, C and D in device memory and keeps them
 * alive until the work on `stream` has finished.  The library never frees caller
 * memory.  A handle owns only a lazily grown device workspace (used by the
 * split-K path and by the transposed copy of a row-major int8 B for large M)
 * and cached device properties; one handle serves one host thread at a time,
 * and calls through one handle on different streams must not overlap (they
 * would share the workspace).  D may alias C exactly (same pointer, same ldc); any other overlap
 * between D and an input is undefined.
 *
 * Caching: D (every output the library writes) is stored with non-temporal
 * stores.  It is written once and is not kept in the caches, so it does not
 * displace operands; a kernel that reads D right afterwards fetches it from
 * HBM.
 *
 * Graph capture: the calls enqueue kernels only (no memset or copy nodes), so
 * they can be captured into a HIP graph once the handle's workspace is large
 * enough, i.e. after an eager call of the same (or a larger) shape on the same
 * handle; a call that must grow the workspace synchronises the device and
 * allocates, which capture does not allow.  A graph keeps the workspace's
 * address: replaying it after a later call on the handle has grown (replaced)
 * the workspace is undefined.
 *
 * Errors: every call returns a gemm_status_t.  Arguments are validated before
 * anything is enqueued; on error nothing is launched.  Limits: M, N, K below
 * 2^31 - 1024, batch at most 2^30, leading dimensions at most 2^48, and
 * every operand's extent (the largest element index over all batch entries,
 * from the leading dimensions and batch strides) at most 2^48 elements;
 * beyond them GEMM_ERR_INVALID_ARG.  Launches
 * are asynchronous on `stream` (a hipStream_t, NULL = the null stream), so
 * faults during execution surface at the caller's next synchronisation.
 */
#ifndef DMP_GEMM_H
#define DMP_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gemm_handle *gemm_handle_t;

typedef enum { GEMM_F16 = 0, GEMM_BF16 = 1, GEMM_I8 = 2, GEMM_F64 = 3 } gemm_dtype_t;

/*
 * flags: bitwise OR; default (0) is row-major A and row-major B, each with its
 * own matrix per batch entry.  GEMM_A_SHARED / GEMM_B_SHARED: one A (B) serves
 * every batch entry (batch stride 0), e.g. one small transform applied to many
 * inputs.
 */
enum { GEMM_A_COLMAJOR = 1u, GEMM_B_COLMAJOR = 2u, GEMM_A_SHARED = 4u, GEMM_B_SHARED = 8u };

typedef enum {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_ARG = 1,        /* null pointer, negative size, ld too small, bad dtype/flags */
    GEMM_ERR_UNSUPPORTED_DEVICE = 2, /* current device is not gfx950; there is no fallback */
    GEMM_ERR_ALLOC = 3,              /* workspace allocation failed */
    GEMM_ERR_HIP = 4,                /* a HIP API call or kernel launch reported an error; the
                                        launch status is read with hipGetLastError, so an error an
                                        earlier HIP call of this thread left unread is reported too */
    GEMM_ERR_SCRATCH = 5             /* gemm_run_noalloc: the product needs more scratch than
                                        GEMM_NOALLOC_SCRATCH_BYTES; nothing was enqueued */
} gemm_status_t;

/*
 * Create a handle bound to the current HIP device.  *out receives the handle
 * (NULL on failure).  Fails with GEMM_ERR_UNSUPPORTED_DEVICE unless the device
 * is gfx950.
 */
int gemm_create(gemm_handle_t *out);

/*
 * Enqueue D_b = A_b*B_b + C_b for b < batch on `stream` (layouts above).
 * A, B, C, D: device pointers (must be non-NULL when the product is non-empty).
 * M, N, K, batch >= 0.  M, N or batch == 0 is a no-op returning GEMM_OK.
 * K == 0 gives D = C (A, B and their leading dimensions are then not used).
 * dtype: a gemm_dtype_t.  flags: any OR of GEMM_A_COLMAJOR, GEMM_B_COLMAJOR,
 * GEMM_A_SHARED and GEMM_B_SHARED.  Pointers must be aligned to their element size; any such
 * pointer and any leading dimension is accepted, and 16-byte aligned pointers
 * with leading dimensions that are multiples of 16 bytes take the fast tiled
 * path (for K-contiguous operands K, for M/N-contiguous ones M or N, must also
 * be a whole number of 16-byte granules).
 */
int gemm_run(gemm_handle_t h, const void *A, const void *B, const void *C, void *D,
             int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
             int dtype, unsigned flags, int64_t batch, void *stream);

/* Storage types of C and D for gemm_run_ex. */
typedef enum {
    GEMM_OUT_F32 = 0, GEMM_OUT_F16 = 1, GEMM_OUT_BF16 = 2, GEMM_OUT_I32 = 3, GEMM_OUT_F64 = 4
} gemm_out_t;

/*
 * Scaled product with a low-precision output (the fp16/bf16-result variants of
 * the matrix instructions; pages: "RDNA3 dense WMMA builtins", FP16- and
 * BF16-accumulate builtins, which keep the result in 16-bit storage).  For
 * b < batch:
 *
 *     D_b = cvt_D( alpha * (A_b * B_b)  +  beta * cvt(C_b) )
 *
 * computed as: the fp32 accumulation of gemm_run, then t = alpha*acc and
 * u = beta*c (each an fp32 round-to-nearest-even product; c decoded exactly
 * from C's storage type), s = t + u (fp32 RNE add; no fused multiply-add), and
 * finally s converted to D's storage type with round-to-nearest-even.
 * beta == 0: C is not read (may be NULL) and D = cvt_D(alpha*acc).
 * c_type, d_type: gemm_out_t.  fp16/bf16 inputs accept GEMM_OUT_F32, _F16 and
 * _BF16 for each of C and D independently; int8 inputs require GEMM_OUT_I32
 * for both, fp64 inputs GEMM_OUT_F64 for both, and each of them alpha == 1 and
 * beta in {0, 1}.  C and D share ldc (in elements of
 * their own type); D may alias C only when their types are equal.  All other
 * arguments, layouts and errors are those of gemm_run, which equals
 * gemm_run_ex with alpha = beta = 1 and C, D in the accumulator type.
 */
int gemm_run_ex(gemm_handle_t h, const void *A, const void *B, const void *C, void *D,
                int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                int dtype, unsigned flags, int64_t batch, float alpha, float beta,
                int c_type, int d_type, void *stream);

/*
 * 2:4 structured-sparse A (the sparse matrix instructions; pages: "MFMA common
 * parameters", section "Sparse MFMA parameters": two of every four consecutive
 * K positions of A hold the non-zeros, and an index operand names them).
 *
 * gemm_prune24 compresses a row-major A (fp16, bf16 or int8, M x K, lda >= K,
 * batch entries M*lda elements apart): in every group of four consecutive k of
 * a row (the last group of a row may be shorter) the two entries of largest
 * magnitude are kept -- on a tie the lower k; positions past K never win over
 * present ones; float inputs are taken to be finite -- and the others dropped.
 * Output, with KT = 64 (fp16/bf16) or 128 (int8) dense k per sparse k-tile,
 * Kp = KT * ceil(K / KT), T = Kp / KT and Mp = 16 * ceil(M / 16):
 *   row data: for row i, value slot 2q of its Kp/2 slots holds the kept value
 *         of group q (k 4q..4q+3) at the lower position, slot 2q+1 the other;
 *         index word w (of Kp/16) covers groups 4w..4w+3 and its bits
 *         [2j+1:2j] are the position (0..3) inside its group of value slot
 *         8w + j (the same bits for every input type: four per group, groups
 *         in k order, low bits first).  Groups past K and rows M..Mp-1 hold
 *         zero values (their index words name positions 0 and 1).
 *   Ac:   batch x Mp x Kp/2 values of A's type, blocked: value slot s of row
 *         i lies at element ((b*(Mp/16) + i/16)*T + s/(KT/2))*16*(KT/2)
 *         + (i%16)*(KT/2) + s%(KT/2) -- one k-tile of 16 rows is 1 KB,
 *         contiguous, so that the product's copies read whole cache lines;
 *   meta: batch x Mp x Kp/16 uint16, blocked the same way: word w of row i at
 *         ((b*(Mp/16) + i/16)*T + w/(KT/16))*16*(KT/16) + (i%16)*(KT/16)
 *         + w%(KT/16).
 * Pointers need element alignment (meta: 2 bytes) here; gemm_run_sparse24
 * needs Ac and meta 16-byte aligned (hipMalloc'd buffers are).
 */
int gemm_prune24(gemm_handle_t h, const void *A, int64_t M, int64_t K, int64_t lda, int dtype,
                 int64_t batch, void *Ac, void *meta, void *stream);

/*
 * D_b = prune(A_b) * B_b + C_b from the compressed form written by
 * gemm_prune24 (same M, K, dtype and batch), on v_smfmac_f32_32x32x32_{f16,bf16}
 * or v_smfmac_i32_32x32x64_i8.  B is K x N of A's type, row-major (default) or
 * GEMM_B_COLMAJOR (the only flag taken), batch entries (K or N)*ldb elements
 * apart; C and D fp32 (fp16/bf16) or int32 (int8), row-major, ldc >= N, batch
 * entries M*ldc apart; D may alias C exactly.  Accuracy as gemm_run's with the
 * pruned A: the fp16/bf16 bound, int8 exact (int32, wrapping).  Requirements
 * (else GEMM_ERR_INVALID_ARG, nothing enqueued): B 16-byte aligned, ldb a
 * multiple of 16 bytes, and N (row-major B) or K (column-major B) a multiple
 * of 16 bytes' worth of elements (8 for fp16/bf16, 16 for int8).
 * K == 0 gives D = C.
 */
int gemm_run_sparse24(gemm_handle_t h, const void *Ac, const void *meta, const void *B,
                      const void *C, void *D, int64_t M, int64_t N, int64_t K, int64_t ldb,
                      int64_t ldc, int dtype, unsigned flags, int64_t batch, void *stream);

/*
 * For callers that cannot allocate device memory while they run products: code
 * that a HIP graph captures, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, semantics, results (bit for bit) and errors as
 * gemm_run_ex, but the split-K partials and the transposed copy of a row-major
 * int8 B live in a fixed scratch array of GEMM_NOALLOC_SCRATCH_BYTES (64 MiB)
 * that the library holds on every device it runs on until the process ends;
 * the call never allocates or frees device memory (the scratch address is
 * looked up once per device by gemm_create).  A product whose plan needs more
 * scratch fails with GEMM_ERR_SCRATCH and enqueues nothing (gemm_run_ex then
 * serves it).  The current device must be the handle's (else
 * GEMM_ERR_INVALID_ARG).  Every call on one device shares that device's
 * scratch and leaves its contents behind: calls that can run at the same time
 * on one device (different streams, threads or handles) race and must be
 * ordered by the caller.
 */
#define GEMM_NOALLOC_SCRATCH_BYTES (64ll << 20)
int gemm_run_noalloc(gemm_handle_t h, const void *A, const void *B, const void *C, void *D,
                     int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                     int dtype, unsigned flags, int64_t batch, float alpha, float beta,
                     int c_type, int d_type, void *stream);

/* Release the handle's workspace (after synchronising its device) and the handle. */
int gemm_destroy(gemm_handle_t h);

/* Static, human-readable name of a status code. */
const char *gemm_status_string(int status);

/*
 * Describe, without launching anything, which kernel path gemm_run would take
 * for these arguments: writes a NUL-terminated label of at most label_len bytes
 * (e.g. "tile256x256 bf16 a:row b:col splitk=1 grid=256").  Validates
 * the same way gemm_run does, except that no data pointers are needed and
 * pointer alignment is assumed to be 16 bytes.  h may be NULL: the plan is then
 * made for a 256-CU gfx950 without any HIP call (host-only use).
 */
int gemm_plan(gemm_handle_t h, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
              int64_t ldc, int dtype, unsigned flags, int64_t batch, char *label,
              size_t label_len);

#ifdef __cplusplus
}
#endif

#endif /* DMP_GEMM_H */
