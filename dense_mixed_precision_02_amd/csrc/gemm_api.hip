// gemm_api.hip -- the C ABI declared in include/dmp_gemm.h: argument checks,
// kernel-path selection, workspace management and launches on the caller's
// stream.  Host code only; the kernels live in tile_gemm.hpp and aux_kernels.hpp.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>

#include "../../include/dmp_gemm.h"
#include "aux_kernels.hpp"
#include "dgemm.hpp"
#include "sparse_gemm.hpp"
#include "tile_gemm.hpp"
#include "tile16_gemm.hpp"
#include "tiny_gemm.hpp"
#include "plan.hpp"

using namespace dmp;
using namespace dmp::plan;

struct gemm_handle {
    int device = 0;
    int num_cus = 0;
    void *ws = nullptr;   // split-K partials or the transposed int8 B, grown on demand
    size_t ws_bytes = 0;
};

namespace {

template <int E, bool AK, bool BKC>
hipError_t launch_dgemm_t(const DgemmArgs &a, int64_t grid, hipStream_t s) {
    hipLaunchKernelGGL((dgemm_tile<E, E, AK, BKC>), dim3((unsigned)grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int E>
hipError_t launch_dgemm_layout(const DgemmArgs &a, bool a_col, bool b_col, int64_t grid,
                               hipStream_t s) {
    if (!a_col && b_col) return launch_dgemm_t<E, true, true>(a, grid, s);
    if (!a_col && !b_col) return launch_dgemm_t<E, true, false>(a, grid, s);
    if (a_col && b_col) return launch_dgemm_t<E, false, true>(a, grid, s);
    return launch_dgemm_t<E, false, false>(a, grid, s);
}

// fp64 launch for plan P (tile or element-wise kernel).
hipError_t launch_f64(const Plan &P, const void *A, const void *B, const void *C, void *D,
                      int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                      bool a_col, bool b_col, int64_t sA, int64_t sB, int64_t sC, int use_c,
                      hipStream_t s) {
    DgemmArgs a;
    a.A = (const double *)A; a.B = (const double *)B; a.C = (const double *)C; a.D = (double *)D;
    a.M = M; a.N = N; a.K = K; a.lda = lda; a.ldb = ldb; a.ldc = ldc;
    a.sA = sA; a.sB = sB; a.sC = sC;
    a.tiles_m = P.tiles_m; a.tiles_n = P.tiles_n;
    a.use_c = use_c;
    if (P.cfg == CFG_D128) return launch_dgemm_layout<128>(a, a_col, b_col, P.grid, s);
    if (P.cfg == CFG_D64) return launch_dgemm_layout<64>(a, a_col, b_col, P.grid, s);
    hipLaunchKernelGGL(dgemm_generic, dim3((unsigned)P.grid), dim3(64), 0, s, a, (int)a_col, (int)b_col);
    return hipGetLastError();
}

template <class DT, int BM, int BN, bool AK, bool BKC>
hipError_t launch_tile(const TileArgs &a, int64_t grid, hipStream_t s) {
    if constexpr (BM == 64 && BN == 64) {
        if (a.k_chunk <= 128 / DT::ESZ) {  // one k-tile per split
            hipLaunchKernelGGL((tile_gemm<DT, BM, BN, 2, 2, AK, BKC, true>), dim3((unsigned)grid),
                               dim3(256), 0, s, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((tile_gemm<DT, BM, BN, 2, 2, AK, BKC>), dim3((unsigned)grid), dim3(256), 0, s,
                       a);
    return hipGetLastError();
}

template <class DT, int E>
hipError_t launch_tile_layout(const TileArgs &a, bool a_col, bool b_col, int64_t grid,
                              hipStream_t s) {
    // AK: A is K-contiguous (row-major); BKC: B is K-contiguous (col-major)
    if (!a_col && b_col) return launch_tile<DT, E, E, true, true>(a, grid, s);
    if (!a_col && !b_col) return launch_tile<DT, E, E, true, false>(a, grid, s);
    if (a_col && b_col) return launch_tile<DT, E, E, false, true>(a, grid, s);
    return launch_tile<DT, E, E, false, false>(a, grid, s);
}

// 256x256 tiles: the 16x16-instruction kernel (tile16_gemm.hpp).
template <class DT>
hipError_t launch_tile16_layout(const TileArgs &a, bool a_col, bool b_col, int64_t grid,
                                hipStream_t s) {
    const dim3 g((unsigned)grid), blk(256);
    if (!a_col && b_col) hipLaunchKernelGGL((tile16_gemm<DT, true, true>), g, blk, 0, s, a);
    else if (!a_col && !b_col) hipLaunchKernelGGL((tile16_gemm<DT, true, false>), g, blk, 0, s, a);
    else if (a_col && b_col) hipLaunchKernelGGL((tile16_gemm<DT, false, true>), g, blk, 0, s, a);
    else hipLaunchKernelGGL((tile16_gemm<DT, false, false>), g, blk, 0, s, a);
    return hipGetLastError();
}

template <class DT>
hipError_t launch_cfg(int cfg, const TileArgs &a, bool a_col, bool b_col, int64_t grid,
                      hipStream_t s) {
    switch (cfg) {
    case CFG_L: return launch_tile16_layout<DT>(a, a_col, b_col, grid, s);
    case CFG_M: return launch_tile_layout<DT, 128>(a, a_col, b_col, grid, s);
    default: return launch_tile_layout<DT, 64>(a, a_col, b_col, grid, s);
    }
}

int64_t reduce_grid(int64_t items) {
    return std::max<int64_t>(1, std::min<int64_t>(cdiv(items, 256), 256 * 64));
}

template <class T>
hipError_t launch_reduce_t(const void *W, const void *C, void *D, int64_t M, int64_t N, int64_t ldc,
                           int64_t batch, int S, const EpiParams &ep, hipStream_t s) {
    const bool vec = N % 4 == 0 && ldc % 4 == 0 &&
                     (!ep.use_c || (uintptr_t)C % (4u * out_bytes(ep.c_type)) == 0) &&
                     (uintptr_t)D % (4u * out_bytes(ep.d_type)) == 0 && (S == 0 || aligned16(W));
    const int64_t elems = M * N * batch;
    if (vec)
        hipLaunchKernelGGL((splitk_reduce<T, true>), dim3((unsigned)reduce_grid(elems / 4)), dim3(256), 0,
                           s, (const T *)W, C, D, M, N, ldc, batch, S, ep);
    else
        hipLaunchKernelGGL((splitk_reduce<T, false>), dim3((unsigned)reduce_grid(elems)), dim3(256), 0, s,
                           (const T *)W, C, D, M, N, ldc, batch, S, ep);
    return hipGetLastError();
}

// Fixed-order sum of S split-K partials, then the output stage, into D (S == 0: no partials).
hipError_t launch_reduce(int dtype, const void *W, const void *C, void *D, int64_t M, int64_t N,
                         int64_t ldc, int64_t batch, int S, const EpiParams &ep, hipStream_t s) {
    if (dtype == GEMM_I8) return launch_reduce_t<int32_t>(W, C, D, M, N, ldc, batch, S, ep, s);
    if (dtype == GEMM_F64) return launch_reduce_t<double>(W, C, D, M, N, ldc, batch, S, ep, s);
    return launch_reduce_t<float>(W, C, D, M, N, ldc, batch, S, ep, s);
}

template <class DT, int S>
hipError_t launch_tiny_t(const TinyArgs &a, bool sa, bool sb, int64_t grid, hipStream_t s) {
    const dim3 g((unsigned)grid), blk(256);
    if (!sa && !sb) hipLaunchKernelGGL((tiny_gemm<DT, S, false, false>), g, blk, 0, s, a);
    else if (sa && !sb) hipLaunchKernelGGL((tiny_gemm<DT, S, true, false>), g, blk, 0, s, a);
    else if (!sa && sb) hipLaunchKernelGGL((tiny_gemm<DT, S, false, true>), g, blk, 0, s, a);
    else hipLaunchKernelGGL((tiny_gemm<DT, S, true, true>), g, blk, 0, s, a);
    return hipGetLastError();
}

template <class DT>
hipError_t launch_tiny_dt(int cfg, const TinyArgs &a, bool sa, bool sb, int64_t grid, hipStream_t s) {
    return cfg == CFG_TINY4 ? launch_tiny_t<DT, 4>(a, sa, sb, grid, s)
                            : launch_tiny_t<DT, 16>(a, sa, sb, grid, s);
}

// Tiny-product launch: four consecutive k of a K-contiguous operand row are
// loaded as one access when every row start is aligned to four elements.
hipError_t launch_tiny(const Plan &P, int dtype, const void *A, const void *B, const void *C,
                       void *D, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                       int64_t ldc, bool a_col, bool b_col, int64_t sA, int64_t sB, int64_t sC,
                       int64_t batch, const EpiParams &ep, bool sa, bool sb, hipStream_t s) {
    TinyArgs t;
    t.A = A; t.B = B; t.C = C; t.D = D;
    t.M = M; t.N = N; t.K = K; t.lda = lda; t.ldb = ldb; t.ldc = ldc;
    t.sA = sA; t.sB = sB; t.sC = sC; t.batch = batch;
    t.a_col = a_col; t.b_col = b_col;
    const uintptr_t es = (uintptr_t)elem_size(dtype);
    t.a_vec = !a_col && lda % 4 == 0 && sA % 4 == 0 && (uintptr_t)A % (4 * es) == 0;
    t.b_vec = b_col && ldb % 4 == 0 && sB % 4 == 0 && (uintptr_t)B % (4 * es) == 0;
    // LDS staging of a wave's operand region: 16-byte aligned starts, and the
    // region of NB problems (up to the last element of the last one) fits
    const int64_t nb = P.cfg == CFG_TINY4 ? 16 : 4;
    t.ext_a = a_col ? (K - 1) * lda + M : (M - 1) * lda + K;
    t.ext_b = b_col ? (N - 1) * ldb + K : (K - 1) * ldb + N;
    t.stage_a = !sa && (uintptr_t)A % 16 == 0 && (sA * (int64_t)es) % 16 == 0 &&
                ((nb - 1) * sA + t.ext_a) * (int64_t)es <= TINY_STAGE;
    t.stage_b = !sb && (uintptr_t)B % 16 == 0 && (sB * (int64_t)es) % 16 == 0 &&
                ((nb - 1) * sB + t.ext_b) * (int64_t)es <= TINY_STAGE;
    const int acc_ty = acc_type(dtype);
    t.flat_out = ldc == N && ep.d_type == acc_ty && (!ep.use_c || ep.c_type == acc_ty) &&
                 (uintptr_t)D % 16 == 0 && (!ep.use_c || (uintptr_t)C % 16 == 0) &&
                 (sC * 4) % 16 == 0 && nb * sC * 4 <= tiny_out_bytes(P.cfg == CFG_TINY4 ? 4 : 16);
    t.ep = ep;
    if (dtype == GEMM_F16) return launch_tiny_dt<F16>(P.cfg, t, sa, sb, P.grid, s);
    if (dtype == GEMM_BF16) return launch_tiny_dt<BF16>(P.cfg, t, sa, sb, P.grid, s);
    return launch_tiny_dt<I8>(P.cfg, t, sa, sb, P.grid, s);
}

// ---------------------------------------------------------------------------
// Fixed scratch for gemm_run_noalloc: one array per device that loads this
// library, held until the process ends.  Host code never uses the array's name
// as an address (on the host it is only a stand-in for the symbol); the device
// address of each device's copy is looked up once, with that device current,
// and kept in scratch_ptr.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[GEMM_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_lock;
void *scratch_ptr[MAX_DEVICES] = {};

// Device address of the current device's scratch (looked up on first use).
hipError_t scratch_for(int dev, void **out) {
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(scratch_lock);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return hipSuccess;
}

// gemm_run_ex and gemm_run_noalloc: the whole dense path.  ws_fixed == nullptr:
// the handle's workspace, grown on demand; otherwise ws_fixed (ws_cap bytes),
// and a plan that needs more fails with GEMM_ERR_SCRATCH before anything is
// enqueued.
int run_dense(gemm_handle_t h, const void *A, const void *B, const void *C, void *D, int64_t M,
              int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int dtype,
              unsigned flags, int64_t batch, const EpiParams &ep, void *stream, void *ws_fixed,
              size_t ws_cap) {
    int rc = validate(h, A, B, C, D, M, N, K, lda, ldb, ldc, dtype, flags, batch, true, ep);
    if (rc != GEMM_OK) return rc;
    if (M == 0 || N == 0 || batch == 0) return GEMM_OK;
    hipStream_t s = (hipStream_t)stream;
    const bool a_col = flags & GEMM_A_COLMAJOR, b_col = flags & GEMM_B_COLMAJOR;
    const bool a_sh = flags & GEMM_A_SHARED, b_sh = flags & GEMM_B_SHARED;
    // (A and B are not read when K == 0, and their leading dimensions unchecked)
    const int64_t sA = (a_sh || K == 0) ? 0 : (a_col ? K : M) * lda;
    const int64_t sB = (b_sh || K == 0) ? 0 : (b_col ? N : K) * ldb;
    const int64_t sC = M * ldc;
    const Plan P = make_plan(h->num_cus, A, B, M, N, K, lda, ldb, dtype, flags, batch, true);
    if (P.grid > 0x7fffffff) return GEMM_ERR_INVALID_ARG;  // beyond one launch's grid

    if (P.copy_only)
        return launch_reduce(dtype, nullptr, C, D, M, N, ldc, batch, 0, ep, s) == hipSuccess
                   ? GEMM_OK
                   : GEMM_ERR_HIP;

    if (P.cfg == CFG_TINY4 || P.cfg == CFG_TINY16)
        return launch_tiny(P, dtype, A, B, C, D, M, N, K, lda, ldb, ldc, a_col, b_col, sA, sB, sC,
                           batch, ep, a_sh, b_sh, s) == hipSuccess
                   ? GEMM_OK
                   : GEMM_ERR_HIP;

    if (dtype == GEMM_F64)
        return launch_f64(P, A, B, C, D, M, N, K, lda, ldb, ldc, a_col, b_col, sA, sB, sC,
                          ep.use_c, s) == hipSuccess
                   ? GEMM_OK
                   : GEMM_ERR_HIP;

    if (P.cfg == CFG_GENERIC) {
        GenericArgs g;
        g.A = A; g.B = B; g.C = C; g.D = D;
        g.M = M; g.N = N; g.K = K;
        g.a_rs = a_col ? 1 : lda;
        g.a_ks = a_col ? lda : 1;
        g.b_ks = b_col ? 1 : ldb;
        g.b_cs = b_col ? ldb : 1;
        g.ldc = ldc; g.sA = sA; g.sB = sB; g.sC = sC;
        g.tiles_m = P.tiles_m; g.tiles_n = P.tiles_n;
        g.ep = ep;
        const dim3 grid((unsigned)P.grid), blk(64);
        if (dtype == GEMM_F16) hipLaunchKernelGGL(generic_gemm<F16>, grid, blk, 0, s, g);
        else if (dtype == GEMM_BF16) hipLaunchKernelGGL(generic_gemm<BF16>, grid, blk, 0, s, g);
        else hipLaunchKernelGGL(generic_gemm<I8>, grid, blk, 0, s, g);
        return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
    }

    void *ws = ws_fixed;
    if (ws_fixed) {
        if (P.ws_needed > ws_cap) return GEMM_ERR_SCRATCH;
    } else if (P.ws_needed > h->ws_bytes) {
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess || cur != h->device) return GEMM_ERR_INVALID_ARG;
        if (h->ws) {
            // the old workspace may still be read by queued work on some stream
            if (hipDeviceSynchronize() != hipSuccess) return GEMM_ERR_HIP;
            if (hipFree(h->ws) != hipSuccess) return GEMM_ERR_HIP;
            h->ws = nullptr;
            h->ws_bytes = 0;
        }
        if (hipMalloc(&h->ws, P.ws_needed) != hipSuccess) {
            h->ws = nullptr;
            (void)hipGetLastError();
            return GEMM_ERR_ALLOC;
        }
        h->ws_bytes = P.ws_needed;
    }
    if (!ws_fixed) ws = h->ws;

    const void *Bk = B;
    int64_t ldbk = ldb, sBk = sB;
    bool b_colk = b_col;
    if (P.transpose_b) {
        const int tk = (int)cdiv(K, 128), tn = (int)cdiv(N, 128);
        const int64_t tgrid = (int64_t)tk * tn * batch;
        if (tgrid > 0x7fffffff) return GEMM_ERR_INVALID_ARG;
        const int vec_in = aligned16(B) && ldb % 16 == 0 && sB % 16 == 0;
        hipLaunchKernelGGL(transpose_i8, dim3((unsigned)tgrid), dim3(256), 0, s, (const int8_t *)B, K,
                           N, ldb, sB, (int8_t *)ws, P.ldt, N * P.ldt, tk, tn, vec_in);
        if (hipGetLastError() != hipSuccess) return GEMM_ERR_HIP;
        Bk = ws;
        ldbk = P.ldt;
        sBk = N * P.ldt;
        b_colk = true;
    }

    TileArgs t;
    t.A = A; t.B = Bk; t.C = C; t.D = D; t.W = ws;
    t.M = M; t.N = N; t.K = K; t.lda = lda; t.ldb = ldbk; t.ldc = ldc;
    t.sA = sA; t.sB = sBk; t.sC = sC;
    t.k_chunk = P.k_chunk;
    t.tiles_m = P.tiles_m; t.tiles_n = P.tiles_n;
    t.batch = (int)batch; t.splits = P.splits;
    t.partial = P.reduce ? 1 : 0;
    t.ep = ep;
    hipError_t e;
    if (dtype == GEMM_F16) e = launch_cfg<F16>(P.cfg, t, a_col, b_colk, P.grid, s);
    else if (dtype == GEMM_BF16) e = launch_cfg<BF16>(P.cfg, t, a_col, b_colk, P.grid, s);
    else e = launch_cfg<I8>(P.cfg, t, a_col, b_colk, P.grid, s);
    if (e != hipSuccess) return GEMM_ERR_HIP;
    if (P.reduce && launch_reduce(dtype, ws, C, D, M, N, ldc, batch, P.splits, ep, s) != hipSuccess)
        return GEMM_ERR_HIP;
    return GEMM_OK;
}

EpiParams make_epi(float alpha, float beta, int c_type, int d_type) {
    EpiParams ep;
    ep.alpha = alpha;
    ep.beta = beta;
    ep.c_type = c_type;
    ep.d_type = d_type;
    ep.use_c = beta != 0.0f;
    return ep;
}

}  // namespace

extern "C" {

const char *gemm_status_string(int status) {
    switch (status) {
    case GEMM_OK: return "GEMM_OK";
    case GEMM_ERR_INVALID_ARG: return "GEMM_ERR_INVALID_ARG";
    case GEMM_ERR_UNSUPPORTED_DEVICE: return "GEMM_ERR_UNSUPPORTED_DEVICE";
    case GEMM_ERR_ALLOC: return "GEMM_ERR_ALLOC";
    case GEMM_ERR_HIP: return "GEMM_ERR_HIP";
    case GEMM_ERR_SCRATCH: return "GEMM_ERR_SCRATCH";
    default: return "GEMM_ERR_UNKNOWN";
    }
}

int gemm_create(gemm_handle_t *out) {
    if (!out) return GEMM_ERR_INVALID_ARG;
    *out = nullptr;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GEMM_ERR_HIP;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GEMM_ERR_HIP;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return GEMM_ERR_UNSUPPORTED_DEVICE;
    gemm_handle *h = new (std::nothrow) gemm_handle;
    if (!h) return GEMM_ERR_ALLOC;
    h->device = dev;
    h->num_cus = prop.multiProcessorCount;
    // set-up of gemm_run_noalloc: this device's scratch address, once per device
    void *sp = nullptr;
    if (scratch_for(dev, &sp) != hipSuccess) {
        delete h;
        return GEMM_ERR_HIP;
    }
    *out = h;
    return GEMM_OK;
}

int gemm_destroy(gemm_handle_t h) {
    if (!h) return GEMM_ERR_INVALID_ARG;
    int rc = GEMM_OK;
    if (h->ws) {
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess) rc = GEMM_ERR_HIP;
        if (hipSetDevice(h->device) != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
            hipFree(h->ws) != hipSuccess)
            rc = GEMM_ERR_HIP;
        (void)hipSetDevice(cur);
    }
    delete h;
    return rc;
}

int gemm_plan(gemm_handle_t h, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
              int64_t ldc, int dtype, unsigned flags, int64_t batch, char *label, size_t label_len) {
    gemm_handle host_only;  // h == NULL: plan for a 256-CU device without touching HIP
    host_only.num_cus = 256;
    if (!h) h = &host_only;
    int rc = validate(h, nullptr, nullptr, nullptr, nullptr, M, N, K, lda, ldb, ldc, dtype, flags,
                      batch, false, plain_epi(dtype));
    if (rc != GEMM_OK) return rc;
    if (!label || label_len == 0) return GEMM_ERR_INVALID_ARG;
    if (M == 0 || N == 0 || batch == 0) {
        std::snprintf(label, label_len, "noop");
        return GEMM_OK;
    }
    const Plan P = make_plan(h->num_cus, nullptr, nullptr, M, N, K, lda, ldb, dtype, flags, batch, false);
    if (P.copy_only) {
        std::snprintf(label, label_len, "copy_c k=0");
        return GEMM_OK;
    }
    // the 64x64 tile with one k-tile per split runs its single-buffer variant
    const bool one = P.cfg == CFG_S && P.k_chunk <= 128 / elem_size(dtype);
    std::snprintf(label, label_len, "%s %s a:%s b:%s splitk=%d grid=%lld%s", cfg_name(P.cfg),
                  dtype_name(dtype), (flags & GEMM_A_COLMAJOR) ? "col" : "row",
                  P.transpose_b ? "row->col" : (flags & GEMM_B_COLMAJOR) ? "col" : "row", P.splits,
                  (long long)P.grid, one ? " one-ktile" : "");
    return GEMM_OK;
}

int gemm_run_ex(gemm_handle_t h, const void *A, const void *B, const void *C, void *D, int64_t M,
                int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int dtype,
                unsigned flags, int64_t batch, float alpha, float beta, int c_type, int d_type,
                void *stream) {
    return run_dense(h, A, B, C, D, M, N, K, lda, ldb, ldc, dtype, flags, batch,
                     make_epi(alpha, beta, c_type, d_type), stream, nullptr, 0);
}

int gemm_run_noalloc(gemm_handle_t h, const void *A, const void *B, const void *C, void *D,
                     int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                     int dtype, unsigned flags, int64_t batch, float alpha, float beta, int c_type,
                     int d_type, void *stream) {
    if (!h) return GEMM_ERR_INVALID_ARG;
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return GEMM_ERR_HIP;
    if (cur != h->device) return GEMM_ERR_INVALID_ARG;
    void *ws = nullptr;
    if (scratch_for(h->device, &ws) != hipSuccess) return GEMM_ERR_HIP;
    return run_dense(h, A, B, C, D, M, N, K, lda, ldb, ldc, dtype, flags, batch,
                     make_epi(alpha, beta, c_type, d_type), stream, ws,
                     (size_t)GEMM_NOALLOC_SCRATCH_BYTES);
}

int gemm_prune24(gemm_handle_t h, const void *A, int64_t M, int64_t K, int64_t lda, int dtype,
                 int64_t batch, void *Ac, void *meta, void *stream) {
    int rc = validate_sparse(h, M, 1, K, dtype, batch);
    if (rc != GEMM_OK) return rc;
    if (K > 0 && (lda < K || lda > (1ll << 48))) return GEMM_ERR_INVALID_ARG;
    if (M == 0 || batch == 0 || K == 0) return GEMM_OK;
    if (!extent_ok(batch, M, lda, K) ||
        !extent_ok(batch, sparse_mp(M), sparse_kp(K, dtype) / 2, sparse_kp(K, dtype) / 2))
        return GEMM_ERR_INVALID_ARG;
    const int esz = elem_size(dtype);
    if (!A || !Ac || !meta || (uintptr_t)A % esz || (uintptr_t)Ac % esz || (uintptr_t)meta % 2)
        return GEMM_ERR_INVALID_ARG;
    const int64_t kp = sparse_kp(K, dtype), mp = sparse_mp(M), nkt = kp / sparse_kt(dtype);
    const int64_t items = batch * mp * (kp / 16);
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(cdiv(items, 256), 256 * 64));
    hipStream_t s = (hipStream_t)stream;
    if (dtype == GEMM_F16)
        hipLaunchKernelGGL(prune24_kernel<F16>, dim3((unsigned)grid), dim3(256), 0, s, A, M, mp, K,
                           lda, M * lda, batch, Ac, meta, nkt);
    else if (dtype == GEMM_BF16)
        hipLaunchKernelGGL(prune24_kernel<BF16>, dim3((unsigned)grid), dim3(256), 0, s, A, M, mp, K,
                           lda, M * lda, batch, Ac, meta, nkt);
    else
        hipLaunchKernelGGL(prune24_kernel<I8>, dim3((unsigned)grid), dim3(256), 0, s, A, M, mp, K,
                           lda, M * lda, batch, Ac, meta, nkt);
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

int gemm_run_sparse24(gemm_handle_t h, const void *Ac, const void *meta, const void *B,
                      const void *C, void *D, int64_t M, int64_t N, int64_t K, int64_t ldb,
                      int64_t ldc, int dtype, unsigned flags, int64_t batch, void *stream) {
    int rc = validate_sparse(h, M, N, K, dtype, batch);
    if (rc != GEMM_OK) return rc;
    if (flags & ~(unsigned)GEMM_B_COLMAJOR) return GEMM_ERR_INVALID_ARG;
    const bool b_col = flags & GEMM_B_COLMAJOR;
    if (K > 0 && (ldb < std::max<int64_t>(1, b_col ? K : N) || ldb > (1ll << 48)))
        return GEMM_ERR_INVALID_ARG;
    if (ldc < std::max<int64_t>(1, N) || ldc > (1ll << 48)) return GEMM_ERR_INVALID_ARG;
    if (M == 0 || N == 0 || batch == 0) return GEMM_OK;
    if (!extent_ok(batch, M, ldc, N)) return GEMM_ERR_INVALID_ARG;
    if (K > 0 && (!extent_ok(batch, b_col ? N : K, ldb, b_col ? K : N) ||
                  !extent_ok(batch, sparse_mp(M), sparse_kp(K, dtype) / 2, sparse_kp(K, dtype) / 2)))
        return GEMM_ERR_INVALID_ARG;
    if (!C || !D || (uintptr_t)C % 4 || (uintptr_t)D % 4) return GEMM_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    const EpiParams ep = plain_epi(dtype);
    if (K == 0)
        return launch_reduce(dtype, nullptr, C, D, M, N, ldc, batch, 0, ep, s) == hipSuccess
                   ? GEMM_OK
                   : GEMM_ERR_HIP;
    // the operands go straight to LDS in 16-byte granules: aligned starts, whole
    // granules along the contiguous extent of B, offsets within 31 bits
    const int esz = elem_size(dtype), gran = 16 / esz;
    const int64_t kt = sparse_kt(dtype);
    if (!Ac || !meta || !B || !aligned16(Ac) || !aligned16(meta) || !aligned16(B) || ldb % gran ||
        (b_col ? K % gran : N % gran) ||
        (b_col ? 256 * ldb : kt * ldb) * esz >= (1ll << 31) - (1ll << 22))
        return GEMM_ERR_INVALID_ARG;
    const int64_t kp = sparse_kp(K, dtype), mp = sparse_mp(M);
    SparseArgs a;
    a.Ac = Ac; a.meta = meta; a.B = B; a.C = C; a.D = D;
    a.M = M; a.N = N; a.K = K; a.ldb = ldb; a.ldc = ldc;
    a.sAc = mp * (kp / 2); a.sM = mp * (kp / 16); a.sB = (b_col ? N : K) * ldb; a.sC = M * ldc;
    a.tiles_m = (int)cdiv(M, 256); a.tiles_n = (int)cdiv(N, 256); a.batch = (int)batch;
    a.nkt = (int)(kp / kt);
    a.ep = ep;
    const int64_t grid = (int64_t)a.tiles_m * a.tiles_n * batch;
    if (grid > 0x7fffffff) return GEMM_ERR_INVALID_ARG;
    const dim3 g((unsigned)grid), blk(256);
    if (dtype == GEMM_F16) {
        if (b_col) hipLaunchKernelGGL((sparse_gemm<F16, true>), g, blk, 0, s, a);
        else hipLaunchKernelGGL((sparse_gemm<F16, false>), g, blk, 0, s, a);
    } else if (dtype == GEMM_BF16) {
        if (b_col) hipLaunchKernelGGL((sparse_gemm<BF16, true>), g, blk, 0, s, a);
        else hipLaunchKernelGGL((sparse_gemm<BF16, false>), g, blk, 0, s, a);
    } else {
        if (b_col) hipLaunchKernelGGL((sparse_gemm<I8, true>), g, blk, 0, s, a);
        else hipLaunchKernelGGL((sparse_gemm<I8, false>), g, blk, 0, s, a);
    }
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

int gemm_run(gemm_handle_t h, const void *A, const void *B, const void *C, void *D, int64_t M,
             int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int dtype,
             unsigned flags, int64_t batch, void *stream) {
    const int t = acc_type(dtype);
    return gemm_run_ex(h, A, B, C, D, M, N, K, lda, ldb, ldc, dtype, flags, batch, 1.0f, 1.0f, t, t,
                       stream);
}

}  // extern "C"
