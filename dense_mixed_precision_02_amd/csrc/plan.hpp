// plan.hpp -- host-side argument checks and kernel-path selection of the C ABI
// (plain C++: no HIP types, so that it can also be built and checked on its
// own, e.g. under the address and undefined-behaviour sanitizers).
#pragma once
#include <stdint.h>

#include <algorithm>

#include "../../include/dmp_gemm.h"
#include "epi.hpp"

namespace dmp {
namespace plan {

// Workgroup tile shapes of the tiled kernel (4 waves each, 2 x 2); the fp64
// kernels have their own.
enum Cfg { CFG_L = 0, CFG_M = 1, CFG_S = 2, CFG_GENERIC = 3, CFG_D128 = 4, CFG_D64 = 5,
           CFG_DGENERIC = 6, CFG_TINY4 = 7, CFG_TINY16 = 8 };
constexpr unsigned ALL_FLAGS = GEMM_A_COLMAJOR | GEMM_B_COLMAJOR | GEMM_A_SHARED | GEMM_B_SHARED;
constexpr int CFG_EDGE[3] = {256, 128, 64};

struct Plan {
    int cfg = CFG_GENERIC;
    int splits = 1;
    int64_t k_chunk = 0;
    int tiles_m = 0, tiles_n = 0;
    int64_t grid = 0;
    bool reduce = false;     // second launch: fixed-order sum of partials + C
    bool copy_only = false;  // K == 0: D = C
    bool transpose_b = false;  // int8 row-major B copied column-major into the workspace first
    int64_t ldt = 0;           // its leading dimension
    size_t ws_needed = 0;
};

inline int elem_size(int dtype) { return dtype == GEMM_I8 ? 1 : dtype == GEMM_F64 ? 8 : 2; }
inline int out_bytes(int t) {
    return (t == GEMM_OUT_F16 || t == GEMM_OUT_BF16) ? 2 : t == GEMM_OUT_F64 ? 8 : 4;
}
inline int acc_type(int dtype) {
    return dtype == GEMM_I8 ? GEMM_OUT_I32 : dtype == GEMM_F64 ? GEMM_OUT_F64 : GEMM_OUT_F32;
}

// The plain output stage of gemm_run: D = acc + C in the accumulator type.
inline EpiParams plain_epi(int dtype) {
    EpiParams e;
    e.alpha = 1.0f;
    e.beta = 1.0f;
    e.c_type = e.d_type = acc_type(dtype);
    e.use_c = 1;
    return e;
}

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Largest element index (plus one) of `batch` contiguous blocks of `rows` rows
// `ld` apart (`cols` used per row), computed in 128 bits.  Every operand is
// required to stay within 2^48 elements, far above any device's memory, so
// that all index arithmetic on the host and in the kernels fits 64 bits.
inline bool extent_ok(int64_t batch, int64_t rows, int64_t ld, int64_t cols) {
    const __int128 stride = (__int128)rows * ld;
    const __int128 e = (__int128)(batch - 1) * stride + (__int128)(rows - 1) * ld + cols;
    return e <= ((__int128)1 << 48);
}

inline int validate(gemm_handle_t h, const void *A, const void *B, const void *C, const void *D,
             int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int dtype,
             unsigned flags, int64_t batch, bool check_ptrs, const EpiParams &ep) {
    if (!h) return GEMM_ERR_INVALID_ARG;
    if (dtype != GEMM_F16 && dtype != GEMM_BF16 && dtype != GEMM_I8 && dtype != GEMM_F64)
        return GEMM_ERR_INVALID_ARG;
    if (flags & ~ALL_FLAGS) return GEMM_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K < 0 || batch < 0) return GEMM_ERR_INVALID_ARG;
    // output stage: fp16/bf16 inputs take fp32/fp16/bf16 C and D and any alpha,
    // beta; int8 and fp64 inputs keep C and D in their accumulator type, with
    // alpha = 1 and beta in {0, 1}
    if (dtype == GEMM_I8 || dtype == GEMM_F64) {
        const int t = acc_type(dtype);
        if (ep.c_type != t || ep.d_type != t || ep.alpha != 1.0f ||
            (ep.beta != 0.0f && ep.beta != 1.0f))
            return GEMM_ERR_INVALID_ARG;
    } else {
        const auto float_type = [](int t) {
            return t == GEMM_OUT_F32 || t == GEMM_OUT_F16 || t == GEMM_OUT_BF16;
        };
        if (!float_type(ep.c_type) || !float_type(ep.d_type)) return GEMM_ERR_INVALID_ARG;
    }
    const bool a_col = flags & GEMM_A_COLMAJOR, b_col = flags & GEMM_B_COLMAJOR;
    // A and B are not read when K == 0, so their leading dimensions are free then
    if (K > 0 && lda < std::max<int64_t>(1, a_col ? M : K)) return GEMM_ERR_INVALID_ARG;
    if (K > 0 && ldb < std::max<int64_t>(1, b_col ? K : N)) return GEMM_ERR_INVALID_ARG;
    if (ldc < std::max<int64_t>(1, N)) return GEMM_ERR_INVALID_ARG;
    // grid dimensions and element indices are kept well inside their integer types
    if (M > (1ll << 31) - 1024 || N > (1ll << 31) - 1024 || K > (1ll << 31) - 1024 ||
        batch > (1ll << 30))
        return GEMM_ERR_INVALID_ARG;
    // leading dimensions themselves (a one-row operand's ld enters no extent)
    const int64_t ld_max = 1ll << 48;
    if ((K > 0 && (lda > ld_max || ldb > ld_max)) || ldc > ld_max) return GEMM_ERR_INVALID_ARG;
    if (M == 0 || N == 0 || batch == 0) return GEMM_OK;
    const bool a_sh = flags & GEMM_A_SHARED, b_sh = flags & GEMM_B_SHARED;
    const int64_t ar = a_col ? K : M, ac = a_col ? M : K, br = b_col ? N : K, bc = b_col ? K : N;
    if (K > 0 && (!extent_ok(a_sh ? 1 : batch, ar, lda, ac) ||
                  !extent_ok(b_sh ? 1 : batch, br, ldb, bc)))
        return GEMM_ERR_INVALID_ARG;
    if (!extent_ok(batch, M, ldc, N)) return GEMM_ERR_INVALID_ARG;
    if (!check_ptrs) return GEMM_OK;
    if (!D || (ep.use_c && !C)) return GEMM_ERR_INVALID_ARG;
    if (K > 0 && (!A || !B)) return GEMM_ERR_INVALID_ARG;
    if (C == D && ep.use_c && ep.c_type != ep.d_type) return GEMM_ERR_INVALID_ARG;
    const uintptr_t es = (uintptr_t)elem_size(dtype);
    if (((uintptr_t)A % es) || ((uintptr_t)B % es) ||
        (ep.use_c && ((uintptr_t)C % (uintptr_t)out_bytes(ep.c_type))) ||
        ((uintptr_t)D % (uintptr_t)out_bytes(ep.d_type)))
        return GEMM_ERR_INVALID_ARG;
    return GEMM_OK;
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Can the 16-byte granule path handle these operands?  Every granule must be
// 16-byte aligned and wholly inside or wholly outside the matrix, and per-lane
// byte offsets must fit 31 bits.
inline bool granule_ok(const void *A, const void *B, int64_t M, int64_t N, int64_t K, int64_t lda,
                int64_t ldb, int dtype, bool a_col, bool b_col, bool check_ptrs) {
    const int es = elem_size(dtype);
    const int G = 16 / es;
    if (check_ptrs && (!aligned16(A) || !aligned16(B))) return false;
    if ((lda * es) % 16 || (ldb * es) % 16) return false;
    const bool a_k = !a_col, b_k = b_col;
    // the contiguous extent of each operand is a whole number of granules, so no
    // granule reaches past the last element of a row or column
    if ((a_k || b_k) && K % G) return false;
    if ((!a_k && M % G) || (!b_k && N % G)) return false;
    const int64_t kt = 128 / es;
    const int64_t lim = (1ll << 31) - (1ll << 22);
    // offsets inside one k-tile: up to 256 rows (K-contig) or kt k-rows (MN-contig)
    const int64_t span_a = (a_k ? 256 * lda : kt * lda) * es;
    const int64_t span_b = (b_k ? 256 * ldb : kt * ldb) * es;
    return span_a < lim && span_b < lim;
}

// fp64: 128 x 128 tiles when they fill the device, else 64 x 64; the
// element-wise kernel when the 16-byte granule path cannot take the operands.
inline Plan make_plan_f64(int num_cus, const void *A, const void *B, int64_t M, int64_t N,
                   int64_t K, int64_t lda, int64_t ldb, bool a_col, bool b_col, int64_t batch,
                   bool check_ptrs) {
    Plan P;
    if (!granule_ok(A, B, M, N, K, lda, ldb, GEMM_F64, a_col, b_col, check_ptrs)) {
        P.cfg = CFG_DGENERIC;
        P.tiles_m = (int)cdiv(M, 16);
        P.tiles_n = (int)cdiv(N, 16);
        P.grid = (int64_t)P.tiles_m * P.tiles_n * batch;
        return P;
    }
    const int64_t cus = num_cus > 0 ? num_cus : 256;
    const int64_t t128 = cdiv(M, 128) * cdiv(N, 128) * batch;
    const double useful128 = (double)M * (double)N / ((double)cdiv(M, 128) * 128.0 *
                                                      (double)cdiv(N, 128) * 128.0);
    const int e = (t128 >= cus && useful128 >= 0.75) ? 128 : 64;
    P.cfg = e == 128 ? CFG_D128 : CFG_D64;
    P.tiles_m = (int)cdiv(M, e);
    P.tiles_n = (int)cdiv(N, e);
    P.grid = (int64_t)P.tiles_m * P.tiles_n * batch;
    return P;
}

inline Plan make_plan(int num_cus, const void *A, const void *B, int64_t M, int64_t N, int64_t K,
               int64_t lda, int64_t ldb, int dtype, unsigned flags, int64_t batch, bool check_ptrs) {
    Plan P;
    const bool a_col = flags & GEMM_A_COLMAJOR, b_col = flags & GEMM_B_COLMAJOR;
    if (K == 0) {
        P.copy_only = true;
        return P;
    }
    if (dtype == GEMM_F64) return make_plan_f64(num_cus, A, B, M, N, K, lda, ldb, a_col, b_col, batch, check_ptrs);
    if (M <= 16 && N <= 16) {
        // tiny products: several problems per multi-block instruction
        const int nb = (M <= 4 && N <= 4) ? 16 : 4;
        P.cfg = nb == 16 ? CFG_TINY4 : CFG_TINY16;
        P.tiles_m = P.tiles_n = 1;
        P.grid = cdiv(batch, 4 * nb);
        return P;
    }
    const int es = elem_size(dtype);
    const int64_t kt = 128 / es;
    // int8 row-major B with a large M: a transposed copy (one pass over B into the
    // workspace) lets the K loop use plain instead of transposing LDS reads; the
    // copy is column-major with a 16-byte multiple leading dimension, so only A's
    // granule conditions and K % 16 remain
    const bool tb = dtype == GEMM_I8 && !b_col && (flags & GEMM_B_SHARED) == 0 && M >= 4096 &&
                    K % 16 == 0;
    const int64_t ldt = cdiv(K, 16) * 16;
    if (tb ? !granule_ok(A, A, M, N, K, lda, ldt, dtype, a_col, true, check_ptrs)
           : !granule_ok(A, B, M, N, K, lda, ldb, dtype, a_col, b_col, check_ptrs)) {
        P.cfg = CFG_GENERIC;
        P.tiles_m = (int)cdiv(M, 32);
        P.tiles_n = (int)cdiv(N, 32);
        P.grid = (int64_t)P.tiles_m * P.tiles_n * batch;
        return P;
    }
    const int64_t cus = num_cus > 0 ? num_cus : 256;
    auto tiles = [&](int cfg) {
        return cdiv(M, CFG_EDGE[cfg]) * cdiv(N, CFG_EDGE[cfg]) * batch;
    };
    // Fraction of a config's tile area that is inside the matrix.
    auto useful = [&](int cfg) {
        const double e = CFG_EDGE[cfg];
        return (double)M * (double)N / ((double)cdiv(M, CFG_EDGE[cfg]) * e *
                                        (double)cdiv(N, CFG_EDGE[cfg]) * e);
    };
    const int64_t nkt = cdiv(K, kt);
    // Largest tile that wastes at most a quarter of its area to the edges.
    int cfg = CFG_S;
    for (int c = CFG_L; c <= CFG_S; ++c)
        if (useful(c) >= 0.75) {
            cfg = c;
            break;
        }
    int64_t splits = 1;
    if (tiles(cfg) < cus) {
        // Under one workgroup per CU.  A long K is split (each split keeps at
        // least 8 k-tiles) so the large tile's low traffic per flop is kept;
        // a short K instead moves to smaller tiles.
        const int64_t s = std::min(cus / tiles(cfg), nkt / 8);
        if (s >= 2 && !tb) {
            splits = s;
        } else {
            while (cfg < CFG_S && tiles(cfg) < cus && useful(cfg + 1) >= 0.75) ++cfg;
        }
    }
    const int e = CFG_EDGE[cfg];
    P.cfg = cfg;
    P.tiles_m = (int)cdiv(M, e);
    P.tiles_n = (int)cdiv(N, e);
    P.k_chunk = cdiv(nkt, splits) * kt;
    P.splits = (int)cdiv(K, P.k_chunk);  // no empty splits
    P.grid = (int64_t)P.tiles_m * P.tiles_n * batch * P.splits;
    if (P.splits > 1) {
        P.reduce = true;
        P.ws_needed = (size_t)P.splits * (size_t)batch * (size_t)M * (size_t)N * 4u;
    } else if (tb) {
        P.transpose_b = true;
        P.ldt = ldt;
        P.ws_needed = (size_t)batch * (size_t)N * (size_t)P.ldt;
    }
    return P;
}

inline const char *cfg_name(int cfg) {
    switch (cfg) {
    case CFG_L: return "tile256x256";
    case CFG_M: return "tile128x128";
    case CFG_S: return "tile64x64";
    case CFG_D128: return "dtile128x128";
    case CFG_D64: return "dtile64x64";
    case CFG_DGENERIC: return "dgeneric16x16";
    case CFG_TINY4: return "tiny4x4x16b";
    case CFG_TINY16: return "tiny16x16x4b";
    default: return "generic32x32";
    }
}

inline const char *dtype_name(int d) {
    return d == GEMM_F16 ? "f16" : d == GEMM_BF16 ? "bf16" : d == GEMM_F64 ? "f64" : "i8";
}

// Compressed-A geometry: Kp dense k per row (a whole number of the sparse
// kernel's k-tiles: 64 for fp16/bf16, 128 for int8), Kp/2 values and Kp/16
// 16-bit index words per row, Mp = 16 * ceil(M / 16) rows (16-row blocks).
inline int64_t sparse_kt(int dtype) { return dtype == GEMM_I8 ? 128 : 64; }
inline int64_t sparse_kp(int64_t K, int dtype) { return cdiv(K, sparse_kt(dtype)) * sparse_kt(dtype); }
inline int64_t sparse_mp(int64_t M) { return cdiv(M, 16) * 16; }

inline int validate_sparse(gemm_handle_t h, int64_t M, int64_t N, int64_t K, int dtype, int64_t batch) {
    if (!h) return GEMM_ERR_INVALID_ARG;
    if (dtype != GEMM_F16 && dtype != GEMM_BF16 && dtype != GEMM_I8) return GEMM_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K < 0 || batch < 0) return GEMM_ERR_INVALID_ARG;
    if (M > (1ll << 31) - 1024 || N > (1ll << 31) - 1024 || K > (1ll << 31) - 1024 ||
        batch > (1ll << 30))
        return GEMM_ERR_INVALID_ARG;
    // byte offsets inside one 256-row panel of the compressed operand fit 31 bits
    if (256 * (sparse_kp(K, dtype) / 2) * elem_size(dtype) >= (1ll << 31) - (1ll << 22))
        return GEMM_ERR_INVALID_ARG;
    return GEMM_OK;
}

}  // namespace plan
}  // namespace dmp
