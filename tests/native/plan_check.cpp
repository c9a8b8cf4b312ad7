// Host-side check of the C ABI's argument validation and kernel-path
// selection (csrc/plan.hpp), built with the address and undefined-behaviour
// sanitizers by tests/test_sanitizers.py.  Sweeps ordinary and extreme
// arguments and checks the invariants every accepted plan must satisfy; any
// overflow or out-of-range access in the checks themselves is reported by the
// sanitizers.  Exit status 0: all checks held.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../dense_mixed_precision_02_amd/csrc/plan.hpp"

using namespace dmp;
using namespace dmp::plan;

static int failures = 0;
#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            std::fprintf(stderr, "FAILED %s: ", #cond);    \
            std::fprintf(stderr, __VA_ARGS__);             \
            std::fprintf(stderr, "\n");                    \
            ++failures;                                    \
        }                                                  \
    } while (0)

// A fake handle: validate() only tests it against NULL.
static gemm_handle_t fake_handle() { return reinterpret_cast<gemm_handle_t>(0x1000); }

static void check_plan(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                       int dtype, unsigned flags, int64_t batch) {
    const EpiParams ep = plain_epi(dtype);
    const int rc = validate(fake_handle(), nullptr, nullptr, nullptr, nullptr, M, N, K, lda, ldb,
                            ldc, dtype, flags, batch, false, ep);
    if (rc != GEMM_OK || M == 0 || N == 0 || batch == 0) return;
    for (int cus : {0, 80, 256, 304}) {
        const Plan P = make_plan(cus, nullptr, nullptr, M, N, K, lda, ldb, dtype, flags, batch, false);
        if (K == 0) {
            CHECK(P.copy_only, "K=0 must copy C (M=%lld N=%lld)", (long long)M, (long long)N);
            continue;
        }
        CHECK(P.grid >= 1, "empty grid M=%lld N=%lld K=%lld", (long long)M, (long long)N,
              (long long)K);
        CHECK(P.splits >= 1, "splits %d", P.splits);
        if (P.cfg <= CFG_S) {
            const int64_t e = CFG_EDGE[P.cfg];
            CHECK(P.tiles_m == cdiv(M, e) && P.tiles_n == cdiv(N, e), "tile counts");
            CHECK(P.grid == (int64_t)P.tiles_m * P.tiles_n * batch * P.splits, "grid");
            const int64_t kt = 128 / elem_size(dtype);
            CHECK(P.k_chunk % kt == 0 && P.k_chunk > 0, "k_chunk %lld", (long long)P.k_chunk);
            CHECK((P.splits - 1) * P.k_chunk < K && K <= P.splits * P.k_chunk,
                  "splits %d x %lld do not cover K=%lld exactly", P.splits, (long long)P.k_chunk,
                  (long long)K);
            if (P.splits > 1)
                CHECK(P.reduce && P.ws_needed == (size_t)P.splits * batch * M * N * 4, "workspace");
            if (P.transpose_b) {
                CHECK(dtype == GEMM_I8 && !(flags & GEMM_B_COLMAJOR) && K % 16 == 0, "transpose");
                CHECK(P.ws_needed == (size_t)batch * N * P.ldt && P.ldt >= K, "transpose ws");
            }
        } else if (P.cfg == CFG_GENERIC || P.cfg == CFG_DGENERIC) {
            const int64_t e = P.cfg == CFG_GENERIC ? 32 : 16;
            CHECK(P.grid == cdiv(M, e) * cdiv(N, e) * batch, "generic grid");
        } else if (P.cfg == CFG_TINY4 || P.cfg == CFG_TINY16) {
            CHECK(M <= 16 && N <= 16 && dtype != GEMM_F64, "tiny shape");
        }
        CHECK(cfg_name(P.cfg) != nullptr, "name");
    }
}

int main() {
    const std::vector<int64_t> dims = {1, 3, 4, 15, 16, 17, 31, 64, 65, 127, 128, 255, 256, 300,
                                       1000, 1024, 4096, 8192, 65536, (1ll << 31) - 1024};
    const int dtypes[] = {GEMM_F16, GEMM_BF16, GEMM_I8, GEMM_F64};
    int64_t n = 0;
    for (int dt : dtypes)
        for (unsigned flags = 0; flags < 16; ++flags)
            for (int64_t M : {1ll, 16ll, 300ll, 4096ll, 8192ll})
                for (int64_t N : {1ll, 16ll, 96ll, 1024ll, 4096ll})
                    for (int64_t K : dims)
                        for (int64_t batch : {1ll, 3ll, 8192ll}) {
                            const bool a_col = flags & GEMM_A_COLMAJOR, b_col = flags & GEMM_B_COLMAJOR;
                            for (int64_t pad : {0ll, 1ll, 8ll}) {
                                const int64_t lda = (a_col ? M : K) + pad;
                                const int64_t ldb = (b_col ? K : N) + pad;
                                check_plan(M, N, K, lda, ldb, N + pad, dt, flags, batch);
                                ++n;
                            }
                        }
    // extremes: huge dimensions, leading dimensions and batches must be rejected
    // (or planned) without overflow anywhere
    const int64_t big[] = {0, 1, (1ll << 31) - 1024, (1ll << 31), (1ll << 40), (1ll << 48),
                           (1ll << 62), INT64_MAX};
    for (int64_t M : big)
        for (int64_t N : big)
            for (int64_t K : big)
                for (int64_t ld : big)
                    for (int64_t batch : {0ll, 1ll, (1ll << 20), (1ll << 30), (1ll << 31)}) {
                        check_plan(M, N, K, ld, ld, ld, GEMM_BF16, 0, batch);
                        check_plan(M, N, K, ld, ld, ld, GEMM_I8, GEMM_A_SHARED | GEMM_B_COLMAJOR, batch);
                        check_plan(M, N, K, ld, ld, ld, GEMM_F64, GEMM_A_COLMAJOR, batch);
                        (void)validate_sparse(fake_handle(), M, N, K, GEMM_I8, batch);
                        ++n;
                    }
    // an operand of exactly 2^48 elements is accepted, one more element is not
    CHECK(validate(fake_handle(), nullptr, nullptr, nullptr, nullptr, 1ll << 24, 1ll << 24, 16,
                   16, 1ll << 24, 1ll << 24, GEMM_F16, 0, 1, false, plain_epi(GEMM_F16)) == GEMM_OK,
          "2^48 elements");
    CHECK(validate(fake_handle(), nullptr, nullptr, nullptr, nullptr, 1ll << 24, 1ll << 24, 16,
                   16, 1ll << 24, (1ll << 24) + 1, GEMM_F16, 0, 1, false,
                   plain_epi(GEMM_F16)) == GEMM_ERR_INVALID_ARG,
          "2^48 + 2^24 - 1 elements");
    std::printf("plan_check: %lld argument sets, %d failures\n", (long long)n, failures);
    return failures ? 1 : 0;
}
