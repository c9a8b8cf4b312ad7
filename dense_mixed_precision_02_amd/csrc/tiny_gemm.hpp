// tiny_gemm.hpp -- batches of tiny products (M, N <= 16) on the multi-block
// matrix instructions, which compute several independent products at once
// (pages: "CDNA2 dense MFMA builtins", section "Accumulator layout", the 4x4
// (16 blocks) and 16x16 (4 blocks) shapes, and "MFMA common parameters" for
// cbsz / abid / blgp).
//
// Maps, as on the pages and checked on gfx950 with a one-hot probe (S = 4 or
// 16, NB = 64/S blocks; each block is one problem of the batch):
//   A input:  lane L holds row L%S of block L/S, 4 consecutive k in one register
//   B input:  lane L holds column L%S of block L/S, the same 4 k
//   output S=4:  element (i, j) of block b in lane 4b + j, register i
//   output S=16: element (i, j) of block b in lane 16*(i/4) + j, register 4b + i%4
// Shared operands (batch stride 0) are loaded once per wave and spread by the
// instruction itself: A from block 0 to every block with cbsz = log2(NB),
// abid = 0; B from lanes 0-15 to the other three lane groups with blgp = 4.
#pragma once

#include "common.hpp"

namespace dmp {

typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

struct TinyArgs {
    const void *A, *B, *C;
    void *D;
    int64_t M, N, K, lda, ldb, ldc;
    int64_t sA, sB, sC;  // batch strides in elements (0 for a shared operand)
    int64_t batch;
    int a_col, b_col;
    int a_vec, b_vec;    // 4 k of a row (column) of A (B) are contiguous and aligned
    int64_t ext_a, ext_b;  // elements from the start of one problem's A (B) to its last element + 1
    int stage_a, stage_b;  // the wave's A (B) region is copied to LDS with 16-byte accesses
    int flat_out;          // dense fp32/int32 C and D: the output moves as 16-byte vectors
    EpiParams ep;
};

// LDS bytes per wave: one operand region each for A and B, and the output region,
// sized for the dense outputs of the wave's problems (16 of at most 4x4 with the
// 4x4 blocks, 4 of at most 16x16 with the 16x16 ones).
constexpr int TINY_STAGE = 2048;
constexpr int tiny_out_bytes(int S) { return S == 4 ? 16 * 4 * 4 * 4 : 4 * 16 * 16 * 4; }

// Instruction for S x S blocks of element type DT (4 k per instruction).
template <class DT, int S> struct Multi;
template <> struct Multi<F16, 4> {
    using acc = floatx4;
    template <int CB, int AB, int BG>
    __device__ static acc mma(uint64_t a, uint64_t b, acc c) {
        return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(half4, a), __builtin_bit_cast(half4, b),
                                                  c, CB, AB, BG);
    }
};
template <> struct Multi<F16, 16> {
    using acc = floatx16;
    template <int CB, int AB, int BG>
    __device__ static acc mma(uint64_t a, uint64_t b, acc c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f16(__builtin_bit_cast(half4, a), __builtin_bit_cast(half4, b),
                                                    c, CB, AB, BG);
    }
};
template <> struct Multi<BF16, 4> {
    using acc = floatx4;
    template <int CB, int AB, int BG>
    __device__ static acc mma(uint64_t a, uint64_t b, acc c) {
        return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(bf16x4, a),
                                                      __builtin_bit_cast(bf16x4, b), c, CB, AB, BG);
    }
};
template <> struct Multi<BF16, 16> {
    using acc = floatx16;
    template <int CB, int AB, int BG>
    __device__ static acc mma(uint64_t a, uint64_t b, acc c) {
        return __builtin_amdgcn_mfma_f32_16x16x4bf16_1k(__builtin_bit_cast(bf16x4, a),
                                                        __builtin_bit_cast(bf16x4, b), c, CB, AB, BG);
    }
};
template <> struct Multi<I8, 4> {
    using acc = intx4;
    template <int CB, int AB, int BG>
    __device__ static acc mma(uint64_t a, uint64_t b, acc c) {
        return __builtin_amdgcn_mfma_i32_4x4x4i8((int)(uint32_t)a, (int)(uint32_t)b, c, CB, AB, BG);
    }
};
template <> struct Multi<I8, 16> {
    using acc = intx16;
    template <int CB, int AB, int BG>
    __device__ static acc mma(uint64_t a, uint64_t b, acc c) {
        return __builtin_amdgcn_mfma_i32_16x16x4i8((int)(uint32_t)a, (int)(uint32_t)b, c, CB, AB, BG);
    }
};

// Element of type T at byte pointer q, in global memory or in LDS.
template <class T>
__device__ static inline T ld_as(const char *q) { return *(const T *)q; }
template <class T>
__device__ static inline T ld_as(const DMP_LDS char *q) { return *(const DMP_LDS T *)q; }

// Four consecutive k (k0 .. k0+3) of one row of a K-contiguous operand or one
// column of an MN-contiguous one, packed little-endian into 4*ESZ bytes; out of
// range elements (rc >= rows, k >= K) read as zero.  stride_k: element step
// along k; vec: the four are contiguous, aligned and all inside K.
template <int ESZ, class P>
__device__ static inline uint64_t load_k4(P base, int64_t stride_k, int64_t k0, int64_t K,
                                          bool row_ok, bool vec) {
    if (!row_ok) return 0;
    if (vec && k0 + 3 < K) {
        if constexpr (ESZ == 2) return ld_as<uint64_t>(base + k0 * ESZ);
        else return ld_as<uint32_t>(base + k0 * ESZ);
    }
    uint64_t r = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t k = k0 + e;
        if (k < K) {
            const auto q = base + k * stride_k * ESZ;
            const uint64_t v = ESZ == 2 ? (uint64_t)ld_as<uint16_t>(q) : (uint64_t)ld_as<uint8_t>(q);
            r |= v << (8 * ESZ * e);
        }
    }
    return r;
}

// Copy of nbytes (at most TINY_STAGE) from global memory into LDS, in two
// halves so that every load can be in flight before the first store: issue()
// loads the 16-byte pieces into registers, put() stores them and copies the
// tail in ESZ-byte elements.  src is 16-byte aligned; nothing past src + nbytes
// is read.
template <int ESZ>
struct Stager {
    static constexpr int PIECES = TINY_STAGE / 1024;  // 16-byte pieces per lane
    intx4 v[PIECES];
    __device__ void issue(const char *src, int64_t nbytes, int lane) {
        const int64_t full = nbytes / 16;
#pragma unroll
        for (int u = 0; u < PIECES; ++u) {
            const int64_t c = lane + 64 * u;
            // non-temporal: each problem's operands are read by this wave only
            if (c < full) v[u] = __builtin_nontemporal_load((const intx4 *)(src + c * 16));
        }
    }
    __device__ void put(DMP_LDS char *dst, const char *src, int64_t nbytes, int lane) const {
        const int64_t full = nbytes / 16;
#pragma unroll
        for (int u = 0; u < PIECES; ++u) {
            const int64_t c = lane + 64 * u;
            if (c < full) *(DMP_LDS intx4 *)(dst + c * 16) = v[u];
        }
        for (int64_t t = full * 16 + (int64_t)lane * ESZ; t < nbytes; t += 64 * ESZ) {
            if constexpr (ESZ == 2) *(DMP_LDS uint16_t *)(dst + t) = *(const uint16_t *)(src + t);
            else *(DMP_LDS uint8_t *)(dst + t) = *(const uint8_t *)(src + t);
        }
    }
};

// One wave per NB problems (4 waves per workgroup).  SA / SB: A / B shared by
// the whole batch.  The NB problems of a wave are consecutive batch entries, so
// their A (B, C, D) lie in one contiguous region that the wave can move with
// 16-byte accesses through LDS when it fits; the instruction operands are then
// gathered from LDS.  Otherwise each lane loads its own elements.
template <class DT, int S, bool SA, bool SB>
__global__ __launch_bounds__(256) void tiny_gemm(const TinyArgs p) {
    constexpr int NB = 64 / S;
    constexpr int ESZ = DT::ESZ;
    constexpr int CB = SA ? (NB == 16 ? 4 : 2) : 0;  // broadcast block 0's A to all blocks
    constexpr int BG = SB ? 4 : 0;                    // lanes 0-15's B to all lane groups
    using I = Multi<DT, S>;
    using acc_t = typename DT::acc;
    constexpr int TINY_OUT = tiny_out_bytes(S);
    __shared__ __attribute__((aligned(16))) char lds[4 * (2 * TINY_STAGE + TINY_OUT)];
    const int lane = lane_id(), wave = wave_id();
    const int64_t base = ((int64_t)blockIdx.x * 4 + wave) * NB;
    if (base >= p.batch) return;  // whole wave idle (wave-uniform); no barriers below
    const int64_t nprob = p.batch - base < NB ? p.batch - base : NB;
    DMP_LDS char *la = (DMP_LDS char *)lds + wave * (2 * TINY_STAGE + TINY_OUT);
    DMP_LDS char *lb = la + TINY_STAGE;
    DMP_LDS char *lo = lb + TINY_STAGE;

    // input roles of this lane
    const int blk = lane / S, rc = lane % S;
    const int64_t prob = base + blk;
    const bool prob_ok = prob < p.batch;
    // a shared operand is read only by the lanes the instruction takes it from
    const bool a_lane = SA ? blk == 0 : prob_ok;
    const bool b_lane = SB ? lane < 16 : prob_ok;
    const int64_t pa = SA ? 0 : prob, pb = SB ? 0 : prob;
    const int64_t a_off = p.a_col ? (int64_t)rc : (int64_t)rc * p.lda;   // start of row rc
    const int64_t b_off = p.b_col ? (int64_t)rc * p.ldb : (int64_t)rc;   // start of column rc
    const int64_t a_sk = p.a_col ? p.lda : 1, b_sk = p.b_col ? 1 : p.ldb;
    const bool a_ok = a_lane && rc < p.M, b_ok = b_lane && rc < p.N;
    const bool st_a = !SA && p.stage_a, st_b = !SB && p.stage_b;
    typedef acc_t vec4 __attribute__((ext_vector_type(4)));
    // every global load of the wave is issued before any is waited for: C of a
    // dense output region, then the A and B regions
    constexpr int OUTP = TINY_OUT / 1024;  // 16-byte output pieces per lane
    const int64_t chunks = p.flat_out ? nprob * p.sC / 4 : 0;  // sC is a multiple of 4 then
    const acc_t *Cr = (const acc_t *)p.C + base * p.sC;
    vec4 cpre[OUTP];
    if (p.flat_out && p.ep.use_c) {
#pragma unroll
        for (int u = 0; u < OUTP; ++u) {
            const int64_t c = lane + 64 * u;
            if (c < chunks) cpre[u] = *(const vec4 *)(Cr + c * 4);
        }
    }
    const char *Areg = (const char *)p.A + base * p.sA * ESZ;
    const char *Breg = (const char *)p.B + base * p.sB * ESZ;
    const int64_t nba = st_a ? ((nprob - 1) * p.sA + p.ext_a) * ESZ : 0;
    const int64_t nbb = st_b ? ((nprob - 1) * p.sB + p.ext_b) * ESZ : 0;
    Stager<ESZ> sa_, sb_;
    if (st_a) sa_.issue(Areg, nba, lane);
    if (st_b) sb_.issue(Breg, nbb, lane);
    if (st_a) sa_.put(la, Areg, nba, lane);
    if (st_b) sb_.put(lb, Breg, nbb, lane);
    // LDS operations of one wave complete in order; this keeps the compiler
    // from moving the gathers above the copies
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const char *Ag = (const char *)p.A + (pa * p.sA + a_off) * ESZ;
    const char *Bg = (const char *)p.B + (pb * p.sB + b_off) * ESZ;
    const DMP_LDS char *As = la + ((prob - base) * p.sA + a_off) * ESZ;
    const DMP_LDS char *Bs = lb + ((prob - base) * p.sB + b_off) * ESZ;

    typename I::acc acc{};
    for (int64_t k0 = 0; k0 < p.K; k0 += 4) {
        const uint64_t a = st_a ? load_k4<ESZ>(As, a_sk, k0, p.K, a_ok, p.a_vec)
                                : load_k4<ESZ>(Ag, a_sk, k0, p.K, a_ok, p.a_vec);
        const uint64_t b = st_b ? load_k4<ESZ>(Bs, b_sk, k0, p.K, b_ok, p.b_vec)
                                : load_k4<ESZ>(Bg, b_sk, k0, p.K, b_ok, p.b_vec);
        acc = I::template mma<CB, 0, BG>(a, b, acc);
    }

    // output: element (i, j) of problem q held in register g of this lane
    auto where = [&](int g, int64_t &q, int &i, int &j) {
        if (S == 4) {
            q = base + lane / 4;
            i = g;
            j = lane % 4;
        } else {
            q = base + g / 4;
            i = 4 * (lane / 16) + g % 4;
            j = lane % 16;
        }
    };
    if (p.flat_out) {
        // dense C and D in the accumulator type: results go to LDS at their
        // offsets in the wave's region, which then moves as 16-byte vectors
#pragma unroll
        for (int g = 0; g < (S == 4 ? 4 : 16); ++g) {
            int64_t q;
            int i, j;
            where(g, q, i, j);
            if (q < p.batch && i < p.M && j < p.N)
                *(DMP_LDS acc_t *)(lo + ((q - base) * p.sC + (int64_t)i * p.ldc + j) * 4) = acc[g];
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        acc_t *Dr = (acc_t *)p.D + base * p.sC;
#pragma unroll
        for (int u = 0; u < OUTP; ++u) {
            const int64_t c = lane + 64 * u;
            if (c < chunks) {
                const vec4 v = *(const DMP_LDS vec4 *)(lo + c * 16);
                const vec4 cv = p.ep.use_c ? cpre[u] : vec4{0, 0, 0, 0};
                *(vec4 *)(Dr + c * 4) = finish4(v, cv, p.ep);
            }
        }
        return;
    }
    const char *Cb = (const char *)p.C;
    char *Db = (char *)p.D;
#pragma unroll
    for (int g = 0; g < (S == 4 ? 4 : 16); ++g) {
        int64_t q;
        int i, j;
        where(g, q, i, j);
        if (q < p.batch && i < p.M && j < p.N) {
            const int64_t idx = q * p.sC + (int64_t)i * p.ldc + j;
            const vec4 a = {acc[g], 0, 0, 0};
            const vec4 c = p.ep.use_c ? load4<acc_t>(Cb, idx, p.ep.c_type, false, 1) : vec4{0, 0, 0, 0};
            store4<acc_t>(Db, idx, finish4(a, c, p.ep), p.ep.d_type, false, 1);
        }
    }
}

}  // namespace dmp
