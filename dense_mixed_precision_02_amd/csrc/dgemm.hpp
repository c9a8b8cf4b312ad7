// dgemm.hpp -- fp64 D = A*B + C on the double-precision matrix instruction
// v_mfma_f64_16x16x4_f64 (pages: "CDNA2 dense MFMA builtins", section
// "FP64-accumulate builtins" and the 16x16 FP64 accumulator layout).
//
// Operand maps of one instruction (checked on gfx950 with a one-hot probe):
// lane L supplies A[row L%16][k L/16] and B[k L/16][col L%16]; accumulator
// pair G of lane L holds D[4G + L/16][L%16] (the pages' CDNA2 FP64 layout).
// The instruction rounds every step to nearest even.  It cannot overlap with
// vector ALU work of the same wave, so the K loop keeps that work minimal:
// operands go straight from global memory into LDS (no registers), offsets
// are precomputed, and loop control is scalar.
#pragma once

#include "common.hpp"

namespace dmp {

typedef double doublex2 __attribute__((ext_vector_type(2)));
typedef double doublex4 __attribute__((ext_vector_type(4)));

__device__ static inline doublex4 mfma_f64(double a, double b, doublex4 c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

struct DgemmArgs {
    const double *A, *B, *C;
    double *D;
    int64_t M, N, K, lda, ldb, ldc;
    int64_t sA, sB, sC;  // batch strides in elements
    int tiles_m, tiles_n;
    int use_c;           // 0: D = A*B (C not read)
};

// One operand tile of R rows (A: rows of M, B: columns of N) by 16 k (128
// bytes of k per row) in LDS, filled by wave-wide 1 KB direct loads.
//   K-contiguous operand: row r occupies bytes [128 r, 128 r + 128); its 16-byte
//     granule g (k = 2g, 2g+1) sits in slot g ^ swz(r), so that the 16 rows a
//     fragment read touches spread over all banks (SWZ; otherwise slot g).
//   MN-contiguous operand: k-row k occupies bytes [8 R k, 8 R (k+1)); granule p
//     (rows 2p, 2p+1) sits in slot p, unswizzled.  A swizzle that moved every
//     other pair of k-rows by 128 bytes (so that the four k-rows one read touches
//     alternate between the halves of a 256-byte bank window) made the 4096^3
//     launch with a row-major B 7 % slower (2138 against 1981 us, timed
//     interleaved); dropping the K-contiguous operand's swizzle as well made it
//     slower again (2095 us).
template <int R, bool KCONTIG, bool SWZ = true>
struct Op64 {
    static constexpr int BYTES = R * 128;
    static constexpr int CHUNKS = BYTES / 1024;
    static constexpr int CPW = CHUNKS / 4;  // chunks per wave (4 waves)
    static_assert(CHUNKS % 4 == 0, "chunks split evenly over 4 waves");

    int off[CPW];  // byte offset of this lane's granule from the tile origin, per chunk
    int rr[CPW];   // K-contig: row index; MN-contig: first row of the granule
    int kk[CPW];   // k index of the granule's first element within the tile

    __device__ static int swz(int r) { return SWZ ? ((r & 7) ^ ((r >> 3) & 1)) : 0; }

    __device__ void init(int wave, int lane, int64_t ld) {
#pragma unroll
        for (int j = 0; j < CPW; ++j) {
            const int c = j * 4 + wave;
            if (KCONTIG) {
                const int r = c * 8 + (lane >> 3);
                const int g = (lane & 7) ^ swz(r);
                rr[j] = r;
                kk[j] = 2 * g;
                off[j] = (int)(r * ld + 2 * g) * 8;
            } else {
                const int q = c * 64 + lane;          // granule index in k-row-major order
                const int k = q / (R / 2);
                const int p = q % (R / 2);
                rr[j] = 2 * p;
                kk[j] = k;
                off[j] = (int)(k * ld + 2 * p) * 8;
            }
        }
    }

    // Copy this wave's chunks of the tile whose origin is (row0, k0) into lds.
    // rows: valid rows from row0; kleft: valid k from k0 (granules beyond either
    // are zero-filled by the buffer range check).
    __device__ void issue(const double *tile, DMP_LDS char *lds, int wave, int64_t rows,
                          int kleft) const {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(tile);
#pragma unroll
        for (int j = 0; j < CPW; ++j) {
            const bool ok = rr[j] < rows && kk[j] < kleft;
            load_granule_to_lds(rs, lds + (j * 4 + wave) * 1024, ok ? off[j] : OOB_OFFSET);
        }
    }

    // Values of rows [rb, rb+16) for the two instructions of double-step d
    // (k = 8d .. 8d+7): lane L (group q = L/16, row rb + L%16) gets k = 8d+2q in
    // .x (first instruction) and k = 8d+2q+1 in .y (second).
    __device__ static doublex2 frag(const DMP_LDS char *lds, int rb, int d, int lane) {
        const int q = lane >> 4;
        const int row = rb + (lane & 15);
        if (KCONTIG) {
            const int g = 4 * d + q;
            return *(const DMP_LDS doublex2 *)(lds + row * 128 + ((g ^ swz(row)) << 4));
        } else {
            const int k0 = 8 * d + 2 * q;
            doublex2 v;
            const int p = row >> 1, h = (row & 1) * 8;
            v.x = *(const DMP_LDS double *)(lds + k0 * (R * 8) + (p << 4) + h);
            v.y = *(const DMP_LDS double *)(lds + (k0 + 1) * (R * 8) + (p << 4) + h);
            return v;
        }
    }

    // Element (row0, k0) of the operand.
    __device__ static const double *tile_base(const double *X, int64_t ld, int64_t row0, int64_t k0) {
        return KCONTIG ? X + row0 * ld + k0 : X + k0 * ld + row0;
    }
};

// BM x BN output tile per workgroup of 4 waves (2 x 2), each wave (BM/2) x (BN/2)
// in 16 x 16 instruction tiles.  k-tile 16.  AK: A row-major (k-contiguous);
// BKC: B column-major (k-contiguous).
template <int BM, int BN, bool AK, bool BKC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void dgemm_tile(const DgemmArgs p) {
    constexpr int WTM = BM / 2, WTN = BN / 2;
    constexpr int TM = WTM / 16, TN = WTN / 16;
    constexpr int KT = 16;
    // K-contiguous B is swizzled only next to an MN-contiguous A: with a swizzled
    // K-contiguous A the unswizzled B is faster (4096^3: 2075 against 2183 us),
    // with an MN-contiguous A the swizzled one (2026 against 2132 us).
    using OpA = Op64<BM, AK>;
    using OpB = Op64<BN, BKC, !AK>;

    __shared__ __attribute__((aligned(1024))) char lds_a0[OpA::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_b0[OpB::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_a1[OpA::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_b1[OpB::BYTES];

    // tile order: batch-major, then grouped rows of 4 tiles (as the 16-bit kernel),
    // after spreading consecutive ids over the 8 XCDs' L2s
    int wg = blockIdx.x;
    {
        const int total = gridDim.x, per = total / 8;
        if (wg < per * 8) wg = (wg % 8) * per + wg / 8;
    }
    const int tiles = p.tiles_m * p.tiles_n;
    const int b = wg / tiles;
    int t = wg - b * tiles;
    constexpr int GM = 4;
    const int group = t / (GM * p.tiles_n);
    const int first_m = group * GM;
    const int gm = min(p.tiles_m - first_m, GM);
    t -= group * GM * p.tiles_n;
    const int64_t m0 = (int64_t)(first_m + t % gm) * BM, n0 = (int64_t)(t / gm) * BN;

    const int lane = lane_id(), wave = wave_id();
    const int wm = wave >> 1, wn = wave & 1;
    const double *Ab = p.A + b * p.sA;
    const double *Bb = p.B + b * p.sB;
    const int64_t rows_a = p.M - m0, rows_b = p.N - n0;

    OpA opa;
    OpB opb;
    opa.init(wave, lane, p.lda);
    opb.init(wave, lane, p.ldb);

    doublex4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = doublex4{0, 0, 0, 0};

    // An odd k-tile count is made even by a leading all-zero k-tile, so the loop
    // below (two k-tiles per trip, each LDS buffer named statically) has a
    // single exit.  k-tiles outside [0, K) load zeros and touch no memory.
    const int nkt = (int)((p.K + KT - 1) / KT);
    const int ntiles = nkt + (nkt & 1);
    const int64_t k_first = -(int64_t)(nkt & 1) * KT;
    auto stage = [&](int kt, DMP_LDS char *la, DMP_LDS char *lb) {
        const int64_t k0 = k_first + (int64_t)kt * KT;
        const int64_t kl = p.K - k0;
        const bool in = k0 >= 0 && kl > 0;
        const int kleft = !in ? 0 : (kl > KT ? KT : (int)kl);
        const int64_t kb = in ? k0 : 0;
        opa.issue(OpA::tile_base(Ab, p.lda, m0, kb), la, wave, rows_a, kleft);
        opb.issue(OpB::tile_base(Bb, p.ldb, n0, kb), lb, wave, rows_b, kleft);
    };
    auto compute = [&](const DMP_LDS char *la, const DMP_LDS char *lb) {
#pragma unroll
        for (int d = 0; d < KT / 8; ++d) {
            doublex2 fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) fa[i] = OpA::frag(la, wm * WTM + i * 16, d, lane);
#pragma unroll
            for (int j = 0; j < TN; ++j) fb[j] = OpB::frag(lb, wn * WTN + j * 16, d, lane);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma_f64(fa[i].x, fb[j].x, acc[i][j]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma_f64(fa[i].y, fb[j].y, acc[i][j]);
        }
    };

    DMP_LDS char *la0 = (DMP_LDS char *)lds_a0, *lb0 = (DMP_LDS char *)lds_b0;
    DMP_LDS char *la1 = (DMP_LDS char *)lds_a1, *lb1 = (DMP_LDS char *)lds_b1;
    if (nkt > 0) {
        stage(0, la0, lb0);
        wait_vmcnt<0>();
        __syncthreads();
        for (int kt = 0; kt < ntiles; kt += 2) {
            stage(kt + 1, la1, lb1);
            step_sync();
            compute(la0, lb0);
            wait_vmcnt<0>();
            __syncthreads();
            stage(kt + 2, la0, lb0);  // past the last k-tile: zero fill only
            step_sync();
            compute(la1, lb1);
            wait_vmcnt<0>();
            __syncthreads();
        }
    }

    // Epilogue.  Pair G of lane L holds row 4G + L/16, column L%16 of each 16x16
    // tile.  Each wave passes its tile through LDS 16 rows at a time (LDS stores
    // take the accumulator registers directly; vector arithmetic on them would
    // make the compiler keep them in vector registers through the K loop and
    // copy them every trip), then reads whole rows back so that C and D move
    // in runs of consecutive doubles.
    constexpr int SP = WTN + 16;  // padded slab row: rows r and r+1 are 128 bytes apart mod 256
    static_assert(16 * SP * 8 <= OpA::BYTES && 16 * SP * 8 <= OpB::BYTES, "slab must fit");
    constexpr int RPP = 64 / WTN;  // slab rows per pass of 64 lanes
    DMP_LDS double *slab = (DMP_LDS double *)(wave == 0 ? la0 : wave == 1 ? lb0 : wave == 2 ? la1 : lb1);
    const double *Cb = p.C + b * p.sC;
    double *Db = p.D + b * p.sC;
    const int64_t col = n0 + wn * WTN + lane % WTN;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int G = 0; G < 4; ++G)
                // volatile: single stores, which take the accumulator registers
                // as data (paired stores would need vector registers)
                *(volatile DMP_LDS double *)&slab[(4 * G + (lane >> 4)) * SP + j * 16 + (lane & 15)] =
                    acc[i][j][G];
        // LDS instructions of one wave complete in order; this only keeps the
        // compiler from moving the reads above the writes
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
        for (int q = 0; q < 16 / RPP; ++q) {
            const int r = q * RPP + lane / WTN;
            const double v = slab[r * SP + lane % WTN];
            const int64_t row = m0 + wm * WTM + i * 16 + r;
            if (row < p.M && col < p.N) {
                const int64_t idx = row * p.ldc + col;
                __builtin_nontemporal_store(p.use_c ? v + Cb[idx] : v, Db + idx);  // D is written once
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }
}

// Any alignment, leading dimension or K: one wave per 16 x 16 output tile,
// element loads with bounds checks, the same instruction.
__global__ __launch_bounds__(64) void dgemm_generic(const DgemmArgs p, int a_col, int b_col) {
    const int tiles = p.tiles_m * p.tiles_n;
    const int b = blockIdx.x / tiles;
    const int t = blockIdx.x - b * tiles;
    const int64_t m0 = (int64_t)(t / p.tiles_n) * 16, n0 = (int64_t)(t % p.tiles_n) * 16;
    const int lane = threadIdx.x;
    const double *Ab = p.A + b * p.sA;
    const double *Bb = p.B + b * p.sB;
    const int64_t row = m0 + (lane & 15), col = n0 + (lane & 15);
    const int q = lane >> 4;
    doublex4 acc = {0, 0, 0, 0};
    for (int64_t k0 = 0; k0 < p.K; k0 += 4) {
        const int64_t k = k0 + q;
        double a = 0.0, bv = 0.0;
        if (row < p.M && k < p.K) a = a_col ? Ab[row + k * p.lda] : Ab[row * p.lda + k];
        if (col < p.N && k < p.K) bv = b_col ? Bb[k + col * p.ldb] : Bb[k * p.ldb + col];
        acc = mfma_f64(a, bv, acc);
    }
    const double *Cb = p.C + b * p.sC;
    double *Db = p.D + b * p.sC;
    const int64_t c = n0 + (lane & 15);
#pragma unroll
    for (int G = 0; G < 4; ++G) {
        const int64_t r = m0 + 4 * G + q;
        if (r < p.M && c < p.N) {
            const int64_t idx = r * p.ldc + c;
            __builtin_nontemporal_store(p.use_c ? acc[G] + Cb[idx] : acc[G], Db + idx);
        }
    }
}

}  // namespace dmp
