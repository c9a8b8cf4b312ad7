// sparse_gemm.hpp -- D = A*B + C with a 2:4 structured-sparse A on the sparse
// matrix instructions v_smfmac_f32_32x32x32_{f16,bf16} and
// v_smfmac_i32_32x32x64_i8 (pages: "MFMA common parameters", section "Sparse
// MFMA parameters": two of every four consecutive K positions of A hold the
// non-zeros, and an index operand says which, two bits per kept value).
//
// Compressed A (the library's format): per row, every group of four dense k
// keeps two values, the one at the lower position first; the index stream
// holds four bits per group (the two positions, lower one in the low two
// bits), groups in k order, packed into 16-bit words low nibble first.  Rows
// are padded to Kp dense k with zero values: Kp = 64 * ceil(K / 64) for
// fp16/bf16, 128 * ceil(K / 128) for int8 (one sparse k-tile of KT dense k),
// and to Mp = 16 * ceil(M / 16) rows.  Both arrays are blocked so that one
// k-tile of 16 rows is contiguous: values [batch][Mp/16][Kp/KT][16][KT/2]
// (1 KB per block and k-tile), index words [batch][Mp/16][Kp/KT][16][KT/16];
// each copy then reads whole 128-byte lines.
//
// Instruction maps on gfx950 (checked with one-hot and random-operand probes):
// lane L holds row L%32 of A; with h = L/32 its compressed values cover dense k
// [16h, 16h+16) of the 32-k step (16-bit types: eight values) or [32h, 32h+32)
// of the 64-k step (int8: sixteen values), and its 32-bit index operand is
// the index stream of those k, value j's position in bits [2j+1:2j].  B lane L
// holds column L%32 as the two fragments of the dense 32x32 instruction (16-k
// or 32-k) for the step's two halves, so B is staged and read exactly as in the
// dense kernel.
#pragma once

#include "tile_gemm.hpp"

namespace dmp {

typedef int sp_intx8 __attribute__((ext_vector_type(8)));
typedef _Float16 sp_half16 __attribute__((ext_vector_type(16)));
typedef __bf16 sp_bf16x16 __attribute__((ext_vector_type(16)));

template <class DT> struct SparseMma;
template <> struct SparseMma<F16> {
    __device__ static floatx16 mma(intx4 a, intx4 b0, intx4 b1, floatx16 c, int idx) {
        const sp_intx8 b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        return __builtin_amdgcn_smfmac_f32_32x32x32_f16(__builtin_bit_cast(half8, a),
                                                        __builtin_bit_cast(sp_half16, b), c, idx, 0, 0);
    }
};
template <> struct SparseMma<I8> {
    __device__ static intx16 mma(intx4 a, intx4 b0, intx4 b1, intx16 c, int idx) {
        const sp_intx8 b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        return __builtin_amdgcn_smfmac_i32_32x32x64_i8(a, b, c, idx, 0, 0);
    }
};
template <> struct SparseMma<BF16> {
    __device__ static floatx16 mma(intx4 a, intx4 b0, intx4 b1, floatx16 c, int idx) {
        const sp_intx8 b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        return __builtin_amdgcn_smfmac_f32_32x32x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                         __builtin_bit_cast(sp_bf16x16, b), c, idx, 0, 0);
    }
};

struct SparseArgs {
    const void *Ac, *meta, *B, *C;
    void *D;
    int64_t M, N, K, ldb, ldc;
    int64_t sAc, sM, sB, sC;               // batch strides in elements (values, words, B, C)
    int tiles_m, tiles_n, batch, nkt;      // nkt = Kp/KT k-tiles
    EpiParams ep;                          // plain: accumulator-typed C and D, alpha 1, beta 0 or 1
};

// Dense k per k-tile: two instruction steps.  Either way a k-tile is 64 bytes
// of compressed values and 128 bytes of B per row or column; the index stream
// is KT/8 bytes per row.
template <class DT> constexpr int sparse_kt() { return DT::ESZ == 2 ? 64 : 128; }

// Compressed-A panel: R rows x 64 bytes (one k-tile) per row; the 16-byte
// granule g of row r sits in slot g ^ ((r >> 1) & 3), so that any eight
// consecutive rows of one fragment read cover the eight 16-byte slots of a
// 128-byte bank window.  One wave-wide load copies one 16-row block (1 KB,
// contiguous in the blocked format); blk is the distance between blocks.
template <int R, int NW>
struct OpC {
    static constexpr int BYTES = R * 64;
    static constexpr int CHUNKS = BYTES / 1024;  // 16 rows per wave-wide load
    static constexpr int CPW = CHUNKS / NW;
    static_assert(CHUNKS % NW == 0, "chunks split evenly over waves");
    __device__ static int sw(int r) { return (r >> 1) & 3; }
    int off0, r0, step;
    __device__ void init(int wave, int lane, int64_t blk) {
        r0 = wave * 16 + (lane >> 2);
        const int g = (lane & 3) ^ sw(r0);  // sw(r0 + 16*NW*j) == sw(r0)
        off0 = (int)(wave * blk) + (lane >> 2) * 64 + 16 * g;
        step = (int)(NW * blk);
    }
    // chunk j of this wave; rows: valid rows from the tile origin; ok: the k-tile exists
    __device__ void issue(const __amdgpu_buffer_rsrc_t &rs, DMP_LDS char *lds, int wave, int j,
                          int64_t rows, bool ok) const {
        const bool in = ok && r0 + 16 * NW * j < rows;
        load_granule_to_lds(rs, lds + (j * NW + wave) * 1024, in ? off0 + j * step : OOB_OFFSET);
    }
    // values of row rbase + L%32 for step S: granule 2S + L/32
    __device__ static intx4 frag(const DMP_LDS char *lds, int rbase, int S, int lane) {
        const int row = rbase + (lane & 31);
        const int g = 2 * S + (lane >> 5);
        return *(const DMP_LDS intx4 *)(lds + row * 64 + ((g ^ sw(row)) << 4));
    }
};

// Index stream of a panel: R rows x MB bytes (one k-tile) per row, row after
// row in LDS, copied with direct loads of 4 bytes (MB = 8: two lanes per row)
// or 16 bytes (MB = 16).  In the blocked format a 16-row block's index bytes
// for one k-tile are contiguous (16*MB bytes, blocks blk apart), so each
// load reads whole lines.
template <int R, int NW, int MB>
struct OpMeta {
    static constexpr int BYTES = R * MB;
    static constexpr int LB = MB == 8 ? 4 : 16;  // bytes per lane per load
    static constexpr int LPR = MB / LB;          // lanes per row
    static constexpr int ROWS = 64 / LPR;        // rows per wave-wide load
    static constexpr int BPC = ROWS / 16;        // 16-row blocks per load
    static constexpr int CHUNKS = R / ROWS;
    static constexpr int CPW = CHUNKS / NW;
    static_assert(MB == 8 || MB == 16, "index bytes per row");
    static_assert(CHUNKS % NW == 0, "chunks split evenly over waves");
    int off0, r0, step;
    __device__ void init(int wave, int lane, int64_t blk) {
        r0 = wave * ROWS + lane / LPR;
        const int lpb = 64 / BPC;                 // lanes per block
        off0 = (int)((BPC * wave + lane / lpb) * blk) + (lane % lpb) * LB;
        step = (int)(BPC * NW * blk);
    }
    __device__ void issue(const __amdgpu_buffer_rsrc_t &rs, DMP_LDS char *lds, int wave, int j,
                          int64_t rows, bool ok) const {
        const bool in = ok && r0 + ROWS * NW * j < rows;
        DMP_LDS char *dst = lds + (j * NW + wave) * 64 * LB;
        const int off = in ? off0 + j * step : OOB_OFFSET;
        if constexpr (LB == 4) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 4, off, 0, 0, 0);
        else __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, off, 0, 0, 0);
    }
    // index operand of row rbase + L%32 for step S: the 16-bit (MB = 8) or
    // 32-bit (MB = 16) piece 2S + L/32 of the row's k-tile
    __device__ static int word(const DMP_LDS char *lds, int rbase, int S, int lane) {
        const int row = rbase + (lane & 31);
        if constexpr (MB == 8) return *(const DMP_LDS uint16_t *)(lds + row * 8 + (2 * S + (lane >> 5)) * 2);
        else return *(const DMP_LDS int *)(lds + row * 16 + (2 * S + (lane >> 5)) * 4);
    }
};

// 256 x 256 tile of D per workgroup of 4 waves (2 x 2, 128 x 128 each); k-tile
// of two instruction steps; three LDS stages so that the copy of k-tile t+2
// has two k-tiles of work to land behind.  BKC: B column-major.
template <class DT, bool BKC>
__global__ __launch_bounds__(256) void sparse_gemm(const SparseArgs p) {
    constexpr int BM = 256, BN = 256, NW = 4, WN = 2;
    constexpr int WTM = 128, WTN = 128, TM = WTM / 32, TN = WTN / 32;
    constexpr int KT = sparse_kt<DT>();  // dense k per k-tile
    constexpr int ESZ = DT::ESZ;
    using OpA = OpC<BM, NW>;
    using OpM = OpMeta<BM, NW, KT / 8>;
    using OpB = Operand<DT, BN, NW, BKC>;
    using acc_t = typename DT::acc;
    using accv = typename DT::accv;
    using vec4 = vec4_of<acc_t>;
    constexpr int SP = WTN + 8;  // epilogue slab row (floats)
    constexpr int ABYTES = OpA::BYTES > 32 * SP * 4 ? OpA::BYTES : 32 * SP * 4;
    static_assert(32 * SP * 4 <= OpB::BYTES, "epilogue slab must fit a B buffer");
    __shared__ __attribute__((aligned(1024))) char lds_a0[ABYTES];
    __shared__ __attribute__((aligned(1024))) char lds_a1[ABYTES];
    __shared__ __attribute__((aligned(1024))) char lds_a2[ABYTES];
    __shared__ __attribute__((aligned(1024))) char lds_m0[OpM::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_m1[OpM::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_m2[OpM::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_b0[OpB::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_b1[OpB::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_b2[OpB::BYTES];

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
    const int wm = wave / WN, wn = wave % WN;
    // blocked format: 16-row blocks, each k-tile of a block contiguous
    const int64_t vblk = (int64_t)p.nkt * 1024, mblk = (int64_t)p.nkt * 16 * (KT / 8);
    const char *Acb = (const char *)p.Ac + (int64_t)b * p.sAc * ESZ + (m0 / 16) * vblk;
    const char *Mb = (const char *)p.meta + (int64_t)b * p.sM * 2 + (m0 / 16) * mblk;
    const char *Bb = (const char *)p.B + (int64_t)b * p.sB * ESZ;
    const int64_t rows_a = p.M - m0;

    OpA opa;
    OpM opm;
    OpB opb;
    opa.init(wave, lane, vblk);
    opm.init(wave, lane, mblk);
    opb.init(wave, lane, p.ldb, (int)n0, p.N);

    accv acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = accv{};

    // The k-tile count is made a multiple of three (one per LDS stage, named
    // statically) by leading all-zero k-tiles; tiles outside [0, nkt) load zeros
    // and touch no memory.
    const int lead = (3 - p.nkt % 3) % 3;
    const int ntiles = p.nkt + lead;
    auto stage = [&](int tt, DMP_LDS char *la, DMP_LDS char *lm, DMP_LDS char *lb) {
        const int kt = tt - lead;
        const bool ok = kt >= 0 && kt < p.nkt;
        const int64_t ktc = ok ? kt : 0;
        const int64_t kl = p.K - ktc * KT;
        const int kleft = !ok ? 0 : (kl > KT ? KT : (kl < 0 ? 0 : (int)kl));
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(Acb + ktc * 1024);
        const __amdgpu_buffer_rsrc_t rm = make_rsrc(Mb + ktc * 16 * (KT / 8));
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(OpB::tile_base(Bb, p.ldb, n0, ktc * KT));
#pragma unroll
        for (int j = 0; j < OpA::CPW; ++j) opa.issue(ra, la, wave, j, rows_a, ok);
#pragma unroll
        for (int j = 0; j < OpM::CPW; ++j) opm.issue(rm, lm, wave, j, rows_a, ok);
#pragma unroll
        for (int j = 0; j < OpB::CPW; ++j) opb.issue(rb, lb, wave, j, kleft, p.N);
    };
    constexpr int NL = OpA::CPW + OpM::CPW + OpB::CPW;  // loads per wave per k-tile

    struct Frags {
        intx4 a[TM], b0[TN], b1[TN];
        int ix[TM];
    };
    auto read = [&](Frags &f, const DMP_LDS char *la, const DMP_LDS char *lm, const DMP_LDS char *lb,
                    int S) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            f.a[i] = OpA::frag(la, wm * WTM + i * 32, S, lane);
            f.ix[i] = OpM::word(lm, wm * WTM + i * 32, S, lane);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            f.b0[j] = OpB::frag(lb, wn * WTN + j * 32, 2 * S, lane);
            f.b1[j] = OpB::frag(lb, wn * WTN + j * 32, 2 * S + 1, lane);
        }
    };
    auto mma = [&](const Frags &f) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = SparseMma<DT>::mma(f.a[i], f.b0[j], f.b1[j], acc[i][j], f.ix[i]);
    };
    constexpr int NMF = TM * TN;
    constexpr int NRD = TM * 2 + TN * 2 * OpB::READS;

    DMP_LDS char *LA[3] = {(DMP_LDS char *)lds_a0, (DMP_LDS char *)lds_a1, (DMP_LDS char *)lds_a2};
    DMP_LDS char *LM[3] = {(DMP_LDS char *)lds_m0, (DMP_LDS char *)lds_m1, (DMP_LDS char *)lds_m2};
    DMP_LDS char *LB[3] = {(DMP_LDS char *)lds_b0, (DMP_LDS char *)lds_b1, (DMP_LDS char *)lds_b2};

    // k-tile tt in stage c: the copy of tt+2 starts (into the stage freed at the
    // last barrier), step 1 is read while step 0 runs, then every wave waits for
    // tt+1 to land, and step 0 of tt+1 is read while step 1 runs.
    Frags F0, F1;
    auto ktile = [&](int tt, int c) {
        const int n = (c + 1) % 3, f = (c + 2) % 3;
        stage(tt + 2, LA[f], LM[f], LB[f]);
        read(F1, LA[c], LM[c], LB[c], 1);
        mma(F0);
        interleave<NMF, NRD, NL>();
        __builtin_amdgcn_sched_barrier(0);
        step_sync();
        barrier_vmcnt<NL>();  // k-tile tt+1 has landed everywhere; tt+2 may still be in flight
        read(F0, LA[n], LM[n], LB[n], 0);
        mma(F1);
        interleave<NMF, NRD, 0>();
        __builtin_amdgcn_sched_barrier(0);
        step_sync();
    };
    if (p.nkt > 0) {
        stage(0, LA[0], LM[0], LB[0]);
        stage(1, LA[1], LM[1], LB[1]);
        barrier_vmcnt<NL>();
        read(F0, LA[0], LM[0], LB[0], 0);
        for (int tt = 0; tt < ntiles; tt += 3) {
            ktile(tt, 0);
            ktile(tt + 1, 1);
            ktile(tt + 2, 2);
        }
    }

    // ---- epilogue: as the dense kernel's (accumulators through a row-major LDS
    // slab per wave, C and D as 16-byte vectors), fp32 C and D ----
    wait_vmcnt<0>();
    __syncthreads();
    DMP_LDS acc_t *slab = (DMP_LDS acc_t *)(wave == 0 ? LB[0] : wave == 1 ? LB[1] : wave == 2 ? LB[2] : LA[0]);
    constexpr int LPR = WTN / 4, RPP = 64 / LPR, PASSES = 32 / RPP;
    const int64_t col_w = n0 + wn * WTN;
    const acc_t *Cb = (const acc_t *)p.C + (int64_t)b * p.sC;
    acc_t *Db = (acc_t *)p.D + (int64_t)b * p.sC;
    const bool use_c = p.ep.use_c;
    const bool vec_ok = p.ldc % 4 == 0 && (!use_c || (uintptr_t)Cb % 16 == 0) && (uintptr_t)Db % 16 == 0;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int G = 0; G < 16; ++G)
                slab[(8 * (G >> 2) + 4 * (lane >> 5) + (G & 3)) * SP + j * 32 + (lane & 31)] = acc[i][j][G];
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        const int64_t row_s = m0 + wm * WTM + i * 32;
        if (vec_ok && row_s + 32 <= p.M && col_w + WTN <= p.N) {
            vec4 cv[PASSES];
#pragma unroll
            for (int q = 0; q < PASSES; ++q) {
                cv[q] = vec4{0, 0, 0, 0};
                if (use_c) {
                    const int64_t grow = row_s + q * RPP + lane / LPR, gcol = col_w + (lane % LPR) * 4;
                    cv[q] = *(const vec4 *)(Cb + grow * p.ldc + gcol);
                }
            }
#pragma unroll
            for (int q = 0; q < PASSES; ++q) {
                const int r = q * RPP + lane / LPR, cl = (lane % LPR) * 4;
                const vec4 v = *(const DMP_LDS vec4 *)(slab + r * SP + cl);
                *(vec4 *)(Db + (row_s + r) * p.ldc + col_w + cl) = finish4(v, cv[q], p.ep);
            }
        } else {
#pragma unroll 1
            for (int q = 0; q < PASSES; ++q) {
                const int r = q * RPP + lane / LPR, cl = (lane % LPR) * 4;
                const int64_t grow = row_s + r, gcol = col_w + cl;
                const int nn = grow < p.M ? cols_in(p.N, gcol) : 0;
                const vec4 c = use_c ? load4s<acc_t, 4>(Cb, grow * p.ldc + gcol, false, vec_ok, nn)
                                     : vec4{0, 0, 0, 0};
                const vec4 v = *(const DMP_LDS vec4 *)(slab + r * SP + cl);
                store4s<acc_t, 4>(Db, grow * p.ldc + gcol, finish4(v, c, p.ep), false, vec_ok, nn);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }
}

// Compression: one thread per (batch entry, row, 16 dense k), rows up to Mp.
// Keeps in every group of four k the two entries of largest magnitude (ties to
// the lower k; positions past K, and every position of a padding row, never
// win over present ones) and writes the eight kept values and their 16-bit
// piece of the index stream into the blocked format.  A is row-major.
template <class DT>
__global__ __launch_bounds__(256) void prune24_kernel(const void *A, int64_t M, int64_t Mp, int64_t K,
                                                      int64_t lda, int64_t sA, int64_t batch,
                                                      void *Ac, void *meta, int64_t nkt) {
    constexpr int KT = sparse_kt<DT>();
    const int64_t quads = nkt * (KT / 16);  // 16-k pieces per row
    const int64_t total = batch * Mp * quads;
    for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < total;
         x += (int64_t)gridDim.x * blockDim.x) {
        const int64_t c = x % quads, ri = x / quads;
        const int64_t i = ri % Mp, b = ri / Mp;
        const bool row_in = i < M;
        using E = typename DT::elem;
        const E *row = (const E *)A + b * sA + (row_in ? i : 0) * lda;
        E v[16];
        float mag[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t k = c * 16 + e;
            const bool in = row_in && k < K;
            v[e] = in ? row[k] : (E)0;
            float f;  // exact value of the entry
            if constexpr (std::is_same<DT, F16>::value) f = (float)__builtin_bit_cast(_Float16, (uint16_t)v[e]);
            else if constexpr (std::is_same<DT, BF16>::value) f = __builtin_bit_cast(float, (uint32_t)(uint16_t)v[e] << 16);
            else f = (float)v[e];
            mag[e] = in ? __builtin_fabsf(f) : -1.0f;
        }
        E outv[8];
        uint32_t word = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            int keep[2], nk = 0;
#pragma unroll
            for (int x1 = 0; x1 < 4; ++x1) {
                int beaten = 0;
#pragma unroll
                for (int y = 0; y < 4; ++y) {
                    const float my = mag[4 * u + y], mx = mag[4 * u + x1];
                    beaten += (y != x1) && (my > mx || (my == mx && y < x1));
                }
                if (beaten < 2 && nk < 2) keep[nk++] = x1;
            }
            // the two kept positions in increasing order
            outv[2 * u] = v[4 * u + keep[0]];
            outv[2 * u + 1] = v[4 * u + keep[1]];
            word |= (uint32_t)(keep[0] | (keep[1] << 2)) << (4 * u);
        }
        // block (b, i/16), k-tile t, row i%16, piece q of the k-tile
        const int64_t t = c / (KT / 16), q = c % (KT / 16);
        const int64_t blk = (b * (Mp / 16) + i / 16) * nkt + t;
        E *dst = (E *)Ac + blk * 16 * (KT / 2) + (i % 16) * (KT / 2) + q * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[e] = outv[e];
        ((uint16_t *)meta)[blk * 16 * (KT / 16) + (i % 16) * (KT / 16) + q] = (uint16_t)word;
    }
}

}  // namespace dmp
