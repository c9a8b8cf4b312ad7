// tile_gemm.hpp -- the tiled MFMA GEMM kernel for gfx950.
//
// One workgroup owns a BM x BN tile of D (of one batch entry, and one K range
// when split-K is on).  Per 128-byte K panel ("k-tile": 64 fp16/bf16 or 128
// int8 elements) it
//   1. copies the A panel (BM x k-tile) and the B panel (k-tile x BN) from global
//      memory straight into LDS with 16-byte buffer loads that bypass registers
//      (out-of-range granules come back as zero), into the LDS buffer that the
//      MFMAs are not reading (two buffers, alternating);
//   2. reads 16-byte fragments from the other buffer and issues 32x32 MFMAs
//      (the K-panel accumulation of the pages: "CDNA2 dense MFMA builtins",
//      section "Naming convention" -- each instruction adds one K step of an A
//      panel times a B panel to an M x N accumulator tile, the caller loops K).
// After the K loop the epilogue adds C once and writes D (or, under split-K,
// writes the raw partial tile to a workspace).
//
// Operand storage.  Both operands are seen as "R rows x K": A is M x K and B is
// (B^T) N x K.  An operand is K-contiguous (A row-major, B col-major) or
// MN-contiguous (A col-major, B row-major).
//  * K-contiguous panels are stored in LDS as R rows of 128 bytes; the 16-byte
//    granule g of row r sits at slot g ^ swz(r), which makes the fragment reads
//    (32 lanes on 32 consecutive rows, same granule) hit distinct banks.
//  * MN-contiguous panels are stored in 128-byte blocks, each holding 4 k-rows
//    x 16 rows (16-bit types) or 8 k-rows x 16 rows (int8).  A fragment is then
//    read with the gfx950 LDS transpose loads: a group of 16 lanes reads one
//    whole block (128 contiguous bytes) and every lane receives 4 (or 8)
//    consecutive k values of its own row -- the K-contiguous register layout the
//    MFMA needs.
#pragma once
#include <type_traits>

#include "common.hpp"

namespace dmp {

struct TileArgs {
    const void *A, *B, *C;
    void *D, *W;
    int64_t M, N, K, lda, ldb, ldc;
    int64_t sA, sB, sC;      // batch strides in elements
    int64_t k_chunk;         // K elements per split (multiple of the k-tile)
    int tiles_m, tiles_n, batch, splits;
    int partial;             // 1: write raw partials to W (split-K), 0: output stage to D
    EpiParams ep;            // output stage: alpha, beta, C and D storage types
};

// How many of the 4 columns starting at gcol lie inside N columns (0..4).
__device__ static inline int cols_in(int64_t N, int64_t gcol) {
    const int64_t r = N - gcol;
    return r >= 4 ? 4 : (r <= 0 ? 0 : (int)r);
}

// Row swizzle of the K-contiguous LDS layout.  Any 8 consecutive rows (and the
// even/odd rows of any 16) map to distinct 16-byte slots modulo 128 (256) bytes.
__device__ static inline int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// PAD (MN-contiguous operands only): bytes of padding after each row of
// 128-byte blocks (a "block row": 4 k-rows (16-bit) or 8 k-rows (int8) of all
// R rows), so that reads of blocks in consecutive block rows fall on different
// LDS banks; every block row is a whole number of 1 KB copies (R >= 128).
template <class DT, int R, int NW, bool KCONTIG, int PAD = 0>
struct Operand {
    // R rows per tile, NW waves in the workgroup.
    static constexpr int ESZ = DT::ESZ;
    static constexpr int G = DT::G;
    static constexpr int KT = 128 / ESZ;            // k-tile in elements
    static_assert(PAD == 0 || (!KCONTIG && R >= 128 && PAD % 16 == 0), "padding: MN-contiguous, R >= 128");
    static constexpr int ROW_BYTES = R * 8 + PAD;   // one block row (R / 16 blocks) with its padding
    static constexpr int BYTES = R * 128 + 16 * PAD;  // one LDS buffer (16 block rows per k-tile)
    static constexpr int CHUNKS = R * 128 / 1024;   // 1 KB per wave-wide load
    static_assert(CHUNKS % NW == 0, "chunks must split evenly over waves");
    static constexpr int CPW = CHUNKS / NW;         // chunks per wave
    static constexpr int KB = (ESZ == 2) ? 4 : 8;   // k-rows per 128-byte block (MN-contig)
    static_assert((NW * 8) % (R / 16) == 0, "MN-contig chunk stride must be whole block rows");

    // Chunk j of this wave is chunk c = j*NW + wave of the tile.  Successive
    // chunks of one wave differ by a fixed step: 8*NW rows (K-contig) or
    // KB*(8*NW)/(R/16) k-rows (MN-contig), so one offset per lane suffices.
    int off0;      // byte offset of this lane's granule in chunk j = 0
    int row_or_k;  // K-contig: row of chunk 0 (rows step by 8*NW); MN-contig: k of chunk 0
    int fixed;     // K-contig: k offset of the granule; MN-contig: row offset of the granule
    int step;      // byte offset between successive chunks (uniform)

    __device__ void init(int wave, int lane, int64_t ld, int row0, int64_t Rtot) {
        if (KCONTIG) {
            const int r = wave * 8 + (lane >> 3);
            const int g = (lane & 7) ^ swz(r);  // swz(r + 8*NW*j) == swz(r): 8*NW is a multiple of 16
            off0 = (int)(r * ld + g * G) * ESZ;
            row_or_k = row0 + r;
            fixed = g * G;
            step = (int)(8 * NW * ld) * ESZ;
        } else {
            const int bid = wave * 8 + (lane >> 3);
            const int kb = bid / (R / 16), mb = bid % (R / 16);
            int k, mn;
            if (ESZ == 2) {
                k = kb * 4 + ((lane & 7) >> 1);
                mn = mb * 16 + (lane & 1) * 8;
            } else {
                k = kb * 8 + (lane & 7);
                mn = mb * 16;
            }
            off0 = (int)(k * ld + mn) * ESZ;
            row_or_k = k;
            fixed = row0 + mn;
            step = (int)(KSTEP * ld) * ESZ;
        }
        (void)Rtot;
    }
    static constexpr int KSTEP = KB * (8 * NW) / (R / 16);  // MN-contig: k-rows between chunks

    // Issue chunk j of this wave's share of the copy of one k-tile into LDS
    // buffer `lds`.  rs: buffer over element (row0, k0) of the operand.
    // kleft: valid k elements from k0.
    template <int CPOL = 0>
    __device__ void issue(const __amdgpu_buffer_rsrc_t &rs, DMP_LDS char *lds, int wave, int j,
                          int kleft, int64_t Rtot) const {
        const int c = j * NW + wave;
        bool ok;
        if (KCONTIG) ok = (row_or_k + 8 * NW * j < Rtot) && (fixed < kleft);
        else ok = (fixed < Rtot) && (row_or_k + KSTEP * j < kleft);
        load_granule_to_lds<CPOL>(rs, lds + chunk_offset(c), ok ? off0 + j * step : OOB_OFFSET);
    }

    // LDS byte offset of copy chunk c (1 KB; R / 128 chunks per block row).
    __device__ static constexpr int chunk_offset(int c) {
        if constexpr (PAD == 0) return c * 1024;
        else return (c / (R / 128)) * ROW_BYTES + (c % (R / 128)) * 1024;
    }
    // LDS byte offset of 128-byte block (kb, mb) of an MN-contiguous panel.
    __device__ static constexpr int block_offset(int kb, int mb) { return kb * ROW_BYTES + mb * 128; }

    // LDS reads one fragment takes
    static constexpr int READS = KCONTIG ? 1 : 2;

    // 16-byte fragment for MFMA step s (2 granules of K) of rows [rbase, rbase+32):
    // lane L gets row rbase + L%32 and K granule 2s + L/32 of the k-tile.
    __device__ static intx4 frag(const DMP_LDS char *lds, int rbase, int s, int lane) {
        if (KCONTIG) {
            const int row = rbase + (lane & 31);
            const int g = 2 * s + (lane >> 5);
            return *(const DMP_LDS intx4 *)(lds + row * 128 + ((g ^ swz(row)) << 4));
        } else {
            const int grp = lane >> 4, j = lane & 15, h = grp >> 1;
            const int mn = rbase + 16 * (grp & 1);
            intx4 out;
            if (ESZ == 2) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int k = s * 16 + 8 * h + 4 * t;  // multiple of 4: first row of a block
                    const int addr = ((k >> 2) * (R / 16) + (mn >> 4)) * 128 + j * 8;
                    shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (DMP_LDS shortx4 *)(lds + addr));
                    intx2 w = __builtin_bit_cast(intx2, v);
                    out[2 * t] = w[0];
                    out[2 * t + 1] = w[1];
                }
            } else {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int k = s * 32 + 16 * h + 8 * t;  // multiple of 8: first row of a block
                    const int addr = ((k >> 3) * (R / 16) + (mn >> 4)) * 128 + j * 8;
                    intx2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((DMP_LDS intx2 *)(lds + addr));
                    out[2 * t] = w[0];
                    out[2 * t + 1] = w[1];
                }
            }
            return out;
        }
    }

    // Pointer to element (row0, k0) of the operand.
    __device__ static const char *tile_base(const void *X, int64_t ld, int64_t row0, int64_t k0) {
        const char *p = (const char *)X;
        return KCONTIG ? p + (row0 * ld + k0) * ESZ : p + (k0 * ld + row0) * ESZ;
    }
};

// Scheduling hint for one MFMA step: NM MFMAs with ND LDS reads and NV global
// loads spread evenly between them (each read or load sits behind an MFMA).
template <int NM, int ND, int NV, int I = 0>
__device__ static inline void interleave() {
    if constexpr (I < NM) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        constexpr int nd = ND * (I + 1) / NM - ND * I / NM;
        constexpr int nv = NV * (I + 1) / NM - NV * I / NM;
        if constexpr (nd > 0) __builtin_amdgcn_sched_group_barrier(0x100, nd, 0);  // LDS reads
        if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(0x020, nv, 0);  // global loads
        interleave<NM, ND, NV, I + 1>();
    }
}

// The two LDS buffers are distinct arrays so that the compiler can tell that
// copies into one never alias fragment reads from the other.
// ONE: every split holds at most one k-tile (K of a 64x64 batch entry, say).
// Then a single operand buffer suffices and the epilogue's slabs reuse it, so
// the workgroup needs 20 KB of LDS instead of 32 and more of them fit a CU.
template <class DT, int BM, int BN, int WM, int WN, bool AK, bool BKC, bool ONE = false>
__global__ __launch_bounds__(WM *WN * 64) void tile_gemm(const TileArgs p) {
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
    constexpr int TM = WTM / 32, TN = WTN / 32;  // 32x32 MFMA tiles per wave
    constexpr int KT = 128 / DT::ESZ;            // k-tile in elements
    constexpr int STEPS = 4;                     // 32x32 MFMA steps per k-tile
    using OpA = Operand<DT, BM, NW, AK>;
    using OpB = Operand<DT, BN, NW, BKC>;
    using acc_t = typename DT::acc;
    using accv = typename DT::accv;

    constexpr int SLAB_BYTES = 32 * (WTN + 8) * (int)sizeof(acc_t);   // one wave's epilogue slab
    constexpr int ONE_BYTES = OpA::BYTES + OpB::BYTES > NW * SLAB_BYTES ? OpA::BYTES + OpB::BYTES
                                                                        : NW * SLAB_BYTES;
    __shared__ __attribute__((aligned(1024))) char lds_a0[ONE ? ONE_BYTES : OpA::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_b0[OpB::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_a1[OpA::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_b1[OpB::BYTES];

    // ---- which tile: XCD-aware remap, then grouped order ----------------------
    // Workgroup i is dispatched to XCD i % 8.  Renumber so that consecutive tile
    // ids share an XCD (and its L2), then walk tiles in groups of 4 tile-rows.
    int wg = blockIdx.x;
    {
        const int total = gridDim.x, per = total / 8;
        if (wg < per * 8) wg = (wg % 8) * per + wg / 8;
    }
    const int tiles = p.tiles_m * p.tiles_n;
    const int prob = wg / tiles;
    int t = wg - prob * tiles;
    const int split = prob / p.batch, b = prob - split * p.batch;
    constexpr int GM = 4;
    const int group = t / (GM * p.tiles_n);
    const int first_m = group * GM;
    const int gm = min(p.tiles_m - first_m, GM);
    t -= group * GM * p.tiles_n;
    const int tm = first_m + t % gm, tn = t / gm;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int64_t k_begin = (int64_t)split * p.k_chunk;
    const int64_t k_end = min(p.K, k_begin + p.k_chunk);
    const int kspan = k_end > k_begin ? (int)(k_end - k_begin) : 0;  // K < 2^31
    const int nkt = (kspan + KT - 1) / KT;

    const int lane = lane_id(), wave = wave_id();
    const int wm = wave / WN, wn = wave % WN;

    const char *Ab = (const char *)p.A + (int64_t)b * p.sA * DT::ESZ;
    const char *Bb = (const char *)p.B + (int64_t)b * p.sB * DT::ESZ;

    OpA opa;
    OpB opb;
    opa.init(wave, lane, p.lda, (int)m0, p.M);
    opb.init(wave, lane, p.ldb, (int)n0, p.N);

    accv acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = accv{};

    // An odd k-tile count is made even by a leading k-tile that is all zeros
    // (every granule out of range), so the loop below has a single exit.
    const int ntiles = nkt + (nkt & 1);
    const int64_t k_first = k_begin - (int64_t)(nkt & 1) * KT;
    // The copy of one k-tile is NCH wave-wide loads per wave (A chunks, then B
    // chunks), issued in two parts spread over two MFMA steps so that the wave
    // never blocks on a full load queue with MFMAs waiting behind it, and each
    // part still has two steps to land before the next barrier.
    constexpr int NCH = OpA::CPW + OpB::CPW;
    constexpr int P1 = (NCH + 1) / 2, P2 = NCH;
    // 64x64 tiles serve batches of small problems, whose operands no other
    // workgroup reads: their copies are non-temporal.  Larger tiles share
    // panels through L2 and keep the default policy.
    constexpr int CPOL = (BM == 64 && BN == 64) ? CPOL_NT : 0;
    auto stage_part = [&](int kt, DMP_LDS char *la, DMP_LDS char *lb, auto lo_c, auto hi_c) {
        constexpr int LO = decltype(lo_c)::value, HI = decltype(hi_c)::value;
        // k-tiles outside [k_begin, k_end) (the padding tile, and the ones past
        // the end that the loop below still issues) load zeros and touch no memory
        const int64_t k0 = k_first + (int64_t)kt * KT;
        const int koff = (kt - (nkt & 1)) * KT;  // k0 - k_begin
        int kleft = kspan - koff;
        kleft = kleft > KT ? KT : kleft;
        kleft = ((koff < 0) | (kleft < 0)) ? 0 : kleft;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(OpA::tile_base(Ab, p.lda, m0, k0));
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(OpB::tile_base(Bb, p.ldb, n0, k0));
#pragma unroll
        for (int c = LO; c < HI; ++c) {
            if (c < OpA::CPW) opa.template issue<CPOL>(ra, la, wave, c, kleft, p.M);
            else opb.template issue<CPOL>(rb, lb, wave, c - OpA::CPW, kleft, p.N);
        }
    };
    using Z = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, P1>;
    using I2 = std::integral_constant<int, P2>;
    // Fragments for step s of the k-tile held in (la, lb).
    auto read = [&](intx4 (&fa)[TM], intx4 (&fb)[TN], const DMP_LDS char *la,
                    const DMP_LDS char *lb, int s) {
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[i] = OpA::frag(la, wm * WTM + i * 32, s, lane);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[j] = OpB::frag(lb, wn * WTN + j * 32, s, lane);
    };
    auto mma = [&](const intx4 (&fa)[TM], const intx4 (&fb)[TN]) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = DT::mfma(fa[i], fb[j], acc[i][j]);
    };
    constexpr int NMF = TM * TN;                                   // MFMAs per step
    constexpr int NRD = TM * OpA::READS + TN * OpB::READS;        // LDS reads per step

    DMP_LDS char *LA[2], *LB[2];
    if constexpr (ONE) {
        LA[0] = LA[1] = (DMP_LDS char *)lds_a0;
        LB[0] = LB[1] = (DMP_LDS char *)lds_a0 + OpA::BYTES;
    } else {
        LA[0] = (DMP_LDS char *)lds_a0;
        LA[1] = (DMP_LDS char *)lds_a1;
        LB[0] = (DMP_LDS char *)lds_b0;
        LB[1] = (DMP_LDS char *)lds_b1;
    }

    // Software pipeline.  Fragments of step s+1 are read while the MFMAs of step
    // s run.  Before the last step of k-tile kt every wave waits for k-tile kt+1
    // to land and for its own reads of kt to finish; after that barrier the
    // buffer of kt is free: the copy of k-tile kt+2 into it starts in step 3 of
    // kt and finishes in step 0 of kt+1, and step 0 of kt+1 is read from
    // the other buffer while the MFMAs of step 3 of kt run.  Inside each step
    // the LDS reads and loads are interleaved with the MFMAs; to keep each step
    // one branch-free block they are issued even past the last k-tile, where
    // they read nothing (zero-fill) or read a buffer no longer used.
    intx4 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
    auto ktile = [&](int kt, int cur) {
        DMP_LDS char *la = LA[cur], *lb = LB[cur], *na = LA[cur ^ 1], *nb = LB[cur ^ 1];
        // step 0
        read(fa1, fb1, la, lb, 1);
        stage_part(kt + 1, na, nb, I1{}, I2{});
        mma(fa0, fb0);
        interleave<NMF, NRD, P2 - P1>();
        __builtin_amdgcn_sched_barrier(0);
        step_sync();
        // step 1
        read(fa0, fb0, la, lb, 2);
        mma(fa1, fb1);
        interleave<NMF, NRD, 0>();
        __builtin_amdgcn_sched_barrier(0);
        step_sync();
        // step 2
        read(fa1, fb1, la, lb, 3);
        mma(fa0, fb0);
        interleave<NMF, NRD, 0>();
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<0>();
        __syncthreads();
        // step 3
        stage_part(kt + 2, la, lb, Z{}, I1{});
        read(fa0, fb0, na, nb, 0);
        mma(fa1, fb1);
        interleave<NMF, NRD, P1>();
        __builtin_amdgcn_sched_barrier(0);
        step_sync();
    };
    if constexpr (ONE) {
        // nkt is 0 or 1; a single k-tile is k-tile 1 of the padded count
        if (nkt > 0) {
            stage_part(1, LA[0], LB[0], Z{}, I2{});
            wait_vmcnt<0>();
            __syncthreads();
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
                read(fa0, fb0, LA[0], LB[0], s);
                mma(fa0, fb0);
            }
        }
    } else if (nkt > 0) {
        stage_part(0, LA[0], LB[0], Z{}, I2{});
        wait_vmcnt<0>();
        __syncthreads();
        stage_part(1, LA[1], LB[1], Z{}, I1{});
        read(fa0, fb0, LA[0], LB[0], 0);
        // two k-tiles per trip so that each buffer is named statically
        for (int kt = 0; kt < ntiles; kt += 2) {
            ktile(kt, 0);
            ktile(kt + 1, 1);
        }
    }

    // ---- epilogue -----------------------------------------------------------
    // Accumulator register G of lane L in a 32x32 tile holds row
    // 8*(G/4) + 4*(L/32) + G%4 and column L%32: a lane's values are scattered
    // over rows.  Each wave therefore passes its tile through LDS one 32-row
    // slab at a time and leaves it row-major, so that C is read and D written
    // as 16-byte vectors covering whole row segments.
    wait_vmcnt<0>();  // the zero-fill loads issued past the last k-tile have landed
    __syncthreads();  // every wave is done with the operand buffers
    DMP_LDS char *slab_c = ONE ? (DMP_LDS char *)lds_a0 + wave * SLAB_BYTES
                         : wave == 0 ? LA[0] : wave == 1 ? LB[0] : wave == 2 ? LA[1] : LB[1];
    DMP_LDS acc_t *slab = (DMP_LDS acc_t *)slab_c;
    constexpr int SP = WTN + 8;        // padded slab row (elements): rows r and r+4 land 128 B apart mod 256
    static_assert(32 * SP * 4 <= OpA::BYTES && 32 * SP * 4 <= OpB::BYTES, "slab must fit");
    constexpr int LPR = WTN / 4;       // lanes per slab row (4 elements each)
    constexpr int RPP = 64 / LPR;      // slab rows per pass
    constexpr int PASSES = 32 / RPP;
    const int64_t col_w = n0 + wn * WTN;
    // Split-K partials go to W (dense M x N per split and batch entry) unscaled:
    // the output stage with alpha = 1 and no C leaves them unchanged.
    EpiParams ep = p.ep;
    if (p.partial) {
        ep.alpha = 1.0f;
        ep.use_c = 0;
        ep.d_type = OUT_F32;
    }
    const int64_t ldo = p.partial ? p.N : p.ldc;
    const char *Cb = (const char *)p.C + (int64_t)b * p.sC * out_size(ep.c_type);
    char *Ob = p.partial ? (char *)p.W + (((int64_t)split * p.batch + b) * p.M * p.N) * sizeof(acc_t)
                         : (char *)p.D + (int64_t)b * p.sC * out_size(ep.d_type);
    const bool c_f16 = ep.c_type == OUT_F16, d_f16 = ep.d_type == OUT_F16;
    using vec4 = vec4_of<acc_t>;
    // CS, DS: bytes per element of C (0: C not read) and of the output, fixed at
    // compile time so that each variant is a short, fully unrolled loop.
    auto epilogue = [&](auto cs_c, auto ds_c) {
        constexpr int CS = decltype(cs_c)::value, DS = decltype(ds_c)::value;
        // 4-element vector accesses need every row start aligned to 4 elements
        const bool vec_ok = (ldo % 4 == 0) && (CS == 0 || (uintptr_t)Cb % (4 * (CS ? CS : 1)) == 0) &&
                            (uintptr_t)Ob % (4 * DS) == 0;
        const int64_t row_w = m0 + wm * WTM;
        if constexpr (TM > 1) {
            if (vec_ok && row_w + WTM <= p.M && col_w + WTN <= p.N) {
                // Whole wave tile inside the matrix: the C loads of slab i+1 are
                // issued before slab i is transposed and stored, so their latency
                // overlaps that work instead of stalling every slab.
                vec4 cv[2][PASSES];
                auto load_c = [&](int i, vec4 (&dst)[PASSES]) {
#pragma unroll
                    for (int q = 0; q < PASSES; ++q) {
                        dst[q] = vec4{0, 0, 0, 0};
                        if constexpr (CS != 0) {
                            const int64_t grow = row_w + i * 32 + q * RPP + lane / LPR;
                            const int64_t gcol = col_w + (lane % LPR) * 4;
                            dst[q] = load4s<acc_t, CS>(Cb, grow * ldo + gcol, c_f16, true, 4);
                        }
                    }
                };
                load_c(0, cv[0]);
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    if (i + 1 < TM) load_c(i + 1, cv[(i + 1) & 1]);
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int G = 0; G < 16; ++G)
                            slab[(8 * (G >> 2) + 4 * (lane >> 5) + (G & 3)) * SP + j * 32 +
                                 (lane & 31)] = acc[i][j][G];
                    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
                    for (int q = 0; q < PASSES; ++q) {
                        const int r = q * RPP + lane / LPR;
                        const int cl = (lane % LPR) * 4;
                        const vec4 v = *(const DMP_LDS vec4 *)(slab + r * SP + cl);
                        store4s<acc_t, DS>(Ob, (row_w + i * 32 + r) * ldo + col_w + cl,
                                           finish4(v, cv[i & 1][q], ep), d_f16, true, 4);
                    }
                    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                }
                return;
            }
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            // accumulators of rows [i*32, i*32+32) of the wave tile -> LDS, row-major
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int G = 0; G < 16; ++G)
                    slab[(8 * (G >> 2) + 4 * (lane >> 5) + (G & 3)) * SP + j * 32 + (lane & 31)] =
                        acc[i][j][G];
            // LDS instructions of one wave complete in order; this only keeps the
            // compiler from moving the reads above the writes
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            const int64_t row_s = m0 + wm * WTM + i * 32;
            if (vec_ok && row_s + 32 <= p.M && col_w + WTN <= p.N) {
                // whole slab inside the matrix: straight-line vector code, with
                // every C load of the slab issued before the first is used
                vec4 cv[PASSES];
#pragma unroll
                for (int q = 0; q < PASSES; ++q) {
                    cv[q] = vec4{0, 0, 0, 0};
                    if constexpr (CS != 0) {
                        const int64_t grow = row_s + q * RPP + lane / LPR;
                        const int64_t gcol = col_w + (lane % LPR) * 4;
                        cv[q] = load4s<acc_t, CS>(Cb, grow * ldo + gcol, c_f16, true, 4);
                    }
                }
#pragma unroll
                for (int q = 0; q < PASSES; ++q) {
                    const int r = q * RPP + lane / LPR;
                    const int cl = (lane % LPR) * 4;
                    const vec4 v = *(const DMP_LDS vec4 *)(slab + r * SP + cl);
                    const int64_t grow = row_s + r, gcol = col_w + cl;
                    store4s<acc_t, DS>(Ob, grow * ldo + gcol, finish4(v, cv[q], ep), d_f16, true, 4);
                }
            } else {
                // edge slab (or unaligned rows): masked accesses, one pass at a time
#pragma unroll 1
                for (int q = 0; q < PASSES; ++q) {
                    const int r = q * RPP + lane / LPR;
                    const int cl = (lane % LPR) * 4;
                    const int64_t grow = row_s + r, gcol = col_w + cl;
                    const int n = grow < p.M ? cols_in(p.N, gcol) : 0;
                    vec4 c = {0, 0, 0, 0};
                    if constexpr (CS != 0) c = load4s<acc_t, CS>(Cb, grow * ldo + gcol, c_f16, vec_ok, n);
                    const vec4 v = *(const DMP_LDS vec4 *)(slab + r * SP + cl);
                    store4s<acc_t, DS>(Ob, grow * ldo + gcol, finish4(v, c, ep), d_f16, vec_ok, n);
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        }
    };
    using S0 = std::integral_constant<int, 0>;
    using S2 = std::integral_constant<int, 2>;
    using S4 = std::integral_constant<int, 4>;
    if constexpr (is_float_acc<acc_t>) {
        const bool c16 = out_size(ep.c_type) == 2, d16 = out_size(ep.d_type) == 2;
        if (!ep.use_c) {
            if (d16) epilogue(S0{}, S2{});
            else epilogue(S0{}, S4{});
        } else if (c16) {
            if (d16) epilogue(S2{}, S2{});
            else epilogue(S2{}, S4{});
        } else {
            if (d16) epilogue(S4{}, S2{});
            else epilogue(S4{}, S4{});
        }
    } else {
        if (ep.use_c) epilogue(S4{}, S4{});
        else epilogue(S0{}, S4{});
    }
}

}  // namespace dmp
