// tile16_gemm.hpp -- the 256x256 tile on the 16x16 matrix instructions
// (v_mfma_f32_16x16x32_{f16,bf16}, v_mfma_i32_16x16x64_i8).
//
// Same tile, staging and epilogue plan as tile_gemm (tile_gemm.hpp): four
// waves, each owning a 128x128 quarter of a 256x256 tile of D; per 128-byte
// k-tile the A and B panels go from global memory straight into one of two LDS
// buffers, and the waves read 16-byte fragments from the other.  What differs
// is the instruction.  A 16x16 instruction covers twice the K of a 32x32 one
// in half the time on a quarter of the outputs, so a wave tile is 8 x 8 of them
// and a k-tile is two steps of 64 instructions.  On this part a loop of the
// 16x16 instructions alone sustains a markedly higher rate than one of the
// 32x32 instructions (the probe library in tests/native measures both), the
// clock holding higher under the smaller instruction.
//
// The K-panel accumulation is the pages' ("CDNA2 dense MFMA builtins",
// section "Naming convention": each instruction adds one K step of an A panel
// times a B panel to an M x N accumulator tile; the caller loops over K).
// Operand maps of the 16x16 single-block instructions: lane L supplies row (A)
// or column (B) L % 16 and the K slice (L / 16) of the step, 8 consecutive
// 16-bit values or 16 int8 values (one 16-byte granule); the accumulator map
// is block 0 of the page's 16 x 16 layout ("Accumulator layout"): lane L,
// register G hold row 4 * (L / 16) + G, column L % 16.
//
// The instructions are written as inline assembly with the accumulator tied as
// an input-output operand in the accumulation registers.  With the compiler's
// builtins the register allocator of this toolchain moves the 64 four-register
// accumulators around on every loop trip (hundreds of register copies next to
// 128 instructions); tied operands keep each in place.  The compiler does not
// see these statements as matrix instructions, so the two dependences it would
// otherwise resolve are resolved here: the accumulators are written (zeroed)
// well before the first instruction reads them, and after the last one the
// wave idles long enough for every result to land before the epilogue reads
// them (mma_drain).  Waits for the fragments are still inserted by the
// compiler, which tracks the registers an assembly statement reads.  Volatile
// statements also keep their order relative to the memory operations around
// them, which is how the loop body below interleaves fragment reads and copies
// with the instructions: in the order written.
#pragma once
#include "tile_gemm.hpp"

namespace dmp {

template <class DT> struct Mma16;
template <> struct Mma16<F16> {
    __device__ static inline void run(floatx4 &c, const intx4 &a, const intx4 &b) {
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    }
};
template <> struct Mma16<BF16> {
    __device__ static inline void run(floatx4 &c, const intx4 &a, const intx4 &b) {
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    }
};
template <> struct Mma16<I8> {
    __device__ static inline void run(intx4 &c, const intx4 &a, const intx4 &b) {
        asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    }
};

// Idle long enough for the last matrix instructions' results to be written
// back (a 16x16 instruction takes 16 cycles; 96 wait states cover several in
// flight with margin).
__device__ static inline void mma_drain() {
    asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::);
}

// 16-byte fragment of MFMA step s (0 or 1) for rows [rbase, rbase + 16): lane L
// gets row rbase + L % 16 and granule 2 (L / 16) + s of the 8-granule k-tile.
// Which granules a step takes is free as long as A and B agree (each step sums
// over its four granules, and the two steps over all eight); this order puts
// the four 16-lane groups of one read on granules two apart, which keeps the
// reads free of LDS bank conflicts (granules 4 s + L / 16 gave conflicts on
// about half of the LDS cycles).
template <class DT, class Op, int R, bool KCONTIG>
__device__ static inline intx4 frag16(const DMP_LDS char *lds, int rbase, int s, int lane) {
    if constexpr (KCONTIG) {
        const int row = rbase + (lane & 15);
        const int g = 2 * (lane >> 4) + s;
        return *(const DMP_LDS intx4 *)(lds + row * 128 + ((g ^ swz(row)) << 4));
    } else {
        // MN-contiguous panels: 128-byte blocks of 4 k-rows (16-bit) or 8 k-rows
        // (int8) x 16 rows; a group of 16 lanes reads one block with a
        // transposing read and each lane receives 4 (8) consecutive k of its row.
        const int grp = lane >> 4, j = lane & 15;
        intx4 out;
        if constexpr (DT::ESZ == 2) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int kb = 2 * (2 * grp + s) + t;  // granule 2 grp + s: blocks 2 g, 2 g + 1
                const int addr = Op::block_offset(kb, rbase >> 4) + j * 8;
                shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DMP_LDS shortx4 *)(lds + addr));
                intx2 w = __builtin_bit_cast(intx2, v);
                out[2 * t] = w[0];
                out[2 * t + 1] = w[1];
            }
        } else {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int kb = 2 * (2 * grp + s) + t;  // granule 2 grp + s: blocks 2 g, 2 g + 1
                const int addr = Op::block_offset(kb, rbase >> 4) + j * 8;
                intx2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((DMP_LDS intx2 *)(lds + addr));
                out[2 * t] = w[0];
                out[2 * t + 1] = w[1];
            }
        }
        return out;
    }
}

template <class DT, bool AK, bool BKC>
__global__ __launch_bounds__(256) void tile16_gemm(const TileArgs p) {
    constexpr int BM = 256, BN = 256, WM = 2, WN = 2, NW = 4;
    constexpr int WTM = BM / WM, WTN = BN / WN;  // 128 x 128 wave tile
    constexpr int TM = WTM / 16, TN = WTN / 16;  // 8 x 8 instructions per step
    constexpr int KT = 128 / DT::ESZ;            // k-tile in elements
    // An MN-contiguous panel is read four blocks at a time (one per 16-lane
    // group), from block rows four apart.  The LDS serves the groups in pairs
    // (0 with 1, 2 with 3), and a pair is free of bank conflicts when its two
    // 128-byte blocks fill the two halves of the 256 bytes of banks: 32 bytes
    // of padding per block row (2080-byte rows, four of them 128 bytes past a
    // multiple of 256) does that (16 bytes of padding, which puts the four 64
    // bytes apart, left 31 % of the LDS cycles in bank conflicts).
    using OpA = Operand<DT, BM, NW, AK, AK ? 0 : 32>;
    using OpB = Operand<DT, BN, NW, BKC, BKC ? 0 : 32>;
    using acc_t = typename DT::acc;
    using acc4 = vec4_of<acc_t>;
    static_assert(OpA::CPW + OpB::CPW == 16, "16 copies per wave per k-tile");

    __shared__ __attribute__((aligned(1024))) char lds_a0[OpA::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_b0[OpB::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_a1[OpA::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_b1[OpB::BYTES];

    // ---- which tile: XCD-aware remap, then grouped order (as tile_gemm) -------
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
    const int kspan = k_end > k_begin ? (int)(k_end - k_begin) : 0;
    const int nkt = (kspan + KT - 1) / KT;

    const int lane = lane_id(), wave = wave_id();
    const int wm = wave / WN, wn = wave % WN;
    const char *Ab = (const char *)p.A + (int64_t)b * p.sA * DT::ESZ;
    const char *Bb = (const char *)p.B + (int64_t)b * p.sB * DT::ESZ;

    OpA opa;
    OpB opb;
    opa.init(wave, lane, p.lda, (int)m0, p.M);
    opb.init(wave, lane, p.ldb, (int)n0, p.N);

    acc4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = acc4{0, 0, 0, 0};
    // An empty statement that claims to change every accumulator: reads of an
    // accumulator cannot move above it, nor its writes below it.  Used, with
    // idle cycles, where a matrix instruction hands registers to other code.
    auto pin_acc = [&]() {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) asm volatile("" : "+a"(acc[i][j]));
    };

    // k-tile kt (0 .. nkt-1, plus zero-filled ones past the end that the loop
    // still issues) of this split into LDS buffer (la, lb): copy c of this wave
    // (0..15: A chunks, then B chunks).
    auto copy = [&](int kt, DMP_LDS char *la, DMP_LDS char *lb, int c) {
        const int64_t k0 = k_begin + (int64_t)kt * KT;
        int kleft = kspan - kt * KT;
        kleft = kleft > KT ? KT : (kleft < 0 ? 0 : kleft);
        if (c < OpA::CPW) {
            const __amdgpu_buffer_rsrc_t ra = make_rsrc(OpA::tile_base(Ab, p.lda, m0, k0));
            opa.issue(ra, la, wave, c, kleft, p.M);
        } else {
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(OpB::tile_base(Bb, p.ldb, n0, k0));
            opb.issue(rb, lb, wave, c - OpA::CPW, kleft, p.N);
        }
    };
    // fragments of step s of the k-tile in (la, lb): A block i, B block j
    auto fragA = [&](const DMP_LDS char *la, int i, int s) {
        return frag16<DT, OpA, BM, AK>(la, wm * WTM + i * 16, s, lane);
    };
    auto fragB = [&](const DMP_LDS char *lb, int j, int s) {
        return frag16<DT, OpB, BN, BKC>(lb, wn * WTN + j * 16, s, lane);
    };

    DMP_LDS char *LA[2] = {(DMP_LDS char *)lds_a0, (DMP_LDS char *)lds_a1};
    DMP_LDS char *LB[2] = {(DMP_LDS char *)lds_b0, (DMP_LDS char *)lds_b1};

    // Fragment sets.  A K-contiguous operand's fragments of the next step are
    // read while the current step runs, into the other of two sets.  An
    // MN-contiguous operand's are read with the transposing LDS reads, which
    // the compiler cannot tell apart from the buffer that copies in flight are
    // writing: each such read would first wait for every copy.  So they are
    // read only where no copy is in flight -- both steps of the next k-tile,
    // right after the barrier and before the copies of the step are issued --
    // into a pair of sets per LDS buffer (four sets).
    constexpr int NSA = AK ? 2 : 4, NSB = BKC ? 2 : 4;
    intx4 fa[NSA][TM], fb[NSB][TN];
    // set holding step s of a k-tile in buffer `buf`
    auto seta = [](int buf, int s) { return AK ? s : 2 * buf + s; };
    auto setb = [](int buf, int s) { return BKC ? s : 2 * buf + s; };
    // both steps' fragments of the MN-contiguous operands of the k-tile in buffer buf
    auto read_mn = [&](int buf) {
        if constexpr (!AK) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int i = 0; i < TM; ++i) fa[seta(buf, s2)][i] = fragA(LA[buf], i, s2);
        }
        if constexpr (!BKC) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int j = 0; j < TN; ++j) fb[setb(buf, s2)][j] = fragB(LB[buf], j, s2);
        }
    };
    // Per k-tile kt in buffer cur (the next one in the other buffer, nxt):
    //   step 0: 64 instructions on the step-0 fragments; between them the
    //           K-contiguous fragments of step 1 (from cur) are read;
    //   wait for this wave's copies (k-tile kt+1) and meet every wave: kt+1 is
    //           in nxt, and no wave reads cur any more;
    //   step 1: the MN-contiguous fragments of both steps of kt+1 are read from
    //           nxt; then 64 instructions on the step-1 fragments, between them
    //           the K-contiguous fragments of step 0 of kt+1 are read from nxt and
    //           the 16 copies of k-tile kt+2 into cur are issued.
    // So each copy has about two steps to land before the wait that needs it.
    auto ktile = [&](int kt, int cur) {
        DMP_LDS char *la = LA[cur], *lb = LB[cur];
        DMP_LDS char *na = LA[cur ^ 1], *nb = LB[cur ^ 1];
        // step 0
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                Mma16<DT>::run(acc[i][j], fa[seta(cur, 0)][i], fb[setb(cur, 0)][j]);
                if ((j & 3) == 3) {  // two fragment reads per row of 8 instructions
                    const int r = 2 * i + (j >> 2);
                    if (r < TM) {
                        if constexpr (AK) fa[seta(cur, 1)][r] = fragA(la, r, 1);
                    } else {
                        if constexpr (BKC) fb[setb(cur, 1)][r - TM] = fragB(lb, r - TM, 1);
                    }
                }
            }
        }
        wait_vmcnt<0>();
        __syncthreads();
        // step 1
        read_mn(cur ^ 1);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                Mma16<DT>::run(acc[i][j], fa[seta(cur, 1)][i], fb[setb(cur, 1)][j]);
                if ((j & 3) == 1) copy(kt + 2, la, lb, 2 * i + (j >> 2));
                if ((j & 3) == 3) {
                    const int r = 2 * i + (j >> 2);
                    if (r < TM) {
                        if constexpr (AK) fa[seta(cur ^ 1, 0)][r] = fragA(na, r, 0);
                    } else {
                        if constexpr (BKC) fb[setb(cur ^ 1, 0)][r - TM] = fragB(nb, r - TM, 0);
                    }
                }
            }
        }
        step_sync();
    };

    if (nkt > 0) {
        // prologue: k-tile 0 -> buffer 0 (waited for), its step-0 fragments (both
        // steps for MN-contiguous operands) read, then k-tile 1 -> buffer 1
#pragma unroll
        for (int c = 0; c < 16; ++c) copy(0, LA[0], LB[0], c);
        wait_vmcnt<0>();
        __syncthreads();
        read_mn(0);
        if constexpr (AK) {
#pragma unroll
            for (int i = 0; i < TM; ++i) fa[seta(0, 0)][i] = fragA(LA[0], i, 0);
        }
        if constexpr (BKC) {
#pragma unroll
            for (int j = 0; j < TN; ++j) fb[setb(0, 0)][j] = fragB(LB[0], j, 0);
        }
#pragma unroll
        for (int c = 0; c < 16; ++c) copy(1, LA[1], LB[1], c);
        // the zeroed accumulators are written well before the first instruction reads them
        pin_acc();
        asm volatile("s_nop 7" ::);
        // two k-tiles per trip so that each buffer is named statically; an odd
        // count runs one zero-filled k-tile more (its copies read nothing)
        for (int kt = 0; kt < nkt; kt += 2) {
            ktile(kt, 0);
            ktile(kt + 1, 1);
        }
        mma_drain();
        pin_acc();
    }

    // ---- epilogue (as tile_gemm's, with the 16x16 accumulator map) -------------
    wait_vmcnt<0>();  // the zero-fill copies issued past the last k-tile have landed
    __syncthreads();  // every wave is done with the operand buffers
    DMP_LDS char *slab_c = wave == 0 ? LA[0] : wave == 1 ? LB[0] : wave == 2 ? LA[1] : LB[1];
    DMP_LDS acc_t *slab = (DMP_LDS acc_t *)slab_c;
    constexpr int SP = WTN + 4;  // padded slab row (elements): rows 4 apart fall 16 banks apart
    static_assert(32 * SP * 4 <= OpA::BYTES && 32 * SP * 4 <= OpB::BYTES, "slab must fit");
    constexpr int LPR = WTN / 4;   // lanes per slab row (4 elements each)
    constexpr int RPP = 64 / LPR;  // slab rows per pass
    constexpr int PASSES = 32 / RPP;
    const int64_t col_w = n0 + wn * WTN;
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
    // slab q (rows 32 q .. 32 q + 31 of the wave tile) = instruction rows 2q, 2q+1
    auto to_slab = [&](int q) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int G = 0; G < 4; ++G)
                    slab[(16 * h + 4 * (lane >> 4) + G) * SP + j * 16 + (lane & 15)] =
                        acc[2 * q + h][j][G];
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    };
    auto epilogue = [&](auto cs_c, auto ds_c) {
        constexpr int CS = decltype(cs_c)::value, DS = decltype(ds_c)::value;
        const bool vec_ok = (ldo % 4 == 0) && (CS == 0 || (uintptr_t)Cb % (4 * (CS ? CS : 1)) == 0) &&
                            (uintptr_t)Ob % (4 * DS) == 0;
        const int64_t row_w = m0 + wm * WTM;
        if (vec_ok && row_w + WTM <= p.M && col_w + WTN <= p.N) {
            // whole wave tile inside the matrix: the C loads of slab q+1 are
            // issued before slab q is transposed and stored
            vec4 cv[2][PASSES];
            auto load_c = [&](int q, vec4 (&dst)[PASSES]) {
#pragma unroll
                for (int u = 0; u < PASSES; ++u) {
                    dst[u] = vec4{0, 0, 0, 0};
                    if constexpr (CS != 0) {
                        const int64_t grow = row_w + q * 32 + u * RPP + lane / LPR;
                        const int64_t gcol = col_w + (lane % LPR) * 4;
                        dst[u] = load4s<acc_t, CS>(Cb, grow * ldo + gcol, c_f16, true, 4);
                    }
                }
            };
            load_c(0, cv[0]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (q + 1 < 4) load_c(q + 1, cv[(q + 1) & 1]);
                to_slab(q);
#pragma unroll
                for (int u = 0; u < PASSES; ++u) {
                    const int r = u * RPP + lane / LPR;
                    const int cl = (lane % LPR) * 4;
                    const vec4 v = *(const DMP_LDS vec4 *)(slab + r * SP + cl);
                    store4s<acc_t, DS>(Ob, (row_w + q * 32 + r) * ldo + col_w + cl,
                                       finish4(v, cv[q & 1][u], ep), d_f16, true, 4);
                }
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            }
            return;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            to_slab(q);
            const int64_t row_s = row_w + q * 32;
            // edge slab (or unaligned rows): masked accesses, one pass at a time
#pragma unroll 1
            for (int u = 0; u < PASSES; ++u) {
                const int r = u * RPP + lane / LPR;
                const int cl = (lane % LPR) * 4;
                const int64_t grow = row_s + r, gcol = col_w + cl;
                const int n = grow < p.M ? cols_in(p.N, gcol) : 0;
                vec4 c = {0, 0, 0, 0};
                if constexpr (CS != 0) c = load4s<acc_t, CS>(Cb, grow * ldo + gcol, c_f16, vec_ok, n);
                const vec4 v = *(const DMP_LDS vec4 *)(slab + r * SP + cl);
                store4s<acc_t, DS>(Ob, grow * ldo + gcol, finish4(v, c, ep), d_f16, vec_ok, n);
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
