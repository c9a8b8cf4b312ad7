// aux_kernels.hpp -- the any-alignment MFMA kernel, the split-K reduction and
// the K == 0 copy.
#pragma once
#include "common.hpp"

namespace dmp {

struct GenericArgs {
    const void *A, *B, *C;
    void *D;
    int64_t M, N, K;
    int64_t a_rs, a_ks, b_ks, b_cs;  // element strides: A[i][k] = A[i*a_rs + k*a_ks], B[k][j] = B[k*b_ks + j*b_cs]
    int64_t ldc, sA, sB, sC;
    int tiles_m, tiles_n;
    EpiParams ep;  // output stage: alpha, beta, C and D storage types
};

// Element loads for the any-alignment path (no vector loads, no alignment
// assumption beyond the element's own).
__device__ static inline uint32_t load_elem(const uint16_t *p) { return *p; }
__device__ static inline uint32_t load_elem(const int8_t *p) { return (uint8_t)*p; }

// One wave per 32x32 output tile.  Fragments come straight from global memory
// element by element, so any pointer alignment, leading dimension and K work;
// the MFMA, its fragment layout (lane L: row or column L%32, K elements
// G*(L/32) .. G*(L/32)+G-1 of each step) and the epilogue are those of the
// tiled kernel.  Used when the 16-byte granule path does not apply.
template <class DT>
__global__ __launch_bounds__(64) void generic_gemm(const GenericArgs p) {
    using elem = typename DT::elem;
    using acc_t = typename DT::acc;
    using accv = typename DT::accv;
    constexpr int G = DT::G;
    constexpr int EPW = 4 / DT::ESZ;  // elements per 32-bit word
    const int tiles = p.tiles_m * p.tiles_n;
    const int b = blockIdx.x / tiles;
    const int t = blockIdx.x - b * tiles;
    const int64_t m0 = (int64_t)(t / p.tiles_n) * 32, n0 = (int64_t)(t % p.tiles_n) * 32;
    const int lane = threadIdx.x;
    const elem *A = (const elem *)p.A + b * p.sA;
    const elem *B = (const elem *)p.B + b * p.sB;
    const int64_t row = m0 + (lane & 31), col = n0 + (lane & 31);
    const int kh = (lane >> 5) * G;
    accv acc = accv{};
    for (int64_t k0 = 0; k0 < p.K; k0 += 2 * G) {
        intx4 fa, fb;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t wa = 0, wb = 0;
#pragma unroll
            for (int q = 0; q < EPW; ++q) {
                const int64_t k = k0 + kh + w * EPW + q;
                const uint32_t va = (row < p.M && k < p.K) ? load_elem(A + row * p.a_rs + k * p.a_ks) : 0u;
                const uint32_t vb = (col < p.N && k < p.K) ? load_elem(B + k * p.b_ks + col * p.b_cs) : 0u;
                wa |= va << (q * 8 * DT::ESZ);
                wb |= vb << (q * 8 * DT::ESZ);
            }
            fa[w] = (int)wa;
            fb[w] = (int)wb;
        }
        acc = DT::mfma(fa, fb, acc);
    }
    const char *Cb = (const char *)p.C + b * p.sC * out_size(p.ep.c_type);
    char *Db = (char *)p.D + b * p.sC * out_size(p.ep.d_type);
    typedef acc_t vec4 __attribute__((ext_vector_type(4)));
    const int64_t c = n0 + (lane & 31);
    if (c < p.N) {
#pragma unroll
        for (int G2 = 0; G2 < 16; ++G2) {
            const int64_t r = m0 + 8 * (G2 >> 2) + 4 * (lane >> 5) + (G2 & 3);
            if (r < p.M) {
                const int64_t idx = r * p.ldc + c;
                vec4 a = {acc[G2], 0, 0, 0};
                const vec4 cv = p.ep.use_c ? load4<acc_t>(Cb, idx, p.ep.c_type, false, 1) : vec4{0, 0, 0, 0};
                store4<acc_t>(Db, idx, finish4(a, cv, p.ep), p.ep.d_type, false, 1);
            }
        }
    }
}

// Split-K reduction and output stage: D = out(P_0 + P_1 + ... + P_{S-1}, C),
// the partials summed in that fixed order (so the result is the same on every
// run) and the output stage (alpha, beta, C once, conversion) applied at the
// end.  With S == 0 the sum is zero (K == 0).  W holds S*batch dense M x N
// partial tiles.  VEC: each thread handles 4 consecutive elements of a row with
// vector accesses (N and ldc multiples of 4, aligned C, D and W).
template <class T, bool VEC>
__global__ __launch_bounds__(256) void splitk_reduce(const T *__restrict__ W, const void *C, void *D,
                                                     int64_t M, int64_t N, int64_t ldc, int64_t batch,
                                                     int S, EpiParams ep) {
    typedef T vec __attribute__((ext_vector_type(4)));
    constexpr int V = VEC ? 4 : 1;
    const int64_t MN = M * N;
    const int64_t total = MN * batch;
    const int64_t groups = total / V;
    for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups;
         g += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e = g * V;
        const int64_t b = e / MN, rem = e - b * MN;
        const int64_t i = rem / N, j = rem - i * N;
        const int64_t idx = b * M * ldc + i * ldc + j;
        vec acc = {0, 0, 0, 0};
        if (S > 0) {
            if constexpr (VEC) {
                // each partial is read once: non-temporal
                acc = __builtin_nontemporal_load((const vec *)(W + e));
                for (int q = 1; q < S; ++q) {
                    const vec w = __builtin_nontemporal_load((const vec *)(W + (int64_t)q * total + e));
#pragma unroll
                    for (int t = 0; t < 4; ++t) acc[t] = add_acc(acc[t], w[t]);
                }
            } else {
                acc[0] = W[e];
                for (int q = 1; q < S; ++q) acc[0] = add_acc(acc[0], W[(int64_t)q * total + e]);
            }
        }
        const vec cv = ep.use_c ? load4<T>(C, idx, ep.c_type, VEC, V) : vec{0, 0, 0, 0};
        store4<T>(D, idx, finish4(acc, cv, ep), ep.d_type, VEC, V);
    }
}

// Row-major int8 B (K x N, leading dimension ldb) to column-major form Bt
// (Bt[j*ldt + k] = B[k*ldb + j], ldt a multiple of 16), per batch entry, in
// 128 (k) x 128 (j) tiles through LDS.  Rows come in as 16-byte pieces, eight
// lanes to a 128-byte row; each thread then reads 16 k-rows x 4 columns as 16
// dwords, transposes the 4x4 byte blocks in registers (byte permutes) and
// writes 4 columns x 16 k as 16-byte pieces, eight lanes to a 128-byte column
// segment, so both sides move whole cache lines.  The dword column of LDS row r
// is XOR-ed with 4*((r/16)%8), which puts the 64 lanes of a dword read on
// distinct banks and keeps 16-byte pieces contiguous.  The tiled GEMM reads a
// column-major B with plain 16-byte LDS reads where a row-major one needs twice
// as many transposing reads.
__device__ static inline void transpose4x4_bytes(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3,
                                                 uint32_t &o0, uint32_t &o1, uint32_t &o2,
                                                 uint32_t &o3) {
    // w_r holds bytes (c0 c1 c2 c3) of row r; o_c receives (r0 r1 r2 r3) of column c
    const uint32_t t0 = __builtin_amdgcn_perm(w1, w0, 0x05010400u);  // w0b0 w1b0 w0b1 w1b1
    const uint32_t t1 = __builtin_amdgcn_perm(w3, w2, 0x05010400u);  // w2b0 w3b0 w2b1 w3b1
    const uint32_t t2 = __builtin_amdgcn_perm(w1, w0, 0x07030602u);  // w0b2 w1b2 w0b3 w1b3
    const uint32_t t3 = __builtin_amdgcn_perm(w3, w2, 0x07030602u);  // w2b2 w3b2 w2b3 w3b3
    o0 = __builtin_amdgcn_perm(t1, t0, 0x05040100u);
    o1 = __builtin_amdgcn_perm(t1, t0, 0x07060302u);
    o2 = __builtin_amdgcn_perm(t3, t2, 0x05040100u);
    o3 = __builtin_amdgcn_perm(t3, t2, 0x07060302u);
}

__global__ __launch_bounds__(256) void transpose_i8(const int8_t *B, int64_t K, int64_t N, int64_t ldb,
                                                    int64_t sB, int8_t *Bt, int64_t ldt, int64_t sBt,
                                                    int tiles_k, int tiles_n, int vec_in) {
    __shared__ __attribute__((aligned(16))) uint32_t t[128 * 32];
    const int tiles = tiles_k * tiles_n;
    const int64_t b = blockIdx.x / tiles;
    const int tile = blockIdx.x - (int)(b * tiles);
    const int64_t k0 = (int64_t)(tile / tiles_n) * 128, n0 = (int64_t)(tile % tiles_n) * 128;
    const int tid = threadIdx.x;
    const int8_t *Bb = B + b * sB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int f = i * 256 + tid;  // 16-byte piece f: row f/8, bytes 16*(f%8) ..
        const int r = f >> 3, c = (f & 7) * 16;
        const int8_t *src = Bb + (k0 + r) * ldb + n0 + c;
        uint32_t *d = &t[r * 32 + ((c >> 2) ^ (4 * ((r >> 4) & 7)))];
        if (vec_in && k0 + r < K && n0 + c + 15 < N) {
            *(intx4 *)d = __builtin_nontemporal_load((const intx4 *)src);  // B is read once
        } else {
            uint8_t *db = (uint8_t *)d;
#pragma unroll
            for (int e = 0; e < 16; ++e)
                db[e] = (k0 + r < K && n0 + c + e < N) ? (uint8_t)src[e] : (uint8_t)0;
        }
    }
    __syncthreads();
    // thread: columns 4cg .. 4cg+3, k rows 16kq .. 16kq+15
    const int kq = tid & 7, cg = tid >> 3;
    uint32_t w[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) w[e] = t[(16 * kq + e) * 32 + (cg ^ (4 * kq))];
    uint32_t o[4][4];  // o[column][group of four k]
#pragma unroll
    for (int g = 0; g < 4; ++g)
        transpose4x4_bytes(w[4 * g], w[4 * g + 1], w[4 * g + 2], w[4 * g + 3], o[0][g], o[1][g],
                           o[2][g], o[3][g]);
    int8_t *Btb = Bt + b * sBt;
    const int64_t kb = k0 + 16 * kq;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int64_t j = n0 + 4 * cg + jj;
        if (j >= N) continue;
        int8_t *dst = Btb + j * ldt + kb;
        const intx4 v = {(int)o[jj][0], (int)o[jj][1], (int)o[jj][2], (int)o[jj][3]};
        if (kb + 15 < K) {
            *(intx4 *)dst = v;
        } else {
            const uint8_t *vb = (const uint8_t *)&v;
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (kb + e < K) dst[e] = (int8_t)vb[e];
        }
    }
}

}  // namespace dmp
