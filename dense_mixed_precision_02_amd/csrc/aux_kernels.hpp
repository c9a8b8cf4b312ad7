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
                acc = *(const vec *)(W + e);
                for (int q = 1; q < S; ++q) {
                    const vec w = *(const vec *)(W + (int64_t)q * total + e);
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
// 64 x 64 tiles through LDS: 16-byte row pieces in, 16-byte column pieces out.
// The tiled GEMM reads a column-major B with plain 16-byte LDS reads where a
// row-major one needs twice as many transposing reads.
__global__ __launch_bounds__(256) void transpose_i8(const int8_t *B, int64_t K, int64_t N, int64_t ldb,
                                                    int64_t sB, int8_t *Bt, int64_t ldt, int64_t sBt,
                                                    int tiles_k, int tiles_n, int vec_in) {
    __shared__ __attribute__((aligned(16))) uint8_t t[64][80];
    const int tiles = tiles_k * tiles_n;
    const int64_t b = blockIdx.x / tiles;
    const int tile = blockIdx.x - (int)(b * tiles);
    const int64_t k0 = (int64_t)(tile / tiles_n) * 64, n0 = (int64_t)(tile % tiles_n) * 64;
    const int r = threadIdx.x >> 2, c0 = (threadIdx.x & 3) * 16;
    const int8_t *src = B + b * sB + (k0 + r) * ldb + n0 + c0;
    if (vec_in && k0 + r < K && n0 + c0 + 15 < N) {
        *(intx4 *)&t[r][c0] = *(const intx4 *)src;
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e)
            t[r][c0 + e] = (k0 + r < K && n0 + c0 + e < N) ? (uint8_t)src[e] : (uint8_t)0;
    }
    __syncthreads();
    const int j = threadIdx.x >> 2, kk = (threadIdx.x & 3) * 16;
    if (n0 + j >= N) return;
    int8_t *dst = Bt + b * sBt + (n0 + j) * ldt + k0 + kk;
    intx4 v;
    uint8_t *vb = (uint8_t *)&v;
#pragma unroll
    for (int e = 0; e < 16; ++e) vb[e] = t[kk + e][j];
    if (k0 + kk + 15 < K) {
        *(intx4 *)dst = v;
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e)
            if (k0 + kk + e < K) dst[e] = (int8_t)vb[e];
    }
}

}  // namespace dmp
