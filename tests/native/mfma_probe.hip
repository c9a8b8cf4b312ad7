// Test-only probe of the accumulator layouts of the matrix instructions the
// library's kernels use, on gfx950.  It shares no code with the library.
//
// For every output element (block b, row i, column j) one wave runs the
// instruction once on one-hot inputs: the lanes that supply row i of block b
// of A hold ones in every k slot, the lanes that supply column j of block b of
// B hold ones, every other lane zeros.  The product then has exactly one
// non-zero element, (b, i, j), equal to the number of k the instruction sums;
// the wave writes its whole accumulator (64 lanes x up to 16 registers, as
// double) so the test can see in which lane and register that element landed.
// Input maps (which lane supplies which row or column):
//   32x32 single-block instructions (dense and sparse): row/column L % 32;
//   16x16x4 fp64: row/column L % 16;
//   4x4x4 16-block: row/column L % 4 of block L / 4;
//   16x16x4 4-block: row/column L % 16 of block L / 16.
// The sparse instructions get the index word that keeps positions 0 and 1 of
// every group of four, so half of their k slots count.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int intx16 __attribute__((ext_vector_type(16)));
typedef double doublex4 __attribute__((ext_vector_type(4)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef __bf16 b16 __attribute__((ext_vector_type(16)));

enum { P_F16_32 = 0, P_BF16_32 = 1, P_I8_32 = 2, P_SP_BF16_32 = 3, P_SP_I8_32 = 4,
       P_F64_16 = 5, P_F16_4X4 = 6, P_F16_16X4 = 7, P_BF16_4X4 = 8, P_BF16_16X4 = 9,
       P_I8_4X4 = 10, P_I8_16X4 = 11, P_COUNT = 12 };

typedef __bf16 b4 __attribute__((ext_vector_type(4)));

constexpr int REGS = 16;  // registers written per lane (unused ones are zero)

// 16-bit words of 1.0
constexpr uint32_t F16_ONE2 = 0x3C003C00u, BF16_ONE2 = 0x3F803F80u;
constexpr uint32_t I8_ONE4 = 0x01010101u;

template <class V>
__device__ static void put(double *out, const V &acc, int n) {
    const int c = blockIdx.x, L = threadIdx.x;
    for (int g = 0; g < REGS; ++g) out[((size_t)c * 64 + L) * REGS + g] = g < n ? (double)acc[g] : 0.0;
}

template <int WHICH>
__global__ __launch_bounds__(64) void probe_32(double *out) {
    const int c = blockIdx.x, i = c / 32, j = c % 32, L = threadIdx.x;
    const bool ra = (L % 32) == i, rb = (L % 32) == j;
    if constexpr (WHICH == P_F16_32 || WHICH == P_BF16_32) {
        const uint32_t one = WHICH == P_F16_32 ? F16_ONE2 : BF16_ONE2;
        const intx4 a = ra ? intx4{(int)one, (int)one, (int)one, (int)one} : intx4{0, 0, 0, 0};
        const intx4 b = rb ? intx4{(int)one, (int)one, (int)one, (int)one} : intx4{0, 0, 0, 0};
        floatx16 acc = {};
        if constexpr (WHICH == P_F16_32)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), acc, 0, 0, 0);
        else
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), acc, 0, 0, 0);
        put(out, acc, 16);
    } else if constexpr (WHICH == P_I8_32) {
        const int o = (int)I8_ONE4;
        const intx4 a = ra ? intx4{o, o, o, o} : intx4{0, 0, 0, 0};
        const intx4 b = rb ? intx4{o, o, o, o} : intx4{0, 0, 0, 0};
        intx16 acc = {};
        acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc, 0, 0, 0);
        put(out, acc, 16);
    } else if constexpr (WHICH == P_SP_BF16_32) {
        const int o = (int)BF16_ONE2;
        const intx4 a = ra ? intx4{o, o, o, o} : intx4{0, 0, 0, 0};   // 8 kept values
        const intx8 b = rb ? intx8{o, o, o, o, o, o, o, o} : intx8{0, 0, 0, 0, 0, 0, 0, 0};
        floatx16 acc = {};
        acc = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(__builtin_bit_cast(b8, a), __builtin_bit_cast(b16, b),
                                                        acc, 0x4444, 0, 0);
        put(out, acc, 16);
    } else {  // P_SP_I8_32
        const int o = (int)I8_ONE4;
        const intx4 a = ra ? intx4{o, o, o, o} : intx4{0, 0, 0, 0};   // 16 kept values
        const intx8 b = rb ? intx8{o, o, o, o, o, o, o, o} : intx8{0, 0, 0, 0, 0, 0, 0, 0};
        intx16 acc = {};
        acc = __builtin_amdgcn_smfmac_i32_32x32x64_i8(a, b, acc, 0x44444444, 0, 0);
        put(out, acc, 16);
    }
}

__global__ __launch_bounds__(64) void probe_f64(double *out) {
    const int c = blockIdx.x, i = c / 16, j = c % 16, L = threadIdx.x;
    const double a = (L % 16) == i ? 1.0 : 0.0, b = (L % 16) == j ? 1.0 : 0.0;
    doublex4 acc = {0, 0, 0, 0};
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc, 0, 0, 0);
    put(out, acc, 4);
}

// S x S blocks, 64 / S of them: combo c = (b * S + i) * S + j.  T: 0 fp16,
// 1 bf16 (the _1k instructions), 2 int8; four k per lane in every case.
template <int S, int T>
__global__ __launch_bounds__(64) void probe_multi(double *out) {
    const int c = blockIdx.x, j = c % S, i = (c / S) % S, b = c / (S * S), L = threadIdx.x;
    const uint32_t one2 = T == 0 ? F16_ONE2 : BF16_ONE2;
    const uint64_t ones = ((uint64_t)one2 << 32) | one2;
    const uint64_t a = L == b * S + i ? ones : 0, bb = L == b * S + j ? ones : 0;
    const int a8 = L == b * S + i ? (int)I8_ONE4 : 0, b8v = L == b * S + j ? (int)I8_ONE4 : 0;
    if constexpr (S == 4) {
        if constexpr (T == 2) {
            intx4 acc = {};
            acc = __builtin_amdgcn_mfma_i32_4x4x4i8(a8, b8v, acc, 0, 0, 0);
            put(out, acc, 4);
        } else {
            floatx4 acc = {};
            if constexpr (T == 0)
                acc = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(h4, a), __builtin_bit_cast(h4, bb), acc, 0, 0, 0);
            else
                acc = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(b4, a), __builtin_bit_cast(b4, bb), acc, 0, 0, 0);
            put(out, acc, 4);
        }
    } else {
        if constexpr (T == 2) {
            intx16 acc = {};
            acc = __builtin_amdgcn_mfma_i32_16x16x4i8(a8, b8v, acc, 0, 0, 0);
            put(out, acc, 16);
        } else {
            floatx16 acc = {};
            if constexpr (T == 0)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f16(__builtin_bit_cast(h4, a), __builtin_bit_cast(h4, bb), acc, 0, 0, 0);
            else
                acc = __builtin_amdgcn_mfma_f32_16x16x4bf16_1k(__builtin_bit_cast(b4, a), __builtin_bit_cast(b4, bb), acc, 0, 0, 0);
            put(out, acc, 16);
        }
    }
}

extern "C" {

// Output elements (workgroups) of probe `which`; 0 for an unknown probe.
int mfma_probe_combos(int which) {
    switch (which) {
        case P_F16_32: case P_BF16_32: case P_I8_32: case P_SP_BF16_32: case P_SP_I8_32: return 32 * 32;
        case P_F64_16: return 16 * 16;
        case P_F16_4X4: case P_BF16_4X4: case P_I8_4X4: return 16 * 4 * 4;
        case P_F16_16X4: case P_BF16_16X4: case P_I8_16X4: return 4 * 16 * 16;
        default: return 0;
    }
}

// Run probe `which` on `stream`; out: device buffer of at least
// mfma_probe_combos(which) * 64 * 16 doubles.  Returns 0, 1 (unknown probe)
// or 2 (launch error).
int mfma_probe_run(int which, double *out, void *stream) {
    const int n = mfma_probe_combos(which);
    if (n == 0 || out == nullptr) return 1;
    hipStream_t s = (hipStream_t)stream;
    switch (which) {
        case P_F16_32: hipLaunchKernelGGL(probe_32<P_F16_32>, dim3(n), dim3(64), 0, s, out); break;
        case P_BF16_32: hipLaunchKernelGGL(probe_32<P_BF16_32>, dim3(n), dim3(64), 0, s, out); break;
        case P_I8_32: hipLaunchKernelGGL(probe_32<P_I8_32>, dim3(n), dim3(64), 0, s, out); break;
        case P_SP_BF16_32: hipLaunchKernelGGL(probe_32<P_SP_BF16_32>, dim3(n), dim3(64), 0, s, out); break;
        case P_SP_I8_32: hipLaunchKernelGGL(probe_32<P_SP_I8_32>, dim3(n), dim3(64), 0, s, out); break;
        case P_F64_16: hipLaunchKernelGGL(probe_f64, dim3(n), dim3(64), 0, s, out); break;
        case P_F16_4X4: hipLaunchKernelGGL((probe_multi<4, 0>), dim3(n), dim3(64), 0, s, out); break;
        case P_F16_16X4: hipLaunchKernelGGL((probe_multi<16, 0>), dim3(n), dim3(64), 0, s, out); break;
        case P_BF16_4X4: hipLaunchKernelGGL((probe_multi<4, 1>), dim3(n), dim3(64), 0, s, out); break;
        case P_BF16_16X4: hipLaunchKernelGGL((probe_multi<16, 1>), dim3(n), dim3(64), 0, s, out); break;
        case P_I8_4X4: hipLaunchKernelGGL((probe_multi<4, 2>), dim3(n), dim3(64), 0, s, out); break;
        case P_I8_16X4: hipLaunchKernelGGL((probe_multi<16, 2>), dim3(n), dim3(64), 0, s, out); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
