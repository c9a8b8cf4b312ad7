// Test-only probes of the practical ceilings of gfx950 that the GEMM kernels
// are measured against.  They share no code with the library.
//
//  * Matrix-instruction rate.  Every wave of a one-workgroup-per-CU grid runs
//    a loop of independent matrix instructions of one kind (enough
//    accumulators that no instruction waits for another's result), with
//    operands held in registers and alternated between two sets so that the
//    inputs keep changing.  Nothing else runs, so the launch's rate is the
//    instruction's sustained rate on this part: issue rate times whatever
//    clock the part holds under that load.  Each wave also records the
//    shader clock counter and the constant-rate real-time counter at its start
//    and end, which gives the clock the part ran at.
//  * Load bandwidth from the L2: every workgroup sweeps a buffer small enough
//    to stay in each XCD's L2, with 16-byte loads into registers, or with the
//    16-byte buffer loads that write LDS directly (the GEMM kernels' copies).
//  * LDS read bandwidth: 16-byte LDS reads in a loop.
//  * HBM: streaming reads (non-temporal), streaming writes, and a copy, over
//    buffers far larger than the memory-side cache.
//
// Pages: "CDNA2 dense MFMA builtins", section "Instruction throughput" gives a
// matrix instruction's peak as operations / cycles x clock; these probes
// measure what the clock and the memory system allow on this part.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int intx16 __attribute__((ext_vector_type(16)));
typedef double doublex4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef __bf16 b16 __attribute__((ext_vector_type(16)));

enum {
    R_BF16_32X32X16 = 0, R_F16_32X32X16 = 1, R_BF16_16X16X32 = 2, R_F16_16X16X32 = 3,
    R_I8_32X32X32 = 4, R_I8_16X16X64 = 5, R_F64_16X16X4 = 6, R_SP_BF16_32X32X32 = 7,
    R_SP_I8_32X32X64 = 8, R_COUNT = 9
};

// Operations one instruction performs (2 per multiply-add; the sparse ones
// counted at their dense-equivalent work, twice their stored A).
extern "C" long long ceil_ops_per_inst(int which) {
    switch (which) {
        case R_BF16_32X32X16: case R_F16_32X32X16: return 2LL * 32 * 32 * 16;
        case R_BF16_16X16X32: case R_F16_16X16X32: return 2LL * 16 * 16 * 32;
        case R_I8_32X32X32: return 2LL * 32 * 32 * 32;
        case R_I8_16X16X64: return 2LL * 16 * 16 * 64;
        case R_F64_16X16X4: return 2LL * 16 * 16 * 4;
        case R_SP_BF16_32X32X32: return 2LL * 32 * 32 * 32;
        case R_SP_I8_32X32X64: return 2LL * 32 * 32 * 64;
        default: return 0;
    }
}

// Independent accumulators per wave, and instructions per loop trip.
constexpr int NACC = 8;

// Per-wave clock record: shader-clock counter and real-time counter at the
// wave's start and end.
struct ClockRec {
    unsigned long long t0, t1, r0, r1;
};

__device__ static inline void rec_start(ClockRec &c) {
    c.r0 = __builtin_amdgcn_s_memrealtime();
    c.t0 = __builtin_amdgcn_s_memtime();
}
__device__ static inline void rec_end(ClockRec &c, ClockRec *out) {
    c.t1 = __builtin_amdgcn_s_memtime();
    c.r1 = __builtin_amdgcn_s_memrealtime();
    if ((threadIdx.x & 63) == 0) out[blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64] = c;
}

// Keeps the compiler from treating v as known (no code is emitted).
template <class T>
__device__ static inline void opaque(T &v) {
    asm volatile("" : "+v"(v));
}

template <int W>
__global__ __launch_bounds__(256) void mfma_rate(const intx4 *in, float *sink, int iters,
                                                 ClockRec *clk) {
    const int lane = threadIdx.x & 63;
    // two operand sets per lane from the (random) input buffer
    intx4 a0 = in[lane], a1 = in[64 + lane], b0 = in[128 + lane], b1 = in[192 + lane];
    ClockRec c;
    rec_start(c);
    float s = 0.0f;
    if constexpr (W == R_BF16_32X32X16 || W == R_F16_32X32X16 || W == R_I8_32X32X32 ||
                  W == R_SP_BF16_32X32X32 || W == R_SP_I8_32X32X64) {
        using acc_t = typename std::conditional<W == R_I8_32X32X32 || W == R_SP_I8_32X32X64,
                                                intx16, floatx16>::type;
        acc_t acc[NACC / 2];
#pragma unroll
        for (int i = 0; i < NACC / 2; ++i) acc[i] = acc_t{};
        intx8 b0w = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        intx8 b1w = {b1[0], b1[1], b1[2], b1[3], b0[0], b0[1], b0[2], b0[3]};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < NACC / 2; ++i) {
                const intx4 a = (i & 1) ? a1 : a0;
                const intx4 b = (i & 2) ? b1 : b0;
                if constexpr (W == R_BF16_32X32X16)
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), acc[i], 0, 0, 0);
                else if constexpr (W == R_F16_32X32X16)
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        __builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), acc[i], 0, 0, 0);
                else if constexpr (W == R_I8_32X32X32)
                    acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[i], 0, 0, 0);
                else if constexpr (W == R_SP_BF16_32X32X32)
                    acc[i] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(
                        __builtin_bit_cast(b8, a), __builtin_bit_cast(b16, (i & 2) ? b1w : b0w),
                        acc[i], 0x4444, 0, 0);
                else
                    acc[i] = __builtin_amdgcn_smfmac_i32_32x32x64_i8(a, (i & 2) ? b1w : b0w, acc[i],
                                                                     0x44444444, 0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < NACC / 2; ++i)
#pragma unroll
            for (int g = 0; g < 16; ++g) s += (float)acc[i][g];
    } else if constexpr (W == R_F64_16X16X4) {
        double a0d = (double)a0[0] * 1e-9, a1d = (double)a1[0] * 1e-9;
        double b0d = (double)b0[0] * 1e-9, b1d = (double)b1[0] * 1e-9;
        doublex4 acc[NACC];
#pragma unroll
        for (int i = 0; i < NACC; ++i) acc[i] = doublex4{0, 0, 0, 0};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < NACC; ++i)
                acc[i] = __builtin_amdgcn_mfma_f64_16x16x4f64((i & 1) ? a1d : a0d,
                                                              (i & 2) ? b1d : b0d, acc[i], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NACC; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) s += (float)acc[i][g];
    } else {
        using acc_t = typename std::conditional<W == R_I8_16X16X64, intx4, floatx4>::type;
        acc_t acc[NACC];
#pragma unroll
        for (int i = 0; i < NACC; ++i) acc[i] = acc_t{};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < NACC; ++i) {
                const intx4 a = (i & 1) ? a1 : a0;
                const intx4 b = (i & 2) ? b1 : b0;
                if constexpr (W == R_BF16_16X16X32)
                    acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), acc[i], 0, 0, 0);
                else if constexpr (W == R_F16_16X16X32)
                    acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        __builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), acc[i], 0, 0, 0);
                else
                    acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[i], 0, 0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < NACC; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) s += (float)acc[i][g];
    }
    rec_end(c, clk);
    sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Instructions of the measured kind that one wave issues per loop trip.
extern "C" int ceil_insts_per_trip(int which) {
    switch (which) {
        case R_BF16_32X32X16: case R_F16_32X32X16: case R_I8_32X32X32:
        case R_SP_BF16_32X32X32: case R_SP_I8_32X32X64: return NACC / 2;
        case R_BF16_16X16X32: case R_F16_16X16X32: case R_I8_16X16X64: case R_F64_16X16X4:
            return NACC;
        default: return 0;
    }
}

// ---------------------------------------------------------------------------
// Bandwidth probes.  buf: `bytes` of device memory (a multiple of 16 KB);
// every workgroup of 256 lanes sweeps it `passes` times, starting at an
// offset that depends on its id so that workgroups do not move in lockstep.
// ---------------------------------------------------------------------------

// Plain 16-byte loads into registers.
__global__ __launch_bounds__(256) void read_regs(const intx4 *buf, long long n16, int passes,
                                                 intx4 *sink) {
    intx4 x = {0, 0, 0, 0};
    const long long chunk = 256 * 4;  // 16-byte elements per workgroup step (4 per lane)
    const long long steps = n16 / chunk;
    for (int p = 0; p < passes; ++p) {
        for (long long s = 0; s < steps; ++s) {
            const long long base = ((s + blockIdx.x * 7) % steps) * chunk + threadIdx.x;
            const intx4 *q = buf + base;
            opaque(q);
            const intx4 v0 = q[0], v1 = q[256], v2 = q[512], v3 = q[768];
            x ^= v0 ^ v1 ^ v2 ^ v3;
        }
    }
    if ((x[0] ^ x[1] ^ x[2] ^ x[3]) == 0x13572468) sink[blockIdx.x * 256 + threadIdx.x] = x;
}

// 16-byte buffer loads that write LDS directly (no registers), four waves
// each filling its own 4 KB of LDS per step; the LDS contents are not used.
__global__ __launch_bounds__(256) void read_lds_direct(const char *buf, long long bytes, int passes,
                                                       intx4 *sink) {
    __shared__ __attribute__((aligned(1024))) char lds[4 * 4096];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long long chunk = 256 * 16 * 4;  // bytes per workgroup step
    const long long steps = bytes / chunk;
    // The descriptor's base must sit in scalar registers: both halves of the
    // (wave-uniform) address are read from the first lane.  The builtin returns
    // a signed int, so each half is taken back to uint32_t before widening; a
    // sign-extended low half would set the top bits of the base whenever bit 31
    // of the address is set.
    const uint64_t a = (uint64_t)buf;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void *base = (void *)(((uint64_t)hi << 32) | lo);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff),
                                          0x00020000);
    for (int p = 0; p < passes; ++p) {
        for (long long s = 0; s < steps; ++s) {
            // wave w, part q: the 1 KB at step + 4096 q + 1024 w (lane L: 16 bytes at +16 L)
            const int off = (int)(((s + blockIdx.x * 7) % steps) * chunk) + wave * 1024 + lane * 16;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (__attribute__((address_space(3))) void *)(lds + wave * 4096 + q * 1024), 16,
                    off + q * 4096, 0, 0, 0);
            // at most 16 copies of this wave in flight (vmcnt <= 12 before the next 4)
            __builtin_amdgcn_s_waitcnt(12 | (0x7 << 4) | (0xf << 8));
        }
        __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();
    const intx4 v = *(const intx4 *)(lds + threadIdx.x * 16);
    if ((v[0] ^ v[1]) == 0x13572468) sink[blockIdx.x * 256 + threadIdx.x] = v;
}

// 16-byte LDS reads: each lane reads its own 16 bytes of a 64 KB region, 16
// reads per trip spread over the region.
__global__ __launch_bounds__(256) void lds_read(int iters, intx4 *sink) {
    __shared__ __attribute__((aligned(1024))) intx4 lds[4096];
    for (int i = threadIdx.x; i < 4096; i += 256) lds[i] = intx4{i, i + 1, i + 2, i + 3};
    __syncthreads();
    intx4 x = {0, 0, 0, 0};
    int idx = threadIdx.x;
    for (int it = 0; it < iters; ++it) {
        opaque(idx);
#pragma unroll
        for (int q = 0; q < 16; ++q) x ^= lds[(idx + q * 256) & 4095];
    }
    if ((x[0] ^ x[1] ^ x[2] ^ x[3]) == 0x13572468) sink[blockIdx.x * 256 + threadIdx.x] = x;
}

// HBM streams over n16 16-byte elements, grid-stride: 0 read (non-temporal),
// 1 write (non-temporal), 2 copy.
template <int MODE>
__global__ __launch_bounds__(256) void hbm_stream(const intx4 *src, intx4 *dst, long long n16,
                                                  intx4 *sink) {
    intx4 x = {0, 0, 0, 0};
    const long long stride = (long long)gridDim.x * 256;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
        if constexpr (MODE == 0) x ^= __builtin_nontemporal_load(src + i);
        else if constexpr (MODE == 1) __builtin_nontemporal_store(intx4{(int)i, 1, 2, 3}, dst + i);
        else __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
    }
    if (MODE == 0 && (x[0] ^ x[1] ^ x[2] ^ x[3]) == 0x13572468) sink[threadIdx.x] = x;
}

extern "C" {

// Matrix-instruction rate probe `which` (R_*): grid workgroups of 256 lanes.
// in: 256 intx4 (random operand bits); sink: grid*256 floats; clk: grid*4
// ClockRec.  Returns 0, 1 (bad arguments) or 2 (launch error).
int ceil_mfma(int which, int grid, int iters, const void *in, void *sink, void *clk, void *stream) {
    if (which < 0 || which >= R_COUNT || grid <= 0 || iters <= 0 || !in || !sink || !clk) return 1;
    hipStream_t s = (hipStream_t)stream;
    const dim3 g(grid), b(256);
    const intx4 *pi = (const intx4 *)in;
    float *ps = (float *)sink;
    ClockRec *pc = (ClockRec *)clk;
    switch (which) {
        case R_BF16_32X32X16: hipLaunchKernelGGL(mfma_rate<R_BF16_32X32X16>, g, b, 0, s, pi, ps, iters, pc); break;
        case R_F16_32X32X16: hipLaunchKernelGGL(mfma_rate<R_F16_32X32X16>, g, b, 0, s, pi, ps, iters, pc); break;
        case R_BF16_16X16X32: hipLaunchKernelGGL(mfma_rate<R_BF16_16X16X32>, g, b, 0, s, pi, ps, iters, pc); break;
        case R_F16_16X16X32: hipLaunchKernelGGL(mfma_rate<R_F16_16X16X32>, g, b, 0, s, pi, ps, iters, pc); break;
        case R_I8_32X32X32: hipLaunchKernelGGL(mfma_rate<R_I8_32X32X32>, g, b, 0, s, pi, ps, iters, pc); break;
        case R_I8_16X16X64: hipLaunchKernelGGL(mfma_rate<R_I8_16X16X64>, g, b, 0, s, pi, ps, iters, pc); break;
        case R_F64_16X16X4: hipLaunchKernelGGL(mfma_rate<R_F64_16X16X4>, g, b, 0, s, pi, ps, iters, pc); break;
        case R_SP_BF16_32X32X32: hipLaunchKernelGGL(mfma_rate<R_SP_BF16_32X32X32>, g, b, 0, s, pi, ps, iters, pc); break;
        case R_SP_I8_32X32X64: hipLaunchKernelGGL(mfma_rate<R_SP_I8_32X32X64>, g, b, 0, s, pi, ps, iters, pc); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Load-bandwidth probe: kind 0 registers, 1 direct-to-LDS; bytes a multiple
// of 16 KB and below 2^31; sink: grid*256 intx4.
int ceil_read(int kind, int grid, const void *buf, long long bytes, int passes, void *sink,
              void *stream) {
    if (grid <= 0 || passes <= 0 || !buf || !sink || bytes < 16384 || bytes % 16384 ||
        bytes >= 0x7fffffffLL)
        return 1;
    hipStream_t s = (hipStream_t)stream;
    if (kind == 0)
        hipLaunchKernelGGL(read_regs, dim3(grid), dim3(256), 0, s, (const intx4 *)buf, bytes / 16,
                           passes, (intx4 *)sink);
    else if (kind == 1)
        hipLaunchKernelGGL(read_lds_direct, dim3(grid), dim3(256), 0, s, (const char *)buf, bytes,
                           passes, (intx4 *)sink);
    else
        return 1;
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// LDS-read probe: each of grid workgroups does iters * 16 reads of 16 bytes
// per lane; sink: grid*256 intx4.
int ceil_lds(int grid, int iters, void *sink, void *stream) {
    if (grid <= 0 || iters <= 0 || !sink) return 1;
    hipLaunchKernelGGL(lds_read, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters, (intx4 *)sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// HBM stream probe: mode 0 read src, 1 write dst, 2 copy src -> dst; n16
// 16-byte elements; sink: 256 intx4.
int ceil_hbm(int mode, int grid, const void *src, void *dst, long long n16, void *sink,
             void *stream) {
    if (grid <= 0 || n16 <= 0 || !sink || (mode != 1 && !src) || (mode != 0 && !dst)) return 1;
    hipStream_t s = (hipStream_t)stream;
    const dim3 g(grid), b(256);
    if (mode == 0)
        hipLaunchKernelGGL(hbm_stream<0>, g, b, 0, s, (const intx4 *)src, (intx4 *)dst, n16, (intx4 *)sink);
    else if (mode == 1)
        hipLaunchKernelGGL(hbm_stream<1>, g, b, 0, s, (const intx4 *)src, (intx4 *)dst, n16, (intx4 *)sink);
    else if (mode == 2)
        hipLaunchKernelGGL(hbm_stream<2>, g, b, 0, s, (const intx4 *)src, (intx4 *)dst, n16, (intx4 *)sink);
    else
        return 1;
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
