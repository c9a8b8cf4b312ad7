// common.hpp -- types and small device helpers for the gfx950 GEMM kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "epi.hpp"

namespace dmp {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx2 __attribute__((ext_vector_type(2)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx16 __attribute__((ext_vector_type(16)));
typedef short shortx4 __attribute__((ext_vector_type(4)));

#define DMP_LDS __attribute__((address_space(3)))

// ---------------------------------------------------------------------------
// Input-type traits.  A "granule" is 16 bytes: the unit of every global load,
// every LDS store and every fragment read.  One 32x32 MFMA step consumes two
// granules of K per operand: lanes 0..31 supply the first granule of their row
// (or column), lanes 32..63 the second (pages: "CDNA2 dense MFMA builtins",
// "Fragment loading" -- lane groups supply successive K positions, and the lane
// offset inside a group selects the A row or B column).
//
// The accumulator map of the 32x32 single-block instructions is block 0 of the
// 32x32 layout on the same page ("32x32 layout"): lane L, accumulator
// register G hold row 8*(G/4) + 4*(L/32) + (G%4), column L%32.
// ---------------------------------------------------------------------------
struct F16 {
    using elem = uint16_t;
    using acc = float;
    using accv = floatx16;
    static constexpr int ESZ = 2;
    static constexpr int G = 8;  // elements per granule
    __device__ static inline accv mfma(intx4 a, intx4 b, accv c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                                      __builtin_bit_cast(half8, b), c, 0, 0, 0);
    }
};

struct BF16 {
    using elem = uint16_t;
    using acc = float;
    using accv = floatx16;
    static constexpr int ESZ = 2;
    static constexpr int G = 8;
    __device__ static inline accv mfma(intx4 a, intx4 b, accv c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

struct I8 {
    using elem = int8_t;
    using acc = int32_t;
    using accv = intx16;
    static constexpr int ESZ = 1;
    static constexpr int G = 16;
    __device__ static inline accv mfma(intx4 a, intx4 b, accv c) {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
    }
};

// Raw buffer resource over [base, base + 2^31): loads whose byte offset is
// OOB_OFFSET or more return zero, which is how out-of-range granules of a tile
// are zero-filled without branching.
constexpr int OOB_OFFSET = 0x7ffffff0;

__device__ static inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base) {
    // The descriptor must sit in scalar registers.  base is wave-uniform by
    // construction; reading it from the first lane says so to the compiler,
    // which otherwise may compute it in vector registers and wrap every buffer
    // load in a loop over distinct descriptor values.
    const uint64_t a = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void *u = (void *)(((uint64_t)hi << 32) | lo);
    // dword3 0x00020000: 32-bit data format, the gfx9-family raw-buffer setting
    return __builtin_amdgcn_make_buffer_rsrc(u, (short)0, OOB_OFFSET, 0x00020000);
}

// 16-byte global -> LDS copy that bypasses registers.  The LDS destination of
// lane L is lds + 16*L (lds must be wave-uniform).  CPOL: cache policy bits of
// the load (CPOL_NT: non-temporal, for data that no other workgroup reads).
constexpr int CPOL_NT = 2;
template <int CPOL = 0>
__device__ static inline void load_granule_to_lds(__amdgpu_buffer_rsrc_t r, DMP_LDS void *lds,
                                                  int voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voffset, 0, 0, CPOL);
}

// Wait until at most n vector-memory operations of this wave are outstanding
// (the other counters left at their maxima).
template <int n>
__device__ static inline void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// Workgroup barrier after this wave's LDS reads have completed and at most n of
// its vector-memory operations are outstanding.  Unlike __syncthreads() it does
// not wait for every outstanding global load, so copies for later k-tiles stay in
// flight; the empty asm statements keep the compiler from moving memory
// accesses across it.
template <int n>
__device__ static inline void barrier_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Race check.  A build with DMP_EXTRA_SYNC defined waits for every copy and
// meets every wave at each step of the software pipelines (step_sync() is
// empty otherwise); the arithmetic is unchanged, so its results must equal the
// normal build's bit for bit, whatever the timing of copies and reads.
#ifdef DMP_EXTRA_SYNC
constexpr bool EXTRA_SYNC = true;
#else
constexpr bool EXTRA_SYNC = false;
#endif
__device__ static inline void step_sync() {
    if constexpr (EXTRA_SYNC) {
        wait_vmcnt<0>();
        __syncthreads();
    }
}

// C is added once after the reduction: an fp32 round-to-nearest-even add, or an
// int32 add that wraps modulo 2^32 (done in unsigned arithmetic, where wrapping
// is defined).
__device__ static inline float add_acc(float a, float b) { return a + b; }
__device__ static inline double add_acc(double a, double b) { return a + b; }
__device__ static inline int32_t add_acc(int32_t a, int32_t b) {
    return (int32_t)((uint32_t)a + (uint32_t)b);
}

// ---------------------------------------------------------------------------
// Output stage (parameters and semantics in epi.hpp): loads and stores of C and
// D in their storage types, and the alpha/beta combination.
// ---------------------------------------------------------------------------
__device__ static inline int out_size(int t) {
    return (t == OUT_F16 || t == OUT_BF16) ? 2 : t == OUT_F64 ? 8 : 4;
}

typedef uint16_t ushortx4 __attribute__((ext_vector_type(4)));
template <class T> using vec4_of = T __attribute__((ext_vector_type(4)));
template <class T> constexpr bool is_float_acc = T(0.5) != T(0);

// 16-bit storage: fp16 if f16, else bf16 (both conversions are computed and one
// selected, so a uniform flag costs no branch).  fp32 -> 16 bit rounds to
// nearest even.
__device__ static inline float decode16(uint16_t h, bool f16) {
    const float a = (float)__builtin_bit_cast(_Float16, h);
    const float b = __builtin_bit_cast(float, (uint32_t)h << 16);
    return f16 ? a : b;
}
__device__ static inline uint16_t encode16(float x, bool f16) {
    const uint16_t a = __builtin_bit_cast(uint16_t, (_Float16)x);
    const uint16_t b = __builtin_bit_cast(uint16_t, (__bf16)x);
    return f16 ? a : b;
}

// Four consecutive elements [idx, idx + 4) of one row, SZ bytes each in memory
// (sizeof(T): the accumulator type itself; 2: fp16 / bf16, float accumulators only).
// n of them (0..4) lie inside the matrix; vec: one aligned vector access is allowed.
template <class T, int SZ>
__device__ static inline vec4_of<T> load4s(const void *base, int64_t idx, bool f16, bool vec, int n) {
    vec4_of<T> r = {0, 0, 0, 0};
    if constexpr (SZ == sizeof(T)) {
        const T *q = (const T *)base + idx;
        if (vec && n == 4) return *(const vec4_of<T> *)q;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (e < n) r[e] = q[e];
    } else {
        static_assert(is_float_acc<T>, "16-bit storage needs a float accumulator");
        const uint16_t *q = (const uint16_t *)base + idx;
        if (vec && n == 4) {
            const ushortx4 h = *(const ushortx4 *)q;
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = decode16(h[e], f16);
            return r;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (e < n) r[e] = decode16(q[e], f16);
    }
    return r;
}
// Every store of D (and of split-K partials) is non-temporal.  D is written
// once and not read again by the launch, so it need not compete with the
// operands for the caches.  When a step's operands could stay in the 256 MB
// memory-side cache (repeated products over the same inputs), this keeps them
// there.  Batched 64^3 products alternating between two input sets ran in 62
// instead of 76 us.  With inputs that are cold anyway (three or more sets) it
// changes nothing, and the 8192^3 int8 product gains 1.5 %.  The cost is that
// a consumer reading D right after finds it in HBM, not in the cache.  The
// policy is fixed at compile time: the compiler merges a run-time choice
// between a non-temporal and a plain store into one plain store.
template <class T, int SZ>
__device__ static inline void store4s(void *base, int64_t idx, vec4_of<T> v, bool f16, bool vec, int n) {
    if constexpr (SZ == sizeof(T)) {
        T *q = (T *)base + idx;
        if (vec && n == 4) {
            __builtin_nontemporal_store(v, (vec4_of<T> *)q);
            return;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (e < n) __builtin_nontemporal_store((T)v[e], q + e);
    } else {
        static_assert(is_float_acc<T>, "16-bit storage needs a float accumulator");
        uint16_t *q = (uint16_t *)base + idx;
        ushortx4 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = encode16(v[e], f16);
        if (vec && n == 4) {
            __builtin_nontemporal_store(h, (ushortx4 *)q);
            return;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (e < n) __builtin_nontemporal_store((uint16_t)h[e], q + e);
    }
}

// The same with the storage type t (OUT_*) known only at run time.
template <class T>
__device__ static inline vec4_of<T> load4(const void *base, int64_t idx, int t, bool vec, int n) {
    if constexpr (sizeof(T) == 4 && is_float_acc<T>) {
        if (t != OUT_F32) return load4s<T, 2>(base, idx, t == OUT_F16, vec, n);
    }
    return load4s<T, sizeof(T)>(base, idx, false, vec, n);
}
template <class T>
__device__ static inline void store4(void *base, int64_t idx, vec4_of<T> v, int t, bool vec, int n) {
    if constexpr (sizeof(T) == 4 && is_float_acc<T>) {
        if (t != OUT_F32) return store4s<T, 2>(base, idx, v, t == OUT_F16, vec, n);
    }
    store4s<T, sizeof(T)>(base, idx, v, false, vec, n);
}

// alpha * acc + beta * c, each product and the sum rounded separately.
__device__ static inline floatx4 finish4(floatx4 acc, floatx4 c, const EpiParams &ep) {
#pragma clang fp contract(off)
    floatx4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float t = ep.alpha * acc[e];
        r[e] = ep.use_c ? t + ep.beta * c[e] : t;
    }
    return r;
}
// fp64: only alpha = 1 and beta in {0, 1} reach here, so this is acc (+ c).
__device__ static inline vec4_of<double> finish4(vec4_of<double> acc, vec4_of<double> c,
                                                 const EpiParams &ep) {
#pragma clang fp contract(off)
    vec4_of<double> r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const double t = (double)ep.alpha * acc[e];
        r[e] = ep.use_c ? t + (double)ep.beta * c[e] : t;
    }
    return r;
}
__device__ static inline intx4 finish4(intx4 acc, intx4 c, const EpiParams &ep) {
    intx4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = ep.use_c ? add_acc(acc[e], c[e]) : acc[e];
    return r;
}

__device__ static inline int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ static inline int lane_id() { return threadIdx.x & 63; }

}  // namespace dmp
