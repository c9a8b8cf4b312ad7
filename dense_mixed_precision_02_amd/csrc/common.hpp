// common.hpp -- types and small device helpers for the gfx950 GEMM kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

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
    // dword3 0x00020000: 32-bit data format, the gfx9-family raw-buffer setting
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, OOB_OFFSET,
                                             0x00020000);
}

// 16-byte global -> LDS copy that bypasses registers.  The LDS destination of
// lane L is lds + 16*L (lds must be wave-uniform).
__device__ static inline void load_granule_to_lds(__amdgpu_buffer_rsrc_t r, DMP_LDS void *lds,
                                                  int voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voffset, 0, 0, 0);
}

// Wait until at most n vector-memory operations of this wave are outstanding
// (the other counters left at their maxima).
template <int n>
__device__ static inline void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// C is added once after the reduction: an fp32 round-to-nearest-even add, or an
// int32 add that wraps modulo 2^32 (done in unsigned arithmetic, where wrapping
// is defined).
__device__ static inline float add_acc(float a, float b) { return a + b; }
__device__ static inline int32_t add_acc(int32_t a, int32_t b) {
    return (int32_t)((uint32_t)a + (uint32_t)b);
}

__device__ static inline int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ static inline int lane_id() { return threadIdx.x & 63; }

}  // namespace dmp
