// epi.hpp -- parameters of the output stage, shared by the host code and the
// kernels (plain C++: no HIP types).
//
// D = cvt_D(alpha * acc + beta * cvt_C(C)) with every step an fp32
// round-to-nearest-even operation (no fused multiply-add), C decoded exactly
// from its storage type and the final conversion to D's storage type rounding
// to nearest even.  alpha = beta = 1 with fp32 C and D is the plain
// D = acc + C.  The int8 path only has D = acc + C (int32, wrapping) or D = acc.
#pragma once

namespace dmp {

// Storage types of C and D (the values of gemm_out_t in the C header).
enum { OUT_F32 = 0, OUT_F16 = 1, OUT_BF16 = 2, OUT_I32 = 3, OUT_F64 = 4 };

struct EpiParams {
    float alpha, beta;
    int c_type, d_type;
    int use_c;  // beta != 0: C is read
};

}  // namespace dmp
