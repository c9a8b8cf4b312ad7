"""MI355X (gfx950) dense mixed-precision GEMM:  D = A*B + C.

A thin ctypes binding over the C ABI in ``include/dmp_gemm.h`` (shared library
``libdmp_gemm.so`` built from ``csrc/``).  Every arithmetic step runs in the
library's HIP kernels; this module only marshals pointers, sizes and the
stream.  PyTorch is used for device memory and streams only.

    import torch, dense_mixed_precision_02_amd as dmp
    A = torch.randn(4096, 4096, device="cuda").bfloat16()
    B = torch.randn(4096, 4096, device="cuda").bfloat16().t()   # column-major view
    C = torch.zeros(4096, 4096, device="cuda")
    D = dmp.gemm(A, B, C)           # D = A @ B + C, fp32 accumulate
    E = dmp.gemm(A, B, None, alpha=0.5, out_dtype=torch.bfloat16)   # bf16 result
"""
from __future__ import annotations

from .binding import (GEMM_A_COLMAJOR, GEMM_A_SHARED, GEMM_B_COLMAJOR, GEMM_B_SHARED, GEMM_BF16, GEMM_F16, GEMM_F64, GEMM_I8,
                      GEMM_OUT_BF16, GEMM_OUT_F16, GEMM_OUT_F32, GEMM_OUT_F64, GEMM_OUT_I32,
                      GEMM_ERR_SCRATCH, NOALLOC_SCRATCH_BYTES, GemmError, Handle, Sparse24, default_handle, gemm, gemm_sparse24, lib_path, load_library,
                      prune24, release_default_handles, sparse24_kp, sparse24_mp, plan_label, status_string,
                      EXPORTED_SYMBOLS)

__all__ = ["GEMM_A_COLMAJOR", "GEMM_A_SHARED", "GEMM_B_COLMAJOR", "GEMM_B_SHARED", "GEMM_BF16", "GEMM_F16", "GEMM_F64", "GEMM_I8",
           "GEMM_OUT_BF16", "GEMM_OUT_F16", "GEMM_OUT_F32", "GEMM_OUT_F64", "GEMM_OUT_I32",
           "GEMM_ERR_SCRATCH", "NOALLOC_SCRATCH_BYTES", "GemmError", "Handle", "Sparse24", "default_handle", "gemm", "gemm_sparse24", "lib_path", "load_library",
           "prune24", "release_default_handles", "sparse24_kp", "sparse24_mp", "plan_label",
           "status_string", "EXPORTED_SYMBOLS"]
