"""ctypes binding of libdmp_gemm.so (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libdmp_gemm.so"

GEMM_F16, GEMM_BF16, GEMM_I8 = 0, 1, 2
GEMM_A_COLMAJOR, GEMM_B_COLMAJOR = 1, 2
GEMM_OK = 0

EXPORTED_SYMBOLS = ("gemm_create", "gemm_run", "gemm_destroy", "gemm_status_string", "gemm_plan")

_lib = None
_lock = threading.Lock()


class GemmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


def lib_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def load_library():
    """Load the built library.  Raises if it is missing: there is no fallback path."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build() "
                               "(or python -m dense_mixed_precision_02_amd.build)")
        lib = ctypes.CDLL(path)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.gemm_create.restype = ctypes.c_int
        lib.gemm_create.argtypes = [ctypes.POINTER(vp)]
        lib.gemm_destroy.restype = ctypes.c_int
        lib.gemm_destroy.argtypes = [vp]
        lib.gemm_status_string.restype = ctypes.c_char_p
        lib.gemm_status_string.argtypes = [ctypes.c_int]
        lib.gemm_run.restype = ctypes.c_int
        lib.gemm_run.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                 ctypes.c_int, ctypes.c_uint, i64, vp]
        lib.gemm_plan.restype = ctypes.c_int
        lib.gemm_plan.argtypes = [vp, i64, i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_uint,
                                  i64, ctypes.c_char_p, ctypes.c_size_t]
        _lib = lib
        return lib


def status_string(status: int) -> str:
    return load_library().gemm_status_string(int(status)).decode()


def plan_label(M, N, K, lda, ldb, ldc, dtype, flags=0, batch=1, handle=None) -> str:
    """Which kernel path gemm_run takes for these sizes (no launch; handle optional)."""
    lib = load_library()
    buf = ctypes.create_string_buffer(256)
    h = handle.ptr if handle is not None else None
    rc = lib.gemm_plan(h, M, N, K, lda, ldb, ldc, dtype, flags, batch, buf, 256)
    if rc != GEMM_OK:
        raise GemmError(rc, "gemm_plan")
    return buf.value.decode()


class Handle:
    """Owns one gemm_handle_t (bound to the HIP device current at creation)."""

    def __init__(self):
        lib = load_library()
        p = ctypes.c_void_p()
        rc = lib.gemm_create(ctypes.byref(p))
        if rc != GEMM_OK:
            raise GemmError(rc, "gemm_create")
        self.ptr = p

    def close(self):
        if self.ptr:
            rc = load_library().gemm_destroy(self.ptr)
            self.ptr = None
            if rc != GEMM_OK:
                raise GemmError(rc, "gemm_destroy")

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def run(self, A: int, B: int, C: int, D: int, M: int, N: int, K: int, lda: int, ldb: int,
            ldc: int, dtype: int, flags: int = 0, batch: int = 1, stream: int = 0) -> None:
        """Raw-pointer call of gemm_run (device addresses as ints, stream as hipStream_t int)."""
        rc = load_library().gemm_run(self.ptr, A, B, C, D, M, N, K, lda, ldb, ldc, dtype, flags,
                                     batch, stream)
        if rc != GEMM_OK:
            raise GemmError(rc, "gemm_run")

    def status(self, A, B, C, D, M, N, K, lda, ldb, ldc, dtype, flags=0, batch=1, stream=0) -> int:
        """Like run() but returns the status code instead of raising."""
        return load_library().gemm_run(self.ptr, A, B, C, D, M, N, K, lda, ldb, ldc, dtype, flags,
                                       batch, stream)


_default = {}


def default_handle() -> Handle:
    import torch
    dev = torch.cuda.current_device()
    h = _default.get(dev)
    if h is None:
        h = Handle()
        _default[dev] = h
    return h


def _operand_layout(X, rows: int, cols: int, name: str):
    """(col_major, ld) of a logical rows x cols matrix view (last two dims)."""
    s_r, s_c = X.stride(-2), X.stride(-1)
    if s_c == 1 and (s_r >= max(1, cols) or rows == 1):
        return False, max(s_r, cols, 1)
    if s_r == 1 and (s_c >= max(1, rows) or cols == 1):
        return True, max(s_c, rows, 1)
    raise ValueError(f"{name} must be row-major or column-major in its last two dims")


def gemm(A, B, C, out=None, handle: Handle | None = None):
    """D = A @ B + C on the current stream.

    A: (..., M, K) float16 / bfloat16 / int8;  B: (..., K, N) same dtype (row-major, or a
    transposed view = column-major);  C: (..., M, N) float32 (int32 for int8), row-major.
    Leading batch dims (one at most) must be contiguous in the library's sense.  Returns D
    (a new tensor unless ``out`` is given; ``out`` may be C itself)."""
    import torch
    dt = {torch.float16: GEMM_F16, torch.bfloat16: GEMM_BF16, torch.int8: GEMM_I8}.get(A.dtype)
    if dt is None or B.dtype != A.dtype:
        raise TypeError("A and B must both be float16, bfloat16 or int8")
    acc = torch.int32 if dt == GEMM_I8 else torch.float32
    if C.dtype != acc:
        raise TypeError(f"C must be {acc}")
    if not (A.is_cuda and B.is_cuda and C.is_cuda):
        raise ValueError("tensors must be on the GPU")
    if A.dim() != B.dim() or A.dim() != C.dim() or A.dim() not in (2, 3):
        raise ValueError("A, B, C must all be 2-D or all 3-D")
    M, K = A.shape[-2], A.shape[-1]
    N = B.shape[-1]
    if B.shape[-2] != K or C.shape[-2] != M or C.shape[-1] != N:
        raise ValueError("shape mismatch")
    batch = A.shape[0] if A.dim() == 3 else 1
    a_col, lda = _operand_layout(A, M, K, "A")
    b_col, ldb = _operand_layout(B, K, N, "B")
    if C.stride(-1) != 1:
        raise ValueError("C must be row-major")
    ldc = max(C.stride(-2), N, 1)
    if out is None:
        out = torch.empty_strided(C.shape, C.stride(), dtype=acc, device=C.device)
    if out.stride() != C.stride() or out.dtype != acc:
        raise ValueError("out must have C's strides and dtype")
    if batch > 1:
        want_a = (K if a_col else M) * lda
        want_b = (N if b_col else K) * ldb
        if A.stride(0) != want_a or B.stride(0) != want_b or C.stride(0) != M * ldc:
            raise ValueError("batched operands must have contiguous batch strides")
    flags = (GEMM_A_COLMAJOR if a_col else 0) | (GEMM_B_COLMAJOR if b_col else 0)
    h = handle if handle is not None else default_handle()
    stream = torch.cuda.current_stream(A.device).cuda_stream
    h.run(A.data_ptr(), B.data_ptr(), C.data_ptr(), out.data_ptr(), M, N, K, lda, ldb, ldc, dt,
          flags, batch, stream)
    return out
