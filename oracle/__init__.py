"""CPU oracle for D = A*B + C -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The GPU library never imports it and shares no code with it; the
only thing both sides consume is the seeded input generator in ``synth``.

The arithmetic lives in ``oracle_gemm.c`` (a plain fp64/int64 triple loop that
evaluates the definition D = x(C) + sum_k x(A) x(B) with exact decoding x of
every stored element; pages: "CDNA2 dense MFMA builtins", section "Naming
convention" -- the product is the sum over all K panels of the per-step
contributions -- and "RDNA3 dense WMMA builtins", builtin reference, where a
step returns srcA x srcB + srcC).  This module only marshals numpy arrays into
it, and states the float tolerance the GPU result is held to.

Storage conventions (shared with the GPU library's ABI, restated here):
  * fp16 / bf16 inputs are passed as uint16 bit patterns, fp32 C as float32,
    int8 inputs as int8 and int32 C as int32;
  * A row-major: A[i, k] = A_mem[i*lda + k];  col-major: A_mem[i + k*lda];
  * B row-major: B[k, j] = B_mem[k*ldb + j];  col-major: B_mem[k + j*ldb];
  * C row-major with ldc;  batch b is offset by a stride per operand.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_gemm.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPES = {"f16": 0, "bf16": 1, "i8": 2}

_lib = None


def build() -> str:
    """Compile the oracle with the host C compiler (always rebuilds)."""
    tmp = _LIB_PATH + ".tmp"
    # no contraction of a*b+c into fma: the fp64 path's error-free transformations
    # rely on every + and * rounding exactly once
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-shared", "-fPIC", "-pthread",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64 = ctypes.c_int64
    vp = ctypes.c_void_p
    lib.oracle_decode_f16.restype = ctypes.c_double
    lib.oracle_decode_f16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_bf16.restype = ctypes.c_double
    lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_f32.restype = ctypes.c_double
    lib.oracle_decode_f32.argtypes = [ctypes.c_uint32]
    lib.oracle_gemm_float.restype = ctypes.c_int
    lib.oracle_gemm_float.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp,
                                      i64, i64, i64, i64, i64, i64,
                                      ctypes.c_int, ctypes.c_int, i64, i64, i64, i64, ctypes.c_int]
    lib.oracle_gemm_int8.restype = ctypes.c_int
    lib.oracle_gemm_int8.argtypes = [vp, vp, vp, vp,
                                     i64, i64, i64, i64, i64, i64,
                                     ctypes.c_int, ctypes.c_int, i64, i64, i64, i64, ctypes.c_int]
    lib.oracle_gemm_points.restype = ctypes.c_int
    lib.oracle_gemm_points.argtypes = [ctypes.c_int, vp, vp, vp, vp, i64, vp, vp, vp,
                                       i64, i64, i64, i64, i64, i64,
                                       ctypes.c_int, ctypes.c_int, i64, i64, i64, i64]
    f64p = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int,
            i64, i64, i64, i64, ctypes.c_int]
    lib.oracle_gemm_f64.restype = ctypes.c_int
    lib.oracle_gemm_f64.argtypes = f64p
    lib.oracle_gemm_f64_points.restype = ctypes.c_int
    lib.oracle_gemm_f64_points.argtypes = [vp, vp, vp, vp, i64, vp, vp, vp, i64, i64, i64, i64,
                                           i64, i64, ctypes.c_int, ctypes.c_int, i64, i64, i64, i64]
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check_storage(dtype: str, A, B, C):
    if dtype in ("f16", "bf16"):
        assert A.dtype == np.uint16 and B.dtype == np.uint16, "16-bit inputs are uint16 bit patterns"
        assert C.dtype == np.float32
    elif dtype == "i8":
        assert A.dtype == np.int8 and B.dtype == np.int8 and C.dtype == np.int32
    else:
        raise ValueError(dtype)
    for x in (A, B, C):
        assert x.flags["C_CONTIGUOUS"]


def decode(dtype: str, bits: np.ndarray) -> np.ndarray:
    """Exact decode of fp16 / bf16 bit patterns (uint16) to float64, element by element."""
    lib = _load()
    fn = lib.oracle_decode_f16 if dtype == "f16" else lib.oracle_decode_bf16
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    out = np.empty(flat.shape, dtype=np.float64)
    for n, h in enumerate(flat.tolist()):
        out[n] = fn(h)
    return out.reshape(np.shape(bits))


def decode_f32(words: np.ndarray) -> np.ndarray:
    lib = _load()
    flat = np.asarray(words, dtype=np.uint32).ravel()
    out = np.array([lib.oracle_decode_f32(w) for w in flat.tolist()], dtype=np.float64)
    return out.reshape(np.shape(words))


def gemm(dtype: str, A: np.ndarray, B: np.ndarray, C: np.ndarray, M: int, N: int, K: int,
         lda: int, ldb: int, ldc: int, a_col: bool = False, b_col: bool = False, batch: int = 1,
         sa: int | None = None, sb: int | None = None, sc: int | None = None,
         nthreads: int | None = None):
    """Full reference.  Returns (D_ref, S) for float types (float64, shape (batch, M, N)),
    or D_ref (int64, shape (batch, M, N)) for int8.  Batch strides default to contiguous."""
    _check_storage(dtype, A, B, C)
    lib = _load()
    sa = (K * lda if a_col else M * lda) if sa is None else sa
    sb = (N * ldb if b_col else K * ldb) if sb is None else sb
    sc = M * ldc if sc is None else sc
    nthreads = default_threads() if nthreads is None else nthreads
    if dtype == "i8":
        D = np.zeros((batch, M, N), dtype=np.int64)
        rc = lib.oracle_gemm_int8(_ptr(A), _ptr(B), _ptr(C), _ptr(D), M, N, K, lda, ldb, ldc,
                                  int(a_col), int(b_col), batch, sa, sb, sc, nthreads)
        if rc:
            raise ValueError("oracle_gemm_int8 rejected its arguments")
        return D
    D = np.zeros((batch, M, N), dtype=np.float64)
    S = np.zeros((batch, M, N), dtype=np.float64)
    rc = lib.oracle_gemm_float(DTYPES[dtype], _ptr(A), _ptr(B), _ptr(C.view(np.uint32)),
                               _ptr(D), _ptr(S), M, N, K, lda, ldb, ldc,
                               int(a_col), int(b_col), batch, sa, sb, sc, nthreads)
    if rc:
        raise ValueError("oracle_gemm_float rejected its arguments")
    return D, S


def gemm_points(dtype: str, A, B, C, pts: np.ndarray, M: int, N: int, K: int,
                lda: int, ldb: int, ldc: int, a_col: bool = False, b_col: bool = False,
                batch: int = 1, sa: int | None = None, sb: int | None = None, sc: int | None = None):
    """Reference values at the listed (b, i, j) positions only.
    Returns (D, S) float64 vectors for float types, or an int64 vector for int8."""
    _check_storage(dtype, A, B, C)
    lib = _load()
    pts = np.ascontiguousarray(pts, dtype=np.int64).reshape(-1, 3)
    n = pts.shape[0]
    sa = (K * lda if a_col else M * lda) if sa is None else sa
    sb = (N * ldb if b_col else K * ldb) if sb is None else sb
    sc = M * ldc if sc is None else sc
    D = np.zeros(n, dtype=np.float64)
    S = np.zeros(n, dtype=np.float64)
    Di = np.zeros(n, dtype=np.int64)
    rc = lib.oracle_gemm_points(DTYPES[dtype], _ptr(A), _ptr(B), _ptr(C), _ptr(pts), n,
                                _ptr(D), _ptr(S), _ptr(Di), M, N, K, lda, ldb, ldc,
                                int(a_col), int(b_col), batch, sa, sb, sc)
    if rc:
        raise ValueError("oracle_gemm_points rejected its arguments")
    return Di if dtype == "i8" else (D, S)


def prune24(dtype: str, A: np.ndarray, M: int, K: int, lda: int, batch: int = 1,
            return_keep: bool = False):
    """2:4 structured pruning of a row-major A (the form the sparse matrix
    instructions consume; pages: "MFMA common parameters", sparse parameter idx:
    two of every four consecutive K positions hold the non-zeros).  In every
    group of four consecutive k of a row (the last group may be shorter) the two
    entries of largest magnitude are kept -- on a tie the lower k -- and the
    others set to zero.  Returns a copy of A's storage with the dropped entries
    replaced by +0; kept entries keep their exact bit patterns.  return_keep also
    returns the (batch, M, K) mask of kept positions."""
    out = np.array(A, copy=True)
    if dtype in ("f16", "bf16"):
        table = decode(dtype, np.arange(65536, dtype=np.uint32).astype(np.uint16))
        mag = np.abs(table[np.asarray(A, dtype=np.uint16)])
    else:
        mag = np.abs(np.asarray(A, dtype=np.float64))
    mag = mag.reshape(A.shape)[:batch, :M, :K]
    Kp = (K + 3) // 4 * 4
    # absent positions of a short last group never beat anything
    m = np.full((batch, M, Kp), -1.0)
    m[:, :, :K] = mag
    g = m.reshape(batch, M, Kp // 4, 4)
    # entry x is beaten by y (same group) if |y| > |x|, or |y| == |x| and y comes first
    beaten = np.zeros(g.shape, dtype=np.int64)
    for x in range(4):
        for y in range(4):
            if y == x:
                continue
            beats = (g[..., y] > g[..., x]) | ((g[..., y] == g[..., x]) & (y < x))
            beaten[..., x] += beats
    keep = (beaten < 2).reshape(batch, M, Kp)[:, :, :K]
    region = out[:batch, :M, :K]
    region[~keep] = 0
    return (out, keep) if return_keep else out


def _f64_args(A, B, C):
    for x in (A, B, C):
        assert x.dtype == np.float64 and x.flags["C_CONTIGUOUS"], "fp64 operands are float64"


def gemm_f64(A, B, C, M: int, N: int, K: int, lda: int, ldb: int, ldc: int, a_col: bool = False,
             b_col: bool = False, batch: int = 1, sa: int | None = None, sb: int | None = None,
             sc: int | None = None, nthreads: int | None = None):
    """fp64 reference: returns (D_hi, D_lo, S), each float64 (batch, M, N); D_ref = D_hi + D_lo
    to about 106 significant bits (double-double accumulation)."""
    _f64_args(A, B, C)
    lib = _load()
    sa = (K * lda if a_col else M * lda) if sa is None else sa
    sb = (N * ldb if b_col else K * ldb) if sb is None else sb
    sc = M * ldc if sc is None else sc
    nthreads = default_threads() if nthreads is None else nthreads
    Dh = np.zeros((batch, M, N))
    Dl = np.zeros((batch, M, N))
    S = np.zeros((batch, M, N))
    rc = lib.oracle_gemm_f64(_ptr(A), _ptr(B), _ptr(C), _ptr(Dh), _ptr(Dl), _ptr(S), M, N, K,
                             lda, ldb, ldc, int(a_col), int(b_col), batch, sa, sb, sc, nthreads)
    if rc:
        raise ValueError("oracle_gemm_f64 rejected its arguments")
    return Dh, Dl, S


def gemm_f64_points(A, B, C, pts, M: int, N: int, K: int, lda: int, ldb: int, ldc: int,
                    a_col: bool = False, b_col: bool = False, batch: int = 1,
                    sa: int | None = None, sb: int | None = None, sc: int | None = None):
    """fp64 reference at the listed (b, i, j) positions: (D_hi, D_lo, S) vectors."""
    _f64_args(A, B, C)
    lib = _load()
    pts = np.ascontiguousarray(pts, dtype=np.int64).reshape(-1, 3)
    n = pts.shape[0]
    sa = (K * lda if a_col else M * lda) if sa is None else sa
    sb = (N * ldb if b_col else K * ldb) if sb is None else sb
    sc = M * ldc if sc is None else sc
    Dh, Dl, S = np.zeros(n), np.zeros(n), np.zeros(n)
    rc = lib.oracle_gemm_f64_points(_ptr(A), _ptr(B), _ptr(C), _ptr(pts), n, _ptr(Dh), _ptr(Dl),
                                    _ptr(S), M, N, K, lda, ldb, ldc, int(a_col), int(b_col), batch,
                                    sa, sb, sc)
    if rc:
        raise ValueError("oracle_gemm_f64_points rejected its arguments")
    return Dh, Dl, S


def f64_error(D: np.ndarray, D_hi: np.ndarray, D_lo: np.ndarray) -> np.ndarray:
    """|D - (D_hi + D_lo)| evaluated without losing D_lo (D - D_hi is exact when close)."""
    return np.abs((np.asarray(D, dtype=np.float64) - D_hi) - D_lo)


def f64_tolerance(K: int, S: np.ndarray, C: np.ndarray) -> np.ndarray:
    """Bound for fp64 inputs with an fp64 accumulator that rounds to nearest even
    (each product and each addition at most half an ulp): (2K+2)*2^-53*S for the
    reduction, with a factor 2 for any summation order, and 2^-53*|c| for the one
    final addition of C."""
    u = 2.0 ** -53
    return (2.0 * K + 2.0) * u * np.asarray(S, dtype=np.float64) + u * np.abs(np.asarray(C, dtype=np.float64))


OUT_TYPES = {"f32": 0, "f16": 1, "bf16": 2, "i32": 3, "f64": 4}
# unit roundoff of the output storage type, and half its smallest subnormal spacing
_OUT_UNIT = {"f32": 0.0, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}
_OUT_FLOOR = {"f32": 0.0, "f16": 2.0 ** -25, "bf16": 2.0 ** -134}


def decode_c(c_type: str, C: np.ndarray) -> np.ndarray:
    """Exact float64 values of a C array stored as fp32 (float32), fp16 or bf16 (uint16 bits)."""
    if c_type == "f32":
        return np.asarray(C, dtype=np.float32).astype(np.float64)
    table = decode(c_type, np.arange(65536, dtype=np.uint32).astype(np.uint16))
    return table[np.asarray(C, dtype=np.uint16)]


# (significand bits incl. the leading one, smallest normal exponent, largest finite value)
_FORMATS = {"f16": (11, -14, 65504.0), "bf16": (8, -126, float.fromhex("0x1.fep127")),
            "f32": (24, -126, float.fromhex("0x1.fffffep127"))}


def round_to(d_type: str, x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest value of fp16 / bf16 / fp32, ties to the even
    significand (the IEEE default), returned as float64.  From the definition: the
    spacing of representable values around x is 2^(max(e, emin) - p + 1), with e the
    exponent of x; x is divided by that spacing, rounded half-to-even to an integer and
    scaled back.  Magnitudes at or beyond max + spacing/2 become infinities."""
    p, emin, vmax = _FORMATS[d_type]
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e2 = np.frexp(xf)                  # |x| = m * 2^e2 with m in [0.5, 1)
    e = np.maximum(e2 - 1, emin)          # exponent of the leading bit, clamped to emin
    spacing = np.ldexp(1.0, (e - p + 1).astype(np.int64))
    r = np.round(xf / spacing) * spacing  # np.round: ties to even
    top = vmax + np.ldexp(1.0, int(np.floor(np.log2(vmax))) - p)  # max + half its spacing
    r = np.where(np.abs(xf) >= top, np.copysign(np.inf, xf), r)
    out[fin] = r
    return out


def scaled_reference(P: np.ndarray, c_exact: np.ndarray, alpha: float, beta: float) -> np.ndarray:
    """D_exact = alpha * (A B) + beta * C, with P = A B from gemm() run on a zero C (fp64)."""
    out = float(alpha) * np.asarray(P, dtype=np.float64)
    if beta != 0.0:
        out = out + float(beta) * np.asarray(c_exact, dtype=np.float64)
    return out


def scaled_tolerance(K: int, S: np.ndarray, c_exact: np.ndarray, D_ref: np.ndarray,
                     alpha: float, beta: float, d_type: str) -> np.ndarray:
    """Bound on |D - D_exact| for the scaled, converted output stage:
    fp32 accumulation (4*K*2^-24*S), the two fp32 products and the fp32 sum
    (2^-24 of |alpha*S|, |beta*c| and of the sum each), and the final
    round-to-nearest-even conversion (unit roundoff of D's type, plus half the
    smallest fp16 subnormal spacing)."""
    u = 2.0 ** -24
    aS = abs(float(alpha)) * np.asarray(S, dtype=np.float64)
    bc = abs(float(beta)) * np.abs(np.asarray(c_exact, dtype=np.float64)) if beta != 0 else 0.0
    e_acc = abs(float(alpha)) * 4.0 * K * u * np.asarray(S, dtype=np.float64)
    e_fp32 = e_acc + u * (aS + bc) + u * (np.abs(D_ref) + e_acc + 2 * u * (aS + bc))
    return e_fp32 + _OUT_UNIT[d_type] * (np.abs(D_ref) + e_fp32) + _OUT_FLOOR[d_type]


def float_tolerance(K: int, S: np.ndarray, C: np.ndarray) -> np.ndarray:
    """Per-element bound |D - D_ref| <= 4*K*2^-24*S + 2^-24*|c| for fp16/bf16 inputs
    accumulated in fp32, with C added once (the bound the fp paths are held to)."""
    c = np.abs(np.asarray(C, dtype=np.float64))
    return 4.0 * K * 2.0 ** -24 * np.asarray(S, dtype=np.float64) + 2.0 ** -24 * c
