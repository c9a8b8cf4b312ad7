"""Seeded synthetic inputs for the dense GEMM D = A*B + C.

This module is shared by the tests, the benchmark, the CPU oracle's callers and
the GPU library's callers.  It holds none of the method's arithmetic: it only
draws random numbers and rounds them to the storage types (fp16 with numpy's
round-to-nearest-even cast, bf16 with a round-to-nearest-even bit operation on
the binary32 pattern), and lays them out in memory.

Storage conventions (the same on both sides):
  * fp16 / bf16 inputs are uint16 bit patterns; fp32 C is float32;
    int8 inputs are int8, int32 C is int32; fp64 A, B and C are float64;
  * A row-major -> memory shape (batch, M, lda); col-major -> (batch, K, lda);
  * B row-major -> (batch, K, ldb);  col-major -> (batch, N, ldb);
  * C and D row-major -> (batch, M, ldc);  consecutive batches are contiguous.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ACC_DTYPE = {"f16": np.float32, "bf16": np.float32, "i8": np.int32, "f64": np.float64}


@dataclass
class Problem:
    dtype: str              # "f16", "bf16" or "i8"
    M: int
    N: int
    K: int
    batch: int
    lda: int
    ldb: int
    ldc: int
    a_col: bool
    b_col: bool
    A: np.ndarray           # storage arrays, C-contiguous, shapes per the module doc
    B: np.ndarray
    C: np.ndarray
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K * self.batch

    def oracle_args(self):
        return dict(M=self.M, N=self.N, K=self.K, lda=self.lda, ldb=self.ldb, ldc=self.ldc,
                    a_col=self.a_col, b_col=self.b_col, batch=self.batch)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to bfloat16 (nearest, ties to even); returns uint16 bits.
    Inputs here are finite, so no NaN handling is needed."""
    w = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (w + 0x7FFF + ((w >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def f64_to_f16_bits(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def _draw(rng: np.random.Generator, dtype: str, dist: str, shape, lo=None, hi=None):
    if dtype == "i8":
        if dist == "uniform_int":
            return rng.integers(-128, 127, size=shape, endpoint=True, dtype=np.int8)
        if dist == "small_int":
            return rng.integers(-1, 1, size=shape, endpoint=True, dtype=np.int8)
        raise ValueError(dist)
    if dist == "uniform":
        v = rng.uniform(lo, hi, size=shape)
    elif dist == "normal":
        v = rng.standard_normal(size=shape, dtype=np.float32)
    elif dist == "small_int":
        v = rng.integers(-1, 1, size=shape, endpoint=True).astype(np.float64)
    else:
        raise ValueError(dist)
    if dtype == "f64":
        return np.asarray(v, dtype=np.float64)
    if dtype == "f16":
        return f64_to_f16_bits(v)
    return f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def _draw_c(rng, dtype: str, dist: str, shape, lo=None, hi=None):
    if dtype == "i8":
        if dist == "zeros":
            return np.zeros(shape, dtype=np.int32)
        if dist == "uniform_int":
            return rng.integers(lo, hi, size=shape, endpoint=True, dtype=np.int32)
        raise ValueError(dist)
    ct = np.float64 if dtype == "f64" else np.float32
    if dist == "zeros":
        return np.zeros(shape, dtype=ct)
    if dist == "uniform":
        return rng.uniform(lo, hi, size=shape).astype(ct)
    if dist == "small_int":
        return rng.integers(lo, hi, size=shape, endpoint=True).astype(ct)
    raise ValueError(dist)


def make_problem(dtype: str, M: int, N: int, K: int, *, batch: int = 1, a_col: bool = False,
                 b_col: bool = False, pad: int = 0, seed: int = 0, ab_dist: str | None = None,
                 ab_range=(-1.0, 1.0), c_dist: str | None = None, c_range=(-1.0, 1.0),
                 name: str = "") -> Problem:
    """Draw one problem.  Order of draws: A, then B, then C, from PCG64(seed).
    ``pad`` adds that many unused elements to every leading dimension."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if ab_dist is None:
        ab_dist = "uniform_int" if dtype == "i8" else "uniform"
    if c_dist is None:
        c_dist = "uniform_int" if dtype == "i8" else "uniform"
    lda = (M if a_col else K) + pad
    ldb = (K if b_col else N) + pad
    ldc = N + pad
    a_shape = (batch, K, lda) if a_col else (batch, M, lda)
    b_shape = (batch, N, ldb) if b_col else (batch, K, ldb)
    A = _draw(rng, dtype, ab_dist, a_shape, *ab_range)
    B = _draw(rng, dtype, ab_dist, b_shape, *ab_range)
    C = _draw_c(rng, dtype, c_dist, (batch, M, ldc), *c_range)
    return Problem(dtype, M, N, K, batch, lda, ldb, ldc, a_col, b_col,
                   np.ascontiguousarray(A), np.ascontiguousarray(B), np.ascontiguousarray(C),
                   name=name)


# The five workloads, plus a supplementary large fp16 problem and exact-integer
# variants (entries of A and B in {-1, 0, 1}, small-integer C) used as bit-exact
# pins for the float paths.
CONFIGS = {
    # 256^3 fp16, A/B row-major uniform[-1,1], C fp32 uniform[-1,1]
    "C1": dict(dtype="f16", M=256, N=256, K=256, seed=1, ab_dist="uniform", ab_range=(-1.0, 1.0),
               c_dist="uniform", c_range=(-1.0, 1.0)),
    # 4096^3 bf16 N(0,1), A row-major, B column-major, C zeros
    "C2": dict(dtype="bf16", M=4096, N=4096, K=4096, b_col=True, seed=2, ab_dist="normal",
               c_dist="zeros"),
    # 8192^3 int8 uniform integers [-128,127], C int32 uniform [-2^20, 2^20]
    "C3": dict(dtype="i8", M=8192, N=8192, K=8192, seed=3, ab_dist="uniform_int",
               c_dist="uniform_int", c_range=(-(1 << 20), 1 << 20)),
    # 8192 independent 64^3 fp16 problems, contiguous batch stride
    "C4": dict(dtype="f16", M=64, N=64, K=64, batch=8192, seed=4, ab_dist="uniform",
               ab_range=(-1.0, 1.0), c_dist="uniform", c_range=(-1.0, 1.0)),
    # skinny large-K: 1024 x 1024 x 65536 bf16 uniform[-0.5,0.5], C zeros
    "C5": dict(dtype="bf16", M=1024, N=1024, K=65536, seed=5, ab_dist="uniform",
               ab_range=(-0.5, 0.5), c_dist="zeros"),
    # supplementary: 4096^3 fp16 with C1's distributions
    "S1": dict(dtype="f16", M=4096, N=4096, K=4096, seed=6, ab_dist="uniform",
               ab_range=(-1.0, 1.0), c_dist="uniform", c_range=(-1.0, 1.0)),
    # fp64 (the double-precision instruction family): 4096^3, A/B row-major
    # uniform[-1,1], C fp64 uniform[-1,1]
    "F1": dict(dtype="f64", M=4096, N=4096, K=4096, seed=7, ab_dist="uniform",
               ab_range=(-1.0, 1.0), c_dist="uniform", c_range=(-1.0, 1.0)),
    # 2:4 structured-sparse A (the sparse instructions): the 4096^3 bf16 problem of
    # C2 (A pruned on the GPU before the timed products), seed 9
    "SP1": dict(dtype="bf16", M=4096, N=4096, K=4096, b_col=True, seed=9, ab_dist="normal",
                c_dist="zeros"),
    # tiny products (the multi-block instructions): 2^20 independent 4x4x16 fp16
    # problems, A/B row-major uniform[-1,1], C fp32 uniform[-1,1]
    "T1": dict(dtype="f16", M=4, N=4, K=16, batch=1 << 20, seed=8, ab_dist="uniform",
               ab_range=(-1.0, 1.0), c_dist="uniform", c_range=(-1.0, 1.0)),
    # 2:4 structured-sparse int8 A: C3's 8192^3 distributions, B column-major (the
    # layout the sparse kernel reads without transposing), seed 10
    "SP2": dict(dtype="i8", M=8192, N=8192, K=8192, b_col=True, seed=10, ab_dist="uniform_int",
                c_dist="uniform_int", c_range=(-(1 << 20), 1 << 20)),
}

CONFIG_LABELS = {
    "C1": "gemm 256x256x256 fp16 (A,B row-major), C fp32",
    "C2": "gemm 4096x4096x4096 bf16 (A row-major, B col-major), C fp32 zeros",
    "C3": "gemm 8192x8192x8192 int8 (A,B row-major), C int32, bit-exact",
    "C4": "batched gemm 8192 x 64x64x64 fp16 (row-major), C fp32",
    "C5": "gemm 1024x1024x65536 bf16 (row-major), C fp32 zeros",
    "S1": "gemm 4096x4096x4096 fp16 (row-major), C fp32",
    "F1": "gemm 4096x4096x4096 fp64 (row-major), C fp64",
    "T1": "batched gemm 1048576 x 4x4x16 fp16 (row-major), C fp32",
    "SP1": "gemm 4096x4096x4096 bf16, A 2:4-pruned (row-major), B col-major, C fp32 zeros",
    "SP2": "gemm 8192x8192x8192 int8, A 2:4-pruned (row-major), B col-major, C int32, bit-exact",
}


def config_problem(name: str) -> Problem:
    kw = dict(CONFIGS[name])
    p = make_problem(name=name, **kw)
    return p


def exact_variant(name: str) -> Problem:
    """Same shape and layout as a workload, with A, B in {-1,0,1} and C small integers
    (|c| <= 8 for floats), seeds 101..106.  Every partial sum is an integer of magnitude
    below 2^24, so any fp32 summation order gives the exact answer."""
    kw = dict(CONFIGS[name])
    seed = 100 + list(CONFIGS).index(name) + 1
    kw.update(seed=seed, ab_dist="small_int")
    if kw["dtype"] == "i8":
        kw.update(c_dist="uniform_int", c_range=(-8, 8))
    else:
        kw.update(c_dist="small_int", c_range=(-8, 8))
    return make_problem(name=name + "x", **kw)
