"""Pins for the CPU oracle, each against something other than the oracle itself:
library decoders, exact rational brute force, closed forms, and the properties a
matrix product must have (identity, permutation, rank one, all ones, extremes,
an empty reduction).  CPU only."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

DT_FLOAT = ["f16", "bf16"]
LAYOUTS = list(itertools.product([False, True], [False, True]))


def lib_decode(dtype, bits):
    """Library decoders, independent of the oracle's bit-field arithmetic."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def logical(p: synth.Problem, b: int):
    """Logical A (MxK), B (KxN), C (MxN) of batch b as storage-typed numpy views."""
    A = p.A[b]
    B = p.B[b]
    A = A[:p.K, :p.M].T if p.a_col else A[:p.M, :p.K]
    B = B[:p.N, :p.K].T if p.b_col else B[:p.K, :p.N]
    C = p.C[b][:p.M, :p.N]
    return A, B, C


def run_oracle(p: synth.Problem, nthreads=3):
    return oracle.gemm(p.dtype, p.A, p.B, p.C, **p.oracle_args(), nthreads=nthreads)


# ---------------------------------------------------------------- decoders

@pytest.mark.parametrize("dtype", DT_FLOAT)
def test_decode_exhaustive(dtype):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(dtype, bits)
    ref = lib_decode(dtype, bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_decode_f32_sample():
    rng = np.random.default_rng(7)
    words = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    specials = np.array([0, 0x80000000, 1, 0x807fffff, 0x00800000, 0x7f7fffff, 0x7f800000,
                         0xff800000, 0x3f800000, 0x7fc00000], dtype=np.uint32)
    words = np.concatenate([words, specials])
    got = oracle.decode_f32(words)
    ref = words.view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ------------------------------------------------------- exact brute force

def exact_reference(p: synth.Problem):
    """Exact rational D and S by brute force over Python Fractions (tiny sizes only)."""
    out_d, out_s = [], []
    for b in range(p.batch):
        A, B, C = logical(p, b)
        if p.dtype == "i8":
            Af = [[int(v) for v in row] for row in A]
            Bf = [[int(v) for v in row] for row in B]
            Cf = [[int(v) for v in row] for row in C]
        else:
            Af = [[Fraction(float(v)) for v in row] for row in lib_decode(p.dtype, A)]
            Bf = [[Fraction(float(v)) for v in row] for row in lib_decode(p.dtype, B)]
            Cf = [[Fraction(float(v)) for v in row] for row in C.astype(np.float64)]
        D = [[Cf[i][j] + sum(Af[i][k] * Bf[k][j] for k in range(p.K)) for j in range(p.N)]
             for i in range(p.M)]
        S = [[sum(abs(Af[i][k] * Bf[k][j]) for k in range(p.K)) for j in range(p.N)]
             for i in range(p.M)]
        out_d.append(D)
        out_s.append(S)
    return out_d, out_s


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("a_col,b_col", LAYOUTS)
def test_brute_force_tiny(dtype, a_col, b_col):
    rng = np.random.default_rng(11)
    for trial in range(6):
        M, N, K = (int(x) for x in rng.integers(1, 9, size=3))
        batch = int(rng.integers(1, 4))
        pad = int(rng.integers(0, 3))
        p = synth.make_problem(dtype, M, N, K, batch=batch, a_col=a_col, b_col=b_col, pad=pad,
                               seed=1000 + trial, c_range=(-1.0, 1.0) if dtype != "i8" else (-1000, 1000))
        ed, es = exact_reference(p)
        if dtype == "i8":
            D = run_oracle(p)
            for b, i, j in itertools.product(range(batch), range(M), range(N)):
                assert D[b, i, j] == ed[b][i][j]
        else:
            D, S = run_oracle(p)
            for b, i, j in itertools.product(range(batch), range(M), range(N)):
                s_exact = es[b][i][j]
                assert abs(Fraction(D[b, i, j]) - ed[b][i][j]) <= K * Fraction(2) ** -53 * s_exact \
                    + Fraction(2) ** -53 * abs(ed[b][i][j])
                # products are exact in fp64, so S is exact up to the summation rounding
                assert abs(Fraction(S[b, i, j]) - s_exact) <= K * Fraction(2) ** -53 * s_exact


def test_points_match_brute_force():
    for dtype, (a_col, b_col) in itertools.product(["f16", "bf16", "i8"], LAYOUTS):
        p = synth.make_problem(dtype, 5, 7, 6, batch=2, a_col=a_col, b_col=b_col, pad=1, seed=77,
                               c_range=(-1.0, 1.0) if dtype != "i8" else (-50, 50))
        ed, es = exact_reference(p)
        pts = np.array([(b, i, j) for b in range(2) for i in range(5) for j in range(7)])
        r = oracle.gemm_points(p.dtype, p.A, p.B, p.C, pts, **p.oracle_args())
        for n, (b, i, j) in enumerate(pts):
            if dtype == "i8":
                assert r[n] == ed[b][i][j]
            else:
                assert abs(Fraction(r[0][n]) - ed[b][i][j]) <= 6 * Fraction(2) ** -53 * (es[b][i][j] + 1)
                assert abs(Fraction(r[1][n]) - es[b][i][j]) <= 6 * Fraction(2) ** -53 * es[b][i][j]


# ------------------------------------------------------------ library matmul

@pytest.mark.parametrize("dtype", DT_FLOAT)
@pytest.mark.parametrize("a_col,b_col", LAYOUTS)
def test_against_numpy_matmul(dtype, a_col, b_col):
    """Moderate shapes with padding and a batch: fp64 numpy matmul of the library-decoded
    inputs agrees to fp64 summation accuracy."""
    p = synth.make_problem(dtype, 37, 53, 71, batch=2, a_col=a_col, b_col=b_col, pad=3, seed=5)
    D, S = run_oracle(p)
    for b in range(2):
        A, B, C = logical(p, b)
        ref = lib_decode(dtype, A) @ lib_decode(dtype, B) + C.astype(np.float64)
        sref = np.abs(lib_decode(dtype, A)) @ np.abs(lib_decode(dtype, B))
        assert np.all(np.abs(D[b] - ref) <= 2 * p.K * 2.0 ** -52 * (sref + np.abs(ref)))
        assert np.allclose(S[b], sref, rtol=1e-13, atol=0)


@pytest.mark.parametrize("a_col,b_col", LAYOUTS)
def test_int8_against_numpy_matmul(a_col, b_col):
    p = synth.make_problem("i8", 29, 41, 300, batch=2, a_col=a_col, b_col=b_col, pad=2, seed=6,
                           c_range=(-(1 << 20), 1 << 20))
    D = run_oracle(p)
    for b in range(2):
        A, B, C = logical(p, b)
        ref = A.astype(np.int64) @ B.astype(np.int64) + C.astype(np.int64)
        assert np.array_equal(D[b], ref)


# ------------------------------------------------------------ closed forms

def bits_of(dtype, values):
    v = np.asarray(values, dtype=np.float64)
    if dtype == "f16":
        return synth.f64_to_f16_bits(v)
    if dtype == "bf16":
        return synth.f32_to_bf16_bits(v.astype(np.float32))
    return v.astype(np.int8)


def build(dtype, A_log, B_log, C_log, a_col=False, b_col=False):
    """Storage arrays for given logical matrices (tight leading dimensions, batch 1)."""
    M, K = A_log.shape
    N = B_log.shape[1]
    A = bits_of(dtype, A_log.T if a_col else A_log)[None].copy()
    B = bits_of(dtype, B_log.T if b_col else B_log)[None].copy()
    C = np.asarray(C_log, dtype=np.int32 if dtype == "i8" else np.float32)[None].copy()
    lda = M if a_col else K
    ldb = K if b_col else N
    return A, B, C, dict(M=M, N=N, K=K, lda=lda, ldb=ldb, ldc=N, a_col=a_col, b_col=b_col)


def ref_result(dtype, A, B, C, args):
    r = oracle.gemm(dtype, A, B, C, **args, nthreads=2)
    return r if dtype == "i8" else r[0]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("a_col,b_col", LAYOUTS)
def test_identity(dtype, a_col, b_col):
    """A*I + 0 = A and I*B + 0 = B exactly (the identity-B check input)."""
    rng = np.random.default_rng(3)
    M, K = 19, 23
    if dtype == "i8":
        A_log = rng.integers(-128, 128, size=(M, K)).astype(np.float64)
    else:
        A_log = lib_decode(dtype, bits_of(dtype, rng.uniform(-4, 4, size=(M, K))))
    I = np.eye(K)
    A, B, C, args = build(dtype, A_log, I, np.zeros((M, K)), a_col, b_col)
    D = ref_result(dtype, A, B, C, args)[0]
    assert np.array_equal(D, A_log)
    A, B, C, args = build(dtype, np.eye(M), A_log, np.zeros((M, K)), a_col, b_col)
    D = ref_result(dtype, A, B, C, args)[0]
    assert np.array_equal(D, A_log)


@pytest.mark.parametrize("dtype", ["f16", "i8"])
@pytest.mark.parametrize("a_col,b_col", LAYOUTS)
def test_permutation(dtype, a_col, b_col):
    """P*X permutes the rows of X; X*P permutes its columns -- exactly."""
    rng = np.random.default_rng(4)
    n = 17
    perm = rng.permutation(n)
    P = np.zeros((n, n))
    P[np.arange(n), perm] = 1.0          # (P X)[i] = X[perm[i]]
    X = rng.integers(-100, 100, size=(n, n)).astype(np.float64)
    A, B, C, args = build(dtype, P, X, np.zeros((n, n)), a_col, b_col)
    assert np.array_equal(ref_result(dtype, A, B, C, args)[0], X[perm])
    A, B, C, args = build(dtype, X, P, np.zeros((n, n)), a_col, b_col)
    inv = np.argsort(perm)               # (X P)[:, j] = X[:, inv[j]]
    assert np.array_equal(ref_result(dtype, A, B, C, args)[0], X[:, inv])


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
def test_rank_one(dtype):
    """A[i,k] = x_i, B[k,j] = y_j  =>  D = K*x_i*y_j + c_ij exactly."""
    rng = np.random.default_rng(5)
    M, N, K = 13, 11, 40
    x = rng.integers(-4, 5, size=M).astype(np.float64)
    y = rng.integers(-4, 5, size=N).astype(np.float64)
    if dtype != "i8":
        x = x * 2.0 ** rng.integers(-3, 3, size=M)
        y = y * 2.0 ** rng.integers(-3, 3, size=N)
    c = rng.integers(-9, 10, size=(M, N)).astype(np.float64)
    A_log = np.repeat(x[:, None], K, axis=1)
    B_log = np.repeat(y[None, :], K, axis=0)
    A, B, C, args = build(dtype, A_log, B_log, c)
    D = ref_result(dtype, A, B, C, args)[0]
    assert np.array_equal(D, K * np.outer(x, y) + c)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
def test_all_ones(dtype):
    M, N, K = 9, 10, 300
    c = np.arange(M * N).reshape(M, N) % 7 - 3.0
    A, B, C, args = build(dtype, np.ones((M, K)), np.ones((K, N)), c)
    D = ref_result(dtype, A, B, C, args)[0]
    assert np.array_equal(D, K + c)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
def test_all_ones_large_k_points(dtype):
    """Every output equals K (+c) at the skinny workload's K = 65536."""
    M = N = 4
    K = 65536
    A = bits_of(dtype, np.ones((1, M, K)))
    B = bits_of(dtype, np.ones((1, K, N)))
    C = (np.full((1, M, N), 3, dtype=np.int32) if dtype == "i8"
         else np.full((1, M, N), 3.0, dtype=np.float32))
    pts = np.array([(0, i, j) for i in range(M) for j in range(N)])
    r = oracle.gemm_points(dtype, A, B, C, pts, M=M, N=N, K=K, lda=K, ldb=N, ldc=N)
    vals = r if dtype == "i8" else r[0]
    assert np.all(vals == K + 3)
    if dtype != "i8":
        assert np.all(r[1] == K)


@pytest.mark.parametrize("bv,per_k", [(-128, 16384), (127, -16256)])
def test_int8_extremes(bv, per_k):
    M, N, K = 6, 5, 8192
    c = np.arange(M * N).reshape(M, N) * 1000 - 7000
    A, B, C, args = build("i8", np.full((M, K), -128.0), np.full((K, N), float(bv)), c)
    D = ref_result("i8", A, B, C, args)[0]
    assert np.array_equal(D, per_k * K + c)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
def test_k_zero_gives_c(dtype):
    p = synth.make_problem(dtype, 7, 9, 0, batch=2, seed=8,
                           c_range=(-1.0, 1.0) if dtype != "i8" else (-100, 100))
    r = run_oracle(p)
    D = r if dtype == "i8" else r[0]
    assert np.array_equal(D, p.C[:, :7, :9].astype(D.dtype))


def test_thread_count_does_not_change_result():
    p = synth.make_problem("bf16", 33, 29, 64, batch=3, seed=9, pad=1)
    D1, S1 = oracle.gemm(p.dtype, p.A, p.B, p.C, **p.oracle_args(), nthreads=1)
    D7, S7 = oracle.gemm(p.dtype, p.A, p.B, p.C, **p.oracle_args(), nthreads=7)
    assert np.array_equal(D1, D7) and np.array_equal(S1, S7)


# ------------------------------------------------------------ the tolerance

def fp32_sequential(p: synth.Problem, drop_k=None):
    """An fp32 round-to-nearest k-ordered accumulation, C added once at the end:
    one legitimate way hardware may compute the float result."""
    A, B, C = logical(p, 0)
    Ad = lib_decode(p.dtype, A).astype(np.float32)
    Bd = lib_decode(p.dtype, B).astype(np.float32)
    acc = np.zeros((p.M, p.N), dtype=np.float32)
    for k in range(p.K):
        if k == drop_k:
            continue
        acc = acc + np.outer(Ad[:, k], Bd[k, :]).astype(np.float32)
    return acc + C


@pytest.mark.parametrize("dtype", DT_FLOAT)
def test_tolerance_accepts_fp32_and_rejects_dropped_term(dtype):
    p = synth.make_problem(dtype, 24, 24, 48, seed=12)
    D, S = run_oracle(p)
    tol = oracle.float_tolerance(p.K, S[0], p.C[0])
    good = fp32_sequential(p).astype(np.float64)
    assert np.all(np.abs(good - D[0]) <= tol)
    bad = fp32_sequential(p, drop_k=17).astype(np.float64)
    assert np.any(np.abs(bad - D[0]) > tol)


# ------------------------------------------------------ scaled, converted output

def _simulate_stage(acc32, c32, alpha, beta, d_type):
    """The documented output stage in numpy: fp32 products and sum (no fused
    multiply-add), then round-to-nearest-even to D's storage type."""
    a = np.float32(alpha)
    t = (a * acc32).astype(np.float32)
    if beta != 0:
        t = (t + (np.float32(beta) * c32).astype(np.float32)).astype(np.float32)
    if d_type == "f32":
        return t.astype(np.float64)
    if d_type == "f16":
        return t.astype(np.float16).astype(np.float64)
    bits = synth.f32_to_bf16_bits(t)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("d_type", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("c_type", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("alpha,beta", [(1.0, 1.0), (0.75, -2.5), (-3.0, 0.0)])
def test_scaled_output_tolerance(c_type, d_type, alpha, beta):
    """The stage's fp32 + conversion roundings stay inside scaled_tolerance; a
    stage that forgets beta, or truncates instead of rounding, leaves it."""
    p = synth.make_problem("bf16", 20, 24, 40, seed=31)
    P, S = oracle.gemm("bf16", p.A, p.B, np.zeros_like(p.C), **p.oracle_args())
    P, S = P[0], S[0]
    rng = np.random.default_rng(3)
    cvals = rng.uniform(-4, 4, size=(20, 24))
    if c_type == "f32":
        Cst = cvals.astype(np.float32)
    elif c_type == "f16":
        Cst = synth.f64_to_f16_bits(cvals)
    else:
        Cst = synth.f32_to_bf16_bits(cvals.astype(np.float32))
    c_exact = oracle.decode_c(c_type, Cst)
    D_ref = oracle.scaled_reference(P, c_exact, alpha, beta)
    tol = oracle.scaled_tolerance(p.K, S, c_exact, D_ref, alpha, beta, d_type)
    acc32 = fp32_sequential(p)  # C of the generated problem is added at the end: remove it
    acc32 = (acc32 - p.C[0]).astype(np.float32)
    good = _simulate_stage(acc32, c_exact.astype(np.float32), alpha, beta, d_type)
    assert np.all(np.abs(good - D_ref) <= tol)
    if beta != 0:
        no_beta = _simulate_stage(acc32, c_exact.astype(np.float32), alpha, 0.0, d_type)
        assert np.any(np.abs(no_beta - D_ref) > tol)
    if d_type == "bf16":
        t = _simulate_stage(acc32, c_exact.astype(np.float32), alpha, beta, "f32").astype(np.float32)
        trunc = ((t.view(np.uint32) >> 16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert np.any(np.abs(trunc - D_ref) > tol)


def test_decode_c_matches_library():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    f = np.isfinite(bits.view(np.float16))
    assert np.array_equal(oracle.decode_c("f16", bits)[f], bits.view(np.float16)[f].astype(np.float64))
    x = np.float32([1.5, -2.25, 3e-20])
    assert np.array_equal(oracle.decode_c("f32", x), x.astype(np.float64))


# --------------------------------------------------- rounding to the output type

def _all_values(d_type):
    """Every finite value of a 16-bit format (decoded by the pinned decoder), sorted,
    with its bit pattern."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = oracle.decode(d_type, bits)
    ok = np.isfinite(v)
    order = np.argsort(v[ok], kind="stable")
    return v[ok][order], bits[ok][order]


@pytest.mark.parametrize("d_type", ["f16", "bf16"])
def test_round_to_brute_force_nearest(d_type):
    """round_to picks the nearest representable value, and on an exact tie the one whose
    bit pattern is even; found here by search over all 2^16 patterns."""
    vals, bits = _all_values(d_type)
    rng = np.random.default_rng(5)
    finite_max = vals[-1]
    mid = rng.integers(0, len(vals) - 1, 2000)
    # random magnitudes over the whole range, exact midpoints, subnormals, near-overflow
    x = np.concatenate([
        rng.standard_normal(3000) * np.exp2(rng.integers(-30 if d_type == "f16" else -140,
                                                         16 if d_type == "f16" else 127, 3000)),
        (vals[mid] + vals[mid + 1]) / 2,
        rng.uniform(-1, 1, 500) * vals[vals > 0][0] * 8,
        np.array([finite_max * (1 + 2.0 ** -12), -finite_max * (1 - 2.0 ** -30), 0.0, -0.0]),
    ])
    x = x[np.abs(x) < finite_max]      # overflow is checked separately
    got = oracle.round_to(d_type, x)
    idx = np.searchsorted(vals, x)
    lo = vals[np.clip(idx - 1, 0, len(vals) - 1)]
    hi = vals[np.clip(idx, 0, len(vals) - 1)]
    bhi = bits[np.clip(idx, 0, len(vals) - 1)]
    dlo, dhi = np.abs(x - lo), np.abs(hi - x)
    want = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(bhi % 2 == 0, hi, lo)))
    assert np.array_equal(got, want)   # == also equates the two zeros


def test_round_to_matches_numpy_casts():
    """float64 -> float16 and float64 -> float32 casts in numpy round to nearest even."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-20, 15, 20000))
    assert np.array_equal(oracle.round_to("f16", x), x.astype(np.float16).astype(np.float64))
    y = rng.standard_normal(20000) * np.exp2(rng.integers(-140, 120, 20000))
    assert np.array_equal(oracle.round_to("f32", y), y.astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("d_type,big", [("f16", 65520.0), ("bf16", float.fromhex("0x1.ffp127"))])
def test_round_to_overflow_and_specials(d_type, big):
    """max + half a spacing and beyond round to infinity; just below stays finite."""
    vmax = 65504.0 if d_type == "f16" else float.fromhex("0x1.fep127")
    r = oracle.round_to(d_type, np.array([big, -big, np.nextafter(big, 0), np.inf, np.nan]))
    assert r[0] == np.inf and r[1] == -np.inf and r[2] == vmax
    assert r[3] == np.inf and np.isnan(r[4])


# ------------------------------------------------------------------ fp64 path

def f64_logical(p, b):
    A, B = p.A[b], p.B[b]
    A = A[:p.K, :p.M].T if p.a_col else A[:p.M, :p.K]
    B = B[:p.N, :p.K].T if p.b_col else B[:p.K, :p.N]
    return A, B, p.C[b][:p.M, :p.N]


@pytest.mark.parametrize("a_col,b_col", LAYOUTS)
def test_f64_brute_force_exact(a_col, b_col):
    """Rational brute force: D_hi + D_lo equals the exact value to ~2^-100 relative."""
    rng = np.random.default_rng(21)
    for trial in range(5):
        M, N, K = (int(x) for x in rng.integers(1, 8, size=3))
        p = synth.make_problem("f64", M, N, K, batch=2, a_col=a_col, b_col=b_col,
                               pad=int(rng.integers(0, 3)), seed=300 + trial)
        # spread the exponents so that products are not exact in fp64
        p.A *= np.exp2(rng.integers(-30, 30, size=p.A.shape))
        Dh, Dl, S = oracle.gemm_f64(p.A, p.B, p.C, **p.oracle_args())
        for b in range(2):
            A, B, C = f64_logical(p, b)
            for i in range(M):
                for j in range(N):
                    ex = Fraction(float(C[i, j])) + sum(Fraction(float(A[i, k])) * Fraction(float(B[k, j]))
                                                        for k in range(K))
                    s_ex = sum(abs(Fraction(float(A[i, k])) * Fraction(float(B[k, j]))) for k in range(K))
                    got = Fraction(float(Dh[b, i, j])) + Fraction(float(Dl[b, i, j]))
                    assert abs(got - ex) <= Fraction(2) ** -100 * (s_ex + abs(Fraction(float(C[i, j])))) 
                    assert abs(Fraction(float(S[b, i, j])) - s_ex) <= K * Fraction(2) ** -52 * s_ex


def test_f64_cancellation_needs_the_low_part():
    """1e16 + 1 - 1e16 (+ 0.5 from C): plain fp64 summation loses the 1, the pair keeps it."""
    A = np.array([[[1e16, 1.0, -1e16]]])
    B = np.array([[[1.0], [1.0], [1.0]]])
    C = np.array([[[0.5]]])
    Dh, Dl, S = oracle.gemm_f64(A, B, C, M=1, N=1, K=3, lda=3, ldb=1, ldc=1)
    assert Dh[0, 0, 0] + Dl[0, 0, 0] == 1.5 and Dh[0, 0, 0] == 1.5
    assert S[0, 0, 0] == 2e16 + 1
    # the rounding error of a single product is recovered too: (1 + 2^-30)^2
    x = 1.0 + 2.0 ** -30
    Dh, Dl, _ = oracle.gemm_f64(np.array([[[x]]]), np.array([[[x]]]), np.zeros((1, 1, 1)),
                                M=1, N=1, K=1, lda=1, ldb=1, ldc=1)
    assert Fraction(float(Dh[0, 0, 0])) + Fraction(float(Dl[0, 0, 0])) == Fraction(x) ** 2


@pytest.mark.parametrize("a_col,b_col", LAYOUTS)
def test_f64_against_numpy_and_closed_forms(a_col, b_col):
    p = synth.make_problem("f64", 37, 53, 71, batch=2, a_col=a_col, b_col=b_col, pad=3, seed=22)
    Dh, Dl, S = oracle.gemm_f64(p.A, p.B, p.C, **p.oracle_args(), nthreads=3)
    for b in range(2):
        A, B, C = f64_logical(p, b)
        ref = A @ B + C
        assert np.all(np.abs(Dh[b] - ref) <= 2 * p.K * 2.0 ** -52 * (np.abs(A) @ np.abs(B) + np.abs(C)))
    # identity and permutation: exact
    rng = np.random.default_rng(4)
    X = rng.standard_normal((9, 9))
    P = np.eye(9)[rng.permutation(9)]
    for L, R in [(X, np.eye(9)), (np.eye(9), X), (P, X), (X, P)]:
        Dh, Dl, _ = oracle.gemm_f64(L[None].copy(), R[None].copy(), np.zeros((1, 9, 9)),
                                    M=9, N=9, K=9, lda=9, ldb=9, ldc=9)
        assert np.array_equal(Dh[0], L @ R) and np.all(Dl == 0)
    # rank one with powers of two: K * x_i * y_j + c exactly
    x = np.exp2(rng.integers(-20, 20, 6)).astype(np.float64)
    y = np.exp2(rng.integers(-20, 20, 5)).astype(np.float64)
    K = 11
    A = np.repeat(x[:, None], K, axis=1)[None].copy()
    B = np.repeat(y[None, :], K, axis=0)[None].copy()
    C = rng.integers(-9, 9, (1, 6, 5)).astype(np.float64)
    Dh, Dl, _ = oracle.gemm_f64(A, B, C, M=6, N=5, K=K, lda=K, ldb=5, ldc=5)
    want = [[Fraction(K) * Fraction(x[i]) * Fraction(y[j]) + Fraction(C[0, i, j]) for j in range(5)]
            for i in range(6)]
    for i in range(6):
        for j in range(5):
            assert Fraction(float(Dh[0, i, j])) + Fraction(float(Dl[0, i, j])) == want[i][j]


def test_f64_points_match_full():
    p = synth.make_problem("f64", 23, 19, 45, batch=3, b_col=True, pad=1, seed=23)
    Dh, Dl, S = oracle.gemm_f64(p.A, p.B, p.C, **p.oracle_args())
    pts = np.array([(b, i, j) for b in range(3) for i in (0, 7, 22) for j in (0, 5, 18)])
    ph, pl, ps = oracle.gemm_f64_points(p.A, p.B, p.C, pts, **p.oracle_args())
    sel = (pts[:, 0], pts[:, 1], pts[:, 2])
    assert np.array_equal(ph, Dh[sel]) and np.array_equal(pl, Dl[sel]) and np.array_equal(ps, S[sel])


def test_f64_tolerance_accepts_fp64_sum_and_rejects_dropped_term():
    p = synth.make_problem("f64", 16, 16, 512, seed=24)
    Dh, Dl, S = oracle.gemm_f64(p.A, p.B, p.C, **p.oracle_args())
    A, B, C = f64_logical(p, 0)
    seq = np.zeros((16, 16))
    for k in range(p.K):             # plain sequential fp64, C added last
        seq = seq + np.outer(A[:, k], B[k, :])
    seq = seq + C
    tol = oracle.f64_tolerance(p.K, S[0], C)
    assert np.all(oracle.f64_error(seq, Dh[0], Dl[0]) <= tol)
    dropped = seq - np.outer(A[:, 100], B[100, :])
    assert np.any(oracle.f64_error(dropped, Dh[0], Dl[0]) > tol)


# ------------------------------------------------------------ 2:4 pruning

def test_prune24_hand_example():
    vals = np.array([[0.5, -2.0, 1.0, 0.25, 3.0, 3.0, -3.0, 1.0, 0.0, 0.0, 0.0, 7.0, 1.0, -1.0]])
    A = synth.f64_to_f16_bits(vals)[None].copy()
    P = oracle.prune24("f16", A, M=1, K=14, lda=14)
    got = P[0].view(np.float16).astype(np.float64)
    # groups: {0.5,-2,1,0.25} keep -2, 1; {3,3,-3,1} ties keep the first two 3s;
    # {0,0,0,7} keep 7 and the first 0; short group {1,-1}: both kept
    want = np.array([[0, -2.0, 1.0, 0, 3.0, 3.0, 0, 0, 0.0, 0, 0, 7.0, 1.0, -1.0]])
    assert np.array_equal(got, want)


def test_prune24_brute_force_and_properties():
    rng = np.random.default_rng(12)
    for dtype in ("f16", "bf16"):
        p = synth.make_problem(dtype, 9, 3, 37, batch=2, pad=3, seed=13)
        # many exact ties: values from a small set
        if dtype == "f16":
            p.A = synth.f64_to_f16_bits(rng.choice([-2.0, -1.0, 0.0, 1.0, 2.0, 0.5], size=p.A.shape))
        P = oracle.prune24(dtype, p.A, M=p.M, K=p.K, lda=p.lda, batch=2)
        va, vp = lib_decode(dtype, p.A), lib_decode(dtype, P)
        for b in range(2):
            for i in range(p.M):
                for g in range(0, p.K, 4):
                    ks = list(range(g, min(g + 4, p.K)))

                    def beats(x, y):  # x is preferred to y: larger magnitude, else lower k
                        return abs(va[b, i, x]) > abs(va[b, i, y]) or \
                            (abs(va[b, i, x]) == abs(va[b, i, y]) and x < y)
                    # brute force over all candidate pairs: the one whose members
                    # beat every other member of the group
                    cands = [set(x) for x in itertools.combinations(ks, min(2, len(ks)))
                             if all(beats(u, w) for u in x for w in ks if w not in x)]
                    assert len(cands) == 1
                    keep = cands[0]
                    for k in ks:
                        if k in keep:
                            assert P[b, i, k] == p.A[b, i, k]      # exact bits
                        else:
                            assert vp[b, i, k] == 0
                    assert sum(1 for k in ks if vp[b, i, k] != 0) <= 2
                    dropped = [abs(va[b, i, k]) for k in ks if k not in keep]
                    assert all(abs(va[b, i, k]) >= max(dropped, default=0) for k in keep)
            # padding columns untouched
            assert np.array_equal(P[b, :, p.K:], p.A[b, :, p.K:])
        # idempotent, and a 2:4 matrix is its own pruning
        assert np.array_equal(oracle.prune24(dtype, P, M=p.M, K=p.K, lda=p.lda, batch=2), P)


def test_prune24_int8_hand_example_and_brute_force():
    """int8: magnitude is |v| of the integer (-128 has the largest, 128), ties
    keep the lower k; brute force over every candidate pair on random tie-heavy
    rows."""
    A = np.array([[[-128, 127, 0, -127, 3, -3, 3, 1, 0, 0, 0, -1, 5, -5, 2]]], dtype=np.int8)
    P = oracle.prune24("i8", A, M=1, K=15, lda=15)
    # {-128,127,0,-127}: -128 and 127; {3,-3,3,1}: first two (|3| ties, lower k);
    # {0,0,0,-1}: -1 and the first 0; short group {5,-5,2}: 5 and -5
    want = np.array([[[-128, 127, 0, 0, 3, -3, 0, 0, 0, 0, 0, -1, 5, -5, 0]]], dtype=np.int8)
    assert np.array_equal(P, want)
    rng = np.random.default_rng(14)
    A = rng.choice(np.array([-128, -2, -1, 0, 1, 2, 127], dtype=np.int8), size=(2, 7, 41))
    P = oracle.prune24("i8", A, M=7, K=38, lda=41, batch=2)
    v = A.astype(np.int64)
    for b in range(2):
        for i in range(7):
            for g in range(0, 38, 4):
                ks = list(range(g, min(g + 4, 38)))

                def beats(x, y):
                    return abs(v[b, i, x]) > abs(v[b, i, y]) or (abs(v[b, i, x]) == abs(v[b, i, y]) and x < y)
                cands = [set(x) for x in itertools.combinations(ks, min(2, len(ks)))
                         if all(beats(u, w) for u in x for w in ks if w not in x)]
                assert len(cands) == 1
                for k in ks:
                    assert P[b, i, k] == (A[b, i, k] if k in cands[0] else 0)
        assert np.array_equal(P[b, :, 38:], A[b, :, 38:])
