"""GPU parity of the scaled, converted output stage (gemm_run_ex):

    D = cvt_D(alpha * (A B) + beta * cvt(C)),  C and D in fp32, fp16 or bf16.

Random inputs are held to the oracle's scaled_tolerance (fp32 accumulation, the
fp32 products and sum of the stage, and one round-to-nearest-even conversion).
Exact-integer inputs with power-of-two alpha and beta keep every fp32 step
exact, so the only rounding left is the final conversion, and D must equal the
oracle's round_to of the exact value bit for bit -- on every kernel path."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import DTYPE_CODE, log

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

OUT = oracle.OUT_TYPES
FLOAT_TYPES = ["f32", "f16", "bf16"]


@pytest.fixture(scope="module")
def handle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_mixed_precision_02_amd as dmp
    h = dmp.Handle()
    yield h
    h.close()


def store_c(c_type: str, C: np.ndarray) -> np.ndarray:
    """C values (any float array) in the storage of c_type (input generation only)."""
    if c_type == "f32":
        return np.ascontiguousarray(C, dtype=np.float32)
    if c_type == "f16":
        return synth.f64_to_f16_bits(np.asarray(C, dtype=np.float64))
    return synth.f32_to_bf16_bits(np.asarray(C, dtype=np.float32))


def dev(x: np.ndarray):
    return torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).cuda()


def empty_d(d_type: str, shape):
    return torch.empty(shape, dtype=torch.float32 if d_type == "f32" else torch.int16,
                       device="cuda")


def host_d(d_type: str, D) -> np.ndarray:
    """GPU D -> exact float64 values (storage decoded by the pinned oracle decoder)."""
    x = D.cpu().numpy()
    if d_type == "f32":
        return x.astype(np.float64)
    return oracle.decode_c(d_type, x.view(np.uint16))


def run_ex(handle, p, alpha, beta, c_type, d_type, Cst=None, D=None, A=None, B=None,
           c_ptr=None):
    """One gemm_run_ex call on problem p; returns D (device)."""
    if A is None:
        A, B = dev(p.A), dev(p.B)
    Cd = dev(Cst) if Cst is not None else None
    if D is None:
        D = empty_d(d_type, (p.batch, p.M, p.ldc))
    flags = (1 if p.a_col else 0) | (2 if p.b_col else 0)
    cp = c_ptr if c_ptr is not None else (Cd.data_ptr() if Cd is not None else 0)
    handle.run_ex(A.data_ptr(), B.data_ptr(), cp, D.data_ptr(), p.M, p.N, p.K, p.lda, p.ldb,
                  p.ldc, DTYPE_CODE[p.dtype], flags, p.batch, alpha=alpha, beta=beta,
                  c_type=OUT[c_type], d_type=OUT[d_type],
                  stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return D


def product(p):
    """(P, S) = exact A B and sum |a b| from the oracle (C replaced by zeros)."""
    return oracle.gemm(p.dtype, p.A, p.B, np.zeros_like(p.C), **p.oracle_args())


def check_tol(p, Dg, P, S, c_exact, alpha, beta, d_type, what):
    D_ref = oracle.scaled_reference(P, c_exact, alpha, beta)
    tol = oracle.scaled_tolerance(p.K, S, c_exact, D_ref, alpha, beta, d_type)
    assert np.all(np.isfinite(Dg)), what
    err = np.abs(Dg - D_ref)
    bad = np.argwhere(err > tol)
    assert bad.size == 0, f"{what}: {len(bad)} over the bound, first at {bad[0]}"
    return float(np.max(err / np.maximum(tol, 1e-300)))


def logical(p, X):
    return X.reshape(p.batch, p.M, p.ldc)[:, :, :p.N]


# ----------------------------------------------------------- random inputs

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("c_type", FLOAT_TYPES)
@pytest.mark.parametrize("d_type", FLOAT_TYPES)
def test_storage_types_and_scaling(handle, dtype, c_type, d_type):
    """Every C / D storage pair with alpha, beta != 1, on a ragged shape (odd ldc:
    element stores) and a tile-aligned one (vector stores), both layouts of B."""
    alpha, beta = 0.75, -1.25
    for (M, N, K, b_col) in [(257, 263, 200, False), (256, 264, 192, True)]:
        p = synth.make_problem(dtype, M, N, K, b_col=b_col, seed=51)
        Cst = store_c(c_type, p.C)
        c_exact = oracle.decode_c(c_type, Cst)
        D = run_ex(handle, p, alpha, beta, c_type, d_type, Cst=Cst)
        P, S = product(p)
        r = check_tol(p, logical(p, host_d(d_type, D)), P, S, logical(p, c_exact), alpha, beta,
                      d_type, f"{dtype} C:{c_type} D:{d_type} {M}x{N}x{K}")
        log(f"[out] {dtype} C:{c_type} D:{d_type} {M}x{N}x{K}: max err/bound {r:.3g}")


@pytest.mark.parametrize("c_type", FLOAT_TYPES)
@pytest.mark.parametrize("d_type", FLOAT_TYPES)
def test_tile256_every_storage_pair(handle, c_type, d_type):
    """The 256x256 tile's own epilogue (no split) with every C / D storage pair and alpha,
    beta != 1, on a shape with partial tiles on both edges, compared in full: random bf16
    inputs against the bound, exact-integer fp16 inputs bit for bit."""
    import dense_mixed_precision_02_amd as dmp
    M, N, K = 4000, 4112, 256
    p = synth.make_problem("bf16", M, N, K, b_col=True, seed=57)
    lbl = dmp.plan_label(M, N, K, p.lda, p.ldb, p.ldc, DTYPE_CODE["bf16"], 2)
    log(f"[out tile256] C:{c_type} D:{d_type} {lbl}")
    assert lbl.startswith("tile256x256") and "splitk=1 " in lbl, lbl
    Cst = store_c(c_type, p.C)
    c_exact = oracle.decode_c(c_type, Cst)
    D = run_ex(handle, p, 0.75, -1.25, c_type, d_type, Cst=Cst)
    P, S = product(p)
    check_tol(p, logical(p, host_d(d_type, D)), P, S, logical(p, c_exact), 0.75, -1.25, d_type,
              f"tile256 C:{c_type} D:{d_type}")
    e = synth.make_problem("f16", M, N, K, seed=58, ab_dist="small_int", c_dist="small_int",
                           c_range=(-8, 8))
    exact_check(handle, e, d_type, c_type)


@pytest.mark.parametrize("d_type", FLOAT_TYPES)
def test_beta_zero_reads_no_c(handle, d_type):
    """beta = 0 with a NULL C pointer on the tile, split-K and element-wise paths."""
    import dense_mixed_precision_02_amd as dmp
    cases = [("tile", synth.make_problem("bf16", 300, 260, 192, b_col=True, seed=52)),
             ("splitk", synth.make_problem("bf16", 128, 192, 16384, seed=53)),
             ("generic", synth.make_problem("f16", 70, 33, 61, pad=1, seed=54))]
    for what, p in cases:
        flags = (1 if p.a_col else 0) | (2 if p.b_col else 0)
        lbl = dmp.plan_label(p.M, p.N, p.K, p.lda, p.ldb, p.ldc, DTYPE_CODE[p.dtype], flags)
        log(f"[beta0] {what} D:{d_type} {lbl}")
        assert what != "splitk" or "splitk=1 " not in lbl
        assert what != "generic" or lbl.startswith("generic")
        D = run_ex(handle, p, -2.0, 0.0, "f32", d_type)
        P, S = product(p)
        check_tol(p, logical(p, host_d(d_type, D)), P, S, np.zeros_like(P), -2.0, 0.0, d_type,
                  f"beta=0 {what} D:{d_type}")


def test_split_k_low_precision(handle):
    """Split-K partials are summed in fp32 and the stage runs once in the reduction."""
    p = synth.make_problem("bf16", 256, 256, 8192, seed=55)
    for c_type, d_type in [("f16", "bf16"), ("bf16", "f16"), ("f32", "bf16")]:
        Cst = store_c(c_type, p.C)
        c_exact = oracle.decode_c(c_type, Cst)
        D = run_ex(handle, p, 1.5, 0.5, c_type, d_type, Cst=Cst)
        P, S = product(p)
        check_tol(p, logical(p, host_d(d_type, D)), P, S, logical(p, c_exact), 1.5, 0.5, d_type,
                  f"splitk C:{c_type} D:{d_type}")


def test_batched_low_precision(handle):
    p = synth.make_problem("f16", 64, 64, 64, batch=300, seed=56)
    Cst = store_c("f16", p.C)
    c_exact = oracle.decode_c("f16", Cst)
    D = run_ex(handle, p, 0.5, 2.0, "f16", "f16", Cst=Cst)
    P, S = product(p)
    check_tol(p, logical(p, host_d("f16", D)), P, S, logical(p, c_exact), 0.5, 2.0, "f16",
              "batched f16->f16")


# ------------------------------------------------ exact-integer inputs: bit-exact

# (alpha, beta) per output type: powers of two, beta large enough that D needs more
# significand bits than the output type has, so the conversion rounds (with ties).
EXACT_SCALES = {"f32": (-0.5, 4.0), "f16": (-0.5, 1024.0), "bf16": (-0.5, 64.0)}


def exact_check(handle, p, d_type, c_type, pts=None, in_place=False):
    alpha, beta = EXACT_SCALES[d_type]
    Cst = store_c(c_type, p.C)
    c_exact = oracle.decode_c(c_type, Cst)
    if in_place:
        Cd = dev(Cst)
        A, B = dev(p.A), dev(p.B)
        D = run_ex(handle, p, alpha, beta, c_type, d_type, D=Cd, A=A, B=B, c_ptr=Cd.data_ptr())
    else:
        D = run_ex(handle, p, alpha, beta, c_type, d_type, Cst=Cst)
    Dg = logical(p, host_d(d_type, D))
    if pts is None:
        P, _ = product(p)
        exact = oracle.scaled_reference(P, logical(p, c_exact), alpha, beta)
        want = oracle.round_to(d_type, exact)
        # the conversion rounds somewhere, or the case would not test it
        assert d_type == "f32" or np.any(want != exact)
        bad = np.argwhere(Dg != want)
        assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[0]}"
    else:
        P, _ = oracle.gemm_points(p.dtype, p.A, p.B, np.zeros_like(p.C), pts, **p.oracle_args())
        c = c_exact.reshape(p.batch, p.M, p.ldc)[pts[:, 0], pts[:, 1], pts[:, 2]]
        want = oracle.round_to(d_type, oracle.scaled_reference(P, c, alpha, beta))
        got = Dg[pts[:, 0], pts[:, 1], pts[:, 2]]
        assert np.array_equal(got, want), "mismatch at sampled points"
    return Dg


@pytest.mark.parametrize("d_type", FLOAT_TYPES)
@pytest.mark.parametrize("name", ["C1", "C4", "C5"])
def test_exact_inputs_bit_exact(handle, name, d_type):
    """Tile (C1 shape), batched 64x64 tiles (C4) and split-K (C5) paths, every element."""
    p = synth.exact_variant(name)
    c_type = "bf16" if d_type == "f32" else d_type
    log(f"[exact-out] {name} C:{c_type} D:{d_type}")
    exact_check(handle, p, d_type, c_type)


@pytest.mark.parametrize("d_type", ["f16", "bf16"])
def test_exact_ragged_generic_and_in_place(handle, d_type):
    for (M, N, K, pad, b_col) in [(257, 263, 200, 0, True), (70, 33, 61, 1, False),
                                  (300, 260, 192, 0, False)]:
        p = synth.make_problem("f16", M, N, K, b_col=b_col, pad=pad, seed=57, ab_dist="small_int",
                               c_dist="small_int", c_range=(-8, 8))
        log(f"[exact-out] ragged {M}x{N}x{K} pad={pad} D:{d_type}")
        exact_check(handle, p, d_type, d_type)
        exact_check(handle, p, d_type, d_type, in_place=True)


def test_k_zero_scales_c(handle):
    """K = 0: D = cvt_D(beta * c) (alpha * 0 adds nothing), exactly."""
    p = synth.make_problem("bf16", 33, 45, 0, batch=2, seed=58)
    Cst = store_c("bf16", p.C)
    c_exact = oracle.decode_c("bf16", Cst)
    D = run_ex(handle, p, 3.0, 0.5, "bf16", "f16", Cst=Cst)
    want = oracle.round_to("f16", 0.5 * logical(p, c_exact))
    assert np.array_equal(logical(p, host_d("f16", D)), want)
    D0 = run_ex(handle, p, 3.0, 0.0, "f32", "bf16")
    assert np.all(logical(p, host_d("bf16", D0)) == 0.0)


# ------------------------------------------------------------------ int8

def test_int8_beta_zero_and_one(handle):
    import dense_mixed_precision_02_amd as dmp
    for (M, N, K) in [(260, 320, 208), (128, 128, 16384), (70, 33, 61)]:
        p = synth.make_problem("i8", M, N, K, seed=59, c_range=(-(1 << 20), 1 << 20))
        lbl = dmp.plan_label(M, N, K, p.lda, p.ldb, p.ldc, 2)
        log(f"[i8-ex] {M}x{N}x{K} {lbl}")
        P = oracle.gemm("i8", p.A, p.B, np.zeros_like(p.C), **p.oracle_args())
        A, B = dev(p.A), dev(p.B)
        Dt = torch.empty((p.batch, p.M, p.ldc), dtype=torch.int32, device="cuda")
        run_ex(handle, p, 1.0, 0.0, "i32", "i32", D=Dt, A=A, B=B)
        assert np.array_equal(logical(p, Dt.cpu().numpy()).astype(np.int64), P)
        Ct = dev(p.C)
        run_ex(handle, p, 1.0, 1.0, "i32", "i32", D=Dt, A=A, B=B, c_ptr=Ct.data_ptr())
        assert np.array_equal(logical(p, Dt.cpu().numpy()).astype(np.int64),
                              P + logical(p, p.C).astype(np.int64))


# ------------------------------------------------------------ argument errors

def test_invalid_output_stage_arguments(handle):
    Cf = torch.ones(8, 8, device="cuda")
    D = torch.full_like(Cf, 3.0)
    Di = torch.full((8, 8), 3, dtype=torch.int32, device="cuda")
    A = torch.zeros(8, 8, dtype=torch.int16, device="cuda")
    base = dict(A=A.data_ptr(), B=A.data_ptr(), C=Cf.data_ptr(), D=D.data_ptr(), dtype=0,
                alpha=1.0, beta=1.0, c_type=0, d_type=0)
    bad = [
        dict(dtype=2, C=Di.data_ptr(), D=Di.data_ptr()),                    # int8 with fp32 C/D
        dict(dtype=2, c_type=3, d_type=3, alpha=2.0, C=Di.data_ptr(), D=Di.data_ptr()),
        dict(dtype=2, c_type=3, d_type=3, beta=0.5, C=Di.data_ptr(), D=Di.data_ptr()),
        dict(d_type=3), dict(c_type=3), dict(c_type=9), dict(d_type=-1),
        dict(C=0),                                                          # beta != 0 needs C
        dict(C=D.data_ptr(), d_type=2),                                     # alias, types differ
        dict(D=D.data_ptr() + 2),                                           # fp32 D misaligned
        dict(c_type=1, C=Cf.data_ptr() + 1),                                # fp16 C misaligned
    ]
    for b in bad:
        a = dict(base)
        a.update(b)
        rc = handle.status_ex(a["A"], a["B"], a["C"], a["D"], 8, 8, 8, 8, 8, 8, a["dtype"], 0, 1,
                              alpha=a["alpha"], beta=a["beta"], c_type=a["c_type"],
                              d_type=a["d_type"], stream=0)
        assert rc == 1, b
    torch.cuda.synchronize()
    assert torch.all(D == 3.0) and torch.all(Di == 3)
    # beta == 0 accepts a NULL C, and an fp16 D needs only 2-byte alignment
    rc = handle.status_ex(A.data_ptr(), A.data_ptr(), 0, D.data_ptr() + 2, 8, 8, 8, 8, 8, 8, 0, 0,
                          1, alpha=1.0, beta=0.0, c_type=0, d_type=1, stream=0)
    torch.cuda.synchronize()
    assert rc == 0


def test_unaligned_low_precision_d(handle):
    """An fp16/bf16 D at a 2-byte (not 8-byte) aligned address takes element stores."""
    p = synth.make_problem("bf16", 96, 96, 128, seed=60)
    Cst = store_c("bf16", p.C)
    c_exact = oracle.decode_c("bf16", Cst)
    Dbig = torch.empty(p.M * p.ldc + 1, dtype=torch.int16, device="cuda")
    A, B, Cd = dev(p.A), dev(p.B), dev(Cst)
    handle.run_ex(A.data_ptr(), B.data_ptr(), Cd.data_ptr(), Dbig.data_ptr() + 2, p.M, p.N, p.K,
                  p.lda, p.ldb, p.ldc, 1, 0, 1, alpha=1.0, beta=1.0, c_type=OUT["bf16"],
                  d_type=OUT["bf16"], stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    Dg = oracle.decode_c("bf16", Dbig[1:].cpu().numpy().view(np.uint16)).reshape(1, p.M, p.ldc)
    P, S = product(p)
    check_tol(p, logical(p, Dg), P, S, logical(p, c_exact), 1.0, 1.0, "bf16", "unaligned D")


# ------------------------------------------------------------ torch front end

def test_torch_front_end_output_stage(handle):
    import dense_mixed_precision_02_amd as dmp
    p = synth.make_problem("bf16", 200, 136, 256, b_col=True, seed=61)
    A = torch.from_numpy(p.A[0].view(np.int16)).cuda().view(torch.bfloat16)
    Bc = torch.from_numpy(p.B[0].view(np.int16)).cuda().view(torch.bfloat16)   # (N, K)
    P, S = product(p)
    out = dmp.gemm(A, Bc.t(), None, alpha=0.5, out_dtype=torch.bfloat16)
    assert out.dtype == torch.bfloat16 and out.shape == (200, 136)
    Dg = oracle.decode_c("bf16", out.view(torch.int16).cpu().numpy().view(np.uint16))[None]
    check_tol(p, Dg, P, S, np.zeros_like(P), 0.5, 0.0, "bf16", "front end, no C")
    Ch = torch.from_numpy(store_c("f16", p.C)[0].view(np.int16)).cuda().view(torch.float16)
    out = dmp.gemm(A, Bc.t(), Ch, beta=2.0)
    assert out.dtype == torch.float32
    c_exact = oracle.decode_c("f16", store_c("f16", p.C))
    check_tol(p, out.cpu().numpy()[None].astype(np.float64), P, S, c_exact, 1.0, 2.0, "f32",
              "front end, fp16 C")
