"""GPU parity of the fp64 path (GEMM_F64) against the double-double oracle.

Per element |D - D_ref| <= (2K+2)*2^-53*S + 2^-53*|c| (the fp64 instruction
rounds every step to nearest even); inputs whose every partial sum is an
integer below 2^53 must match bit for bit."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from gpu_util import log

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

F64 = 3


@pytest.fixture(scope="module")
def handle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_mixed_precision_02_amd as dmp
    h = dmp.Handle()
    yield h
    h.close()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def flags_of(p):
    return (1 if p.a_col else 0) | (2 if p.b_col else 0)


def run(handle, p, tensors=None, D=None):
    A, B, C = tensors if tensors is not None else (dev(p.A), dev(p.B), dev(p.C))
    if D is None:
        D = torch.empty_like(C)
    handle.run(A.data_ptr(), B.data_ptr(), C.data_ptr(), D.data_ptr(), p.M, p.N, p.K, p.lda,
               p.ldb, p.ldc, F64, flags_of(p), p.batch, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return D


def logical(p, X):
    return np.asarray(X).reshape(p.batch, p.M, p.ldc)[:, :, :p.N]


def check_full(p, D, exact=False):
    Dg = logical(p, D.cpu().numpy())
    Dh, Dl, S = oracle.gemm_f64(p.A, p.B, p.C, **p.oracle_args())
    assert np.all(np.isfinite(Dg))
    if exact:
        bad = np.argwhere((Dg != Dh) | (Dl != 0))
        assert bad.size == 0, f"{len(bad)} mismatches on exact inputs, first at {bad[0]}"
        return 0.0
    err = oracle.f64_error(Dg, Dh, Dl)
    tol = oracle.f64_tolerance(p.K, S, logical(p, p.C))
    bad = np.argwhere(err > tol)
    assert bad.size == 0, f"{len(bad)} over the bound, first at {bad[0]}"
    return float(np.max(err / np.maximum(tol, 1e-300)))


def check_row_sums(p, D, exact=False):
    """sum_j D_ij = sum_j C_ij + sum_k A_ik (sum_j B_kj) for every row: any dropped or
    doubled tile or k-tile breaks it."""
    Dg = logical(p, D.cpu().numpy())
    for b in range(p.batch):
        A = p.A[b][:p.K, :p.M].T if p.a_col else p.A[b][:p.M, :p.K]
        B = p.B[b][:p.N, :p.K].T if p.b_col else p.B[b][:p.K, :p.N]
        C = p.C[b][:p.M, :p.N]
        want = C.sum(1) + A @ B.sum(1)
        got = Dg[b].sum(1)
        if exact:
            assert np.array_equal(got, want), f"row sums differ in batch {b}"
            continue
        sabs = np.abs(A) @ np.abs(B).sum(1)
        u = 2.0 ** -53
        tol = (2 * p.K + 2) * u * sabs + u * np.abs(C).sum(1) \
            + 4 * (p.N + p.K) * u * (sabs + np.abs(C).sum(1) + np.abs(got))
        assert np.all(np.abs(got - want) <= tol), f"row sums over the bound in batch {b}"


def test_workload_4096_cubed(handle):
    import dense_mixed_precision_02_amd as dmp
    p = synth.config_problem("F1")
    lbl = dmp.plan_label(p.M, p.N, p.K, p.lda, p.ldb, p.ldc, F64, flags_of(p))
    log(f"[f64] {synth.CONFIG_LABELS['F1']} plan={lbl}")
    assert lbl.startswith("dtile128x128")
    D = run(handle, p)
    r = check_full(p, D)
    check_row_sums(p, D)
    log(f"[f64] ok, every element, max err/bound {r:.3g}")


def test_workload_exact_integer_inputs(handle):
    p = synth.exact_variant("F1")
    D = run(handle, p)
    check_full(p, D, exact=True)
    check_row_sums(p, D, exact=True)


SHAPES = [(1, 1, 1), (7, 9, 4), (16, 16, 16), (33, 65, 24), (130, 66, 136), (257, 264, 200),
          (300, 520, 1040), (64, 64, 31), (63, 62, 33)]


@pytest.mark.parametrize("a_col,b_col", [(False, False), (False, True), (True, False), (True, True)])
def test_ragged_shapes_all_layouts(handle, a_col, b_col):
    import dense_mixed_precision_02_amd as dmp
    for n, (M, N, K) in enumerate(SHAPES):
        for pad in (0, 1):
            p = synth.make_problem("f64", M, N, K, a_col=a_col, b_col=b_col, pad=pad, seed=80 + n)
            lbl = dmp.plan_label(M, N, K, p.lda, p.ldb, p.ldc, F64, flags_of(p))
            log(f"[f64-ragged] {M}x{N}x{K} pad={pad} a_col={a_col} b_col={b_col} {lbl}")
            check_full(p, run(handle, p))
            e = synth.make_problem("f64", M, N, K, a_col=a_col, b_col=b_col, pad=pad,
                                   seed=90 + n, ab_dist="small_int", c_dist="small_int",
                                   c_range=(-8, 8))
            check_full(e, run(handle, e), exact=True)


def test_paths_covered():
    """The ragged set reaches the 64x64 tile and the element-wise kernel in every layout."""
    import dense_mixed_precision_02_amd as dmp
    seen = set()
    for a_col in (False, True):
        for b_col in (False, True):
            for (M, N, K) in SHAPES:
                for pad in (0, 1):
                    lda = (M if a_col else K) + pad
                    ldb = (K if b_col else N) + pad
                    fl = (1 if a_col else 0) | (2 if b_col else 0)
                    seen.add(dmp.plan_label(M, N, K, lda, ldb, N + pad, F64, fl).split()[0])
    assert {"dtile64x64", "dgeneric16x16"} <= seen


def test_batched_and_large_tiles(handle):
    for (M, N, K, batch) in [(64, 64, 64, 300), (40, 72, 48, 5), (512, 512, 256, 4)]:
        p = synth.make_problem("f64", M, N, K, batch=batch, b_col=True, seed=73)
        log(f"[f64-batched] {batch} x {M}x{N}x{K}")
        check_full(p, run(handle, p))


def test_k_zero_beta_zero_alias_and_invalid(handle):
    # K = 0: D = C exactly
    p = synth.make_problem("f64", 33, 45, 0, batch=2, seed=74)
    A, B, C = dev(p.A), dev(p.B), dev(p.C)
    D = torch.full_like(C, 7.0)
    run(handle, p, tensors=(A, B, C), D=D)
    assert torch.equal(D, C)
    # beta = 0 with a NULL C
    q = synth.make_problem("f64", 200, 136, 96, seed=75)
    A, B = dev(q.A), dev(q.B)
    D = torch.empty((1, q.M, q.ldc), dtype=torch.float64, device="cuda")
    handle.run_ex(A.data_ptr(), B.data_ptr(), 0, D.data_ptr(), q.M, q.N, q.K, q.lda, q.ldb, q.ldc,
                  F64, 0, 1, alpha=1.0, beta=0.0, c_type=4, d_type=4,
                  stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    Dh, Dl, S = oracle.gemm_f64(q.A, q.B, np.zeros_like(q.C), **q.oracle_args())
    assert np.all(oracle.f64_error(D.cpu().numpy(), Dh, Dl) <= oracle.f64_tolerance(q.K, S, 0.0))
    # D aliasing C
    C = dev(q.C)
    run(handle, q, tensors=(A, B, C), D=C)
    check_full(q, C)
    # invalid output-stage arguments for fp64 inputs enqueue nothing
    Dd = torch.full((1, q.M, q.ldc), 3.0, dtype=torch.float64, device="cuda")
    for kw in [dict(c_type=0, d_type=0), dict(c_type=4, d_type=0), dict(alpha=2.0),
               dict(beta=0.5)]:
        a = dict(alpha=1.0, beta=1.0, c_type=4, d_type=4)
        a.update(kw)
        rc = handle.status_ex(A.data_ptr(), B.data_ptr(), C.data_ptr(), Dd.data_ptr(), q.M, q.N,
                              q.K, q.lda, q.ldb, q.ldc, F64, 0, 1, stream=0, **a)
        assert rc == 1, kw
    rc = handle.status(A.data_ptr() + 4, B.data_ptr(), C.data_ptr(), Dd.data_ptr(), q.M, q.N,
                       q.K, q.lda, q.ldb, q.ldc, F64, 0, 1, 0)
    assert rc == 1  # A not aligned to its element size
    torch.cuda.synchronize()
    assert torch.all(Dd == 3.0)


def test_misaligned_operands_take_the_element_path(handle):
    """8-byte but not 16-byte aligned A and B."""
    p = synth.make_problem("f64", 96, 96, 128, seed=76)
    A = torch.empty(p.A.size + 1, dtype=torch.float64, device="cuda")
    B = torch.empty(p.B.size + 1, dtype=torch.float64, device="cuda")
    A[1:] = dev(p.A).reshape(-1)
    B[1:] = dev(p.B).reshape(-1)
    C = dev(p.C)
    D = torch.empty_like(C)
    handle.run(A.data_ptr() + 8, B.data_ptr() + 8, C.data_ptr(), D.data_ptr(), p.M, p.N, p.K,
               p.lda, p.ldb, p.ldc, F64, 0, 1, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    check_full(p, D)


def test_run_to_run_bit_identical(handle):
    p = synth.make_problem("f64", 1024, 1024, 2048, seed=77)
    T = (dev(p.A), dev(p.B), dev(p.C))
    D1 = run(handle, p, tensors=T).clone()
    D2 = run(handle, p, tensors=T)
    assert torch.equal(D1, D2)


def test_torch_front_end(handle):
    import dense_mixed_precision_02_amd as dmp
    p = synth.make_problem("f64", 200, 136, 256, b_col=True, seed=78)
    A = dev(p.A[0])
    Bt = dev(p.B[0])       # (N, K): its transpose is a column-major (K, N) view
    C = dev(p.C[0])
    out = dmp.gemm(A, Bt.t(), C)
    assert out.dtype == torch.float64
    check_full(p, out[None])


def _rne_inputs(M, K, rng):
    """A (M x K) with full 52-bit mantissas and the diagonal d of B, plus two
    exact ties in row 0: (1 + 2^-52)*1.5 sits halfway between 1.5 + 2^-52 (odd
    last bit) and 1.5 + 2^-51 (even), (1 + 3*2^-52)*1.5 halfway between
    1.5 + 4*2^-52 (even) and 1.5 + 5*2^-52 (odd)."""
    A = np.ldexp(1.0 + rng.integers(0, 1 << 52, size=(M, K)) * 2.0 ** -52,
                 rng.integers(-20, 21, size=(M, K))) * rng.choice([-1.0, 1.0], size=(M, K))
    d = np.ldexp(1.0 + rng.integers(0, 1 << 52, size=K) * 2.0 ** -52, rng.integers(-20, 21, size=K))
    A[0, 0], A[0, 1] = 1.0 + 2.0 ** -52, 1.0 + 3 * 2.0 ** -52
    d[0] = d[1] = 1.5
    return A, d


@pytest.mark.parametrize("shape", [(256, 256), (2048, 2048), (37, 37)],
                         ids=["dtile64", "dtile128", "dgeneric"])
def test_products_round_to_nearest_even(handle, shape):
    """The fp64 matrix instruction rounds products to nearest, ties to even (the
    FP64-accumulate builtins section of the CDNA2 dense MFMA builtins page; round
    toward zero is what it does not do).  With B = diag(d) every output holds one
    nonzero product and every other step adds an exact zero, so D_ij must be
    exactly the correctly rounded a_ij * d_j, which numpy's fp64 product is.
    Round toward zero would miss about half of the elements and both ties; round
    half away from zero would miss the second tie."""
    import dense_mixed_precision_02_amd as dmp
    M, K = shape
    rng = np.random.default_rng(91)
    A, d = _rne_inputs(M, K, rng)
    B = np.diag(d)
    want = A * d[None, :]
    assert want[0, 0] == 1.5 + 2.0 ** -51 and want[0, 1] == 1.5 + 4 * 2.0 ** -52
    for i, j in [(0, 0), (0, 1), (1, 2), (M - 1, K - 1)]:
        assert want[i, j] == float(Fraction(A[i, j]) * Fraction(d[j]))
    label = dmp.plan_label(M, K, K, K, K, K, F64, 0).split()[0]
    log(f"[f64-rne] {M}x{K}x{K} path {label}")
    Ad, Bd = dev(A), dev(B)
    C = torch.zeros((M, K), dtype=torch.float64, device="cuda")
    D = torch.empty_like(C)
    handle.run(Ad.data_ptr(), Bd.data_ptr(), C.data_ptr(), D.data_ptr(), M, K, K, K, K, K, F64, 0, 1,
               torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = D.cpu().numpy()
    assert got[0, 0] == want[0, 0] and got[0, 1] == want[0, 1], "ties not rounded to even"
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} products not rounded to nearest, first at {bad[0]}"


def test_rne_shapes_reach_every_fp64_path():
    import dense_mixed_precision_02_amd as dmp
    seen = {dmp.plan_label(M, K, K, K, K, K, F64, 0).split()[0] for M, K in
            [(256, 256), (2048, 2048), (37, 37)]}
    assert seen == {"dtile64x64", "dtile128x128", "dgeneric16x16"}, seen


def test_subnormal_inputs_are_kept(handle):
    """fp64 subnormal A (m * 2^-1060) times ordinary B with C = 0: a flush would
    return zeros; the results must be non-zero and within the fp64 bound on the
    tile and element-wise kernels."""
    for (M, N, K) in [(128, 128, 64), (37, 37, 37)]:
        p = synth.make_problem("f64", M, N, K, seed=81)
        rng = np.random.default_rng(82)
        p.A[...] = np.ldexp(rng.integers(1, 1 << 20, size=p.A.shape).astype(np.float64), -1060) \
            * rng.choice([-1.0, 1.0], size=p.A.shape)
        p.C[...] = 0
        log(f"[f64-subnormal] {M}x{N}x{K}")
        D = run(handle, p)
        assert np.all(logical(p, D.cpu().numpy()) != 0), "subnormal terms were flushed"
        check_full(p, D)
