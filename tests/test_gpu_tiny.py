"""GPU parity of the tiny-product path (M, N <= 16: several batch entries per
multi-block instruction) and of batches with a shared A or B (batch stride 0,
broadcast by the instruction's cbsz/abid and blgp modifiers on this path)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import DTYPE_CODE, check_full, log, run, to_device

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

A_SHARED, B_SHARED = 4, 8


@pytest.fixture(scope="module")
def handle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_mixed_precision_02_amd as dmp
    h = dmp.Handle()
    yield h
    h.close()


def gpu_result(handle, p):
    D = run(handle, p)
    torch.cuda.synchronize()
    return D.cpu().numpy()


def c_range(dtype):
    return (-1000, 1000) if dtype == "i8" else (-1.0, 1.0)


def test_workload_batched_4x4x16(handle):
    import dense_mixed_precision_02_amd as dmp
    p = synth.config_problem("T1")
    lbl = dmp.plan_label(p.M, p.N, p.K, p.lda, p.ldb, p.ldc, 0, 0, p.batch)
    log(f"[tiny] {synth.CONFIG_LABELS['T1']} plan={lbl}")
    assert lbl.startswith("tiny4x4x16b")
    r = check_full(p, gpu_result(handle, p))
    e = synth.make_problem("f16", 4, 4, 16, batch=1 << 20, seed=108, ab_dist="small_int",
                           c_dist="small_int", c_range=(-8, 8))
    check_full(e, gpu_result(handle, e), exact=True)
    log(f"[tiny] ok, max err/bound {r:.3g}")


SHAPES = [(1, 1, 1), (4, 4, 4), (3, 2, 7), (4, 1, 100), (5, 4, 16), (16, 16, 16), (9, 13, 33),
          (16, 3, 5), (2, 16, 64)]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("a_col,b_col", [(False, False), (False, True), (True, False), (True, True)])
def test_shapes_layouts_batches(handle, dtype, a_col, b_col):
    import dense_mixed_precision_02_amd as dmp
    for n, (M, N, K) in enumerate(SHAPES):
        for batch, pad in [(1, 0), (67, 1), (300, 0)]:
            p = synth.make_problem(dtype, M, N, K, batch=batch, a_col=a_col, b_col=b_col, pad=pad,
                                   seed=200 + n, c_range=c_range(dtype))
            fl = (1 if a_col else 0) | (2 if b_col else 0)
            lbl = dmp.plan_label(M, N, K, p.lda, p.ldb, p.ldc, DTYPE_CODE[dtype], fl, batch)
            assert lbl.startswith("tiny"), lbl
            log(f"[tiny] {dtype} {batch} x {M}x{N}x{K} pad={pad} a_col={a_col} b_col={b_col} {lbl}")
            check_full(p, gpu_result(handle, p))


def shared_problem(dtype, M, N, K, batch, shared, seed, b_col=False, exact=False):
    """A problem whose A (or B) is one matrix for every batch entry; returns the
    problem (with a single-matrix A/B array) and the flags."""
    kw = dict(ab_dist="small_int", c_dist="small_int" if dtype != "i8" else "uniform_int",
              c_range=(-8, 8)) if exact else dict(c_range=c_range(dtype))
    p = synth.make_problem(dtype, M, N, K, batch=batch, b_col=b_col, seed=seed, **kw)
    if "A" in shared:
        p.A = np.ascontiguousarray(p.A[:1])
    if "B" in shared:
        p.B = np.ascontiguousarray(p.B[:1])
    flags = (2 if b_col else 0) | (A_SHARED if "A" in shared else 0) | (B_SHARED if "B" in shared else 0)
    return p, flags


def run_shared(handle, p, flags):
    A, B, C = to_device(p)
    D = torch.empty_like(C)
    handle.run(A.data_ptr(), B.data_ptr(), C.data_ptr(), D.data_ptr(), p.M, p.N, p.K, p.lda, p.ldb,
               p.ldc, DTYPE_CODE[p.dtype], flags, p.batch, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return D.cpu().numpy()


def check_shared(p, flags, D, exact=False):
    sa = 0 if flags & A_SHARED else None
    sb = 0 if flags & B_SHARED else None
    args = p.oracle_args()
    Dg = D.reshape(p.batch, p.M, p.ldc)[:, :, :p.N]
    if p.dtype == "i8":
        ref = oracle.gemm("i8", p.A, p.B, p.C, **args, sa=sa, sb=sb)
        assert np.array_equal(Dg.astype(np.int64), ref)
        return
    ref, S = oracle.gemm(p.dtype, p.A, p.B, p.C, **args, sa=sa, sb=sb)
    if exact:
        assert np.array_equal(Dg.astype(np.float64), ref)
        return
    tol = oracle.float_tolerance(p.K, S, p.C[:, :p.M, :p.N])
    assert np.all(np.abs(Dg - ref) <= tol)


@pytest.mark.parametrize("shared", ["A", "B", "AB"])
@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
def test_shared_operand_batches(handle, shared, dtype):
    """Tiny shapes (broadcast by the instruction) and larger ones (batch stride 0 in
    the tiled and element-wise kernels), random and exact-integer inputs."""
    for n, (M, N, K, batch, b_col) in enumerate([(4, 4, 16, 1000, False), (3, 4, 9, 77, True),
                                                  (16, 16, 32, 301, False), (12, 7, 20, 64, True),
                                                  (96, 80, 64, 5, True), (70, 33, 61, 3, False)]):
        if dtype == "i8" and M > 16:
            K = (K + 15) // 16 * 16
        for exact in (False, True):
            p, fl = shared_problem(dtype, M, N, K, batch, shared, seed=300 + n, b_col=b_col,
                                   exact=exact)
            log(f"[shared {shared}] {dtype} {batch} x {M}x{N}x{K} b_col={b_col} exact={exact}")
            check_shared(p, fl, run_shared(handle, p, fl), exact=exact)


def test_output_stage_on_tiny_path(handle):
    """gemm_run_ex through the tiny kernel: bf16 D, no C; fp16 C, fp16 D with alpha, beta."""
    p = synth.make_problem("bf16", 4, 4, 16, batch=5000, seed=310)
    A, B, _ = to_device(p)
    D = torch.empty((p.batch, p.M, p.ldc), dtype=torch.int16, device="cuda")
    handle.run_ex(A.data_ptr(), B.data_ptr(), 0, D.data_ptr(), p.M, p.N, p.K, p.lda, p.ldb,
                  p.ldc, 1, 0, p.batch, alpha=0.5, beta=0.0, c_type=0, d_type=2,
                  stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    P, S = oracle.gemm("bf16", p.A, p.B, np.zeros_like(p.C), **p.oracle_args())
    Dg = oracle.decode_c("bf16", D.cpu().numpy().view(np.uint16))
    ref = oracle.scaled_reference(P, 0.0, 0.5, 0.0)
    tol = oracle.scaled_tolerance(p.K, S, 0.0, ref, 0.5, 0.0, "bf16")
    assert np.all(np.abs(Dg - ref) <= tol)


def test_torch_front_end_shared_a(handle):
    import dense_mixed_precision_02_amd as dmp
    p, _ = shared_problem("f16", 4, 4, 16, 2000, "A", seed=311)
    A = torch.from_numpy(p.A[0].view(np.int16)).cuda().view(torch.float16)      # (4, 16)
    B = torch.from_numpy(p.B.view(np.int16)).cuda().view(torch.float16)         # (2000, 16, 4)
    C = torch.from_numpy(p.C).cuda()
    out = dmp.gemm(A, B, C)
    assert out.shape == (2000, 4, 4)
    check_shared(p, A_SHARED, out.cpu().numpy())
