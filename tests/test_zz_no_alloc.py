"""gemm_run_noalloc (fixed device scratch, no allocation) against gemm_run_ex,
the entry point it is a variant of: the same kernels run, so every output must
be identical bit for bit (int8 exactly, fp16/bf16 too, since the same
instructions run in the same order).  Two calls in a row per path, the second
on a smaller input, so the second finds the first's contents in the scratch.
Also: a plan that needs more than the scratch is refused before anything is
enqueued, and one result is held to the oracle directly."""
import numpy as np
import pytest

import synth
from gpu_util import DTYPE_CODE, check_full, log, logical_D, to_device

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def handle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_mixed_precision_02_amd as dmp
    h = dmp.Handle()
    yield h
    h.close()


def acc_code(dtype):
    import dense_mixed_precision_02_amd as dmp
    return dmp.GEMM_OUT_I32 if dtype == "i8" else dmp.GEMM_OUT_F32


def both(handle, p):
    """(D from gemm_run_ex, D from gemm_run_noalloc) for problem p, same inputs."""
    A, B, C = to_device(p)
    flags = (1 if p.a_col else 0) | (2 if p.b_col else 0)
    s = torch.cuda.current_stream().cuda_stream
    t = acc_code(p.dtype)
    outs = []
    for fn in (handle.status_ex, handle.status_noalloc):
        D = torch.full_like(C, 7)
        rc = fn(A.data_ptr(), B.data_ptr(), C.data_ptr(), D.data_ptr(), p.M, p.N, p.K, p.lda,
                p.ldb, p.ldc, DTYPE_CODE[p.dtype], flags, p.batch, 1.0, 1.0, t, t, s)
        assert rc == 0, rc
        outs.append(D)
    torch.cuda.synchronize()
    return outs[0].cpu().numpy(), outs[1].cpu().numpy()


# (dtype, M, N, K, batch, b_col): split-K products (partials in the scratch) and
# large-M int8 products with a row-major B (its transposed copy in the scratch);
# in each pair the second call is smaller than the first.
CASES = [
    [("bf16", 1024, 1024, 65536, 1, False), ("bf16", 256, 512, 8192, 1, True)],
    [("i8", 512, 384, 32768, 1, False), ("i8", 200, 96, 16384, 1, False)],
    [("i8", 4096, 520, 272, 1, False), ("i8", 4100, 96, 1040, 2, False)],
    [("f16", 384, 256, 24576, 2, True), ("f16", 128, 128, 8192, 1, False)],
]


@pytest.mark.parametrize("pair", CASES, ids=[f"{c[0][0]}-{c[0][1]}x{c[0][2]}x{c[0][3]}" for c in CASES])
def test_noalloc_matches_gemm_run_ex(handle, pair):
    import dense_mixed_precision_02_amd as dmp
    for n, (dt, M, N, K, batch, b_col) in enumerate(pair):
        p = synth.make_problem(dt, M, N, K, batch=batch, b_col=b_col, seed=500 + n,
                               c_range=(-1.0, 1.0) if dt != "i8" else (-(1 << 20), 1 << 20))
        lbl = dmp.plan_label(M, N, K, p.lda, p.ldb, p.ldc, DTYPE_CODE[dt], 2 if b_col else 0, batch)
        log(f"[noalloc] call {n + 1}: {dt} {batch} x {M}x{N}x{K} b_col={b_col} {lbl}")
        assert "splitk=1 " not in lbl or "row->col" in lbl, lbl  # the scratch is used
        ref, got = both(handle, p)
        assert np.array_equal(logical_D(p, got), logical_D(p, ref)), "noalloc differs from gemm_run_ex"
        if n == 1:
            check_full(p, got)  # and the oracle's bar itself on the second (smaller) call


def test_noalloc_refuses_beyond_the_scratch(handle):
    """A plan whose scratch exceeds the fixed array (the transposed copy of a
    16384-column row-major int8 B: 128 MiB): GEMM_ERR_SCRATCH, D untouched; the
    same product through gemm_run_ex is served (its workspace grows)."""
    import dense_mixed_precision_02_amd as dmp
    M, N, K = 4096, 16384, 8192
    lbl = dmp.plan_label(M, N, K, K, N, N, dmp.GEMM_I8)
    assert "row->col" in lbl and N * K > dmp.NOALLOC_SCRATCH_BYTES, lbl
    A = torch.zeros(M, K, dtype=torch.int8, device="cuda")
    B = torch.zeros(K, N, dtype=torch.int8, device="cuda")
    C = torch.ones(M, N, dtype=torch.int32, device="cuda")
    D = torch.full_like(C, 3)
    s = torch.cuda.current_stream().cuda_stream
    args = (A.data_ptr(), B.data_ptr(), C.data_ptr(), D.data_ptr(), M, N, K, K, N, N, dmp.GEMM_I8,
            0, 1, 1.0, 1.0, dmp.GEMM_OUT_I32, dmp.GEMM_OUT_I32, s)
    rc = handle.status_noalloc(*args)
    assert rc == dmp.GEMM_ERR_SCRATCH
    assert dmp.status_string(rc) == "GEMM_ERR_SCRATCH"
    torch.cuda.synchronize()
    assert torch.all(D == 3)
    assert handle.status_ex(*args) == 0
    torch.cuda.synchronize()
    assert torch.all(D == 1)


def test_noalloc_paths_without_scratch(handle):
    """Products that need no scratch (one tile pass, batched 64^3) give the same result."""
    for (dt, M, N, K, batch) in [("bf16", 520, 300, 256, 1), ("f16", 64, 64, 64, 64)]:
        p = synth.make_problem(dt, M, N, K, batch=batch, seed=520)
        ref, got = both(handle, p)
        assert np.array_equal(got, ref)
