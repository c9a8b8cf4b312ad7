"""int8 products accumulate in int32 modulo 2^32 on every path.

Wrapping addition is associative, so a result whose true value fits int32 is
exact even when partial sums leave the int32 range on the way: in the MFMA
accumulators of one long K loop (256/64-tile, any-alignment and tiny-batch
kernels) or in the split-K reduction.  A true result outside the range comes
back reduced modulo 2^32 into [-2^31, 2^31).

Inputs are built so the exact result is a closed form: A is constant along
each row (a_i), and column j of B holds -128 in its first h_j entries and 127
in the rest, so

    D_ij = C_ij + a_i * (127 K - 255 h_j),

and for |a_i| = 128 the running sum of the first h_j products is 16384 h_j,
beyond 2^31 - 1 for every h_j > 131072.  The oracle (int64, no wrapping)
confirms the closed form at sampled positions."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import log

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

I8 = 2


@pytest.fixture(scope="module")
def handle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_mixed_precision_02_amd as dmp
    h = dmp.Handle()
    yield h
    h.close()


def wrap32(x):
    return ((np.asarray(x, dtype=np.int64) + (1 << 31)) % (1 << 32)) - (1 << 31)


def overflow_problem(M, N, K, batch, b_col, seed):
    """Row-constant A, two-valued B columns, small C; every row with |a_i| >= 100
    overflows its partial sums, every final value fits int32."""
    rng = np.random.default_rng(seed)
    a = rng.integers(-128, 128, size=(batch, M)).astype(np.int64)
    a[:, 0], a[:, -1] = -128, 127
    lo = -(-(127 * K - ((1 << 31) - (1 << 21)) // 128) // 255)   # |127K - 255h| * 128 < 2^31 - 2^21
    hi = (127 * K + ((1 << 31) - (1 << 21)) // 128) // 255
    lo = max(lo, 131073 if K > 131073 else 0)
    assert lo <= hi <= K, (lo, hi, K)
    h = rng.integers(lo, hi + 1, size=(batch, N)).astype(np.int64)
    A = np.empty((batch, M, K), dtype=np.int8)
    A[...] = a[:, :, None].astype(np.int8)
    Bnk = np.full((batch, N, K), 127, dtype=np.int8)      # column j of B as a row
    for b in range(batch):
        for j in range(N):
            Bnk[b, j, :h[b, j]] = -128
    B = Bnk if b_col else np.ascontiguousarray(Bnk.transpose(0, 2, 1))
    C = rng.integers(-(1 << 20), 1 << 20, size=(batch, M, N)).astype(np.int32)
    want = C.astype(np.int64) + a[:, :, None] * (127 * K - 255 * h[:, None, :])
    assert np.all(np.abs(want) < (1 << 31))
    assert np.max(np.abs(a)) * 128 * np.max(h) >= (1 << 31)   # some partial sum overflows
    p = synth.Problem("i8", M, N, K, batch, K, K if b_col else N, N, False, b_col, A, B, C)
    return p, want


CASES = [
    # (M, N, K, batch, b_col, expected path)
    (4096, 4096, 139264, 1, True, "tile256x256 i8 a:row b:col splitk=1"),
    (4096, 64, 139264, 1, False, "tile64x64 i8 a:row b:row->col splitk=1"),
    (256, 256, 262144, 1, False, "tile256x256 i8 a:row b:row splitk=256"),
    (2048, 2048, 196608, 1, True, "tile256x256 i8 a:row b:col splitk=4"),
    (40, 40, 262143, 1, False, "generic32x32"),
    (16, 16, 262144, 6, False, "tiny16x16x4b"),
    (4, 4, 262144, 20, True, "tiny4x4x16b"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[3]}x{c[0]}x{c[1]}x{c[2]}-{'bcol' if c[4] else 'brow'}")
def test_partial_sums_beyond_int32_final_exact(handle, case):
    import dense_mixed_precision_02_amd as dmp
    M, N, K, batch, b_col, path = case
    p, want = overflow_problem(M, N, K, batch, b_col, seed=M + N + batch)
    label = dmp.plan_label(M, N, K, p.lda, p.ldb, p.ldc, I8, 2 if b_col else 0, batch)
    log(f"[int-wrap] {batch} x {M}x{N}x{K} b_col={b_col}: {label}")
    assert label.startswith(path), label
    pts = np.array([(b, i, j) for b in {0, batch - 1} for i in {0, M // 2, M - 1}
                    for j in {0, N // 3, N - 1}], dtype=np.int64)
    ref = oracle.gemm_points("i8", p.A, p.B, p.C, pts, **p.oracle_args())
    assert np.array_equal(ref, want[pts[:, 0], pts[:, 1], pts[:, 2]]), "closed form"
    A, B, C = (torch.from_numpy(x).cuda() for x in (p.A, p.B, p.C))
    D = torch.empty_like(C)
    handle.run(A.data_ptr(), B.data_ptr(), C.data_ptr(), D.data_ptr(), M, N, K, p.lda, p.ldb,
               p.ldc, I8, 2 if b_col else 0, batch, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = D.cpu().numpy().astype(np.int64)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[0]}"


@pytest.mark.parametrize("shape", [(256, 256, 64, 1), (40, 40, 63, 1), (8, 8, 64, 30)],
                         ids=["tile", "generic", "tiny"])
def test_results_beyond_int32_wrap(handle, shape):
    """C within 2^14 of INT32_MAX (first half of the rows) or INT32_MIN (second
    half) plus full-range int8 products: about half of the results leave the
    int32 range and must come back as the true value modulo 2^32."""
    M, N, K, batch = shape
    p = synth.make_problem("i8", M, N, K, batch=batch, seed=93)
    rng = np.random.default_rng(94)
    off = rng.integers(0, 1 << 14, size=(batch, M, N))
    C = np.where(np.arange(M)[None, :, None] < M // 2, (1 << 31) - 1 - off, -(1 << 31) + off)
    p.C[...] = C.astype(np.int32)
    exact = oracle.gemm("i8", p.A, p.B, p.C, **p.oracle_args())
    assert np.mean(np.abs(exact) >= (1 << 31)) > 0.25
    log(f"[int-wrap] final {batch} x {M}x{N}x{K}")
    A, B, Cd = (torch.from_numpy(x).cuda() for x in (p.A, p.B, p.C))
    D = torch.empty_like(Cd)
    handle.run(A.data_ptr(), B.data_ptr(), Cd.data_ptr(), D.data_ptr(), M, N, K, p.lda, p.ldb,
               p.ldc, I8, 0, batch, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = D.cpu().numpy().astype(np.int64).reshape(batch, M, p.ldc)[:, :, :N]
    assert np.array_equal(got, wrap32(exact))


def test_sparse_partial_sums_beyond_int32_final_exact(handle):
    """The 2:4 int8 product: A holds a_i at k = 0, 1 (mod 4) and zeros at k = 2, 3,
    so the compressor keeps exactly the a_i entries; with c_j = #{k < h_j : k mod 4 < 2}
    D_ij = C_ij + a_i (127 K/2 - 255 c_j), and a running sum of a row with
    a_i = -128 passes 2^31 once c_j > 131072."""
    from test_gpu_sparse import compress, run_sparse
    M = N = 512
    K = 786432
    rng = np.random.default_rng(95)
    a = rng.integers(-128, 128, size=M).astype(np.int64)
    a[0], a[-1] = -128, 127
    L = ((1 << 31) - (1 << 21)) // 128
    cmax = (127 * K // 2 + L) // 255
    h = rng.integers(2 * 131073 + 4, 2 * cmax - 4, size=N).astype(np.int64)
    cnt = 2 * (h // 4) + np.minimum(h % 4, 2)
    assert cnt.min() > 131072 and cnt.max() <= cmax
    A = np.zeros((1, M, K), dtype=np.int8)
    A[0, :, 0::4] = a[:, None].astype(np.int8)
    A[0, :, 1::4] = a[:, None].astype(np.int8)
    Bnk = np.full((1, N, K), 127, dtype=np.int8)
    for j in range(N):
        Bnk[0, j, :h[j]] = -128
    C = rng.integers(-(1 << 20), 1 << 20, size=(1, M, N)).astype(np.int32)
    want = C.astype(np.int64) + a[None, :, None] * (127 * K // 2 - 255 * cnt[None, None, :])
    assert np.all(np.abs(want) < (1 << 31))
    p = synth.Problem("i8", M, N, K, 1, K, K, N, False, True, A, Bnk, C)
    pts = np.array([(0, i, j) for i in (0, 100, M - 1) for j in (0, 7, N - 1)], dtype=np.int64)
    pruned = oracle.prune24("i8", A[:, :, :4096], M, 4096, 4096, 1)
    assert np.array_equal(pruned, A[:, :, :4096]), "the compressor keeps the a_i entries"
    assert np.array_equal(oracle.gemm_points("i8", A, Bnk, C, pts, **p.oracle_args()),
                          want[0][pts[:, 1], pts[:, 2]])
    log(f"[int-wrap] sparse {M}x{N}x{K}")
    Ac, meta = compress(handle, p)
    got = run_sparse(handle, p, Ac, meta).astype(np.int64)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[0]}"


def test_sparse_results_beyond_int32_wrap(handle):
    from test_gpu_sparse import compress, run_sparse
    M, N, K = 256, 256, 256
    p = synth.make_problem("i8", M, N, K, b_col=True, seed=96)
    rng = np.random.default_rng(97)
    off = rng.integers(0, 1 << 13, size=(1, M, N))
    C = np.where(np.arange(M)[None, :, None] < M // 2, (1 << 31) - 1 - off, -(1 << 31) + off)
    p.C[...] = C.astype(np.int32)
    pruned = oracle.prune24("i8", p.A, M, K, p.lda, 1)
    exact = oracle.gemm("i8", pruned, p.B, p.C, **p.oracle_args())
    assert np.mean(np.abs(exact) >= (1 << 31)) > 0.25
    log(f"[int-wrap] sparse final {M}x{N}x{K}")
    Ac, meta = compress(handle, p)
    got = run_sparse(handle, p, Ac, meta).astype(np.int64).reshape(1, M, p.ldc)[:, :, :N]
    assert np.array_equal(got, wrap32(exact))
