"""GPU parity of the 2:4 structured-sparse path: the compressor against the
oracle's pruning (values and index words bit for bit), and the sparse product
against the dense oracle on the pruned A."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import DTYPE_CODE, log

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


def kt_of(dtype):
    """Dense k per sparse k-tile."""
    return 128 if dtype == "i8" else 64


def kp_of(K, dtype="f16"):
    g = kt_of(dtype)
    return -(-K // g) * g


def mp_of(M):
    return -(-M // 16) * 16


def blocked(x, per_kt, fill):
    """Row-major compressed rows (batch, M, n) -> the library's blocked layout
    (batch, Mp/16, n/per_kt, 16, per_kt); padding rows hold `fill`."""
    b, M, n = x.shape
    Mp = mp_of(M)
    y = np.full((b, Mp, n), fill, dtype=x.dtype)
    y[:, :M] = x
    return y.reshape(b, Mp // 16, 16, n // per_kt, per_kt).transpose(0, 1, 3, 2, 4)


def gpu_blocked(t, dtype, per_kt, cols):
    """Device compressed array -> (batch, Mp/16, cols/per_kt, 16, per_kt)."""
    x = t.cpu().numpy()
    if x.dtype != np.int8:
        x = x.view(np.uint16)
    b, Mp = x.shape[0], x.shape[1]
    return x.reshape(b, Mp // 16, cols // per_kt, 16, per_kt)


def same_compressed(p, Ac, meta, eAc, emeta, blocks=slice(None)):
    """GPU (Ac, meta) equal to the expected row-major forms (rows of `blocks` only)."""
    kt = kt_of(p.dtype)
    kp = kp_of(p.K, p.dtype)
    ga = gpu_blocked(Ac, p.dtype, kt // 2, kp // 2)[:, blocks]
    gm = gpu_blocked(meta, p.dtype, kt // 16, kp // 16)[:, blocks]
    # rows past M: zero values, index words naming positions 0 and 1
    return (np.array_equal(ga, blocked(eAc, kt // 2, 0)) and
            np.array_equal(gm, blocked(emeta, kt // 16, 0x4444)))


def dev16(x):
    """Operand storage on the device (16-bit patterns as int16, int8 as is)."""
    x = np.ascontiguousarray(x)
    return torch.from_numpy(x if x.dtype == np.int8 else x.view(np.int16)).cuda()


def compress(handle, p, Ad=None):
    """gemm_prune24 on p's A; returns device (Ac, meta)."""
    kp, mp = kp_of(p.K, p.dtype), mp_of(p.M)
    Ad = dev16(p.A) if Ad is None else Ad
    Ac = torch.empty((p.batch, mp, kp // 2), dtype=torch.int8 if p.dtype == "i8" else torch.int16,
                     device="cuda")
    meta = torch.empty((p.batch, mp, kp // 16), dtype=torch.int16, device="cuda")
    rc = handle.prune24(Ad.data_ptr(), p.M, p.K, p.lda, DTYPE_CODE[p.dtype], p.batch,
                        Ac.data_ptr(), meta.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    return Ac, meta


def expected_compressed(p):
    """Ac and index words (row-major, M rows) built from the oracle's kept positions."""
    pruned, keep = oracle.prune24(p.dtype, p.A, p.M, p.K, p.lda, p.batch, return_keep=True)
    kp = kp_of(p.K, p.dtype)
    keep_p = np.zeros((p.batch, p.M, kp), dtype=bool)
    keep_p[:, :, :p.K] = keep
    vals = np.zeros((p.batch, p.M, kp), dtype=p.A.dtype)
    vals[:, :, :p.K] = p.A[:, :p.M, :p.K]
    # groups with fewer than two present positions keep the lowest absent ones
    g = keep_p.reshape(p.batch, p.M, kp // 4, 4)
    for q in range(4):
        need = g.sum(-1) < 2
        g[..., q] |= need & ~g[..., q] & (np.arange(kp // 4)[None, None, :] * 4 + q >= p.K)
    pos = np.argsort(~g, axis=-1, kind="stable")[..., :2]          # kept positions, ascending
    v4 = vals.reshape(p.batch, p.M, kp // 4, 4)
    Ac = np.take_along_axis(v4, pos, axis=-1).reshape(p.batch, p.M, kp // 2)
    Ac = np.where(np.take_along_axis(g, pos, -1).reshape(Ac.shape), Ac, 0).astype(p.A.dtype)
    bits = (pos[..., 0] | (pos[..., 1] << 2)).astype(np.uint32)    # 4 bits per group
    w = bits.reshape(p.batch, p.M, kp // 16, 4)
    meta = (w[..., 0] | (w[..., 1] << 4) | (w[..., 2] << 8) | (w[..., 3] << 12)).astype(np.uint16)
    return pruned, Ac, meta


def run_sparse(handle, p, Ac, meta, C=None, D=None):
    B = dev16(p.B)
    C = torch.from_numpy(p.C).cuda() if C is None else C
    D = torch.empty_like(C) if D is None else D
    rc = handle.run_sparse24(Ac.data_ptr(), meta.data_ptr(), B.data_ptr(), C.data_ptr(),
                             D.data_ptr(), p.M, p.N, p.K, p.ldb, p.ldc, DTYPE_CODE[p.dtype],
                             2 if p.b_col else 0, p.batch, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    return D.cpu().numpy()


def check(p, pruned, Dg, exact=False, pts=None):
    args = p.oracle_args()
    Dg = Dg.reshape(p.batch, p.M, p.ldc)[:, :, :p.N]
    if p.dtype == "i8":   # int32 results: bit for bit
        if pts is not None:
            ref = oracle.gemm_points(p.dtype, pruned, p.B, p.C, pts, **args)
            got = Dg[pts[:, 0], pts[:, 1], pts[:, 2]].astype(np.int64)
        else:
            ref = oracle.gemm(p.dtype, pruned, p.B, p.C, **args)
            got = Dg.astype(np.int64)
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"{len(bad)} int32 results differ, first at {bad[0]}"
        return 0.0
    if pts is not None:
        ref, S = oracle.gemm_points(p.dtype, pruned, p.B, p.C, pts, **args)
        got = Dg[pts[:, 0], pts[:, 1], pts[:, 2]].astype(np.float64)
        c = p.C[pts[:, 0], pts[:, 1], pts[:, 2]]
    else:
        ref, S = oracle.gemm(p.dtype, pruned, p.B, p.C, **args)
        got = Dg.astype(np.float64)
        c = p.C[:, :p.M, :p.N]
    if exact:
        assert np.array_equal(got, ref)
        return 0.0
    tol = oracle.float_tolerance(p.K, S, c)
    bad = np.argwhere(np.abs(got - ref) > tol)
    assert bad.size == 0, f"{len(bad)} over the bound, first at {bad[0]}"
    return float(np.max(np.abs(got - ref) / np.maximum(tol, 1e-300)))


def test_workload_4096_cubed(handle):
    p = synth.config_problem("SP1")
    log(f"[sparse] {synth.CONFIG_LABELS['SP1']}")
    Ac, meta = compress(handle, p)
    pruned, eAc, emeta = expected_compressed(p)
    assert same_compressed(p, Ac, meta, eAc, emeta), "compressed values or index words differ"
    Dg = run_sparse(handle, p, Ac, meta)
    r = check(p, pruned, Dg)
    log(f"[sparse] ok, every element, max err/bound {r:.3g}")


def test_workload_int8_8192_cubed(handle):
    p = synth.config_problem("SP2")
    log(f"[sparse] {synth.CONFIG_LABELS['SP2']}")
    Ac, meta = compress(handle, p)
    # compressor against the oracle's pruning on a block of rows (the whole
    # expected form at this size would hold ~1 GB of host temporaries)
    rows = 512
    q = synth.Problem("i8", rows, p.N, p.K, 1, p.lda, p.ldb, p.ldc, False, True,
                      np.ascontiguousarray(p.A[:, 4096:4096 + rows]), p.B[:, :1],
                      p.C[:, :rows], name="SP2 rows 4096..4607")
    _, eAc, emeta = expected_compressed(q)
    assert same_compressed(p, Ac, meta, eAc, emeta, blocks=slice(4096 // 16, (4096 + rows) // 16))
    del eAc, emeta
    C = torch.from_numpy(p.C).cuda()
    D = torch.empty_like(C)
    Dg = run_sparse(handle, p, Ac, meta, C=C, D=D)
    pruned = oracle.prune24(p.dtype, p.A, p.M, p.K, p.lda, p.batch)
    check(p, pruned, Dg)
    log("[sparse] int8 ok (every element, bit-exact)")


def test_int8_ties_and_extremes(handle):
    """Equal magnitudes of opposite sign (-v and v tie; the lower k wins), -128
    (magnitude 128, above every other value), zeros, K not a multiple of four."""
    rng = np.random.default_rng(97)
    p = synth.make_problem("i8", 200, 48, 203, c_range=(-(1 << 20), 1 << 20), seed=98)
    p.A = rng.choice(np.array([-128, -3, 3, 0, 127, -127, 1, -1], dtype=np.int8),
                     size=p.A.shape).astype(np.int8)
    Ac, meta = compress(handle, p)
    pruned, eAc, emeta = expected_compressed(p)
    assert same_compressed(p, Ac, meta, eAc, emeta)
    check(p, pruned, run_sparse(handle, p, Ac, meta))


SHAPES = [(256, 256, 64), (300, 264, 200), (1, 8, 1000), (520, 136, 64 * 5), (256, 512, 4096 + 64),
          (77, 40, 24), (264, 272, 128 * 3 + 16)]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("b_col", [False, True])
def test_shapes_layouts(handle, dtype, b_col):
    gran = 16 if dtype == "i8" else 8   # elements per 16-byte granule
    for n, (M, N, K) in enumerate(SHAPES):
        if (K if b_col else N) % gran:
            continue
        ckw = dict(c_range=(-(1 << 20), 1 << 20)) if dtype == "i8" else {}
        for batch in (1, 3):
            p = synth.make_problem(dtype, M, N, K, batch=batch, b_col=b_col, seed=400 + n, **ckw)
            log(f"[sparse] {dtype} {batch} x {M}x{N}x{K} b_col={b_col}")
            Ac, meta = compress(handle, p)
            pruned, eAc, emeta = expected_compressed(p)
            assert same_compressed(p, Ac, meta, eAc, emeta)
            check(p, pruned, run_sparse(handle, p, Ac, meta))
            # exact-integer inputs: every partial sum an integer, so bit for bit
            e = synth.make_problem(dtype, M, N, K, batch=batch, b_col=b_col, seed=500 + n,
                                   ab_dist="small_int",
                                   c_dist="uniform_int" if dtype == "i8" else "small_int",
                                   c_range=(-8, 8))
            Ac, meta = compress(handle, e)
            pruned, _, _ = expected_compressed(e)
            check(e, pruned, run_sparse(handle, e, Ac, meta), exact=True)


def test_ties_padding_and_lda(handle):
    """Tie-heavy values (many equal magnitudes, zeros), a padded lda, K not a
    multiple of four."""
    rng = np.random.default_rng(92)
    p = synth.make_problem("f16", 130, 64, 203, seed=93)
    # A with a padded leading dimension (B keeps whole 16-byte granules)
    p.lda = p.K + 5
    p.A = synth.f64_to_f16_bits(rng.choice([-1.0, 0.0, 1.0, 0.5, -0.5], size=(1, p.M, p.lda)))
    Ac, meta = compress(handle, p)
    pruned, eAc, emeta = expected_compressed(p)
    assert same_compressed(p, Ac, meta, eAc, emeta)
    check(p, pruned, run_sparse(handle, p, Ac, meta))


def test_k_zero_alias_and_invalid(handle):
    p = synth.make_problem("bf16", 64, 64, 0, seed=94)
    C = torch.from_numpy(p.C).cuda()
    D = torch.full_like(C, 5.0)
    z = torch.zeros(16, dtype=torch.int16, device="cuda")
    rc = handle.run_sparse24(z.data_ptr(), z.data_ptr(), z.data_ptr(), C.data_ptr(), D.data_ptr(),
                             64, 64, 0, 64, 64, 1, 0, 1, 0)
    torch.cuda.synchronize()
    assert rc == 0 and torch.equal(D, C)
    q = synth.make_problem("bf16", 256, 256, 128, seed=95)
    Ac, meta = compress(handle, q)
    pruned, _, _ = expected_compressed(q)
    C = torch.from_numpy(q.C).cuda()
    check(q, pruned, run_sparse(handle, q, Ac, meta, C=C, D=C))   # D aliases C
    B = dev16(q.B)
    D = torch.full_like(C, 3.0)
    bad = [dict(dtype=3), dict(dtype=5), dict(dtype=0, flags=1), dict(flags=4), dict(Bp=B.data_ptr() + 2),
           dict(N=100), dict(ldb=260), dict(ldc=100), dict(Acp=Ac.data_ptr() + 2),
           dict(dtype=2, N=248), dict(dtype=2, ldb=264)]   # int8: whole 16-element granules
    for kw in bad:
        a = dict(Acp=Ac.data_ptr(), Mp=meta.data_ptr(), Bp=B.data_ptr(), N=256, ldb=256, ldc=256,
                 dtype=1, flags=0)
        a.update(kw)
        rc = handle.run_sparse24(a["Acp"], a["Mp"], a["Bp"], C.data_ptr(), D.data_ptr(), 256,
                                 a["N"], 128, a["ldb"], a["ldc"], a["dtype"], a["flags"], 1, 0)
        assert rc == 1, kw
    torch.cuda.synchronize()
    assert torch.all(D == 3.0)


def test_torch_front_end_sparse(handle):
    """dmp.prune24 / dmp.gemm_sparse24 on tensors: 2-D bf16 with row-major and
    column-major B, a batched int8 product, a zero C, and rejected arguments."""
    import dense_mixed_precision_02_amd as dmp
    for dt, M, N, K, batch, b_col in [("bf16", 300, 256, 520, 1, False), ("bf16", 300, 256, 520, 1, True),
                                      ("i8", 130, 96, 384, 3, True), ("f16", 64, 64, 64, 2, False)]:
        kw = dict(c_range=(-(1 << 20), 1 << 20)) if dt == "i8" else {}
        p = synth.make_problem(dt, M, N, K, batch=batch, b_col=b_col, seed=610, **kw)
        log(f"[sparse torch] {dt} {batch} x {M}x{N}x{K} b_col={b_col}")
        tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "i8": torch.int8}[dt]
        A = dev16(p.A).view(tdt)
        Bs = dev16(p.B).view(tdt)                     # (batch, K, N) or (batch, N, K)
        B = Bs.transpose(-1, -2) if b_col else Bs
        C = torch.from_numpy(p.C).cuda()
        if batch == 1:
            A, B, C = A[0], B[0], C[0]
        sp = dmp.prune24(A)
        D = dmp.gemm_sparse24(sp, B, C)
        torch.cuda.synchronize()
        pruned = oracle.prune24(dt, p.A, p.M, p.K, p.lda, p.batch)
        check(p, pruned, D.cpu().numpy().reshape(p.batch, p.M, p.ldc))
        # zero C
        D0 = dmp.gemm_sparse24(sp, B)
        torch.cuda.synchronize()
        z = synth.Problem(dt, M, N, K, batch, p.lda, p.ldb, p.ldc, False, b_col, p.A, p.B,
                          np.zeros_like(p.C))
        check(z, pruned, D0.cpu().numpy().reshape(p.batch, p.M, p.ldc))
    A = torch.zeros((64, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(TypeError):
        dmp.prune24(A)
    sp = dmp.prune24(torch.zeros((64, 64), dtype=torch.float16, device="cuda"))
    with pytest.raises(TypeError):
        dmp.gemm_sparse24(sp, torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        dmp.gemm_sparse24(sp, torch.zeros((32, 64), dtype=torch.float16, device="cuda"))
