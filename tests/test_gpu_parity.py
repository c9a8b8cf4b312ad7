"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Float paths are held to |D - D_ref| <= 4*K*2^-24*sum|a*b| + 2^-24*|c| per element;
int8 and exact-integer float inputs must match bit for bit."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import DTYPE_CODE, check_full, check_row_sums, log, logical_D, run, to_device

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


def gpu_result(handle, p, **kw):
    D = run(handle, p, **kw)
    torch.cuda.synchronize()
    return D.cpu().numpy()


# ------------------------------------------------------------------ workloads

@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5", "S1"])
def test_workload_parity(handle, name):
    """Every element of D at each workload's full size against the full oracle: int8
    bit for bit, fp16/bf16 within the per-element bound.  The row sums are an
    extra check of the same output."""
    import dense_mixed_precision_02_amd as dmp
    p = synth.config_problem(name)
    flags = (1 if p.a_col else 0) | (2 if p.b_col else 0)
    lbl = dmp.plan_label(p.M, p.N, p.K, p.lda, p.ldb, p.ldc, DTYPE_CODE[p.dtype], flags, p.batch)
    log(f"[parity] {name}: {synth.CONFIG_LABELS[name]} plan={lbl}")
    D = gpu_result(handle, p)
    r = check_full(p, D)
    check_row_sums(p, D)
    log(f"[parity] {name}: ok, every element, max err/bound {r:.3g}")


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5", "S1"])
def test_workload_exact_integer_inputs(handle, name):
    """A, B in {-1, 0, 1} and small-integer C at each workload's shape: every partial sum is
    an integer below 2^24 in magnitude, so every element must equal the oracle exactly."""
    p = synth.exact_variant(name)
    log(f"[exact] {name}")
    D = gpu_result(handle, p)
    check_full(p, D, exact=True)
    check_row_sums(p, D, exact=True)
    log(f"[exact] {name}: every element identical")


# ------------------------------------------------------------ shapes / layouts

SHAPES = [(1, 1, 8), (7, 9, 16), (33, 65, 24), (64, 64, 64), (130, 67, 136), (257, 263, 200),
          (300, 520, 1040), (520, 300, 256)]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("a_col,b_col", [(False, False), (False, True), (True, False), (True, True)])
def test_ragged_shapes_all_layouts(handle, dtype, a_col, b_col):
    for n, (M, N, K) in enumerate(SHAPES):
        if dtype == "i8" and K % 16:
            K = (K // 16 + 1) * 16
        for pad in (0, 8):
            p = synth.make_problem(dtype, M, N, K, a_col=a_col, b_col=b_col, pad=pad, seed=100 + n,
                                   c_range=(-1.0, 1.0) if dtype != "i8" else (-1000, 1000))
            log(f"[ragged] {dtype} a_col={a_col} b_col={b_col} {M}x{N}x{K} pad={pad}")
            check_full(p, gpu_result(handle, p))


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("a_col,b_col", [(False, False), (False, True), (True, False), (True, True)])
def test_tile256_ragged_edges(handle, dtype, a_col, b_col):
    """The 256x256 tile with partial tiles on both edges and a last k-tile that is only part
    full (K not a multiple of the k-tile), for every operand layout, compared in full."""
    import dense_mixed_precision_02_amd as dmp
    M, N = 4000, 4112  # 16 x 17 tiles, both edges partial
    K = 1008 if dtype == "i8" else 1000  # 7.9 int8 / 15.6 16-bit k-tiles
    p = synth.make_problem(dtype, M, N, K, a_col=a_col, b_col=b_col, seed=31,
                           c_range=(-1.0, 1.0) if dtype != "i8" else (-(1 << 20), 1 << 20))
    flags = (dmp.GEMM_A_COLMAJOR if a_col else 0) | (dmp.GEMM_B_COLMAJOR if b_col else 0)
    lbl = dmp.plan_label(M, N, K, p.lda, p.ldb, p.ldc, DTYPE_CODE[dtype], flags)
    log(f"[tile256 edges] {dtype} a_col={a_col} b_col={b_col} {M}x{N}x{K} {lbl}")
    assert lbl.startswith("tile256x256") and "splitk=1 " in lbl, lbl
    check_full(p, gpu_result(handle, p))


@pytest.mark.parametrize("dtype", ["f16", "i8"])
def test_generic_path_odd_k_and_unaligned(handle, dtype):
    """K not a multiple of the 16-byte granule, odd leading dimensions, and operands at
    an address that is not 16-byte aligned all go through the element-wise kernel."""
    import dense_mixed_precision_02_amd as dmp
    for (M, N, K, pad) in [(5, 7, 3, 0), (70, 33, 61, 1), (129, 130, 77, 3)]:
        for a_col, b_col in [(False, False), (True, True), (False, True)]:
            p = synth.make_problem(dtype, M, N, K, a_col=a_col, b_col=b_col, pad=pad, seed=7,
                                   c_range=(-1.0, 1.0) if dtype != "i8" else (-99, 99))
            log(f"[generic] {dtype} {M}x{N}x{K} pad={pad} a_col={a_col} b_col={b_col}")
            check_full(p, gpu_result(handle, p))
    # misaligned base pointers (shift by one element) on an otherwise aligned problem
    p = synth.make_problem(dtype, 96, 96, 128, seed=9,
                           c_range=(-1.0, 1.0) if dtype != "i8" else (-99, 99))
    A, B, C = to_device(p)
    A2 = torch.empty(A.numel() + 1, dtype=A.dtype, device=A.device)
    A2[1:] = A.reshape(-1)
    B2 = torch.empty(B.numel() + 1, dtype=B.dtype, device=B.device)
    B2[1:] = B.reshape(-1)
    D = torch.empty_like(C)
    handle.run(A2.data_ptr() + A.element_size(), B2.data_ptr() + B.element_size(), C.data_ptr(),
               D.data_ptr(), p.M, p.N, p.K, p.lda, p.ldb, p.ldc,
               {"f16": 0, "bf16": 1, "i8": 2}[dtype], 0, 1, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    check_full(p, D.cpu().numpy())


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
def test_split_k(handle, dtype):
    """Small M x N with long K takes the split-K path (fixed-order reduction, C added once)."""
    import dense_mixed_precision_02_amd as dmp
    for (M, N, K) in [(128, 128, 8192), (200, 96, 16384), (256, 512, 4096 + 128)]:
        p = synth.make_problem(dtype, M, N, K, seed=11,
                               c_range=(-1.0, 1.0) if dtype != "i8" else (-(1 << 20), 1 << 20))
        lbl = dmp.plan_label(M, N, K, p.lda, p.ldb, p.ldc, {"bf16": 1, "i8": 2}[dtype])
        log(f"[splitk] {dtype} {M}x{N}x{K} {lbl}")
        assert "splitk=1 " not in lbl
        check_full(p, gpu_result(handle, p))
        e = synth.make_problem(dtype, M, N, K, seed=12, ab_dist="small_int",
                               c_dist="small_int" if dtype != "i8" else "uniform_int",
                               c_range=(-8, 8))
        check_full(e, gpu_result(handle, e), exact=True)


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
def test_tile256_batched_and_batched_split_k(handle, dtype):
    """Batch entries on the 256x256 tile (one tile per workgroup across four 2048^2 products)
    and split-K over a batch of two skinny products, compared in full; the exact-integer
    inputs must come out bit for bit."""
    import dense_mixed_precision_02_amd as dmp
    for (M, N, K, batch, want) in [(2048, 2048, 512, 4, "splitk=1 "), (512, 512, 8192, 2, "splitk=")]:
        p = synth.make_problem(dtype, M, N, K, batch=batch, seed=41,
                               c_range=(-1.0, 1.0) if dtype != "i8" else (-(1 << 20), 1 << 20))
        lbl = dmp.plan_label(M, N, K, p.lda, p.ldb, p.ldc, DTYPE_CODE[dtype], 0, batch)
        log(f"[tile256 batched] {dtype} {batch} x {M}x{N}x{K} {lbl}")
        assert lbl.startswith("tile256x256") and want in lbl, lbl
        if want == "splitk=":
            assert "splitk=1 " not in lbl, lbl
        check_full(p, gpu_result(handle, p))
        e = synth.make_problem(dtype, M, N, K, batch=batch, seed=42, ab_dist="small_int",
                               c_dist="small_int" if dtype != "i8" else "uniform_int",
                               c_range=(-8, 8))
        check_full(e, gpu_result(handle, e), exact=True)


@pytest.mark.parametrize("dtype", ["f16", "i8"])
def test_batched(handle, dtype):
    for (M, N, K, batch, pad) in [(64, 64, 64, 512, 0), (17, 40, 48, 5, 0), (64, 64, 256, 3, 8),
                                  (100, 70, 96, 4, 0)]:
        p = synth.make_problem(dtype, M, N, K, batch=batch, pad=pad, seed=13,
                               c_range=(-1.0, 1.0) if dtype != "i8" else (-999, 999))
        log(f"[batched] {dtype} {batch} x {M}x{N}x{K} pad={pad}")
        check_full(p, gpu_result(handle, p))


# ------------------------------------------------------------ semantics / edges

def test_d_aliases_c(handle):
    p = synth.make_problem("bf16", 300, 260, 192, seed=21)
    A, B, C = to_device(p)
    run(handle, p, tensors=(A, B, C), D=C)
    torch.cuda.synchronize()
    check_full(p, C.cpu().numpy())


@pytest.mark.parametrize("dtype", ["f16", "i8"])
def test_k_zero_copies_c(handle, dtype):
    p = synth.make_problem(dtype, 33, 45, 0, batch=2, seed=22,
                           c_range=(-1.0, 1.0) if dtype != "i8" else (-9, 9))
    A, B, C = to_device(p)
    D = torch.full_like(C, 7)
    run(handle, p, tensors=(A, B, C), D=D)
    torch.cuda.synchronize()
    assert torch.equal(D, C)


def test_empty_is_noop(handle):
    C = torch.ones(4, 4, device="cuda")
    D = torch.full_like(C, 5.0)
    for (M, N, batch) in [(0, 4, 1), (4, 0, 1), (4, 4, 0)]:
        handle.run(0, 0, C.data_ptr(), D.data_ptr(), M, N, 4, 4, 4, 4, 0, 0, batch, 0)
    torch.cuda.synchronize()
    assert torch.all(D == 5.0)


def test_invalid_arguments_enqueue_nothing(handle):
    C = torch.ones(8, 8, device="cuda")
    D = torch.full_like(C, 3.0)
    A = torch.zeros(8, 8, dtype=torch.int16, device="cuda")
    bad = [
        dict(M=-1), dict(K=-1), dict(lda=7), dict(ldb=7), dict(ldc=7), dict(dtype=5),
        dict(flags=16), dict(batch=-1), dict(Aptr=0), dict(Cptr=0), dict(Dptr=0),
        dict(Cptr=C.data_ptr() + 2),
    ]
    for b in bad:
        args = dict(Aptr=A.data_ptr(), Bptr=A.data_ptr(), Cptr=C.data_ptr(), Dptr=D.data_ptr(),
                    M=8, N=8, K=8, lda=8, ldb=8, ldc=8, dtype=0, flags=0, batch=1)
        args.update(b)
        rc = handle.status(args["Aptr"], args["Bptr"], args["Cptr"], args["Dptr"], args["M"],
                           args["N"], args["K"], args["lda"], args["ldb"], args["ldc"],
                           args["dtype"], args["flags"], args["batch"], 0)
        assert rc == 1, b
    torch.cuda.synchronize()
    assert torch.all(D == 3.0)


def test_run_to_run_bit_identical(handle):
    for p in [synth.make_problem("bf16", 1024, 1024, 4096, b_col=True, seed=31, ab_dist="normal",
                                 c_dist="zeros"),
              synth.make_problem("bf16", 256, 256, 32768, seed=32),
              synth.make_problem("i8", 512, 384, 2048, seed=33)]:
        T = to_device(p)
        D1 = run(handle, p, tensors=T).clone()
        D2 = run(handle, p, tensors=T)
        torch.cuda.synchronize()
        assert torch.equal(D1, D2)


def test_nondefault_stream(handle):
    p = synth.make_problem("f16", 260, 300, 320, b_col=True, seed=41)
    T = to_device(p)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        D = run(handle, p, tensors=T, stream=s)
    s.synchronize()
    check_full(p, D.cpu().numpy())


def test_torch_front_end(handle):
    """dmp.gemm on torch tensors: layouts are read from strides, out= may be C."""
    import dense_mixed_precision_02_amd as dmp
    g = torch.Generator(device="cpu").manual_seed(5)
    A = (torch.rand(200, 136, generator=g) * 2 - 1).to(torch.bfloat16).cuda()
    Bt = (torch.rand(96, 136, generator=g) * 2 - 1).to(torch.bfloat16).cuda()
    C = (torch.rand(200, 96, generator=g) * 2 - 1).cuda()
    D = dmp.gemm(A, Bt.t(), C)
    ref = A.double().cpu() @ Bt.double().cpu().t() + C.double().cpu()
    sabs = A.double().abs().cpu() @ Bt.double().abs().cpu().t()
    tol = 4 * 136 * 2.0 ** -24 * sabs + 2.0 ** -24 * C.double().abs().cpu()
    torch.cuda.synchronize()
    assert torch.all((D.double().cpu() - ref).abs() <= tol)
    A8 = torch.randint(-128, 128, (3, 64, 128), dtype=torch.int8, generator=g).cuda()
    B8 = torch.randint(-128, 128, (3, 128, 32), dtype=torch.int8, generator=g).cuda()
    C8 = torch.randint(-1000, 1000, (3, 64, 32), dtype=torch.int32, generator=g).cuda()
    ref8 = torch.bmm(A8.cpu().long(), B8.cpu().long()) + C8.cpu().long()
    D8 = dmp.gemm(A8, B8, C8, out=C8)
    torch.cuda.synchronize()
    assert torch.equal(D8.cpu().long(), ref8)


def test_torch_front_end_rejects(handle):
    """Layouts the C ABI cannot express raise before anything is launched."""
    import dense_mixed_precision_02_amd as dmp
    A = torch.zeros(64, 32, dtype=torch.float16, device="cuda")
    B = torch.zeros(32, 48, dtype=torch.float16, device="cuda")
    C = torch.zeros(64, 48, device="cuda")
    bad = [
        lambda: dmp.gemm(A, B, torch.zeros(1, 48, device="cuda").expand(64, 48)),  # row stride 0
        lambda: dmp.gemm(A, B, C.t().contiguous().t()),                          # column-major C
        lambda: dmp.gemm(A, B, C[:, :47]),                                        # shape
        lambda: dmp.gemm(A, B.float(), C),                                        # dtype
        lambda: dmp.gemm(A, B, C.cpu()),                                          # device
        lambda: dmp.gemm(A[:, ::2], B[:16], C),                                   # strided k
        lambda: dmp.gemm(A, B, C, out=torch.empty(64, 48, device="cuda")[:, :47]),
        # batched A and B with a C of one batch entry: C's batch extent must match
        lambda: dmp.gemm(A.expand(3, 64, 32).contiguous(), B.expand(3, 32, 48).contiguous(),
                         torch.zeros(1, 64, 48, device="cuda")),
    ]
    for i, f in enumerate(bad):
        with pytest.raises((ValueError, TypeError)):
            f()
    torch.cuda.synchronize()


def test_int8_transposed_b_path(handle):
    """Large-M int8 with row-major B goes through a transposed copy of B; ragged N and
    K (multiples of 16) exercise the copy's edges, and a batch its batch stride."""
    import dense_mixed_precision_02_amd as dmp
    for (M, N, K, batch, pad) in [(4096, 520, 272, 1, 0), (4100, 96, 1040, 2, 16)]:
        p = synth.make_problem("i8", M, N, K, batch=batch, pad=pad, seed=61,
                               c_range=(-(1 << 20), 1 << 20))
        lbl = dmp.plan_label(M, N, K, p.lda, p.ldb, p.ldc, 2, 0, batch)
        log(f"[i8-bT] {batch} x {M}x{N}x{K} pad={pad} {lbl}")
        assert "row->col" in lbl
        check_full(p, gpu_result(handle, p))


def test_front_end_streams_get_their_own_workspace(handle):
    """Two split-K products issued on two streams without synchronising in between:
    the front end's default handle differs per stream (each has its own workspace),
    so both results are right."""
    import dense_mixed_precision_02_amd as dmp
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    probs = [synth.make_problem("bf16", 256, 256, 8192, seed=s, b_col=True) for s in (71, 72)]
    outs = []
    with torch.cuda.stream(s1):
        h1 = dmp.default_handle()
    with torch.cuda.stream(s2):
        h2 = dmp.default_handle()
    assert h1 is not h2 and h1.ptr.value != h2.ptr.value
    torch.cuda.synchronize()
    for p, st in zip(probs, (s1, s2)):
        A, B, C = to_device(p)
        with torch.cuda.stream(st):
            At = A.view(torch.bfloat16)[0]
            Bt = B.view(torch.bfloat16)[0].t()        # column-major view
            outs.append(dmp.gemm(At, Bt, C[0]))
    torch.cuda.synchronize()
    for p, D in zip(probs, outs):
        log(f"[streams] bf16 {p.M}x{p.N}x{p.K} {dmp.plan_label(p.M, p.N, p.K, p.lda, p.ldb, p.ldc, 1, 2)}")
        check_full(p, D.cpu().numpy().reshape(1, p.M, p.ldc))
    # the two streams' cached handles (and their workspaces) are released on request
    assert dmp.release_default_handles() >= 2
    assert dmp.default_handle() is not h1


@pytest.mark.parametrize("case", ["f16-subnormal-inputs", "bf16-subnormal-inputs",
                                  "bf16-subnormal-results"])
def test_subnormals_are_kept(handle, case):
    """Subnormal fp16/bf16 inputs and fp32-subnormal products are not flushed to
    zero: with C = 0 every output is a sum of tiny products that a flush would
    lose entirely, so the result must be non-zero and within the bound (whose
    S-term is itself tiny) on the tile, element-wise and tiny-batch kernels."""
    dt = case.split("-")[0]
    for (M, N, K, b_col, batch) in [(64, 64, 64, False, 1), (256, 256, 256, True, 1),
                                    (37, 41, 29, False, 1), (4, 4, 16, False, 50)]:
        p = synth.make_problem(dt, M, N, K, b_col=b_col, batch=batch, seed=5)
        rng = np.random.default_rng(6)
        sign = rng.choice([-1, 1], size=p.A.shape)
        if case == "f16-subnormal-inputs":      # m * 2^-24: fp16 subnormals
            p.A[...] = synth.f64_to_f16_bits(rng.integers(1, 1024, size=p.A.shape) * 2.0 ** -24 * sign)
        else:                                  # m * 2^-133: bf16 subnormals
            a = rng.integers(1, 128, size=p.A.shape) * 2.0 ** -133 * sign
            p.A[...] = synth.f32_to_bf16_bits(a.astype(np.float32))
        if case == "bf16-subnormal-results":   # products near 2^-140: fp32 subnormals
            b = rng.integers(1, 128, size=p.B.shape) * 2.0 ** -16
            p.B[...] = synth.f32_to_bf16_bits(b.astype(np.float32))
        p.C[...] = 0
        log(f"[subnormal] {case} {batch} x {M}x{N}x{K} b_col={b_col}")
        D = run(handle, p)
        torch.cuda.synchronize()
        Dg = logical_D(p, D.cpu().numpy())
        assert np.all(Dg != 0), "subnormal terms were flushed"
        check_full(p, D.cpu().numpy())
