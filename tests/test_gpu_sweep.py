"""Seeded random sweep of gemm_run and gemm_run_ex against the oracle.

Each case draws a type (fp16, bf16, int8, fp64), sizes from a list that
straddles every tile edge (1 ... 300, sometimes up to 1024; K 0 ... 4096, half
of the time a multiple of 16), a batch of 1 to 3 (or up to 70 for tiny
products), both layouts of A and B, a leading-dimension padding of
0, 1 or 8 elements (odd paddings send the product to the element-wise kernel),
and sometimes a shared A or B.  A quarter of the fp16/bf16 cases go through
gemm_run_ex with random alpha, beta and C/D storage types.  Every result is
compared with the oracle in full: int8 bit for bit, floats within their bounds.
The sweep must reach every kernel path."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import log

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

CODE = {"f16": 0, "bf16": 1, "i8": 2, "f64": 3}
OUT = {"f32": 0, "f16": 1, "bf16": 2}
A_SHARED, B_SHARED = 4, 8
DIMS = [1, 3, 4, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 200, 255, 256, 257, 300]
BIG = [384, 512, 640, 1024]
KS = [0, 1, 4, 7, 8, 15, 16, 17, 63, 64, 65, 127, 128, 129, 255, 256, 257, 520]
KS_ALIGNED = [16, 64, 128, 256, 512, 1024, 2048, 4096]
CHUNKS, PER_CHUNK = 10, 50
MAX_MACS = 1.5e8


@pytest.fixture(scope="module")
def handle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_mixed_precision_02_amd as dmp
    h = dmp.Handle()
    yield h
    h.close()


def dev(x):
    x = np.ascontiguousarray(x)
    return torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).cuda()


def draw_case(rng):
    dt = ["f16", "bf16", "i8", "f64"][rng.integers(4)]
    M, N = (int(rng.choice(BIG if rng.random() < 0.2 else DIMS)) for _ in range(2))
    K = int(rng.choice(KS_ALIGNED if rng.random() < 0.5 else KS))
    tiny = M <= 16 and N <= 16 and dt != "f64"
    batch = int(rng.integers(1, 71)) if tiny and rng.random() < 0.5 else int(rng.integers(1, 4))
    if M * N * K * batch > MAX_MACS:       # keep the oracle's share of the sweep to seconds
        K = max(16, int(MAX_MACS // (M * N * batch)) // 16 * 16)
    if rng.random() < 0.06:                # a large shape: 256x256 and 128x128 tiles, split-K
        M, N, K = [(4096, 4096, 64), (1024, 1024, 4096), (2048, 1024, 1024),
                   (2048, 2048, 512)][rng.integers(4)]
        batch = 1
    a_col, b_col = bool(rng.integers(2)), bool(rng.integers(2))
    pad = int(rng.choice([0, 0, 0, 8, 1]))
    shared = ["", "", "", "", "A", "B", "AB"][rng.integers(7)] if batch > 1 else ""
    ex = None
    if dt in ("f16", "bf16") and rng.random() < 0.25:
        ex = dict(alpha=float(rng.choice([1.0, 0.5, -2.0, 0.75])),
                  beta=float(rng.choice([0.0, 1.0, -1.25, 2.0])),
                  c_type=str(rng.choice(["f32", "f16", "bf16"])),
                  d_type=str(rng.choice(["f32", "f16", "bf16"])))
    return dt, M, N, K, batch, a_col, b_col, pad, shared, ex


def store_c(c_type, C):
    if c_type == "f32":
        return C
    if c_type == "f16":
        return synth.f64_to_f16_bits(C.astype(np.float64))
    return synth.f32_to_bf16_bits(C.astype(np.float32))


PATHS = set()


@pytest.mark.parametrize("chunk", range(CHUNKS))
def test_random_sweep_against_the_oracle(handle, chunk):
    import dense_mixed_precision_02_amd as dmp
    rng = np.random.default_rng(2026 + chunk)
    paths = PATHS
    for n in range(chunk * PER_CHUNK, (chunk + 1) * PER_CHUNK):
        dt, M, N, K, batch, a_col, b_col, pad, shared, ex = draw_case(rng)
        kw = dict(c_range=(-(1 << 20), 1 << 20)) if dt == "i8" else {}
        p = synth.make_problem(dt, M, N, K, batch=batch, a_col=a_col, b_col=b_col, pad=pad,
                               seed=5000 + n, **kw)
        if "A" in shared:
            p.A = np.ascontiguousarray(p.A[:1])
        if "B" in shared:
            p.B = np.ascontiguousarray(p.B[:1])
        flags = (1 if a_col else 0) | (2 if b_col else 0) | \
                (A_SHARED if "A" in shared else 0) | (B_SHARED if "B" in shared else 0)
        label = dmp.plan_label(M, N, K, p.lda, p.ldb, p.ldc, CODE[dt], flags, batch)
        paths.add(label.split()[0] + (" split" if "splitk=1 " not in label + " " else "") +
                  (" one-ktile" if label.endswith("one-ktile") else ""))
        log(f"[sweep {n}] {dt} {batch} x {M}x{N}x{K} a_col={a_col} b_col={b_col} pad={pad} "
            f"shared={shared or '-'} ex={ex} {label}")
        A, B = dev(p.A), dev(p.B)
        s = torch.cuda.current_stream().cuda_stream
        sa = 0 if "A" in shared else None
        sb = 0 if "B" in shared else None
        args = p.oracle_args()
        if ex is None:
            C = dev(p.C)
            D = torch.empty_like(C)
            handle.run(A.data_ptr(), B.data_ptr(), C.data_ptr(), D.data_ptr(), M, N, K, p.lda,
                       p.ldb, p.ldc, CODE[dt], flags, batch, s)
            torch.cuda.synchronize()
            Dg = D.cpu().numpy().reshape(batch, M, p.ldc)[:, :, :N]
            if dt == "i8":
                ref = oracle.gemm("i8", p.A, p.B, p.C, **args, sa=sa, sb=sb)
                assert np.array_equal(Dg.astype(np.int64), ref), f"case {n}"
            elif dt == "f64":
                Dh, Dl, S = oracle.gemm_f64(p.A, p.B, p.C, **args, sa=sa, sb=sb)
                err = oracle.f64_error(Dg, Dh, Dl)
                tol = oracle.f64_tolerance(K, S, p.C[:, :M, :N])
                assert np.all(err <= tol), f"case {n}: {np.max(err / np.maximum(tol, 1e-300))}"
            else:
                ref, S = oracle.gemm(dt, p.A, p.B, p.C, **args, sa=sa, sb=sb)
                tol = oracle.float_tolerance(K, S, p.C[:, :M, :N])
                err = np.abs(Dg.astype(np.float64) - ref)
                assert np.all(err <= tol), f"case {n}: {np.max(err / np.maximum(tol, 1e-300))}"
            continue
        # output stage: D = cvt_D(alpha*AB + beta*cvt(C))
        Cst = store_c(ex["c_type"], p.C)
        C = dev(Cst)
        D = torch.empty(p.C.shape, dtype=torch.float32 if ex["d_type"] == "f32" else torch.int16,
                        device="cuda")
        handle.run_ex(A.data_ptr(), B.data_ptr(), C.data_ptr() if ex["beta"] != 0 else 0,
                      D.data_ptr(), M, N, K, p.lda, p.ldb, p.ldc, CODE[dt], flags, batch,
                      alpha=ex["alpha"], beta=ex["beta"], c_type=OUT[ex["c_type"]],
                      d_type=OUT[ex["d_type"]], stream=s)
        torch.cuda.synchronize()
        Dh = D.cpu().numpy()
        Dg = (Dh if ex["d_type"] == "f32" else
              oracle.decode_c(ex["d_type"], Dh.view(np.uint16))).reshape(batch, M, p.ldc)[:, :, :N]
        c_exact = oracle.decode_c(ex["c_type"], Cst).reshape(batch, M, p.ldc)[:, :, :N]
        P, S = oracle.gemm(dt, p.A, p.B, np.zeros_like(p.C), **args, sa=sa, sb=sb)
        ref = oracle.scaled_reference(P, c_exact, ex["alpha"], ex["beta"])
        tol = oracle.scaled_tolerance(K, S, c_exact, ref, ex["alpha"], ex["beta"], ex["d_type"])
        err = np.abs(np.asarray(Dg, dtype=np.float64) - ref)
        assert np.all(err <= tol), f"case {n}: {np.max(err / np.maximum(tol, 1e-300))}"


def test_sweep_reached_every_path():
    """Runs after the chunks (file order): every kernel path was exercised."""
    if len(PATHS) == 0:
        pytest.skip("the sweep did not run")
    log(f"[sweep] paths reached: {sorted(PATHS)}")
    for need in ("tile64x64", "tile64x64 one-ktile", "tile128x128", "tile256x256", "generic32x32", "tiny4x4x16b",
                 "tiny16x16x4b", "dtile64x64", "dgeneric16x16", "copy",
                 "tile256x256 split", "tile64x64 split"):
        assert any(x.startswith(need) for x in PATHS), (need, sorted(PATHS))


SP_CHUNKS, SP_PER_CHUNK = 4, 30


@pytest.mark.parametrize("chunk", range(SP_CHUNKS))
def test_random_sparse_sweep_against_the_oracle(handle, chunk):
    """The 2:4 path: random type, sizes, batch, B layout and padding (B's leading
    dimension stays a whole number of 16-byte granules, as the entry point
    requires); the compressed form must equal the one built from the oracle's
    kept positions, and the product the oracle's product of the pruned A."""
    from test_gpu_sparse import check, compress, expected_compressed, run_sparse, same_compressed
    rng = np.random.default_rng(3030 + chunk)
    for n in range(chunk * SP_PER_CHUNK, (chunk + 1) * SP_PER_CHUNK):
        dt = ["f16", "bf16", "i8"][rng.integers(3)]
        gran = 16 if dt == "i8" else 8
        b_col = bool(rng.integers(2))
        M = int(rng.choice(DIMS + BIG[:2]))
        N = int(rng.choice(DIMS + BIG[:2]))
        K = int(rng.choice(KS + KS_ALIGNED[:6]))
        if b_col:
            K = max(gran, (K + gran - 1) // gran * gran)
        else:
            N = max(gran, (N + gran - 1) // gran * gran)
        batch = int(rng.integers(1, 4))
        if M * N * K * batch > MAX_MACS:
            K = max(gran * 8, int(MAX_MACS // (M * N * batch)) // (gran * 8) * (gran * 8))
        pad = int(rng.choice([0, gran]))
        kw = dict(c_range=(-(1 << 20), 1 << 20)) if dt == "i8" else {}
        p = synth.make_problem(dt, M, N, K, batch=batch, b_col=b_col, pad=pad, seed=7000 + n, **kw)
        log(f"[sparse sweep {n}] {dt} {batch} x {M}x{N}x{K} b_col={b_col} pad={pad}")
        Ac, meta = compress(handle, p)
        pruned, eAc, emeta = expected_compressed(p)
        assert same_compressed(p, Ac, meta, eAc, emeta), f"case {n}: compressed form"
        check(p, pruned, run_sparse(handle, p, Ac, meta))
