#!/usr/bin/env python3
"""Throughput of the gfx950 GEMM D = A*B + C on one MI355X.

Default workload: the single 4096 x 4096 x 4096 bf16 GEMM (A row-major, B
column-major, A and B drawn from N(0,1) with a fixed seed, C fp32 zeros, fp32
accumulation).  One "step" is one gemm_run call on that problem, with inputs
already resident in HBM.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C2] [--no-cpu]

--config picks another workload (C1, C3, C4, C5, S1; F1 fp64; SP1, SP2 with a
2:4-sparse A; T1 tiny batched products); the headline line is the default one.
--rotate N times the steps over N device copies of the operands (default 4 for
the bandwidth-bound C4, C5 and T1), so no step finds its inputs in the
memory-side cache.  --d-type / --c-type /
--alpha / --beta time the scaled, converted output stage instead
(D = cvt_D(alpha*A*B + beta*C) through gemm_run_ex; --c-type none means beta = 0
and no C read).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Published MI355X dense peaks (256 CUs x 2.4 GHz): fp16/bf16 4096 FLOP/clk/CU,
# int8 8192 OP/clk/CU, fp64 matrix 128 FLOP/clk/CU; HBM3E 8 TB/s.
PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "i8": 5033.2, "f64": 78.6}
# the sparse instructions do the dense-equivalent work of a 2:4 A at twice the dense rate
SPARSE_PEAK_TFLOPS = {"f16": 5033.2, "bf16": 5033.2, "i8": 10066.4}
SPARSE_CONFIGS = {"SP1", "SP2"}
PEAK_HBM_GBS = 8000.0
DTYPE_CODE = {"f16": 0, "bf16": 1, "i8": 2, "f64": 3}
# Configs whose bounding roof is HBM rather than the matrix cores (arithmetic
# intensity below the ~315 FLOP/byte ridge).
HBM_BOUND = {"C4", "T1"}
# Configs whose HBM traffic matters: the timed steps rotate over ROTATE_SETS
# device copies of the operands and outputs, so that a step does not find its
# inputs in the 256 MB memory-side cache.  D is stored non-temporally and does
# not enter that cache, so what must exceed it is the inputs read (A, B, C):
# 268 MB per set for the batched 64^3 products.  Two such sets still gave 18 %
# cache hits in time (62 against 75.5 us per step); three and four sets gave
# the same 75.5 us.  Four sets put every rotated workload's reads above 1 GB.
ROTATE = {"C4", "C5", "T1"}
ROTATE_SETS = 4
METRIC = "GEMM TFLOPS/TOPS (fp16, bf16, int8) on 1 MI355X; % of dense MFMA peak"
COPY_BYTES = 512 << 20
# rocprofv3 HBM-traffic summary of the dominant kernel of each workload
TRAFFIC_FILES = {
    "C1": "profiles/tile_gemm_f16_256x256x256_traffic.md",
    "C2": "profiles/tile16_gemm_bf16_4096x4096x4096_traffic.md",
    "C3": "profiles/tile16_gemm_i8_8192x8192x8192_traffic.md",
    "C4": "profiles/tile_gemm_f16_batch8192_64x64x64_traffic.md",
    "C5": "profiles/tile16_gemm_splitk_bf16_1024x1024x65536_traffic.md",
    "S1": "profiles/tile16_gemm_f16_4096x4096x4096_traffic.md",
    "F1": "profiles/dgemm_tile_f64_4096x4096x4096_traffic.md",
    "SP1": "profiles/sparse_gemm_bf16_4096x4096x4096_traffic.md",
    "SP2": "profiles/sparse_gemm_i8_8192x8192x8192_traffic.md",
    "T1": "profiles/tiny_gemm_f16_batch1048576_4x4x16_traffic.md",
}


OUT_SIZE = {"f32": 4, "f16": 2, "bf16": 2, "i32": 4, "none": 0}


def algorithmic_bytes(p, c_type=None, d_type=None, sparse=False) -> int:
    """Compulsory HBM traffic of one call: A, B and C read once, D written once
    (a 2:4 A: its kept half plus four index bits per group of four k)."""
    elems = p.C.size
    csz = p.C.itemsize if c_type is None else OUT_SIZE[c_type]
    dsz = p.C.itemsize if d_type is None else OUT_SIZE[d_type]
    a_bytes = p.A.nbytes
    if sparse:
        a_bytes = p.batch * p.M * p.K * (p.A.itemsize // 2 if p.A.itemsize > 1 else 0.5) \
            + p.batch * p.M * p.K // 8
    return int(a_bytes + p.B.nbytes + elems * (csz + dsz))


def store_c(c_type, C):
    """C values in the storage of c_type (input generation only)."""
    import numpy as np

    import synth
    if c_type == "f16":
        return synth.f64_to_f16_bits(C.astype(np.float64))
    if c_type == "bf16":
        return synth.f32_to_bf16_bits(C.astype(np.float32))
    return C


def cpu_baseline(p, budget_s: float = 15.0):
    """The CPU oracle (as it stands) on a bounded row sample of the same problem."""
    import numpy as np

    import oracle
    threads = min(oracle.default_threads(), 16)

    def ref(dtype, A, B, C, **kw):
        if dtype == "f64":
            return oracle.gemm_f64(A, B, C, **kw)
        return oracle.gemm(dtype, A, B, C, **kw)

    def run_rows(r):
        if p.batch > 1:
            nb = max(1, min(p.batch, r))
            A = p.A[:nb]
            B = p.B[:nb]
            C = p.C[:nb]
            t = time.perf_counter()
            ref(p.dtype, A, B, C, M=p.M, N=p.N, K=p.K, lda=p.lda, ldb=p.ldb, ldc=p.ldc,
                a_col=p.a_col, b_col=p.b_col, batch=nb, nthreads=threads)
            return time.perf_counter() - t, 2 * nb * p.M * p.N * p.K, f"{nb} of {p.batch} batch entries"
        r = max(1, min(p.M, r))
        if p.a_col:
            A = p.A  # column-major A: rows are a strided subset; pass the whole operand
            C = np.ascontiguousarray(p.C[:, :r, :])
            M = r
        else:
            A = np.ascontiguousarray(p.A[:, :r, :])
            C = np.ascontiguousarray(p.C[:, :r, :])
            M = r
        t = time.perf_counter()
        ref(p.dtype, A, p.B, C, M=M, N=p.N, K=p.K, lda=p.lda, ldb=p.ldb, ldc=p.ldc,
            a_col=p.a_col, b_col=p.b_col, batch=1, sa=0 if p.a_col else None, nthreads=threads)
        return time.perf_counter() - t, 2 * M * p.N * p.K, f"rows 0..{M - 1} of {p.M}"

    # calibrate on a small sample, then size the measured sample to ~budget_s
    probe = threads if p.batch == 1 else threads * 8
    dt, fl, _ = run_rows(probe)
    rows = int(probe * budget_s / max(dt, 1e-3))
    rows = max(probe, (rows // threads) * threads)
    dt, fl, what = run_rows(rows)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s" if p.dtype != "i8" else "TOP/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{what} of the same seeded problem ({fl / 2:.3g} MACs, {dt:.1f} s)"}


def _err_over_bound(err, tol):
    """Largest error / bound over the sampled positions; an exact result counts 0 even where
    the bound is 0 (a zero row of A or column of B with a zero C)."""
    import numpy as np
    err = np.asarray(err, dtype=np.float64)
    tol = np.asarray(tol, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(err == 0, 0.0, err / tol)
    return float(np.max(r))


def parity_sample(p, D_host, ex=None, sparse=False):
    """Oracle check of the benchmarked output at sampled positions (not timed)."""
    import numpy as np

    import oracle
    rng = np.random.default_rng(123)
    n = 64 if p.K >= 65536 else 256
    pts = np.stack([rng.integers(0, p.batch, n), rng.integers(0, p.M, n),
                    rng.integers(0, p.N, n)], 1).astype(np.int64)
    Dg = D_host.reshape(p.batch, p.M, p.ldc)[pts[:, 0], pts[:, 1], pts[:, 2]]
    if ex is not None:
        c_type, d_type, alpha, beta, Cst = ex
        P, S = oracle.gemm_points(p.dtype, p.A, p.B, np.zeros_like(p.C), pts, **p.oracle_args())
        if d_type != "f32":
            Dg = oracle.decode_c(d_type, Dg.view(np.uint16))
        c = (oracle.decode_c(c_type, Cst).reshape(p.batch, p.M, p.ldc)[pts[:, 0], pts[:, 1], pts[:, 2]]
             if c_type != "none" else np.zeros(n))
        Dref = oracle.scaled_reference(P, c, alpha, beta)
        tol = oracle.scaled_tolerance(p.K, S, c, Dref, alpha, beta, d_type)
        ratio = _err_over_bound(np.abs(Dg.astype(np.float64) - Dref), tol)
        return {"checked": n, "max_err_over_bound": ratio, "ok": ratio <= 1.0}
    if sparse:
        pruned = oracle.prune24(p.dtype, p.A, p.M, p.K, p.lda, p.batch)
        r = oracle.gemm_points(p.dtype, pruned, p.B, p.C, pts, **p.oracle_args())
        if p.dtype == "i8":
            ok = bool(np.array_equal(Dg.astype(np.int64), r))
            return {"checked": n, "exact": ok, "ok": ok}
        Dref, S = r
        tol = oracle.float_tolerance(p.K, S, p.C[pts[:, 0], pts[:, 1], pts[:, 2]])
        ratio = _err_over_bound(np.abs(Dg.astype(np.float64) - Dref), tol)
        return {"checked": n, "max_err_over_bound": ratio, "ok": ratio <= 1.0}
    if p.dtype == "f64":
        Dh, Dl, S = oracle.gemm_f64_points(p.A, p.B, p.C, pts, **p.oracle_args())
        tol = oracle.f64_tolerance(p.K, S, p.C[pts[:, 0], pts[:, 1], pts[:, 2]])
        ratio = _err_over_bound(oracle.f64_error(Dg, Dh, Dl), tol)
        return {"checked": n, "max_err_over_bound": ratio, "ok": ratio <= 1.0}
    r = oracle.gemm_points(p.dtype, p.A, p.B, p.C, pts, **p.oracle_args())
    if p.dtype == "i8":
        ok = bool(np.array_equal(Dg.astype(np.int64), r))
        return {"checked": n, "exact": ok, "ok": ok}
    Dref, S = r
    tol = oracle.float_tolerance(p.K, S, p.C[pts[:, 0], pts[:, 1], pts[:, 2]])
    ratio = _err_over_bound(np.abs(Dg.astype(np.float64) - Dref), tol)
    return {"checked": n, "max_err_over_bound": ratio, "ok": ratio <= 1.0}


CEIL_LIB = os.path.join(ROOT, "tests", "native", "libceiling_probe.so")
# matrix-instruction probes of tests/native/ceiling_probe.hip: (id, name, dtype, work per CU-clock
# at the datasheet rate, for the fraction of the published peak)
CEIL_MFMA = [(0, "mfma_f32_32x32x16_bf16", "bf16"), (1, "mfma_f32_32x32x16_f16", "f16"),
             (2, "mfma_f32_16x16x32_bf16", "bf16"), (3, "mfma_f32_16x16x32_f16", "f16"),
             (4, "mfma_i32_32x32x32_i8", "i8"), (5, "mfma_i32_16x16x64_i8", "i8"),
             (6, "mfma_f64_16x16x4_f64", "f64"), (7, "smfmac_f32_32x32x32_bf16", "sp_bf16"),
             (8, "smfmac_i32_32x32x64_i8", "sp_i8")]
CEIL_PEAK = {"bf16": 2516.6, "f16": 2516.6, "i8": 5033.2, "f64": 78.6, "sp_bf16": 5033.2,
             "sp_i8": 10066.4}


def ceiling_probes(quick: bool = False, target_ms: float = 20.0, launches: int = 8):
    """Sustained ceilings of this part, measured by the test-side probe library:
    each matrix instruction alone (one workgroup of four waves per CU, plus two per
    CU for bf16 32x32x16), L2-resident loads into registers and straight into LDS,
    LDS reads, and HBM streams.  Returns a list of dicts (one per probe); each
    launch is timed with HIP events on the launch stream, the first launch of
    each probe calibrates its length to about target_ms and is not counted."""
    import ctypes

    import numpy as np
    import torch
    if not os.path.exists(CEIL_LIB):
        raise RuntimeError(f"{CEIL_LIB} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(CEIL_LIB)
    vp, i64 = ctypes.c_void_p, ctypes.c_longlong
    lib.ceil_ops_per_inst.restype = i64
    lib.ceil_ops_per_inst.argtypes = [ctypes.c_int]
    lib.ceil_insts_per_trip.argtypes = [ctypes.c_int]
    lib.ceil_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp]
    lib.ceil_read.argtypes = [ctypes.c_int, ctypes.c_int, vp, i64, ctypes.c_int, vp, vp]
    lib.ceil_lds.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp]
    lib.ceil_hbm.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, i64, vp, vp]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    if quick:
        target_ms, launches = 2.0, 3

    def timed(launch, n):
        ts = []
        for _ in range(n):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            assert launch() == 0
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return ts

    out = []
    rng = np.random.default_rng(77)
    bits = torch.from_numpy(rng.integers(-2**31, 2**31, size=256 * 4, dtype=np.int64)
                            .astype(np.int32)).to(dev)
    # bf16 / fp16 operand bits: keep exponents moderate so the sums stay finite
    bits16 = torch.from_numpy((rng.integers(0, 2**16, size=256 * 8) & 0x3FFF | 0x3000)
                              .astype(np.uint16).view(np.int16)).to(dev)
    for which, name, dt in CEIL_MFMA:
        for per_cu in ((1, 2) if which == 0 else (1,)):
            grid = cus * per_cu
            sink = torch.empty(grid * 256, dtype=torch.float32, device=dev)
            clk = torch.zeros(grid * 4 * 4, dtype=torch.int64, device=dev)
            src = bits16 if dt in ("bf16", "f16", "sp_bf16") else bits
            iters = 2000
            t = timed(lambda: lib.ceil_mfma(which, grid, iters, src.data_ptr(), sink.data_ptr(),
                                            clk.data_ptr(), sp), 1)[0]
            iters = max(100, int(iters * (target_ms * 1e-3) / max(t, 1e-6)))
            ts = timed(lambda: lib.ceil_mfma(which, grid, iters, src.data_ptr(), sink.data_ptr(),
                                             clk.data_ptr(), sp), launches)
            c = clk.view(grid * 4, 4).cpu().numpy().astype(np.float64)
            ops = float(lib.ceil_ops_per_inst(which)) * lib.ceil_insts_per_trip(which) * iters \
                * grid * 4
            rates = [ops / x / 1e12 for x in ts]
            med = float(np.median(ts))
            # shader-clock counter ticks per second over the last launch
            clock = float(np.mean(c[:, 1] - c[:, 0])) / ts[-1] / 1e9
            rt = float(np.mean(c[:, 3] - c[:, 2])) / ts[-1] / 1e6
            out.append({"probe": name, "waves_per_simd": per_cu, "grid": grid, "iters": iters,
                        "launch_ms": round(med * 1e3, 3),
                        "rate": round(ops / med / 1e12, 1),
                        "unit": "TOP/s" if "i8" in dt else "TFLOP/s",
                        "first_last": [round(rates[0], 1), round(rates[-1], 1)],
                        "frac_of_datasheet": round(ops / med / 1e12 / CEIL_PEAK[dt], 4),
                        "clock_counter_ghz": round(clock, 3), "realtime_counter_mhz": round(rt, 2)})
            print(f"[ceiling] {out[-1]}", file=sys.stderr, flush=True)
    # loads from an L2-resident buffer (1 MB, every workgroup sweeps all of it)
    l2 = torch.zeros(1 << 20, dtype=torch.uint8, device=dev)
    for kind, what in ((0, "l2_read_to_registers"), (1, "l2_read_direct_to_lds")):
        for per_cu in (1, 2):
            grid = cus * per_cu
            sink = torch.empty(grid * 256 * 4, dtype=torch.int32, device=dev)
            passes = 4
            t = timed(lambda: lib.ceil_read(kind, grid, l2.data_ptr(), l2.numel(), passes,
                                            sink.data_ptr(), sp), 1)[0]
            passes = max(1, int(passes * (target_ms * 1e-3) / max(t, 1e-6)))
            ts = timed(lambda: lib.ceil_read(kind, grid, l2.data_ptr(), l2.numel(), passes,
                                             sink.data_ptr(), sp), launches)
            med = float(np.median(ts))
            nbytes = float(grid) * passes * l2.numel()
            out.append({"probe": what, "workgroups_per_cu": per_cu, "grid": grid,
                        "buffer_bytes": l2.numel(), "passes": passes,
                        "launch_ms": round(med * 1e3, 3), "rate": round(nbytes / med / 1e12, 2),
                        "unit": "TB/s"})
            print(f"[ceiling] {out[-1]}", file=sys.stderr, flush=True)
    # LDS reads
    grid = cus
    sink = torch.empty(grid * 256 * 4, dtype=torch.int32, device=dev)
    iters = 1000
    t = timed(lambda: lib.ceil_lds(grid, iters, sink.data_ptr(), sp), 1)[0]
    iters = max(10, int(iters * (target_ms * 1e-3) / max(t, 1e-6)))
    ts = timed(lambda: lib.ceil_lds(grid, iters, sink.data_ptr(), sp), launches)
    med = float(np.median(ts))
    nbytes = float(grid) * 256 * 16 * 16 * iters
    out.append({"probe": "lds_read_b128", "grid": grid, "iters": iters,
                "launch_ms": round(med * 1e3, 3), "rate": round(nbytes / med / 1e12, 2),
                "unit": "TB/s", "bytes_per_cu_per_ns": round(nbytes / med / 1e9 / cus, 1)})
    print(f"[ceiling] {out[-1]}", file=sys.stderr, flush=True)
    # HBM streams over 2 GiB (far beyond the 256 MB memory-side cache)
    nbytes = (256 << 20) if quick else (2 << 30)
    a = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    b = torch.empty_like(a)
    sink = torch.empty(256 * 4, dtype=torch.int32, device=dev)
    n16 = nbytes // 16
    for mode, what, moved in ((0, "hbm_read_nt", 1), (1, "hbm_write_nt", 1), (2, "hbm_copy_nt", 2)):
        grid = cus * 8
        ts = timed(lambda: lib.ceil_hbm(mode, grid, a.data_ptr(), b.data_ptr(), n16, sink.data_ptr(),
                                        sp), launches + 1)[1:]
        med = float(np.median(ts))
        out.append({"probe": what, "bytes": nbytes, "grid": grid, "launch_ms": round(med * 1e3, 3),
                    "rate": round(moved * nbytes / med / 1e12, 2), "unit": "TB/s"})
        print(f"[ceiling] {out[-1]}", file=sys.stderr, flush=True)
    del a, b
    torch.cuda.synchronize()
    return out


def time_workload(name, steps, warmup, reps, ex_args=None, rotate=None, dev=None, settle_ms=0.0,
                  zero_operands=False):
    """Upload workload `name`, run `warmup` untimed steps, then untimed steps for
    at least `settle_ms` more milliseconds (the clock settle described at
    SETTLE_MS), then `reps` repetitions of exactly `steps` timed steps each (HIP
    events on the launch stream, with a device synchronisation before and after
    each repetition).  One step is one call of the library on the whole problem.
    Returns a dict with the problem, the per-repetition times, the median, the
    plan label, the number of settle steps and the last output.  zero_operands:
    A and B are all zeros (the same shapes, kernels and memory traffic; the
    matrix units' inputs never change), for measuring how the operands' values
    move the clock."""
    import numpy as np
    import torch

    import dense_mixed_precision_02_amd as dmp
    import synth

    p = synth.config_problem(name)
    if zero_operands:
        p.A[...] = 0
        p.B[...] = 0

    def up(x):
        t = torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x)
        return t.to(dev)

    ex = None
    sparse = name in SPARSE_CONFIGS
    A, B = up(p.A), up(p.B)
    if ex_args is not None:
        c_type, d_type, alpha, beta_in = ex_args
        if p.dtype == "i8":
            raise SystemExit("--d-type applies to fp16/bf16 workloads")
        beta = 0.0 if c_type == "none" else beta_in
        Cst = store_c(c_type, p.C) if c_type != "none" else None
        ex = (c_type, d_type, alpha, beta, Cst)
        C = up(Cst) if Cst is not None else None
        D = torch.empty(p.C.shape, dtype=torch.float32 if d_type == "f32" else torch.int16,
                        device=dev)
    else:
        C = up(p.C)
        D = torch.empty_like(C)
    h = dmp.Handle()
    flags = (dmp.GEMM_A_COLMAJOR if p.a_col else 0) | (dmp.GEMM_B_COLMAJOR if p.b_col else 0)
    code = DTYPE_CODE[p.dtype]
    label = dmp.plan_label(p.M, p.N, p.K, p.lda, p.ldb, p.ldc, code, flags, p.batch, handle=h)
    if sparse:
        ins = "smfmac32x32x64" if p.dtype == "i8" else "smfmac32x32x32"
        label = f"sparse24 {ins} tile256x256 grid={-(-p.M // 256) * -(-p.N // 256) * p.batch}"
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    nsets = rotate if rotate else (ROTATE_SETS if name in ROTATE else 1)
    if sparse:
        nsets = 1  # the sparse products time one compressed A
    # set 0 is (A, B, C, D); further sets are device copies of the same inputs
    sets = [(A, B, C, D)] + [(A.clone(), B.clone(), None if C is None else C.clone(),
                              torch.empty_like(D)) for _ in range(nsets - 1)]
    runs = [(a.data_ptr(), b.data_ptr(), c.data_ptr() if c is not None else 0, d.data_ptr(),
             p.M, p.N, p.K, p.lda, p.ldb, p.ldc, code, flags, p.batch) for (a, b, c, d) in sets]
    prune_us = None
    if sparse:
        kp, mp = dmp.sparse24_kp(p.K, code), dmp.sparse24_mp(p.M)
        Ac = torch.empty((p.batch, mp, kp // 2),
                         dtype=torch.int8 if p.dtype == "i8" else torch.int16, device=dev)
        meta = torch.empty((p.batch, mp, kp // 16), dtype=torch.int16, device=dev)
        # the compression is a one-off preparation of A, timed on its own (after
        # one untimed call that loads the kernel)
        rc = h.prune24(A.data_ptr(), p.M, p.K, p.lda, code, p.batch, Ac.data_ptr(), meta.data_ptr(),
                       sp)
        assert rc == 0, rc
        q0 = torch.cuda.Event(enable_timing=True)
        q1 = torch.cuda.Event(enable_timing=True)
        q0.record(stream)
        rc = h.prune24(A.data_ptr(), p.M, p.K, p.lda, code, p.batch, Ac.data_ptr(), meta.data_ptr(),
                       sp)
        q1.record(stream)
        torch.cuda.synchronize()
        assert rc == 0, rc
        prune_us = q0.elapsed_time(q1) * 1e3

        def step(i):
            rc2 = h.run_sparse24(Ac.data_ptr(), meta.data_ptr(), B.data_ptr(), C.data_ptr(),
                                 D.data_ptr(), p.M, p.N, p.K, p.ldb, p.ldc, code, flags, p.batch, sp)
            assert rc2 == 0, rc2
    elif ex is None:
        def step(i):
            h.run(*runs[i % nsets], sp)
    else:
        OUTC = {"f32": dmp.GEMM_OUT_F32, "f16": dmp.GEMM_OUT_F16, "bf16": dmp.GEMM_OUT_BF16,
                "none": dmp.GEMM_OUT_F32}
        kw = dict(alpha=ex[2], beta=ex[3], c_type=OUTC[ex[0]], d_type=OUTC[ex[1]], stream=sp)

        def step(i):
            h.run_ex(*runs[i % nsets], **kw)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    settle_steps = 0
    if settle_ms > 0:
        # batches of launches of about 20 ms, sized from one synchronised step
        t_w = time.perf_counter()
        step(warmup)
        torch.cuda.synchronize()
        settle_steps = 1
        per = (time.perf_counter() - t_w) * 1e3
        batch = max(1, min(4096, int(20.0 / max(per, 1e-3))))
        t_s = time.perf_counter()
        while (time.perf_counter() - t_s) * 1e3 < settle_ms:
            for i in range(batch):
                step(warmup + settle_steps + i)
            torch.cuda.synchronize()
            settle_steps += batch
    rep_ms = []
    t_all = time.perf_counter()
    for r in range(reps):
        # events on the stream the kernels are launched on
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(steps):
            step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        rep_ms.append(e0.elapsed_time(e1) / steps)
    wall = time.perf_counter() - t_all
    D_host = D.cpu().numpy()
    h.close()
    return {"p": p, "ex": ex, "sparse": sparse, "label": label, "nsets": nsets,
            "rep_ms": rep_ms, "ms": float(np.median(rep_ms)), "wall": wall, "D_host": D_host,
            "prune_us": prune_us, "settle_steps": settle_steps}


def roofline_of(name, r):
    """(throughput, unit, peak, roofline dict, algorithmic bytes) of a timed workload."""
    p, ex, sparse, ms = r["p"], r["ex"], r["sparse"], r["ms"]
    tflops = p.flops / (ms * 1e-3) / 1e12
    peak = SPARSE_PEAK_TFLOPS[p.dtype] if sparse else PEAK_TFLOPS[p.dtype]
    unit = "TOP/s" if p.dtype == "i8" else "TFLOP/s"
    nbytes = algorithmic_bytes(p, *(ex[:2] if ex else (None, None)), sparse=sparse)
    if name in HBM_BOUND:
        gbs = nbytes / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": peak, "unit": unit,
                "frac": round(tflops / peak, 4), "traffic": None}
    # measured HBM bytes per launch, only while the kernel sources are unchanged
    from bench_profile import kernel_source_hash, read_traffic
    tf = TRAFFIC_FILES.get(name)
    rt = read_traffic(os.path.join(ROOT, tf)) if tf and ex is None else None
    if rt is not None and rt[1] == kernel_source_hash():
        roof["traffic"] = round(rt[0])
    return tflops, unit, peak, roof, nbytes


# Clock settle (a study switch, off by default).  Once a sustained
# matrix-instruction load starts, this part's power management moves the shader
# clock for some milliseconds before it holds steady, and repetitions timed in
# that transient are slow and scattered (on the 4096^3 bf16 product, 20-step
# repetitions right after a 5-step warm-up read 116 to 135 us per step, against
# about 105 us in a continuous run).  The default line keeps exactly the
# requested warm-up and times what follows it.  --settle-ms T adds untimed steps
# for T more milliseconds after the warm-up (reported as config.settle_ms and
# config.settle_steps), for comparisons of steady-state rates; such a line is a
# study, not the benchmark.
SETTLE_MS = 0.0

# Workloads timed beside the headline one in the default run, so that every input
# type the metric names is measured: the 4096^3 fp16 product and the 8192^3 int8 one.
EXTRA_WORKLOADS = ("S1", "C3")


def single_core_c1():
    """The oracle on one host thread over the whole 256^3 fp16 workload."""
    import oracle
    import synth
    p = synth.config_problem("C1")
    oracle.gemm(p.dtype, p.A, p.B, p.C, nthreads=1, **p.oracle_args())  # loads the library
    t = time.perf_counter()
    oracle.gemm(p.dtype, p.A, p.B, p.C, nthreads=1, **p.oracle_args())
    dt = time.perf_counter() - t
    return {"value": p.flops / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"whole 256x256x256 fp16 workload ({p.flops // 2} MACs, {dt:.3f} s)"}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--reps", type=int, default=5,
                    help="repetitions of the timed steps; the line reports the median")
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="study switch: untimed steps for this many milliseconds after the "
                         "warm-up steps (default 0: the line's warm-up is exactly --warmup)")
    ap.add_argument("--config", default="C2")
    ap.add_argument("--zero-operands", action="store_true",
                    help="A and B all zeros (a study of how operand values move the clock; "
                         "never the headline)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    ap.add_argument("--no-extra", action="store_true",
                    help=f"skip the workloads timed beside the default one ({', '.join(EXTRA_WORKLOADS)})")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--d-type", choices=["f32", "f16", "bf16"], default=None,
                    help="time gemm_run_ex with this D storage type")
    ap.add_argument("--c-type", choices=["f32", "f16", "bf16", "none"], default="f32")
    ap.add_argument("--alpha", type=float, default=1.0)
    ap.add_argument("--beta", type=float, default=1.0)
    ap.add_argument("--rotate", type=int, default=None,
                    help="device copies of the inputs and outputs the timed steps rotate over "
                         f"(default {ROTATE_SETS} for {sorted(ROTATE)}, else 1)")
    ap.add_argument("--ceiling", action="store_true",
                    help="only run the ceiling probes (matrix-instruction rates, L2 / LDS / HBM "
                         "bandwidth) and print one JSON line per probe")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain device copy of COPY_BYTES (counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.ceiling:
        for r in ceiling_probes():
            print(json.dumps(r), flush=True)
        return

    if args.copy_probe:
        x = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
        y = torch.empty_like(x)
        for _ in range(6):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": COPY_BYTES, "launches": 6}))
        return

    import synth

    name = args.config
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ex_args = (args.c_type, args.d_type, args.alpha, args.beta) if args.d_type else None
    r = time_workload(name, args.steps, args.warmup, args.reps, ex_args, args.rotate, dev,
                      args.settle_ms, args.zero_operands)
    p, ex, sparse, ms = r["p"], r["ex"], r["sparse"], r["ms"]
    tflops, unit, peak, roof, nbytes = roofline_of(name, r)
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic",
        "config": {"workload": synth.CONFIG_LABELS[name], "M": p.M, "N": p.N, "K": p.K,
                   "batch": p.batch, "a_layout": "col" if p.a_col else "row",
                   "b_layout": "col" if p.b_col else "row", "plan": r["label"],
                   "pct_of_dense_peak": round(100 * tflops / peak, 2),
                   "hbm_gbs_algorithmic": round(nbytes / (ms * 1e-3) / 1e9, 1),
                   "repetitions": args.reps,
                   "rep_ms_per_step": [round(x, 5) for x in r["rep_ms"]],
                   "timed_wall_s": round(r["wall"], 3), "input_sets": r["nsets"],
                   "settle_ms": args.settle_ms, "settle_steps": r["settle_steps"]},
        "roofline": roof,
        "parity": parity_sample(p, r["D_host"], ex, sparse),
    }
    if args.zero_operands:
        line["data"] = "synthetic, A and B all zeros"
        line["config"]["zero_operands"] = True
    if sparse:
        line["config"]["prune_us"] = round(r["prune_us"], 1)
        line["config"]["note"] = ("value = 2*M*N*K / time, the dense-equivalent rate of the 2:4 "
                                  "product; peak = the sparse instructions' rate (2x dense)")
    if ex is not None:
        line["config"]["output_stage"] = {"c_type": ex[0], "d_type": ex[1], "alpha": ex[2],
                                          "beta": ex[3]}
    del r
    if name == "C2" and ex is None and not args.no_extra and not args.zero_operands:
        # the other input types the metric names, timed the same way (full-size
        # inputs, every step the whole product)
        others = {}
        for o in EXTRA_WORKLOADS:
            ro = time_workload(o, args.steps, args.warmup, args.reps, None, None, dev,
                               args.settle_ms)
            t_o, u_o, pk_o, roof_o, _ = roofline_of(o, ro)
            others[o] = {"workload": synth.CONFIG_LABELS[o], "dtype": ro["p"].dtype,
                         "plan": ro["label"], "value": round(t_o, 2), "unit": u_o,
                         "ms_per_step": round(ro["ms"], 5),
                         "rep_ms_per_step": [round(x, 5) for x in ro["rep_ms"]],
                         "settle_steps": ro["settle_steps"],
                         "pct_of_dense_peak": round(100 * t_o / pk_o, 2), "roofline": roof_o,
                         "parity": parity_sample(ro["p"], ro["D_host"])}
            del ro
            torch.cuda.empty_cache()
        line["other_dtypes"] = others
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(p, args.cpu_budget)
        line["cpu_baseline"]["single_core_c1"] = single_core_c1()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
