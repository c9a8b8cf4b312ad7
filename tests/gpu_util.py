"""Helpers for the GPU parity tests: upload a synthetic problem, run it through
the C ABI, and compare with the CPU oracle (every element, plus row-sum
properties that hold at any size)."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import synth

DTYPE_CODE = {"f16": 0, "bf16": 1, "i8": 2}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(p: synth.Problem, dev="cuda"):
    import torch
    if p.dtype == "i8":
        A = torch.from_numpy(p.A).to(dev)
        B = torch.from_numpy(p.B).to(dev)
    else:
        A = torch.from_numpy(p.A.view(np.int16)).to(dev)
        B = torch.from_numpy(p.B.view(np.int16)).to(dev)
    C = torch.from_numpy(p.C).to(dev)
    return A, B, C


def run(handle, p: synth.Problem, tensors=None, D=None, stream=None):
    """Launch D = A*B + C for problem p through gemm_run; returns D (device tensor)."""
    import torch
    A, B, C = tensors if tensors is not None else to_device(p)
    if D is None:
        D = torch.empty_like(C)
    flags = (1 if p.a_col else 0) | (2 if p.b_col else 0)
    s = stream if stream is not None else torch.cuda.current_stream()
    handle.run(A.data_ptr(), B.data_ptr(), C.data_ptr(), D.data_ptr(), p.M, p.N, p.K, p.lda,
               p.ldb, p.ldc, DTYPE_CODE[p.dtype], flags, p.batch, s.cuda_stream)
    return D


def logical_D(p: synth.Problem, D_host: np.ndarray) -> np.ndarray:
    """(batch, M, N) view of a D storage array (batch, M, ldc)."""
    return D_host.reshape(p.batch, p.M, p.ldc)[:, :, :p.N]


def check_full(p: synth.Problem, D_host: np.ndarray, exact: bool = False) -> float:
    """Element-by-element comparison with the full oracle.  Returns max err / bound."""
    Dg = logical_D(p, D_host)
    if p.dtype == "i8":
        Dref = oracle.gemm("i8", p.A, p.B, p.C, **p.oracle_args())
        assert np.all(np.abs(Dref) < 2 ** 31), "reference does not fit int32"
        bad = np.argwhere(Dg.astype(np.int64) != Dref)
        assert bad.size == 0, f"{len(bad)} int mismatches, first at {bad[0]}"
        return 0.0
    Dref, S = oracle.gemm(p.dtype, p.A, p.B, p.C, **p.oracle_args())
    Dg64 = Dg.astype(np.float64)
    assert np.all(np.isfinite(Dg64))
    if exact:
        bad = np.argwhere(Dg64 != Dref)
        assert bad.size == 0, f"{len(bad)} mismatches on exact-integer inputs, first at {bad[0]}"
        return 0.0
    tol = oracle.float_tolerance(p.K, S, p.C[:, :p.M, :p.N])
    err = np.abs(Dg64 - Dref)
    ratio = err / np.maximum(tol, np.finfo(np.float64).tiny)
    bad = np.argwhere(err > tol)
    assert bad.size == 0, f"{len(bad)} elements over the bound, worst ratio {ratio.max():.3g} at {bad[0]}"
    return float(ratio.max())


def _decoded(p: synth.Problem, which: str) -> np.ndarray:
    """Logical matrix of batch b as float64/int64 (library decode; test-side arithmetic)."""
    X = p.A if which == "A" else p.B
    if p.dtype == "i8":
        v = X.astype(np.int64)
    elif p.dtype == "f16":
        v = X.view(np.float16).astype(np.float64)
    else:
        v = (X.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return v


def check_row_sums(p: synth.Problem, D_host: np.ndarray, exact: bool = False) -> None:
    """Property valid at any size: sum_j D[i,j] = sum_j C[i,j] + sum_k A[i,k] (sum_j B[k,j]).
    Every output element enters one row sum, so a dropped or doubled tile, K panel or
    split shows up; integer results must satisfy it exactly."""
    Dg = logical_D(p, D_host)
    Ad, Bd = _decoded(p, "A"), _decoded(p, "B")
    for b in range(p.batch):
        Av = Ad[b]
        Bv = Bd[b]
        Al = Av[:p.K, :p.M].T if p.a_col else Av[:p.M, :p.K]
        Bl = Bv[:p.N, :p.K].T if p.b_col else Bv[:p.K, :p.N]
        Cl = p.C[b][:p.M, :p.N]
        if p.dtype == "i8" or exact:
            Ai = Al.astype(np.int64)
            Bi = Bl.astype(np.int64)
            want = Cl.astype(np.int64).sum(1) + Ai @ Bi.sum(1)
            got = Dg[b].astype(np.int64).sum(1)
            assert np.array_equal(got, want), f"row sums differ in batch {b}"
        else:
            want = Cl.astype(np.float64).sum(1) + Al @ Bl.sum(1)
            got = Dg[b].astype(np.float64).sum(1)
            # per-element bound summed over the row, plus fp64 rounding of the check itself
            sabs = np.abs(Al) @ np.abs(Bl).sum(1)
            tol = 4.0 * p.K * 2.0 ** -24 * sabs + 2.0 ** -24 * np.abs(Cl).sum(1) \
                + 1e-12 * (np.abs(want) + sabs + 1.0)
            assert np.all(np.abs(got - want) <= tol), f"row sums over the bound in batch {b}"
