"""Accumulator layouts of the matrix instructions the kernels use.

tests/golden/mfma_output_layouts.txt holds the layout tables printed on the page
"CDNA2 dense MFMA builtins" (section "Accumulator layout").  The CPU test checks
that transcription against the forward formulas the same page prints next to
each table (lane and accVGPR of element (i, j) of block b); the GPU test runs
one-hot probes of the gfx950 instructions (tests/native/mfma_probe.hip) and
checks that every output element lands in the lane and register the table
names, with the value the instruction's k count gives."""
import ctypes
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden", "mfma_output_layouts.txt")
PROBE = os.path.join(ROOT, "tests", "native", "libmfma_probe.so")
SIZE = {"32x32": (1, 32), "16x16": (4, 16), "4x4": (16, 4), "16x16f64": (1, 16)}


def _span(text):
    if "," in text:
        return [int(x) for x in text.split(",")]
    a, b = (int(x) for x in text.split("-"))
    return list(range(a, b + 1))


def load_golden():
    """shape -> {(block, row, col): (lane, register)}"""
    table = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        shape, block, rows, lanes, regs = line.split()
        rows, lanes, regs = _span(rows), _span(lanes), _span(regs)
        assert len(rows) == len(regs), line
        m = table.setdefault(shape, {})
        for r, g in zip(rows, regs):
            for j in range(len(lanes)):
                key = (int(block), r, j)
                assert key not in m, f"{shape} {key} listed twice"
                m[key] = (lanes[0] + j, g)
    return table


def formula(shape, b, i, j):
    """The page's forward formulas: (lane, accVGPR) of element (i, j) of block b."""
    if shape == "32x32":
        return (32 * (i // 4)) % 64 + j, 16 * b + 4 * (i // 8) + i % 4
    if shape == "16x16":
        return 16 * (i // 4) + j, 4 * b + i % 4
    if shape == "4x4":
        return 4 * b + j, i
    if shape == "16x16f64":
        return 16 * (i % 4) + j, i // 4
    raise KeyError(shape)


def test_golden_tables_match_the_printed_formulas():
    table = load_golden()
    assert set(table) == set(SIZE)
    for shape, (blocks, s) in SIZE.items():
        m = table[shape]
        assert len(m) == blocks * s * s, shape          # every element exactly once
        for b in range(blocks):
            for i in range(s):
                for j in range(s):
                    assert m[(b, i, j)] == formula(shape, b, i, j), (shape, b, i, j)
        # each (lane, register) holds one element
        assert len(set(m.values())) == len(m), shape


def converse(shape, lane, g):
    """The page's converse formulas: (block, row, col) held in lane L, register G."""
    if shape == "32x32":
        return g // 16, (8 * (g // 4)) % 32 + 4 * (lane // 32) + g % 4, lane % 32
    if shape == "16x16":
        return g // 4, 4 * (lane // 16) + g % 4, lane % 16
    if shape == "4x4":
        return lane // 4, g % 4, lane % 4
    if shape == "16x16f64":
        return 0, 4 * g + lane // 16, lane % 16
    raise KeyError(shape)


def test_golden_tables_match_the_printed_converse_formulas():
    for shape, m in load_golden().items():
        for (b, i, j), (lane, g) in m.items():
            assert converse(shape, lane, g) == (b, i, j), (shape, b, i, j, lane, g)


# probe id, table shape, k summed per output element
PROBES = [
    (0, "32x32", 16, "mfma_f32_32x32x16_f16"),
    (1, "32x32", 16, "mfma_f32_32x32x16_bf16"),
    (2, "32x32", 32, "mfma_i32_32x32x32_i8"),
    (3, "32x32", 16, "smfmac_f32_32x32x32_bf16"),
    (4, "32x32", 32, "smfmac_i32_32x32x64_i8"),
    (5, "16x16f64", 4, "mfma_f64_16x16x4f64"),
    (6, "4x4", 4, "mfma_f32_4x4x4f16 (16 blocks)"),
    (7, "16x16", 4, "mfma_f32_16x16x4f16 (4 blocks)"),
    (8, "4x4", 4, "mfma_f32_4x4x4bf16_1k (16 blocks)"),
    (9, "16x16", 4, "mfma_f32_16x16x4bf16_1k (4 blocks)"),
    (10, "4x4", 4, "mfma_i32_4x4x4i8 (16 blocks)"),
    (11, "16x16", 4, "mfma_i32_16x16x4i8 (4 blocks)"),
]


@pytest.mark.gpu
@pytest.mark.parametrize("probe", PROBES, ids=[p[3] for p in PROBES])
def test_gfx950_accumulator_layout_matches_the_tables(probe):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(PROBE):
        raise RuntimeError(f"{PROBE} is not built (build() builds it)")
    which, shape, kcount, name = probe
    lib = ctypes.CDLL(PROBE)
    lib.mfma_probe_combos.argtypes = [ctypes.c_int]
    lib.mfma_probe_run.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    blocks, s = SIZE[shape]
    n = lib.mfma_probe_combos(which)
    assert n == blocks * s * s
    print(f"[layout] {name}: {n} one-hot products", flush=True)
    out = torch.zeros(n * 64 * 16, dtype=torch.float64, device="cuda")
    assert lib.mfma_probe_run(which, out.data_ptr(), torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    acc = out.cpu().numpy().reshape(n, 64, 16)
    table = load_golden()[shape]
    for b in range(blocks):
        for i in range(s):
            for j in range(s):
                c = (b * s + i) * s + j
                nz = np.argwhere(acc[c] != 0)
                lane, reg = table[(b, i, j)]
                assert nz.tolist() == [[lane, reg]], (name, b, i, j, nz.tolist()[:4])
                assert acc[c, lane, reg] == kcount, (name, b, i, j, acc[c, lane, reg])
