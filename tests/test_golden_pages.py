"""Facts the pages print as tables, checked on the CPU.

tests/golden/cdna2_mfma_throughput.txt transcribes the instruction throughput
table of the page "CDNA2 dense MFMA builtins" (section "Instruction
throughput").  Three things are pinned against it:
  - the reading of the block count that the library's instruction choices rely
    on: an instruction M x N x K whose lanes each supply e elements of A per
    step computes blocks = 64 e / (M K) independent products, and its ops are
    2 M N K blocks (every row of the table satisfies this; the section
    "Accumulator layout" states blocks = 64 / M for packed inputs, which the
    single-block rows contradict);
  - the peak-rate arithmetic the page states (ops / cycles per SIMD);
  - the figure quoted as context for the method: 1024 bf16 FLOPs per cycle per
    CU for the _1k instructions against 512 for the others (four SIMDs per CU).
The converse layout formulas of section "Accumulator layout" are checked in
tests/test_mfma_layouts.py."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TABLE = os.path.join(ROOT, "tests", "golden", "cdna2_mfma_throughput.txt")

# elements of A each lane supplies per instruction, by the builtin's input type
# (one 32-bit register for fp32 and packed bf16 pairs, two for four fp16 /
# bf16 (_1k) values, one for four int8 values, a register pair for fp64)
LANE_ELEMS = {"f32": 1, "f16": 4, "bf16": 2, "bf16_1k": 4, "i8": 4, "f64": 1}


def rows():
    out = []
    for line in open(TABLE):
        if line.startswith("#") or not line.strip():
            continue
        name, ops, cycles, coexec = line.split()
        m = re.fullmatch(r"mfma_(f32|f64|i32)_(\d+)x(\d+)x(\d+)(f32|f16|bf16|i8|f64)(_1k)?", name)
        assert m, name
        M, N, K = int(m.group(2)), int(m.group(3)), int(m.group(4))
        t = m.group(5) + ("_1k" if m.group(6) else "")
        out.append((name, M, N, K, t, int(ops), int(cycles), int(coexec)))
    return out


def test_table_transcribed_whole():
    r = rows()
    assert len(r) == 27
    assert len({x[0] for x in r}) == 27


def test_ops_equal_2mnk_times_blocks():
    for name, M, N, K, t, ops, cycles, coexec in rows():
        assert M == N, name
        e = LANE_ELEMS[t]
        assert (64 * e) % (M * K) == 0, name
        blocks = 64 * e // (M * K)
        assert blocks in (1, 2, 4, 16), (name, blocks)
        assert ops == 2 * M * N * K * blocks, (name, ops, blocks)
    # "blocks = 64 / M" would give the single-block rows 2, 4 or 16 blocks and the
    # fp64 4x4 row 16 (it has 4): it fails on the table, the reading above does not
    r = {x[0]: x for x in rows()}
    assert r["mfma_f32_32x32x8f16"][5] != 2 * 32 * 32 * 8 * (64 // 32)
    assert r["mfma_f64_4x4x4f64"][5] == 2 * 4 * 4 * 4 * 4


def test_cycles_and_coexecution():
    for name, M, N, K, t, ops, cycles, coexec in rows():
        # cycle counts by output size; fp64 instructions do not co-execute with VALU work
        assert cycles == {32: 64, 16: 32, 4: 8}[M] or (t == "f64" and M == 4 and cycles == 16), name
        if t == "f64":
            assert coexec == 0, name
        else:
            assert coexec == cycles - 4, name


def test_bf16_rate_quoted_for_the_method():
    """1024 bf16 FLOPs per cycle per CU with the _1k instructions, 512 without."""
    r = {x[0]: x for x in rows()}
    per_cu = lambda n: r[n][5] // r[n][6] * 4          # ops per cycle per SIMD, four SIMDs
    assert per_cu("mfma_f32_32x32x8bf16_1k") == 1024
    assert per_cu("mfma_f32_16x16x16bf16_1k") == 1024
    assert per_cu("mfma_f32_32x32x4bf16") == 512
    assert per_cu("mfma_f32_16x16x8bf16") == 512
    # and the fp16 instructions run at the _1k rate
    assert per_cu("mfma_f32_32x32x8f16") == 1024
