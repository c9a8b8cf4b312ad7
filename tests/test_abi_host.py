"""Host-side checks of the C ABI: the library loads and exports every function
the header declares, the header is valid C, status strings, argument validation
and kernel-path selection (gemm_plan with a NULL handle makes no HIP call)."""
import ctypes
import os
import re
import subprocess

import pytest

import dense_mixed_precision_02_amd as dmp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dmp_gemm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gemm_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(dmp.EXPORTED_SYMBOLS)


def test_noalloc_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define GEMM_NOALLOC_SCRATCH_BYTES \((\d+)ll << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == dmp.NOALLOC_SCRATCH_BYTES


def test_header_is_plain_c():
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", HEADER],
                   check=True)


def test_library_exports_every_declared_symbol():
    lib = dmp.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", dmp.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_status_strings():
    assert dmp.status_string(0) == "GEMM_OK"
    assert dmp.status_string(1) == "GEMM_ERR_INVALID_ARG"
    assert dmp.status_string(2) == "GEMM_ERR_UNSUPPORTED_DEVICE"
    assert dmp.status_string(3) == "GEMM_ERR_ALLOC"
    assert dmp.status_string(4) == "GEMM_ERR_HIP"
    assert dmp.status_string(5) == "GEMM_ERR_SCRATCH"
    assert dmp.status_string(99) == "GEMM_ERR_UNKNOWN"


def plan_status(*args):
    lib = dmp.load_library()
    buf = ctypes.create_string_buffer(128)
    return lib.gemm_plan(None, *args, buf, 128), buf.value.decode()


@pytest.mark.parametrize("args", [
    (-1, 4, 4, 4, 4, 4, 0, 0, 1),          # negative M
    (4, 4, -2, 4, 4, 4, 0, 0, 1),          # negative K
    (4, 4, 8, 7, 4, 4, 0, 0, 1),           # lda < K (row-major A)
    (4, 4, 8, 8, 3, 4, 0, 0, 1),           # ldb < N (row-major B)
    (4, 4, 8, 8, 7, 4, 0, 2, 1),           # ldb < K (col-major B)
    (5, 4, 8, 4, 4, 4, 0, 1, 1),           # lda < M (col-major A)
    (4, 6, 8, 8, 6, 5, 0, 0, 1),           # ldc < N
    (4, 4, 8, 8, 4, 4, 5, 0, 1),           # bad dtype
    (4, 4, 8, 8, 4, 4, -1, 0, 1),          # bad dtype
    (4, 4, 8, 8, 4, 4, 0, 16, 1),          # unknown flag bit
    (4, 4, 8, 8, 4, 4, 0, 0, -1),          # negative batch
    (4, 4, 8, 1 << 62, 4, 4, 0, 0, 1),     # lda beyond 2^48 elements
    (4, 4, 8, 8, 1 << 50, 4, 0, 0, 1),     # ldb beyond 2^48 elements
    (4, 4, 8, 8, 4, 1 << 62, 0, 0, 1),     # ldc beyond 2^48 elements
    (1 << 20, 1 << 20, 8, 8, 1 << 20, 1 << 20, 0, 0, 1 << 9),  # C: 2^49 elements
    (4, 4, 1 << 30, 1 << 30, 4, 4, 0, 0, 1 << 20),  # A: batch x M x lda > 2^48
    (1, 4, 8, (1 << 48) + 1, 4, 4, 0, 0, 1),  # one-row A: its lda alone beyond 2^48
])
def test_validation_rejects(args):
    rc, _ = plan_status(*args)
    assert rc == 1


def test_extent_limit_is_inclusive_and_shared_operands_count_once():
    # C of 2^24 x 2^24 elements is exactly 2^48: accepted
    rc, _ = plan_status(1 << 24, 1 << 24, 16, 16, 1 << 24, 1 << 24, 0, 0, 1)
    assert rc == 0
    # a shared A (batch stride 0) counts once: 2^20 batches of a 2^20 x 2^20 A pass
    # only because A is shared (B and C are small per entry)
    big = (1 << 20, 16, 1 << 20, 1 << 20, 16, 16, 0)
    assert plan_status(*big, 4, 1 << 20)[0] == 0         # GEMM_A_SHARED
    assert plan_status(*big, 0, 1 << 20)[0] == 1


def test_noop_and_k0_plans():
    assert plan_status(0, 4, 8, 8, 4, 4, 0, 0, 1) == (0, "noop")
    assert plan_status(4, 4, 8, 8, 4, 4, 0, 0, 0) == (0, "noop")
    assert plan_status(4, 4, 0, 1, 4, 4, 0, 0, 1) == (0, "copy_c k=0")
    assert plan_status(4, 4, 0, 0, 0, 4, 0, 0, 1) == (0, "copy_c k=0")  # lda, ldb unused


def test_plans_of_the_workloads():
    # 4096^3 bf16, B col-major: one 256x256 tile per CU, no split
    assert dmp.plan_label(4096, 4096, 4096, 4096, 4096, 4096, dmp.GEMM_BF16,
                          dmp.GEMM_B_COLMAJOR) == "tile256x256 bf16 a:row b:col splitk=1 grid=256"
    # 8192^3 int8
    assert dmp.plan_label(8192, 8192, 8192, 8192, 8192, 8192, dmp.GEMM_I8) == \
        "tile256x256 i8 a:row b:row->col splitk=1 grid=1024"
    # skinny 1024 x 1024 x 65536: 16 tiles x 16 K-splits
    assert dmp.plan_label(1024, 1024, 65536, 65536, 1024, 1024, dmp.GEMM_BF16) == \
        "tile256x256 bf16 a:row b:row splitk=16 grid=256"
    # 8192 batched 64^3: one k-tile, so the single-buffer variant of the 64x64 tile
    assert dmp.plan_label(64, 64, 64, 64, 64, 64, dmp.GEMM_F16, 0, 8192) == \
        "tile64x64 f16 a:row b:row splitk=1 grid=8192 one-ktile"
    # 256^3 fp16: four k-tiles, the pipelined kernel
    assert dmp.plan_label(256, 256, 256, 256, 256, 256, dmp.GEMM_F16) == \
        "tile64x64 f16 a:row b:row splitk=1 grid=16"


def test_single_buffer_variant_only_for_one_ktile():
    """The k-tile is 128 bytes of K: 64 fp16/bf16 elements, 128 int8 ones."""
    f16 = lambda K, b=1: dmp.plan_label(64, 64, K, K, 64, 64, dmp.GEMM_F16, 0, b)
    i8 = lambda K: dmp.plan_label(64, 64, K, K, 64, 64, dmp.GEMM_I8, 0, 1)
    assert f16(64).endswith("one-ktile") and f16(16).endswith("one-ktile")
    assert not f16(72).endswith("one-ktile") and not f16(128).endswith("one-ktile")
    assert i8(128).endswith("one-ktile") and not i8(144).endswith("one-ktile")
    # other tiles never use it
    assert not dmp.plan_label(4096, 4096, 64, 64, 4096, 4096, dmp.GEMM_F16).endswith("one-ktile")


def test_generic_path_when_granules_do_not_fit():
    # K not a multiple of 8 with K-contiguous A -> element-wise path
    assert dmp.plan_label(64, 64, 30, 30, 64, 64, dmp.GEMM_F16).startswith("generic32x32")
    # leading dimension not a multiple of 16 bytes
    assert dmp.plan_label(64, 64, 64, 65, 64, 64, dmp.GEMM_F16).startswith("generic32x32")
    # MN-contiguous operands only: any K works on the tiled path
    assert dmp.plan_label(64, 64, 30, 64, 64, 64, dmp.GEMM_F16,
                          dmp.GEMM_A_COLMAJOR).startswith("tile64x64")
    # an MN-contiguous extent that is not whole granules -> element-wise path
    assert dmp.plan_label(60, 64, 32, 64, 64, 64, dmp.GEMM_F16,
                          dmp.GEMM_A_COLMAJOR).startswith("generic32x32")


def test_f64_plans():
    # 4096^3 fp64: 128 x 128 tiles (1024 of them, two per CU resident)
    assert dmp.plan_label(4096, 4096, 4096, 4096, 4096, 4096, dmp.GEMM_F64) == \
        "dtile128x128 f64 a:row b:row splitk=1 grid=1024"
    # fewer 128-tiles than CUs -> 64 x 64
    assert dmp.plan_label(512, 512, 512, 512, 512, 512, dmp.GEMM_F64).startswith("dtile64x64")
    # odd K with K-contiguous A, odd leading dimension, odd M with column-major A
    assert dmp.plan_label(64, 64, 31, 31, 64, 64, dmp.GEMM_F64).startswith("dgeneric16x16")
    assert dmp.plan_label(64, 64, 64, 65, 64, 64, dmp.GEMM_F64).startswith("dgeneric16x16")
    assert dmp.plan_label(63, 64, 64, 64, 64, 64, dmp.GEMM_F64,
                          dmp.GEMM_A_COLMAJOR).startswith("dgeneric16x16")
    # MN-contiguous operands only: odd K is fine on the tiled path
    assert dmp.plan_label(64, 64, 31, 64, 64, 64, dmp.GEMM_F64,
                          dmp.GEMM_A_COLMAJOR).startswith("dtile64x64")
    assert plan_status(4, 4, 0, 1, 4, 4, dmp.GEMM_F64, 0, 1) == (0, "copy_c k=0")


def test_tiny_plans():
    # 2^20 independent 4x4x16 fp16 products: 16 per instruction, 64 per workgroup
    assert dmp.plan_label(4, 4, 16, 16, 4, 4, dmp.GEMM_F16, 0, 1 << 20) == \
        "tiny4x4x16b f16 a:row b:row splitk=1 grid=16384"
    assert dmp.plan_label(16, 16, 16, 16, 16, 16, dmp.GEMM_BF16, 0, 1000).startswith("tiny16x16x4b")
    assert dmp.plan_label(5, 3, 7, 7, 3, 3, dmp.GEMM_I8).startswith("tiny16x16x4b")
    # shared operands are accepted on every path
    for fl in (dmp.GEMM_A_SHARED, dmp.GEMM_B_SHARED, dmp.GEMM_A_SHARED | dmp.GEMM_B_SHARED):
        assert plan_status(4, 4, 16, 16, 4, 4, 0, fl, 100)[0] == 0
        assert plan_status(512, 512, 512, 512, 512, 512, 0, fl, 4)[0] == 0
    # fp64 keeps its own kernels
    assert dmp.plan_label(4, 4, 16, 16, 4, 4, dmp.GEMM_F64, 0, 100).startswith("dgeneric") or \
        dmp.plan_label(4, 4, 16, 16, 4, 4, dmp.GEMM_F64, 0, 100).startswith("dtile")
