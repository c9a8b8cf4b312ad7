"""Host code under the address and undefined-behaviour sanitizers (CPU only):
the library's argument checks and path selection (csrc/plan.hpp, plain C++) and
the CPU oracle (oracle/oracle_gemm.c), each driven by a small program under
tests/native/ that sweeps ordinary and extreme arguments."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def build_and_run(tmp_path, compiler, sources, extra, name):
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not available")
    exe = str(tmp_path / name)
    cmd = [compiler, *SAN, "-Wall", "-Wextra", "-Werror", *extra, "-o", exe, *sources]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
    return r.stdout


def test_plan_logic_under_sanitizers(tmp_path):
    out = build_and_run(tmp_path, "g++", [os.path.join(NATIVE, "plan_check.cpp")],
                        ["-std=c++17"], "plan_check")
    assert "0 failures" in out


def test_oracle_under_sanitizers(tmp_path):
    out = build_and_run(tmp_path, "gcc",
                        [os.path.join(NATIVE, "oracle_check.c"), os.path.join(ROOT, "oracle", "oracle_gemm.c")],
                        ["-std=c11", "-pthread", "-lm"], "oracle_check")
    assert "0 failures" in out
