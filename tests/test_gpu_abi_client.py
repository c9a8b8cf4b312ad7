"""The C ABI from plain C: tests/native/abi_client.c (built with gcc against
include/dmp_gemm.h, the HIP runtime and libdmp_gemm.so, no Python in the loop)
runs fp16, int8, fp64, output-stage and 2:4 products on small-integer inputs
and checks them exactly against its own triple loop, plus rejected arguments
and gemm_plan without a handle.  It runs as a child process."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "native", "abi_client")


def test_plain_c_client_of_the_abi():
    torch = pytest.importorskip("torch")
    if torch.cuda.device_count() == 0:
        pytest.skip("no GPU")
    if not os.path.exists(CLIENT):
        raise RuntimeError(f"{CLIENT} is not built (build() builds it)")
    print("[abi-client] running the C client", flush=True)
    r = subprocess.run([CLIENT], capture_output=True, text=True, timeout=100)
    assert r.returncode == 0, r.stdout + r.stderr
    assert ", 0 failures" in r.stdout, r.stdout + r.stderr
