"""Build libdmp_gemm.so for gfx950 with hipcc (in-tree)."""
from __future__ import annotations

import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = [os.path.join(_HERE, "csrc", "gemm_api.hip")]
OUT = os.path.join(_HERE, "libdmp_gemm.so")
# The race-check variant: every pipeline step waits for its copies and meets
# every wave; its results must equal the library's bit for bit.
OUT_SYNC = os.path.join(_HERE, "libdmp_gemm_sync.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU forms stay off; the compiler still emits the scalar forms
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(out: str, extra: list) -> subprocess.Popen:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, *HIPCC_FLAGS, *extra, "-o", out + ".tmp", *SOURCES]
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


def build(verbose: bool = False) -> str:
    """Builds the library and its race-check variant (in parallel); returns the library's path."""
    jobs = [(OUT, _compile(OUT, [])), (OUT_SYNC, _compile(OUT_SYNC, ["-DDMP_EXTRA_SYNC"]))]
    failed = []
    for out, proc in jobs:
        _, err = proc.communicate()
        if proc.returncode != 0:
            sys.stderr.write(err)
            failed.append(os.path.basename(out))
            continue
        if verbose:
            sys.stderr.write(err)
        os.replace(out + ".tmp", out)
    if failed:
        raise RuntimeError("hipcc failed for " + ", ".join(failed))
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
