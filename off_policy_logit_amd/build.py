"""Build libsc.so in-tree with hipcc for gfx950.

Every call compiles from source (no up-to-date check), then swaps the new
library in atomically.
"""
from __future__ import annotations

import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = [os.path.join(CSRC, "sc_api.cpp"), os.path.join(CSRC, "sc_kernels.hip"),
           os.path.join(CSRC, "sc_lmhead.hip"), os.path.join(CSRC, "sc_record.hip")]
LIB = os.path.join(HERE, "libsc.so")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose=False):
    """Compile libsc.so; raises CalledProcessError with the compiler output."""
    fd, tmp = tempfile.mkstemp(prefix="libsc.", suffix=".so.tmp", dir=HERE)
    os.close(fd)
    cmd = [hipcc(), *FLAGS, "-o", tmp, *SOURCES]
    try:
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise subprocess.CalledProcessError(res.returncode, cmd, res.stdout, res.stderr)
        if verbose:
            print(" ".join(cmd))
        os.replace(tmp, LIB)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
