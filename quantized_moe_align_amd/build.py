"""Build libqma.so for gfx950 in-tree with hipcc.

Run as ``python -m quantized_moe_align_amd.build`` or through
``__graft_entry__.build()``. The library is written next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libqma.so")
SOURCES = [os.path.join(HERE, "csrc", "qma_host.cpp"),
           os.path.join(HERE, "csrc", "qma_kernels.hip")]
ARCH = "gfx950"

# Packed-FP32 VALU forms are disabled for all device code. MFMA accumulators
# are kept in architectural VGPRs: the 128-token GEMM tile fits there, and
# the AGPR form made the register allocator shuffle accumulators every
# iteration.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-function", *DEVICE_FLAGS,
           "-I", os.path.join(ROOT, "include"), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
