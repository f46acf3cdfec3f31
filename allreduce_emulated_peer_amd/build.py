"""Build the HIP library libmscl.so in-tree for gfx950.

One translation unit (csrc/mscl.hip: the C ABI, including the kernels of
csrc/kernels.hpp), compiled with hipcc:
-O3, no fast-math, no FP contraction, packed-FP32 instructions disabled.
"""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "mscl.hip")
LIB = os.path.join(HERE, "libmscl.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
# the port channel's proxy drives the SDMA engines through HSA
LIBS = ["-L/opt/rocm/lib", "-lhsa-runtime64"]


def build(verbose: bool = False, extra=()) -> str:
    tmp = LIB + ".tmp"
    cmd = ["/opt/rocm/bin/hipcc", *FLAGS, *extra, "-o", tmp, SRC, *LIBS]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def asm(out_path: str) -> str:
    """Device assembly of the library (for inspection)."""
    cmd = ["/opt/rocm/bin/hipcc", *[f for f in FLAGS if f not in ("-shared", "-fPIC")],
           "--cuda-device-only", "-S", "-o", out_path, SRC]
    subprocess.run(cmd, check=True)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
