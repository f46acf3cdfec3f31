"""Compile the plain-C oracle (test infrastructure) into oracle/liborc_allreduce.so.

gcc, -O2 without fast-math or FP contraction, pthreads.  Called from
__graft_entry__.build() and, if the library is missing, lazily from
oracle.cpu.load().
"""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "allreduce_cpu.c")
LIB = os.path.join(HERE, "liborc_allreduce.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [
        "gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
        "-Wall", "-Wextra", "-o", tmp, SRC, "-lpthread",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
