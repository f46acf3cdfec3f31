"""Builds tests/c_abi_driver (a plain-C consumer of the library's C ABI) with
gcc against the in-tree libmscl.so and the HIP runtime.  The binary finds both
through its rpath, so it runs from any working directory."""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi_driver.c")
OUT = os.path.join(HERE, "c_abi_driver")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", "-o", OUT, SRC,
           f"-L{os.path.join(ROOT, 'allreduce_emulated_peer_amd')}", "-l:libmscl.so", f"-L{ROCM}/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../allreduce_emulated_peer_amd", f"-Wl,-rpath,{ROCM}/lib"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
