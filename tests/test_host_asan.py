"""The library's host code under AddressSanitizer (CPU only).

Builds an ASan-instrumented copy of libmscl.so (host code only: every
-fsanitize flag is passed through -Xarch_host, device code is compiled as
usual) plus tests/host_asan_driver.c, and runs the driver, which walks every
C-ABI path that needs no GPU for every rank count.  Any out-of-bounds access
or leak report from ASan, or an unexpected status, fails the test.
"""

import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"  # the host compiler hipcc drives; same ASan runtime


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not installed")
def test_host_code_is_asan_clean(tmp_path):
    src = os.path.join(ROOT, "allreduce_emulated_peer_amd", "csrc", "mscl.hip")
    lib = tmp_path / "libmscl_asan.so"
    exe = tmp_path / "driver"
    common = ["-I", os.path.join(ROOT, "include"), "-O1", "-g", "-fno-omit-frame-pointer",
              "-Xarch_host", "-fsanitize=address"]
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *common, "-o", str(lib), src,
                    "-L/opt/rocm/lib", "-lhsa-runtime64"],
                   check=True, capture_output=True)
    subprocess.run([CLANG, *common, "-o", str(exe), os.path.join(HERE, "host_asan_driver.c"),
                    str(lib), f"-Wl,-rpath,{tmp_path}"], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "0 failures" in r.stdout
