"""MSCL_LOG (environment, read once by the host library): level 0 prints
nothing, level 1 every failure a call returns, level 2 also the plan of each
call (here: the selector's pick, which needs no GPU)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SNIPPET = """
from allreduce_emulated_peer_amd import mscl as M
assert M.select_algo(8192 * 8192, M.BFLOAT16, 8) == M.ALGO_TWO_SHOT
assert M.raw_allreduce([16] * 2, [4096] * 2, 10, M.FLOAT32, 0, M.ALGO_AUTO, 0) == M.ERR_INVALID_ARGUMENT
print("done")
"""


def run(level):
    env = dict(os.environ)
    env.pop("MSCL_LOG", None)
    if level is not None:
        env["MSCL_LOG"] = str(level)
    r = subprocess.run([sys.executable, "-c", SNIPPET], capture_output=True, text=True, timeout=120, cwd=ROOT, env=env)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "done"
    return [line for line in r.stderr.splitlines() if line.startswith("[mscl]")]


def test_level_0_and_unset_print_nothing():
    assert run(None) == []
    assert run(0) == []


def test_level_1_prints_failures_only():
    lines = run(1)
    assert len(lines) == 1 and "error 1" in lines[0] and "nranks" in lines[0]


def test_level_2_prints_the_plan():
    lines = run(2)
    assert any("select R=8 count=67108864" in line and "two_shot" in line for line in lines), lines
    assert any("error 1" in line for line in lines)
