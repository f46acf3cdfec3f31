"""The C ABI driven from plain C (tests/c_abi_driver.c: HIP runtime and
mscl.h only, no Python binding, no torch) on the GPU, checked bit for bit
against the oracle.  Covers every algorithm, every element type, a ragged
tail at R = 16 and an in-place call; out-of-place cases run three calls in a
row on one channel."""

import os
import subprocess

import numpy as np
import pytest

from allreduce_emulated_peer_amd import workloads as W
from oracle import allreduce as O

pytestmark = pytest.mark.gpu

DRIVER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_driver")
CODES = {"fp32": 0, "fp16": 1, "bf16": 2}
ALGOS = {"auto": 0, "one_shot": 1, "two_shot": 2, "two_shot_fused": 3, "two_shot_port": 4}
STORAGE = {"fp32": np.uint32, "fp16": np.uint16, "bf16": np.uint16}

CASES = [
    (4, "fp32", 4096, "int8range", "auto", False),
    (8, "bf16", 100_003, "normal", "auto", False),
    (16, "bf16", 1_000_003, "normal", "two_shot", False),
    (3, "fp16", 77_777, "uniform", "two_shot_fused", False),
    (8, "bf16", 262_147, "normal", "two_shot", True),
    (5, "bf16", 300_001, "normal", "two_shot_port", False),
]

# Plan controls read from the environment once per process, so these run the
# driver with them set: the put policy forced by MSCL_CACHED_PUTS_MAX_BYTES
# (streaming puts at sizes whose default is device-scope puts, device-scope
# puts at a size whose default is streaming), the two-shot's LDS hold with
# its default and turned off by MSCL_TWO_SHOT_HOLD=0, and the interleaved
# tiles of held slices with their default and turned off by
# MSCL_TILE_INTERLEAVE=0; (case, environment, what the driver must report
# about the plan).
ENV_CASES = [
    ((8, "bf16", 1_000_003, "normal", "two_shot_fused", False), {"MSCL_CACHED_PUTS_MAX_BYTES": "0"}, "cached_puts=0"),
    ((8, "bf16", 1_000_003, "normal", "two_shot", True), {"MSCL_CACHED_PUTS_MAX_BYTES": "0"}, "cached_puts=0"),
    ((4, "fp16", 9_000_001, "uniform", "two_shot", False), {"MSCL_CACHED_PUTS_MAX_BYTES": "1000000000"},
     "cached_puts=1"),
    ((8, "bf16", 12_000_007, "normal", "auto", False), {}, "held_tiles=23"),
    ((8, "bf16", 12_000_007, "normal", "two_shot", True), {"MSCL_TWO_SHOT_HOLD": "0"}, "held_tiles=0"),
    ((8, "bf16", 24_000_017, "normal", "two_shot", False), {}, "slices=2 tile_interleave=1"),
    ((8, "bf16", 24_000_017, "normal", "two_shot", True), {"MSCL_TILE_INTERLEAVE": "0"}, "slices=2 tile_interleave=0"),
]


def _case_id(c):
    return f"r{c[0]}_{c[1]}_{c[2]}_{c[4]}{'_inplace' if c[5] else ''}"


@pytest.mark.parametrize("R,dtype,n,dist,algo,in_place", CASES, ids=[_case_id(c) for c in CASES])
def test_c_driver_matches_oracle(tmp_path, R, dtype, n, dist, algo, in_place):
    _run_driver(tmp_path, R, dtype, n, dist, algo, in_place)


@pytest.mark.parametrize("case,env,expect", ENV_CASES,
                         ids=[f"{_case_id(c)}_{'_'.join(f'{k}={v}' for k, v in e.items()) or 'default'}"
                              for c, e, _ in ENV_CASES])
def test_c_driver_plan_controls(tmp_path, case, env, expect):
    out = _run_driver(tmp_path, *case, env=env)
    assert expect in out, out


def _run_driver(tmp_path, R, dtype, n, dist, algo, in_place, env=None):
    assert os.path.exists(DRIVER), "tests/c_abi_driver is not built: run __graft_entry__.build()"
    w = W.custom(R, dtype, n, dist, seed_index=11)
    xs = W.generate_all(w)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        for x in xs:
            f.write(np.ascontiguousarray(x).view(STORAGE[dtype]).tobytes())
    args = [DRIVER, str(R), str(CODES[dtype]), str(n), str(ALGOS[algo]), str(src), str(dst)]
    if in_place:
        args.append("inplace")
    print(f"[gpu-case] c driver {' '.join(args[1:5])} {'in place' if in_place else ''}", flush=True)
    r = subprocess.run(args, capture_output=True, text=True, timeout=120,
                       env=None if env is None else {**os.environ, **env})
    assert r.returncode == 0, f"driver failed ({r.returncode}): {r.stderr}"
    got = np.fromfile(dst, dtype=STORAGE[dtype]).reshape(R, n)
    want = O.bits_of(O.allreduce(xs, dtype), dtype)
    for rank in range(R):
        if not np.array_equal(got[rank], want):
            bad = np.nonzero(O.ulp_distance(got[rank], want, dtype))[0]
            raise AssertionError(f"rank {rank}: {bad.size} elements differ, first at {bad[:8].tolist()}")
    return r.stdout
