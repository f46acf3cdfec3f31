"""GPU tests of the protocol checks (mscl_channel_set_checks): with checks on,
calls ordered on one stream never record MSCL_ERR_PROTOCOL, whatever the
algorithm, size, workgroup count or in-place flag; and a rank made to signal
twice (the host-side test control standing in for two overlapping calls on
one channel set) is caught within a few calls by every kernel that waits on
the semaphores.  Every kernel still exits normally: doubled signals only let
waits finish sooner."""

import ctypes

import pytest
import torch

import gpu_helpers as G
import oracle_pins as P
from allreduce_emulated_peer_amd import mscl as M

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    M.load()
    yield


def raw_call(ins, outs, n, dtype, algo):
    R = len(ins)
    lib = M.load()
    return lib.mscl_allreduce((ctypes.c_void_p * R)(*[t.data_ptr() for t in ins]),
                              (ctypes.c_void_p * R)(*[t.data_ptr() for t in outs]), n, G.CODES[dtype], R,
                              G.ALGOS[algo], ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_ordered_calls_pass_the_checks():
    """Checks on, a mixed sequence of calls on two channel sets (every
    algorithm, sizes from one tile to 8 held slices, in and out of place,
    repeated in-place one-shots with a barrier per batch): the status stays
    SUCCESS and every algorithm's result equals AUTO's."""
    for R, dtype, sizes in ((8, "bf16", (4099, 262_147, 4_194_311, (64 << 20) // 2)),
                            (5, "fp32", (1000, 1_000_003, 5_000_011))):
        h = G.channel(R)
        M.channel_set_checks(h, True, -1)
        try:
            for n in sizes:
                xs = P.rand_inputs(R, n, dtype, seed=n % 991)
                dev_in = [G.to_device(x, dtype) for x in xs]
                ref = G.run(None, dtype, "auto", dev_inputs=dev_in)
                for algo in G.EXPLICIT:
                    G.note(f"checks on: R={R} {dtype} n={n} {algo}")
                    outs = G.run(None, dtype, algo, dev_inputs=dev_in)
                    for a, b in zip(outs, ref):
                        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), algo
                    if algo != "two_shot_port":
                        G.run(None, dtype, algo, in_place=True, dev_inputs=[t.clone() for t in dev_in])
                assert M.channel_check(h) == M.SUCCESS, f"R={R} n={n}: {M.status_string(M.channel_check(h))}"
            # many barriers per call: the in-place one-shot waits once per batch of tiles
            xs = P.rand_inputs(R, 65_539, dtype, seed=7)
            dev_in = [G.to_device(x, dtype) for x in xs]
            G.note(f"checks on: R={R} 200 in-place one-shots")
            for _ in range(200):
                assert raw_call(dev_in, dev_in, 65_539, dtype, "one_shot") == M.SUCCESS
            torch.cuda.synchronize()
            assert M.channel_check(h) == M.SUCCESS
        finally:
            M.channel_set_checks(h, False, -1)


@pytest.mark.parametrize("algo,in_place,n", [("two_shot", False, 4_194_311), ("two_shot", False, (64 << 20) // 2),
                                             ("two_shot_fused", False, 262_147), ("one_shot", True, 200_003),
                                             ("two_shot_pertile", False, 1_000_003)],
                         ids=["two_shot_held", "two_shot_sliced", "fused", "one_shot_in_place", "pertile"])
def test_doubled_signals_are_caught(algo, in_place, n):
    """Rank 1 signals twice: within six calls the checks record PROTOCOL
    (later calls are then refused); a reset clears it and ordered calls pass
    again."""
    R, dtype = 8, "bf16"
    h = G.channel(R)
    xs = P.rand_inputs(R, n, dtype, seed=n % 983)
    dev_in = [G.to_device(x, dtype) for x in xs]
    outs = dev_in if in_place else [torch.empty_like(t) for t in dev_in]
    M.channel_reset(h)
    M.channel_set_checks(h, True, 1)
    try:
        caught_at = None
        for i in range(6):
            G.note(f"doubled signals: {algo} n={n} call {i}")
            st = raw_call(dev_in, outs, n, dtype, algo)
            if st != M.SUCCESS:
                assert st == M.ERR_PROTOCOL, M.status_string(st)
                caught_at = i
                break
            torch.cuda.synchronize()
            if M.channel_check(h) != M.SUCCESS:
                assert M.channel_check(h) == M.ERR_PROTOCOL, M.status_string(M.channel_check(h))
                caught_at = i
                break
        assert caught_at is not None, f"{algo}: doubled signals not caught in 6 calls"
        assert raw_call(dev_in, outs, n, dtype, algo) == M.ERR_PROTOCOL  # refused until reset
    finally:
        torch.cuda.synchronize()
        M.channel_set_checks(h, True, -1)
        M.channel_reset(h)
    G.note(f"after reset: {algo} n={n}")
    for _ in range(3):
        assert raw_call(dev_in, outs, n, dtype, algo) == M.SUCCESS
    torch.cuda.synchronize()
    assert M.channel_check(h) == M.SUCCESS
    M.channel_set_checks(h, False, -1)


def test_environment_turns_checks_on_for_new_sets_and_the_noalloc_entry():
    """MSCL_CHECK_PROTOCOL=1 (read once per process) starts every channel set
    with the checks on: a child process runs ordered calls of every waiting
    algorithm and must see no failure recorded.  The allocation-free entry
    point runs its kernels with the checks on too, between those calls (its
    status word is device-only, so it can only show here as a call that does
    not return or a channel set that records something)."""
    import os
    import subprocess
    import sys

    code = r"""
import torch
from allreduce_emulated_peer_amd import mscl as M
dev = torch.cuda.current_device()
h = M.channel_create(8, dev)
for n in (4099, 262147, 4194311, (64 << 20) // 2):
    ins = [torch.randn(n, device="cuda").to(torch.bfloat16) for _ in range(8)]
    outs = [torch.empty_like(t) for t in ins]
    s = torch.cuda.current_stream().cuda_stream
    for algo in (M.ALGO_AUTO, M.ALGO_ONE_SHOT, M.ALGO_TWO_SHOT, M.ALGO_TWO_SHOT_FUSED, M.ALGO_TWO_SHOT_PERTILE):
        M.allreduce([t.data_ptr() for t in ins], [t.data_ptr() for t in outs], n, M.BFLOAT16, 8, algo, s)
        if n <= 262147:
            M.allreduce_noalloc([t.data_ptr() for t in ins], [t.data_ptr() for t in outs], n, M.BFLOAT16, 8, algo, s)
    torch.cuda.synchronize()
    assert M.channel_check(h) == M.SUCCESS, M.status_string(M.channel_check(h))
print("checks on, nothing recorded", flush=True)
"""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, MSCL_CHECK_PROTOCOL="1", PYTHONPATH=root)
    G.note("child process with MSCL_CHECK_PROTOCOL=1")
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=root, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "nothing recorded" in r.stdout
