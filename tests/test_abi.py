"""C-ABI checks that need no GPU: exports, validation codes, the selector.

Every call here fails validation (or is pure host logic) before the library
makes any HIP call, so nothing touches a device.
"""

import os
import re

import pytest

from allreduce_emulated_peer_amd import mscl as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "mscl.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mscl_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = M.load()
    decl = declared_functions()
    assert len(decl) >= 11
    for name in decl:
        assert hasattr(lib, name), f"{name} declared in mscl.h but not exported"
    assert sorted(M.EXPORTS) == decl


def test_missing_library_fails_loudly(tmp_path):
    import importlib

    mod = importlib.reload(M)
    try:
        mod._lib = None
        with pytest.raises(FileNotFoundError):
            mod.load(str(tmp_path / "nope.so"))
    finally:
        importlib.reload(M)


def test_version_and_strings():
    assert M.version() == 100
    for code in range(9):
        assert M.status_string(code) != "unknown status"
    assert M.status_string(99) == "unknown status"


A = 0x100000  # aligned fake addresses: never dereferenced (validation fails or count == 0)


def addrs(R, base, step=0x10000000):
    return [base + r * step for r in range(R)]


@pytest.mark.parametrize("R", [0, -1, 17])
def test_bad_nranks(R):
    assert M.raw_allreduce(addrs(1, A), addrs(1, A * 2), 10, M.BFLOAT16, R, 0, 0) == M.ERR_INVALID_ARGUMENT


def test_bad_dtype_and_algo():
    assert M.raw_allreduce(addrs(2, A), addrs(2, A * 64), 10, 3, 2, 0, 0) == M.ERR_INVALID_ARGUMENT
    assert M.raw_allreduce(addrs(2, A), addrs(2, A * 64), 10, -1, 2, 0, 0) == M.ERR_INVALID_ARGUMENT
    assert M.raw_allreduce(addrs(2, A), addrs(2, A * 64), 10, 0, 2, 7, 0) == M.ERR_INVALID_ARGUMENT
    assert M.raw_allreduce(addrs(2, A), addrs(2, A * 64), 10, 0, 2, -1, 0) == M.ERR_INVALID_ARGUMENT


def test_null_arrays_and_pointers():
    assert M.raw_allreduce(None, addrs(2, A), 10, 0, 2, 0, 0) == M.ERR_INVALID_ARGUMENT
    assert M.raw_allreduce(addrs(2, A), None, 10, 0, 2, 0, 0) == M.ERR_INVALID_ARGUMENT
    ins = addrs(2, A)
    ins[1] = 0
    assert M.raw_allreduce(ins, addrs(2, A * 64), 10, 0, 2, 0, 0) == M.ERR_INVALID_ARGUMENT
    assert "null" in M.last_error_string()


def test_misaligned():
    ins = addrs(4, A)
    ins[2] += 8
    assert M.raw_allreduce(ins, addrs(4, A * 64), 10, 0, 4, 0, 0) == M.ERR_MISALIGNED
    outs = addrs(4, A * 64)
    outs[3] += 2
    assert M.raw_allreduce(addrs(4, A), outs, 10, 0, 4, 0, 0) == M.ERR_MISALIGNED


def test_overlaps():
    n = 1024  # fp32: 4 KiB per buffer
    ins = addrs(3, A, step=0x1000)
    # outputs overlapping each other
    outs = [A * 64, A * 64 + 0x800, A * 64 + 0x2000]
    assert M.raw_allreduce(ins, outs, n, 0, 3, 0, 0) == M.ERR_INVALID_ARGUMENT
    # an output overlapping another rank's input
    outs = [A * 64, ins[2], A * 64 + 0x4000]
    assert M.raw_allreduce(ins, outs, n, 0, 3, 0, 0) == M.ERR_INVALID_ARGUMENT
    # an output partially overlapping its own input
    outs = [ins[0] + 0x10, A * 64, A * 64 + 0x4000]
    assert M.raw_allreduce(ins, outs, n, 0, 3, 0, 0) == M.ERR_INVALID_ARGUMENT
    # in place but inputs alias, so the in-place output overlaps another input
    ins2 = [A, A, A + 0x1000]
    outs = [A, A * 64, A * 64 + 0x4000]
    assert M.raw_allreduce(ins2, outs, n, 0, 3, 0, 0) == M.ERR_INVALID_ARGUMENT


def test_count_zero_is_a_noop():
    assert M.raw_allreduce(addrs(8, A), addrs(8, A * 64), 0, M.BFLOAT16, 8, 0, 0) == M.SUCCESS


def test_size_overflow():
    assert M.raw_allreduce(addrs(2, A), addrs(2, A * 64), 2 ** 63, M.FLOAT32, 2, 0, 0) == M.ERR_INVALID_ARGUMENT
    assert M.raw_allreduce(addrs(2, A), addrs(2, A * 64), 2 ** 62, M.FLOAT32, 2, 0, 0) == M.ERR_INVALID_ARGUMENT


def test_selector():
    # one-shot up to a limit that falls with R, fused two-shot (with its
    # completion barrier) up to a limit, two-shot above; bytes per rank buffer
    KiB, MiB = 1024, 1024 * 1024
    one_limit = {2: 8 * MiB, 3: 2 * MiB, 4: MiB, 5: MiB, 6: 512 * KiB, 7: 512 * KiB, 8: 256 * KiB, 9: 256 * KiB,
                 11: 256 * KiB, 12: 128 * KiB, 16: 128 * KiB}
    fused_limit = {4: 16 * MiB, 5: 8 * MiB, 6: MiB, 7: MiB, 8: 2 * MiB, 9: MiB, 11: MiB, 12: MiB, 15: MiB,
                   16: 256 * KiB}
    for R, limit in one_limit.items():
        assert M.select_algo(1, M.BFLOAT16, R) == M.ALGO_ONE_SHOT
        assert M.select_algo(limit // 2, M.BFLOAT16, R) == M.ALGO_ONE_SHOT
        assert M.select_algo(limit // 2 + 1, M.BFLOAT16, R) == M.ALGO_TWO_SHOT_FUSED
        assert M.select_algo(limit // 4, M.FLOAT32, R) == M.ALGO_ONE_SHOT
        assert M.select_algo(limit // 4 + 1, M.FLOAT32, R) == M.ALGO_TWO_SHOT_FUSED
        if R in fused_limit:
            f = fused_limit[R]
            assert M.select_algo(f // 2, M.BFLOAT16, R) == M.ALGO_TWO_SHOT_FUSED
            assert M.select_algo(f // 2 + 1, M.BFLOAT16, R) == M.ALGO_TWO_SHOT
            assert M.select_algo(f // 4 + 1, M.FLOAT32, R) == M.ALGO_TWO_SHOT
        else:  # R = 2, 3: fused at every size above the one-shot band
            assert M.select_algo(2 ** 40, M.BFLOAT16, R) == M.ALGO_TWO_SHOT_FUSED
    assert M.select_algo(1, M.BFLOAT16, 1) == M.ALGO_ONE_SHOT
    assert M.select_algo(2 ** 40, M.BFLOAT16, 1) == M.ALGO_ONE_SHOT  # one buffer: a copy at every size
    assert M.select_algo(4096, M.FLOAT32, 4) == M.ALGO_ONE_SHOT  # the 16 KiB integer workload
    assert M.select_algo(32 * 8192, M.BFLOAT16, 8) == M.ALGO_TWO_SHOT_FUSED  # 512 KiB decode shape
    assert M.select_algo(8192 * 8192, M.BFLOAT16, 8) == M.ALGO_TWO_SHOT  # 128 MiB prefill shape
    assert M.select_algo(2 ** 24 - 1, M.BFLOAT16, 16) == M.ALGO_TWO_SHOT  # ragged R = 16 workload
    with pytest.raises(M.MsclError):
        M.select_algo(10, 7, 8)
    with pytest.raises(M.MsclError):
        M.select_algo(10, M.FLOAT32, 0)


def test_channel_calls_reject_unknown_handles():
    lib = M.load()
    import ctypes

    bogus = ctypes.c_void_p(0x1234)
    assert lib.mscl_channel_destroy(None) == M.ERR_INVALID_ARGUMENT
    assert lib.mscl_channel_destroy(bogus) == M.ERR_INVALID_ARGUMENT
    assert lib.mscl_channel_check(bogus) == M.ERR_INVALID_ARGUMENT
    assert lib.mscl_channel_reset(bogus) == M.ERR_INVALID_ARGUMENT
    assert lib.mscl_channel_set_fault_controls(bogus, 0, -1) == M.ERR_INVALID_ARGUMENT
    assert lib.mscl_channel_set_checks(bogus, 1, -1) == M.ERR_INVALID_ARGUMENT
    assert lib.mscl_channel_set_checks(None, 0, -1) == M.ERR_INVALID_ARGUMENT
    plan = M.Plan()
    assert lib.mscl_channel_plan(bogus, 10, 0, 0, 0, ctypes.byref(plan)) == M.ERR_INVALID_ARGUMENT
    count = ctypes.c_uint64()
    assert lib.mscl_channel_selftest(bogus, 10, ctypes.byref(count)) == M.ERR_INVALID_ARGUMENT
    assert lib.mscl_channel_selftest(bogus, 10, None) == M.ERR_INVALID_ARGUMENT
    out = ctypes.c_void_p()
    assert lib.mscl_channel_create(0, 0, ctypes.byref(out)) == M.ERR_INVALID_ARGUMENT
    assert lib.mscl_channel_create(17, 0, ctypes.byref(out)) == M.ERR_INVALID_ARGUMENT
    assert lib.mscl_channel_create(4, -1, ctypes.byref(out)) == M.ERR_INVALID_ARGUMENT
    assert lib.mscl_channel_create(4, 0, None) == M.ERR_INVALID_ARGUMENT


# ---------------------------------------------------------------- ReduceScatter / AllGather validation

@pytest.mark.parametrize("fn", ["raw_reduce_scatter", "raw_allgather"])
def test_blocks_bad_arguments(fn):
    call = getattr(M, fn)
    ins, outs = addrs(4, A), addrs(4, A * 64)
    assert call(ins, outs, 10, M.FLOAT32, 0, 0) == M.ERR_INVALID_ARGUMENT
    assert call(ins, outs, 10, M.FLOAT32, 17, 0) == M.ERR_INVALID_ARGUMENT
    assert call(ins, outs, 10, 3, 4, 0) == M.ERR_INVALID_ARGUMENT
    assert call(None, outs, 10, M.FLOAT32, 4, 0) == M.ERR_INVALID_ARGUMENT
    assert call(ins, None, 10, M.FLOAT32, 4, 0) == M.ERR_INVALID_ARGUMENT
    bad = list(ins)
    bad[1] = 0
    assert call(bad, outs, 10, M.FLOAT32, 4, 0) == M.ERR_INVALID_ARGUMENT
    assert call(ins, outs, 2 ** 62, M.FLOAT32, 4, 0) == M.ERR_INVALID_ARGUMENT
    assert call(ins, outs, 0, M.FLOAT32, 4, 0) == M.SUCCESS  # no-op, nothing launched


@pytest.mark.parametrize("fn", ["raw_reduce_scatter", "raw_allgather"])
def test_blocks_element_alignment(fn):
    call = getattr(M, fn)
    ins, outs = addrs(2, A), addrs(2, A * 64)
    odd = list(ins)
    odd[0] += 2  # 2-byte aligned: fine for bf16 (would need a GPU), wrong for fp32
    assert call(odd, outs, 8, M.FLOAT32, 2, 0) == M.ERR_MISALIGNED
    odd = list(outs)
    odd[1] += 1
    assert call(ins, odd, 8, M.BFLOAT16, 2, 0) == M.ERR_MISALIGNED


def test_reduce_scatter_overlaps():
    R, rc = 3, 256  # fp32: blocks of 1 KiB, inputs of 3 KiB
    blk = rc * 4
    ins = [A + r * 0x10000 for r in range(R)]
    outs = [A * 64 + r * 0x10000 for r in range(R)]
    outs2 = list(outs)
    outs2[1] = outs2[0] + blk // 2  # outputs overlap each other
    assert M.raw_reduce_scatter(ins, outs2, rc, M.FLOAT32, R, 0) == M.ERR_INVALID_ARGUMENT
    outs2 = list(outs)
    outs2[0] = ins[1]  # output inside another rank's input
    assert M.raw_reduce_scatter(ins, outs2, rc, M.FLOAT32, R, 0) == M.ERR_INVALID_ARGUMENT
    outs2 = list(outs)
    outs2[2] = ins[2] + 1 * blk  # own input, but not block 2
    assert M.raw_reduce_scatter(ins, outs2, rc, M.FLOAT32, R, 0) == M.ERR_INVALID_ARGUMENT


def test_allgather_overlaps():
    R, sc = 3, 256
    blk = sc * 4
    ins = [A + r * 0x10000 for r in range(R)]
    outs = [A * 64 + r * 0x10000 for r in range(R)]
    outs2 = list(outs)
    outs2[2] = outs2[1] + blk  # outputs (3 KiB each) overlap
    assert M.raw_allgather(ins, outs2, sc, M.FLOAT32, R, 0) == M.ERR_INVALID_ARGUMENT
    ins2 = list(ins)
    ins2[0] = outs[1]  # input inside another rank's output
    assert M.raw_allgather(ins2, outs, sc, M.FLOAT32, R, 0) == M.ERR_INVALID_ARGUMENT
    ins2 = list(ins)
    ins2[1] = outs[1]  # own output, but block 0 instead of block 1
    assert M.raw_allgather(ins2, outs, sc, M.FLOAT32, R, 0) == M.ERR_INVALID_ARGUMENT


def test_plain_c_consumer_links_and_loads():
    """tests/c_abi_driver is built against include/mscl.h and libmscl.so with
    gcc alone; it loads the library through its rpath from any directory."""
    import subprocess

    driver = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_driver")
    assert os.path.exists(driver), "tests/c_abi_driver is not built: run __graft_entry__.build()"
    r = subprocess.run([driver, "--version"], capture_output=True, text=True, timeout=60, cwd="/")
    assert r.returncode == 0 and r.stdout.strip() == f"mscl version {M.load().mscl_version()}"
    r = subprocess.run([driver, "0", "2", "16", "0", "/nonexistent", "/nonexistent"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 1 and "bad R" in r.stderr


def test_allreduce_tensors_rejects_bad_arguments_before_any_gpu_call():
    import torch

    cpu = [torch.zeros(8, dtype=torch.bfloat16) for _ in range(2)]
    with pytest.raises(ValueError, match="one output per input"):
        M.allreduce_tensors(cpu, cpu[:1])
    with pytest.raises(ValueError, match="one output per input"):
        M.allreduce_tensors([], [])
    with pytest.raises(ValueError, match="on a GPU"):
        M.allreduce_tensors(cpu, [torch.empty_like(t) for t in cpu])
