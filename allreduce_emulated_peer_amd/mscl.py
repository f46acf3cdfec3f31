"""Thin ctypes binding over libmscl.so (C ABI in include/mscl.h).

Argument marshalling only: every step of the AllReduce runs in the HIP
library.  Names mirror the C entry points without the ``mscl_`` prefix.
There is no fallback: if the library is missing, loading raises.

Pointers are plain integers (device addresses, e.g. ``tensor.data_ptr()``),
streams are ``hipStream_t`` values as integers (``torch.cuda.Stream.cuda_stream``;
0 = default stream).  ``allreduce_tensors`` is a convenience wrapper that
takes torch tensors and the current torch stream.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmscl.so")

FLOAT32, FLOAT16, BFLOAT16 = 0, 1, 2
ALGO_AUTO, ALGO_ONE_SHOT, ALGO_TWO_SHOT, ALGO_TWO_SHOT_FUSED, ALGO_TWO_SHOT_PORT = 0, 1, 2, 3, 4
ALGO_TWO_SHOT_FUSED_NOBARRIER = 5
ALGO_TWO_SHOT_PERTILE = 6
MAX_RANKS = 16

SUCCESS = 0
ERR_INVALID_ARGUMENT = 1
ERR_UNSUPPORTED = 2
ERR_MISALIGNED = 3
ERR_NOT_INITIALIZED = 4
ERR_OUT_OF_MEMORY = 5
ERR_HIP = 6
ERR_TIMEOUT = 7
ERR_PROTOCOL = 8

DTYPE_CODES = {"fp32": FLOAT32, "fp16": FLOAT16, "bf16": BFLOAT16}
ALGO_CODES = {"auto": ALGO_AUTO, "one_shot": ALGO_ONE_SHOT, "two_shot": ALGO_TWO_SHOT,
              "two_shot_fused": ALGO_TWO_SHOT_FUSED, "two_shot_port": ALGO_TWO_SHOT_PORT,
              "two_shot_fused_nobarrier": ALGO_TWO_SHOT_FUSED_NOBARRIER, "two_shot_pertile": ALGO_TWO_SHOT_PERTILE}

# every function include/mscl.h declares
EXPORTS = (
    "mscl_version", "mscl_status_string", "mscl_last_error_string", "mscl_channel_create",
    "mscl_channel_destroy", "mscl_channel_check", "mscl_channel_reset", "mscl_allreduce",
    "mscl_select_algo", "mscl_channel_plan", "mscl_channel_set_fault_controls", "mscl_channel_set_checks",
    "mscl_reduce_scatter", "mscl_allgather", "mscl_channel_selftest", "mscl_allreduce_noalloc",
)


class MsclError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


class Plan(ctypes.Structure):
    _fields_ = [
        ("algo", ctypes.c_int),
        ("nranks", ctypes.c_int),
        ("workgroups_per_rank", ctypes.c_int),
        ("threads_per_workgroup", ctypes.c_int),
        ("vectors_per_thread", ctypes.c_int),
        ("uses_barrier", ctypes.c_int),
        ("chunk_elems", ctypes.c_size_t),
        ("cached_puts", ctypes.c_int),
        ("held_tiles", ctypes.c_int),
        ("slices", ctypes.c_int),
        ("slice_elems", ctypes.c_size_t),
        ("tile_interleave", ctypes.c_int),
    ]


_lib = None


def load(path: str = LIB_PATH):
    """Open libmscl.so once; raises FileNotFoundError if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} is missing: build it with allreduce_emulated_peer_amd/build.py")
    lib = ctypes.CDLL(path)
    c_int, c_size, vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
    lib.mscl_version.restype = c_int
    lib.mscl_version.argtypes = []
    lib.mscl_status_string.restype = ctypes.c_char_p
    lib.mscl_status_string.argtypes = [c_int]
    lib.mscl_last_error_string.restype = ctypes.c_char_p
    lib.mscl_last_error_string.argtypes = []
    lib.mscl_channel_create.restype = c_int
    lib.mscl_channel_create.argtypes = [c_int, c_int, ctypes.POINTER(vp)]
    for name in ("mscl_channel_destroy", "mscl_channel_check", "mscl_channel_reset"):
        getattr(lib, name).restype = c_int
        getattr(lib, name).argtypes = [vp]
    for name in ("mscl_allreduce", "mscl_allreduce_noalloc"):
        getattr(lib, name).restype = c_int
        getattr(lib, name).argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), c_size, c_int, c_int, c_int, vp]
    for name in ("mscl_reduce_scatter", "mscl_allgather"):
        getattr(lib, name).restype = c_int
        getattr(lib, name).argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), c_size, c_int, c_int, vp]
    lib.mscl_channel_selftest.restype = c_int
    lib.mscl_channel_selftest.argtypes = [vp, ctypes.c_uint32, ctypes.POINTER(ctypes.c_uint64)]
    lib.mscl_select_algo.restype = c_int
    lib.mscl_select_algo.argtypes = [c_size, c_int, c_int, ctypes.POINTER(c_int)]
    lib.mscl_channel_plan.restype = c_int
    lib.mscl_channel_plan.argtypes = [vp, c_size, c_int, c_int, c_int, ctypes.POINTER(Plan)]
    lib.mscl_channel_set_fault_controls.restype = c_int
    lib.mscl_channel_set_fault_controls.argtypes = [vp, ctypes.c_uint64, c_int]
    lib.mscl_channel_set_checks.restype = c_int
    lib.mscl_channel_set_checks.argtypes = [vp, c_int, c_int]
    _lib = lib
    return lib


def _check(status: int, where: str) -> None:
    if status != SUCCESS:
        lib = load()
        detail = lib.mscl_last_error_string().decode() or lib.mscl_status_string(status).decode()
        raise MsclError(status, where, detail)


def version() -> int:
    return load().mscl_version()


def status_string(status: int) -> str:
    return load().mscl_status_string(status).decode()


def last_error_string() -> str:
    return load().mscl_last_error_string().decode()


def _ptr_array(ptrs):
    return (ctypes.c_void_p * len(ptrs))(*[ctypes.c_void_p(int(p)) if p else None for p in ptrs])


def raw_allreduce(inputs, outputs, count: int, dtype: int, nranks: int, algo: int, stream: int) -> int:
    """mscl_allreduce with no exception: returns the status code."""
    ins = _ptr_array(inputs) if inputs is not None else None
    outs = _ptr_array(outputs) if outputs is not None else None
    return load().mscl_allreduce(ins, outs, count, dtype, nranks, algo, ctypes.c_void_p(int(stream) or None))


def allreduce(inputs, outputs, count: int, dtype: int, nranks: int, algo: int = ALGO_AUTO, stream: int = 0) -> None:
    """mscl_allreduce: `inputs` / `outputs` are sequences of device addresses."""
    _check(raw_allreduce(inputs, outputs, count, dtype, nranks, algo, stream), "mscl_allreduce")


def raw_allreduce_noalloc(inputs, outputs, count: int, dtype: int, nranks: int, algo: int, stream: int) -> int:
    """mscl_allreduce_noalloc with no exception: returns the status code."""
    ins = _ptr_array(inputs) if inputs is not None else None
    outs = _ptr_array(outputs) if outputs is not None else None
    return load().mscl_allreduce_noalloc(ins, outs, count, dtype, nranks, algo, ctypes.c_void_p(int(stream) or None))


def allreduce_noalloc(inputs, outputs, count: int, dtype: int, nranks: int, algo: int = ALGO_AUTO,
                      stream: int = 0) -> None:
    """mscl_allreduce_noalloc: mscl_allreduce with no channel set and no allocation."""
    _check(raw_allreduce_noalloc(inputs, outputs, count, dtype, nranks, algo, stream), "mscl_allreduce_noalloc")


def raw_reduce_scatter(inputs, outputs, recvcount: int, dtype: int, nranks: int, stream: int) -> int:
    ins = _ptr_array(inputs) if inputs is not None else None
    outs = _ptr_array(outputs) if outputs is not None else None
    return load().mscl_reduce_scatter(ins, outs, recvcount, dtype, nranks, ctypes.c_void_p(int(stream) or None))


def reduce_scatter(inputs, outputs, recvcount: int, dtype: int, nranks: int, stream: int = 0) -> None:
    """mscl_reduce_scatter: inputs hold nranks*recvcount elements, outputs recvcount."""
    _check(raw_reduce_scatter(inputs, outputs, recvcount, dtype, nranks, stream), "mscl_reduce_scatter")


def raw_allgather(inputs, outputs, sendcount: int, dtype: int, nranks: int, stream: int) -> int:
    ins = _ptr_array(inputs) if inputs is not None else None
    outs = _ptr_array(outputs) if outputs is not None else None
    return load().mscl_allgather(ins, outs, sendcount, dtype, nranks, ctypes.c_void_p(int(stream) or None))


def allgather(inputs, outputs, sendcount: int, dtype: int, nranks: int, stream: int = 0) -> None:
    """mscl_allgather: inputs hold sendcount elements, outputs nranks*sendcount."""
    _check(raw_allgather(inputs, outputs, sendcount, dtype, nranks, stream), "mscl_allgather")


def channel_create(nranks: int, device: int) -> int:
    h = ctypes.c_void_p()
    _check(load().mscl_channel_create(nranks, device, ctypes.byref(h)), "mscl_channel_create")
    return h.value


def channel_destroy(handle: int) -> None:
    _check(load().mscl_channel_destroy(ctypes.c_void_p(handle)), "mscl_channel_destroy")


def channel_check(handle: int) -> int:
    """Status recorded on the device by earlier calls (SUCCESS, ERR_TIMEOUT, ERR_PROTOCOL, ...)."""
    return load().mscl_channel_check(ctypes.c_void_p(handle))


def channel_reset(handle: int) -> None:
    _check(load().mscl_channel_reset(ctypes.c_void_p(handle)), "mscl_channel_reset")


def channel_set_fault_controls(handle: int, wait_timeout_us: int = 0, drop_signal_rank: int = -1) -> None:
    _check(load().mscl_channel_set_fault_controls(ctypes.c_void_p(handle), wait_timeout_us, drop_signal_rank),
           "mscl_channel_set_fault_controls")


def channel_set_checks(handle: int, check_protocol: bool = True, double_signal_rank: int = -1) -> None:
    """mscl_channel_set_checks: protocol checks of every device-side wait, and
    the test control that makes one rank signal twice."""
    _check(load().mscl_channel_set_checks(ctypes.c_void_p(handle), int(bool(check_protocol)), double_signal_rank),
           "mscl_channel_set_checks")


def channel_selftest(handle: int, rounds: int) -> int:
    """mscl_channel_selftest: returns the number of mismatching words (expected 0)."""
    out = ctypes.c_uint64()
    _check(load().mscl_channel_selftest(ctypes.c_void_p(handle), rounds, ctypes.byref(out)), "mscl_channel_selftest")
    return out.value


def select_algo(count: int, dtype: int, nranks: int) -> int:
    out = ctypes.c_int()
    _check(load().mscl_select_algo(count, dtype, nranks, ctypes.byref(out)), "mscl_select_algo")
    return out.value


def channel_plan(handle: int, count: int, dtype: int, algo: int = ALGO_AUTO, in_place: bool = False) -> Plan:
    plan = Plan()
    _check(load().mscl_channel_plan(ctypes.c_void_p(handle), count, dtype, algo, int(in_place), ctypes.byref(plan)),
           "mscl_channel_plan")
    return plan


def allreduce_tensors(inputs, outputs, algo: int = ALGO_AUTO, stream=None) -> None:
    """AllReduce over lists of equal-shape contiguous CUDA(HIP) tensors.

    dtype comes from the tensors (float32 / float16 / bfloat16); the call
    runs with the tensors' device current (the channel set is looked up per
    device, so mscl_channel_create must have been called for that device and
    rank count); the stream defaults to torch's current stream there.
    """
    import torch

    codes = {torch.float32: FLOAT32, torch.float16: FLOAT16, torch.bfloat16: BFLOAT16}
    if len(inputs) != len(outputs) or not inputs:
        raise ValueError("need one output per input")
    t0 = inputs[0]
    if not t0.is_cuda:
        raise ValueError("tensors must be on a GPU")
    for t in list(inputs) + list(outputs):
        if t.dtype != t0.dtype or t.numel() != t0.numel() or not t.is_contiguous() or t.device != t0.device:
            raise ValueError("tensors must share dtype, size and device and be contiguous")
    if t0.dtype not in codes:
        raise ValueError(f"unsupported dtype {t0.dtype}")
    with torch.cuda.device(t0.device):
        if stream is None:
            stream = torch.cuda.current_stream(t0.device)
        handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        allreduce([t.data_ptr() for t in inputs], [t.data_ptr() for t in outputs], t0.numel(), codes[t0.dtype],
                  len(inputs), algo, handle)
