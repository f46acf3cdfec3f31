"""ctypes wrapper for the plain-C oracle (oracle/allreduce_cpu.c).

TEST INFRASTRUCTURE ONLY.  Same storage convention as oracle/allreduce.py.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_CODES = {"fp32": 0, "fp16": 1, "bf16": 2}
_STORAGE = {"fp32": np.float32, "fp16": np.float16, "bf16": np.uint16}
_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        lib.orc_allreduce.restype = ctypes.c_int
        lib.orc_allreduce.argtypes = [
            ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p),
            ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ]
        for name in ("orc_round_f16", "orc_round_bf16", "orc_widen_f16"):
            getattr(lib, name).restype = None
            getattr(lib, name).argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t]
        _lib = lib
    return _lib


def allreduce(inputs, dtype: str, nthreads: int | None = None, outputs=None):
    """Reduce R host arrays; returns the list of R outputs (all equal)."""
    lib = load()
    n = len(inputs[0])
    ins = [np.ascontiguousarray(x, dtype=_STORAGE[dtype]) for x in inputs]
    if outputs is None:
        outputs = [np.empty(n, dtype=_STORAGE[dtype]) for _ in inputs]
    R = len(ins)
    in_arr = (ctypes.c_void_p * R)(*[x.ctypes.data for x in ins])
    out_arr = (ctypes.c_void_p * R)(*[y.ctypes.data for y in outputs])
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    rc = lib.orc_allreduce(in_arr, out_arr, n, _CODES[dtype], R, int(nthreads))
    if rc != 0:
        raise ValueError("orc_allreduce rejected its arguments")
    return outputs


def round_f16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    load().orc_round_f16(a.ctypes.data, out.ctypes.data, a.size)
    return out.view(np.float16)


def round_bf16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    load().orc_round_bf16(a.ctypes.data, out.ctypes.data, a.size)
    return out


def widen_f16(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.float16).view(np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    load().orc_widen_f16(h.ctypes.data, out.ctypes.data, h.size)
    return out
