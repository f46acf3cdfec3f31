"""MemoryChannel-style AllReduce over R emulated peer buffers on one MI355X.

The compute path is the HIP library ``libmscl.so`` (C ABI in
``include/mscl.h``); ``mscl.py`` is a thin ctypes binding over it.  Importing
this package loads nothing: the binding opens the library on first use and
raises if it is missing (there is no CPU fallback).
"""

__all__ = ["mscl", "workloads"]
