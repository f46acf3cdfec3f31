"""NumPy oracle: the plain definition of the emulated-peer AllReduce.

TEST INFRASTRUCTURE ONLY — imported by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg, never by the product path.

Element storage convention (shared by every caller of this module):
  "fp32" -> numpy float32 array
  "fp16" -> numpy float16 array
  "bf16" -> numpy uint16 array holding bfloat16 bit patterns

Definition followed (see the package docstring for the sources and the
reading taken where the pages are silent):

    for each element i:
        a = f32(x_0[i])
        for p = 1 .. R-1:  a = a (+)_f32 f32(x_p[i])      # binary32 add, RNE
        y[i] = RNE_dtype(a)                                # identity for fp32
    outputs = [y] * R                                      # replicated

The work is cut into element blocks only to bound host memory; the blocks are
independent because the definition is element-wise.
"""

from __future__ import annotations

import numpy as np

DTYPES = ("fp32", "fp16", "bf16")
ELEM_BYTES = {"fp32": 4, "fp16": 2, "bf16": 2}
STORAGE = {"fp32": np.float32, "fp16": np.float16, "bf16": np.uint16}


def _check_dtype(dtype: str) -> None:
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}; expected one of {DTYPES}")


def to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored elements to binary32 exactly.

    fp16 -> fp32 and bf16 -> fp32 are exact: every binary16 / bfloat16 value
    (subnormals, infinities and NaNs included) is a binary32 value.  bfloat16
    is the upper half of a binary32 pattern, so widening is a 16-bit shift.
    """
    _check_dtype(dtype)
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "fp16":
        return np.asarray(x, dtype=np.float16).astype(np.float32)
    bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return bits.view(np.float32)


def f32_to_bf16_rne(a: np.ndarray) -> np.ndarray:
    """Round binary32 values to bfloat16 bit patterns, nearest-even.

    bfloat16 keeps the top 16 bits of a binary32 pattern.  For a finite value
    the discarded low half L decides the rounding: L above 0x8000 rounds the
    kept part up, below rounds down, and exactly 0x8000 (a tie) rounds to the
    kept part with an even last bit.  Adding 0x7FFF plus the kept part's last
    bit and truncating does exactly that; a carry out of the mantissa bumps the
    exponent, which is also how the largest finite values round to infinity.
    Infinities pass unchanged (their low half is zero).  NaNs keep their sign
    and top payload bits and are made quiet (bit 6 set) so truncation can never
    turn one into an infinity.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    is_nan = (u & 0x7F800000) == 0x7F800000
    is_nan &= (u & 0x007FFFFF) != 0
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    quiet_nan = ((u >> 16) | 0x0040) & 0xFFFF
    return np.where(is_nan, quiet_nan, rounded).astype(np.uint16)


def round_to(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round binary32 totals to the element type (round-to-nearest-even).

    fp32: identity.  fp16: NumPy's binary32 -> binary16 conversion, which
    rounds to nearest-even, produces subnormals and overflows to infinity (a
    library routine used as one step; pinned in the tests against torch and a
    from-definition rounding).  bf16: f32_to_bf16_rne.
    """
    _check_dtype(dtype)
    a = np.asarray(a, dtype=np.float32)
    if dtype == "fp32":
        return a.copy()
    if dtype == "fp16":
        with np.errstate(over="ignore"):
            return a.astype(np.float16)
    return f32_to_bf16_rne(a)


def accumulate_f32(inputs, dtype: str, lo: int = 0, hi: int | None = None) -> np.ndarray:
    """binary32 running sum over ranks 0..R-1 in rank order, elements [lo, hi).

    Starts from rank 0's value itself (not from +0.0), so an all-(-0.0)
    column stays -0.0.
    """
    _check_dtype(dtype)
    if len(inputs) == 0:
        raise ValueError("need at least one rank")
    if hi is None:
        hi = len(inputs[0])
    acc = to_f32(inputs[0][lo:hi], dtype).copy()
    with np.errstate(over="ignore", invalid="ignore"):  # IEEE Inf/NaN results are intended
        for x in inputs[1:]:
            acc += to_f32(x[lo:hi], dtype)
    return acc


def allreduce(inputs, dtype: str, block: int = 1 << 22) -> np.ndarray:
    """The reduced buffer y (one copy).  Every output of the AllReduce is y."""
    _check_dtype(dtype)
    n = len(inputs[0])
    for x in inputs:
        if len(x) != n:
            raise ValueError("all rank buffers must have the same length")
    y = np.empty(n, dtype=STORAGE[dtype])
    for lo in range(0, n, block):
        hi = min(n, lo + block)
        y[lo:hi] = round_to(accumulate_f32(inputs, dtype, lo, hi), dtype)
    return y


def allreduce_outputs(inputs, dtype: str) -> list:
    """All R outputs of the AllReduce: R copies of the reduced buffer."""
    y = allreduce(inputs, dtype)
    return [y.copy() for _ in inputs]


def allreduce_elements(inputs, dtype: str, index: np.ndarray) -> np.ndarray:
    """The reduced value at selected element indices only (for sampled checks
    of buffers too large to reduce whole)."""
    _check_dtype(dtype)
    idx = np.asarray(index, dtype=np.int64)
    acc = to_f32(np.asarray(inputs[0])[idx], dtype).copy()
    with np.errstate(over="ignore", invalid="ignore"):
        for x in inputs[1:]:
            acc += to_f32(np.asarray(x)[idx], dtype)
    return round_to(acc, dtype)


def bits_of(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored elements as unsigned integer bit patterns (u32 for fp32, else u16)."""
    _check_dtype(dtype)
    if dtype == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if dtype == "fp16":
        return np.ascontiguousarray(x, dtype=np.float16).view(np.uint16)
    return np.ascontiguousarray(x, dtype=np.uint16)


def ulp_distance(got: np.ndarray, want: np.ndarray, dtype: str) -> np.ndarray:
    """Distance in units in the last place of the element type.

    Bit patterns are sign-magnitude; mapping them to a monotone integer line
    (negative values to minus their magnitude, so +0 and -0 both map to 0)
    makes adjacent representable values differ by one.  Two NaNs are distance
    0 (payloads are not compared); a NaN against a non-NaN is reported as
    2**40.
    """
    g = bits_of(got, dtype).astype(np.int64)
    w = bits_of(want, dtype).astype(np.int64)
    if dtype == "fp32":
        sign, mag, exp_mask, man_mask = 1 << 31, (1 << 31) - 1, 0x7F800000, 0x007FFFFF
    elif dtype == "fp16":
        sign, mag, exp_mask, man_mask = 1 << 15, (1 << 15) - 1, 0x7C00, 0x03FF
    else:
        sign, mag, exp_mask, man_mask = 1 << 15, (1 << 15) - 1, 0x7F80, 0x007F

    def ordinal(b):
        return np.where(b & sign, -(b & mag), b & mag)

    def nan(b):
        return ((b & exp_mask) == exp_mask) & ((b & man_mask) != 0)

    d = np.abs(ordinal(g) - ordinal(w))
    gn, wn = nan(g), nan(w)
    d = np.where(gn & wn, 0, d)
    d = np.where(gn ^ wn, 1 << 40, d)
    return d


def reduce_scatter(inputs, dtype: str) -> list:
    """ReduceScatter (sum) of R buffers of R*c elements each: output r holds
    elements [r*c, (r+1)*c) of the element-wise sum, accumulated and rounded
    exactly as in `allreduce` (the standard collective that hands each rank
    one block of the reduced result; the MSCCL++ ASPLOS'26 abstract places
    the method in a library offering the usual collective interface)."""
    _check_dtype(dtype)
    R = len(inputs)
    n = len(inputs[0])
    if n % R:
        raise ValueError("each input must hold R * recvcount elements")
    c = n // R
    return [round_to(accumulate_f32(inputs, dtype, r * c, (r + 1) * c), dtype) for r in range(R)]


def allgather(inputs, dtype: str) -> list:
    """AllGather of R buffers of c elements each: every output is rank 0's
    buffer, then rank 1's, ..., then rank R-1's (R*c elements), bit for bit."""
    _check_dtype(dtype)
    joined = np.concatenate([np.asarray(x, dtype=STORAGE[dtype]) for x in inputs])
    return [joined.copy() for _ in inputs]
