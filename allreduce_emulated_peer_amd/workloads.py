"""Seeded synthetic inputs for the emulated-peer AllReduce.

This module is shared by the tests, the benchmark and the oracle checks, and
therefore holds none of the reduction's arithmetic: it only draws random
values and stores them in the element type.  Storage convention:
fp32 -> numpy float32, fp16 -> numpy float16, bf16 -> numpy uint16 bit
patterns.

Every rank buffer comes from its own generator,
``numpy.random.default_rng(SeedSequence([20261202, workload_id, size_index,
rank]))``.  Values are drawn in binary32/binary64 and converted to the
element type by library routines (NumPy for binary16, torch's CPU cast for
bfloat16), both round-to-nearest-even.

The shapes stand in for the tensor-parallel hidden-state all-reduces that the
MSCCL++ pages name as the target use (project summary, "Highlighted
Details"): decode-step (32 tokens x 8192 hidden) and prefill (8192 x 8192)
activations, plus a latency/bandwidth sweep and a ragged, outlier-heavy
stress case.  No dataset or trained weights are involved.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED_ROOT = 20261202
STORAGE = {"fp32": np.float32, "fp16": np.float16, "bf16": np.uint16}
ELEM_BYTES = {"fp32": 4, "fp16": 2, "bf16": 2}


@dataclass(frozen=True)
class Workload:
    name: str
    workload_id: int      # seeds the generators
    size_index: int       # seeds the generators (sweep point)
    nranks: int
    dtype: str
    count: int            # elements per rank buffer
    dist: str             # "int8range" | "normal" | "uniform" | "normal_outliers"
    sigma: float = 1.0
    meta: dict = field(default_factory=dict, compare=False)

    @property
    def bytes_per_rank(self) -> int:
        return self.count * ELEM_BYTES[self.dtype]

    @property
    def algorithmic_bytes(self) -> int:
        """R*S read plus R*S written."""
        return 2 * self.nranks * self.bytes_per_rank


def integer_small() -> Workload:
    """R=4, fp32, 4096 elements (16 KiB); integers in [-8, 8], sums exact."""
    return Workload("r4_fp32_16KiB_int", 0, 0, 4, "fp32", 4096, "int8range")


def decode_bf16() -> Workload:
    """R=8, bf16, 32 tokens x 8192 hidden (512 KiB), N(0,1)."""
    return Workload("r8_bf16_512KiB_decode", 1, 0, 8, "bf16", 32 * 8192, "normal", 1.0)


def prefill_bf16() -> Workload:
    """R=8, bf16, 8192 tokens x 8192 hidden (128 MiB), N(0, sigma=0.5)."""
    return Workload("r8_bf16_128MiB_prefill", 2, 0, 8, "bf16", 8192 * 8192, "normal", 0.5)


def sweep_fp16(k: int) -> Workload:
    """R=8, fp16, 2**k bytes per buffer (k = 10..28), uniform[-1, 1]."""
    if not 10 <= k <= 28:
        raise ValueError("sweep point k must be in 10..28")
    return Workload(f"r8_fp16_sweep_2^{k}B", 3, k, 8, "fp16", 2 ** (k - 1), "uniform")


def ragged_outliers_bf16() -> Workload:
    """R=16, bf16, 2**24 - 1 elements; N(0,1) with 1% large-magnitude outliers."""
    return Workload("r16_bf16_ragged_outliers", 4, 0, 16, "bf16", 2 ** 24 - 1, "normal_outliers", 1.0)


def sweep_bf16(k: int) -> Workload:
    """R=8, bf16, 2**k bytes per buffer, N(0,1): the 512 KiB..128 MiB range
    (k = 19..27) plus the 16 KiB latency point (k = 14)."""
    if not 10 <= k <= 28:
        raise ValueError("sweep point k must be in 10..28")
    return Workload(f"r8_bf16_sweep_2^{k}B", 5, k, 8, "bf16", 2 ** (k - 1), "normal", 1.0)


def custom(nranks: int, dtype: str, count: int, dist: str = "normal", seed_index: int = 0,
           sigma: float = 1.0) -> Workload:
    """Small ad-hoc cases for the tests (workload id 9)."""
    return Workload(f"custom_r{nranks}_{dtype}_{count}_{dist}_{seed_index}", 9, seed_index,
                    nranks, dtype, count, dist, sigma)


def named() -> dict:
    """The five reference workloads by their index."""
    return {0: integer_small(), 1: decode_bf16(), 2: prefill_bf16(), 3: sweep_fp16(20),
            4: ragged_outliers_bf16()}


def rng_for(w: Workload, rank: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([SEED_ROOT, w.workload_id, w.size_index, rank]))


def _to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    import torch  # CPU cast only

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp16":
        return np.ascontiguousarray(x).astype(np.float16)
    return _to_bf16_bits(np.asarray(x, dtype=np.float32))


def generate(w: Workload, rank: int) -> np.ndarray:
    """Rank `rank`'s input buffer for workload `w`, in storage form."""
    rng = rng_for(w, rank)
    n = w.count
    if w.dist == "int8range":
        x = rng.integers(-8, 9, size=n).astype(np.float32)
    elif w.dist == "normal":
        x = rng.standard_normal(n, dtype=np.float32)
        if w.sigma != 1.0:
            x *= np.float32(w.sigma)
    elif w.dist == "uniform":
        x = rng.uniform(-1.0, 1.0, size=n)
    elif w.dist == "normal_outliers":
        x = rng.standard_normal(n, dtype=np.float32)
        mask = rng.random(n, dtype=np.float32) < np.float32(0.01)
        k = int(mask.sum())
        mag = rng.uniform(32768.0, 65504.0, size=k).astype(np.float32)
        sign = np.where(rng.random(k) < 0.5, np.float32(-1.0), np.float32(1.0))
        x[mask] = sign * mag
    else:
        raise ValueError(f"unknown distribution {w.dist!r}")
    return _store(x, w.dtype)


def generate_all(w: Workload) -> list:
    return [generate(w, r) for r in range(w.nranks)]
