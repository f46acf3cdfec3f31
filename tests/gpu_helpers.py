"""Shared helpers for the GPU parity tests (HIP path vs the CPU oracle).

Inputs are generated on the host (seeded), copied into device tensors, the
library is called through its C ABI, and every output is compared with the
oracle bit for bit (ulp distance 0; NaNs compared as NaN), plus the invariant
that all R outputs are identical.  Outputs are filled with a poison pattern
(0xA5 bytes) before each call so unwritten elements show up.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

from allreduce_emulated_peer_amd import mscl as M
from oracle import allreduce as O

TORCH_DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}
CODES = {"fp32": M.FLOAT32, "fp16": M.FLOAT16, "bf16": M.BFLOAT16}
ALGOS = {"one_shot": M.ALGO_ONE_SHOT, "two_shot": M.ALGO_TWO_SHOT, "two_shot_fused": M.ALGO_TWO_SHOT_FUSED,
         "two_shot_port": M.ALGO_TWO_SHOT_PORT, "two_shot_fused_nobarrier": M.ALGO_TWO_SHOT_FUSED_NOBARRIER,
         "two_shot_pertile": M.ALGO_TWO_SHOT_PERTILE, "auto": M.ALGO_AUTO}
EXPLICIT = ("one_shot", "two_shot", "two_shot_fused", "two_shot_port", "two_shot_fused_nobarrier", "two_shot_pertile")
POISON = 0xA5

_channels = {}


def note(msg: str) -> None:
    """Name the case before a GPU step (stderr, flushed)."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def channel(R: int) -> int:
    if R not in _channels:
        _channels[R] = M.channel_create(R, torch.cuda.current_device())
    return _channels[R]


def to_device(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to("cuda")


def to_host_bits(t: torch.Tensor, dtype: str) -> np.ndarray:
    c = t.detach().cpu()
    if dtype == "fp32":
        return c.view(torch.int32).numpy().view(np.uint32)
    return c.view(torch.int16).numpy().view(np.uint16)


def poison_like(t: torch.Tensor) -> torch.Tensor:
    out = torch.empty_like(t)
    out.view(torch.uint8).fill_(POISON)
    return out


def run(xs, dtype, algo="auto", in_place=False, stream=None, dev_inputs=None):
    """Run the HIP AllReduce on host inputs (or on `dev_inputs`, already on the
    device, when given); returns the device outputs."""
    R = len(dev_inputs) if dev_inputs is not None else len(xs)
    channel(R)
    ins = dev_inputs if dev_inputs is not None else [to_device(x, dtype) for x in xs]
    if in_place:
        outs = ins
    else:
        outs = [poison_like(t) for t in ins]
    s = stream if stream is not None else torch.cuda.current_stream()
    M.allreduce([t.data_ptr() for t in ins], [t.data_ptr() for t in outs], ins[0].numel(), CODES[dtype], R,
                ALGOS[algo], s.cuda_stream)
    s.synchronize()
    return outs


def assert_outputs_equal_each_other(outs) -> None:
    ref = outs[0].view(torch.uint8)
    for r, o in enumerate(outs[1:], 1):
        assert torch.equal(o.view(torch.uint8), ref), f"output {r} differs from output 0"


def assert_matches_oracle(outs, want: np.ndarray, dtype: str, what: str) -> None:
    """Bit-exact (ulp distance 0, NaN == NaN) comparison of every output."""
    assert_outputs_equal_each_other(outs)
    got = to_host_bits(outs[0], dtype)
    wb = O.bits_of(want, dtype)
    if np.array_equal(got, wb):
        return
    d = O.ulp_distance(got, wb, dtype)
    bad = np.nonzero(d)[0]
    assert bad.size == 0, (f"{what}: {bad.size} elements differ, first at {bad[:8].tolist()}: "
                           f"got {[hex(int(v)) for v in got[bad[:8]]]} want {[hex(int(v)) for v in wb[bad[:8]]]}, "
                           f"max ulp {int(d.max())}")


def assert_matches_oracle_on_device(outs, want: np.ndarray, dtype: str, what: str) -> None:
    """Full-size version: ship the oracle's result to the device and compare
    bits there (NaN positions compared as NaN)."""
    assert_outputs_equal_each_other(outs)
    w = to_device(want, dtype)
    got = outs[0]
    if torch.equal(got.view(torch.uint8), w.view(torch.uint8)):
        return
    gn, wn = torch.isnan(got.float()), torch.isnan(w.float())
    same = (got.view(torch.uint8).view(-1, got.element_size()) == w.view(torch.uint8).view(-1, w.element_size())).all(1)
    ok = same | (gn & wn)
    bad = torch.nonzero(~ok).flatten()[:8].cpu().tolist()
    assert not bad, f"{what}: elements differ, first at {bad}"


def oracle_full(xs, dtype: str) -> np.ndarray:
    """The oracle's whole result for buffers too large for the NumPy oracle to
    finish quickly: the plain-C oracle (checked bit for bit against the NumPy
    oracle in tests/test_oracle_c.py), on at most 16 host threads, writing one
    output array."""
    import os

    from oracle import cpu as C

    out = np.empty(len(xs[0]), dtype=xs[0].dtype)
    C.allreduce(xs, dtype, nthreads=min(16, os.cpu_count() or 1), outputs=[out] * len(xs))
    return out


def sample_indices(n: int, k: int = 1 << 16, seed: int = 0) -> np.ndarray:
    g = np.random.default_rng(seed)
    edge = np.concatenate([np.arange(min(n, 2048)), np.arange(max(0, n - 2048), n)])
    return np.unique(np.concatenate([edge, g.integers(0, n, size=min(k, n))]))
