"""Plausible mistakes planted in copies of the oracle must fail a pin.

Each mutant below is the oracle with one thing wrong (order, start value, a
dropped or negated term, rounding rule, accumulation precision, subnormal
flushing).  The pins of oracle_pins.py must reject every one of them; if a
mutant slipped through, the pins would not be pinning the oracle.
"""

import numpy as np
import pytest

import oracle_pins as P
from oracle import allreduce as O


def _acc(xs, dtype):
    return [O.to_f32(x, dtype) for x in xs]


def m_reverse_order(xs, dtype):
    return O.allreduce(xs[::-1], dtype)


def m_start_from_zero(xs, dtype):
    a = np.zeros(len(xs[0]), dtype=np.float32)
    for x in _acc(xs, dtype):
        a = a + x
    return O.round_to(a, dtype)


def m_drop_last_rank(xs, dtype):
    return O.allreduce(xs[:-1] if len(xs) > 1 else xs, dtype)


def m_negate_last_rank(xs, dtype):
    vs = _acc(xs, dtype)
    a = vs[0].copy()
    for k, x in enumerate(vs[1:], 1):
        a = a - x if k == len(vs) - 1 else a + x
    return O.round_to(a, dtype)


def m_pairwise_tree(xs, dtype):
    vs = _acc(xs, dtype)
    while len(vs) > 1:
        nxt = [vs[i] + vs[i + 1] for i in range(0, len(vs) - 1, 2)]
        if len(vs) % 2:
            nxt.append(vs[-1])
        vs = nxt
    return O.round_to(vs[0], dtype)


def m_f64_accumulate(xs, dtype):
    vs = [v.astype(np.float64) for v in _acc(xs, dtype)]
    a = vs[0].copy()
    for v in vs[1:]:
        a += v
    return O.round_to(a.astype(np.float32), dtype)


def m_exact_then_round_direct(xs, dtype):
    # accumulate in binary64 and round straight to the element type (single rounding)
    vs = [v.astype(np.float64) for v in _acc(xs, dtype)]
    a = vs[0].copy()
    for v in vs[1:]:
        a += v
    if dtype == "fp16":
        return a.astype(np.float16)
    if dtype == "bf16":
        import torch
        return torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return a.astype(np.float32)


def m_truncate_bf16(xs, dtype):
    a = O.accumulate_f32(xs, dtype)
    if dtype == "bf16":
        return (a.view(np.uint32) >> 16).astype(np.uint16)
    return O.round_to(a, dtype)


def m_ties_away_bf16(xs, dtype):
    a = O.accumulate_f32(xs, dtype)
    if dtype != "bf16":
        return O.round_to(a, dtype)
    u = a.view(np.uint32).astype(np.uint64)
    return (((u + 0x8000) >> 16) & 0xFFFF).astype(np.uint16)


def m_flush_subnormals(xs, dtype):
    y = O.allreduce(xs, dtype)
    b = P.bits_of(y, dtype).copy()
    ebits, fbits = P.FIELDS[dtype]
    exp = (b >> fbits) & ((1 << ebits) - 1)
    sign = b & (1 << (ebits + fbits))
    b = np.where(exp == 0, sign, b).astype(b.dtype)
    return P.from_bits(b, dtype)


def m_rank0_counted_twice(xs, dtype):
    return O.allreduce([xs[0]] + list(xs), dtype)


MUTANTS = [m_reverse_order, m_start_from_zero, m_drop_last_rank, m_negate_last_rank,
           m_pairwise_tree, m_f64_accumulate, m_exact_then_round_direct, m_truncate_bf16,
           m_ties_away_bf16, m_flush_subnormals, m_rank0_counted_twice]


def caught(impl):
    for check in P.ALL_CHECKS:
        try:
            check(impl)
        except AssertionError:
            return check.__name__
    return None


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_mutant_is_caught(mutant):
    assert caught(mutant) is not None, f"{mutant.__name__} passed every pin"


def test_real_oracle_is_not_caught():
    assert caught(lambda xs, d: O.allreduce(xs, d)) is None
