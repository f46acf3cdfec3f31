"""The NumPy oracle against facts that do not come from it (CPU only)."""

import numpy as np
import pytest

import oracle_pins as P
from oracle import allreduce as O
from allreduce_emulated_peer_amd import workloads as W


def impl(xs, dtype):
    return O.allreduce(xs, dtype)


def test_integer_closed_form():
    P.check_integer_closed_form(impl)


def test_integer_workload_16KiB():
    w = W.integer_small()
    P.check_integer_workload(impl, W.generate_all(w))


@pytest.mark.parametrize("dtype,R", [("bf16", 8), ("fp16", 8), ("bf16", 16), ("fp32", 4)])
def test_fraction_exact(dtype, R):
    P.check_fraction_exact(impl, dtype=dtype, R=R, n=1200, seed=R)


def test_brute_force():
    P.check_brute_force(impl)


def test_hand_cases():
    P.check_hand_cases(impl)


def test_invariants():
    P.check_invariants(impl)


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_replication(dtype):
    xs = P.rand_inputs(5, 333, dtype, 9)
    P.check_replication(O.allreduce_outputs, xs, dtype)


def test_blocking_does_not_change_results():
    # the oracle cuts work into blocks only to bound memory
    xs = P.rand_inputs(8, 10007, "bf16", 77)
    a = O.allreduce(xs, "bf16", block=1 << 22)
    b = O.allreduce(xs, "bf16", block=129)
    assert np.array_equal(a, b)


def test_sampled_elements_match_full():
    xs = P.rand_inputs(8, 5000, "fp16", 78)
    full = O.allreduce(xs, "fp16")
    idx = np.array([0, 1, 17, 4095, 4999])
    assert np.array_equal(O.allreduce_elements(xs, "fp16", idx).view(np.uint16), full[idx].view(np.uint16))


def test_outlier_workload_is_order_sensitive():
    """The ragged outlier workload exists to make the accumulation order
    matter; check that it does (reverse order changes some results) on a
    prefix, so the parity tests really pin the order."""
    w = W.ragged_outliers_bf16()
    xs = [W.generate(w, r)[:200_000] for r in range(w.nranks)]
    fwd = O.allreduce(xs, "bf16")
    rev = O.allreduce(xs[::-1], "bf16")
    assert np.count_nonzero(fwd != rev) > 0


def test_ulp_distance():
    a = np.array([0x3F80, 0x3F81, 0x8000, 0x0000, 0x0001, 0x8001, 0x7FC0], dtype=np.uint16)
    b = np.array([0x3F81, 0x3F80, 0x0000, 0x8000, 0x8001, 0x0001, 0x7FC1], dtype=np.uint16)
    assert list(O.ulp_distance(a, b, "bf16")) == [1, 1, 0, 0, 2, 2, 0]
