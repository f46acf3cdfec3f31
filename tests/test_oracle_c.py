"""The plain-C oracle against the NumPy oracle (bit-for-bit) and the pins."""

import numpy as np
import pytest

import oracle_pins as P
from oracle import allreduce as O
from oracle import cpu as C
from allreduce_emulated_peer_amd import workloads as W


def c_impl(xs, dtype):
    return C.allreduce(xs, dtype, nthreads=3)[0]


def test_c_passes_pins():
    P.check_integer_closed_form(c_impl)
    P.check_hand_cases(c_impl)
    P.check_brute_force(c_impl, ranks=(1, 2, 3, 8, 16), sizes=(7, 67))
    P.check_invariants(c_impl)


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_c_matches_numpy_with_specials(dtype):
    g = np.random.default_rng(12)
    for R in (1, 2, 7, 16):
        xs = P.rand_inputs(R, 4099, dtype, 300 + R, scale=1000.0)
        bitsx = [P.bits_of(x, dtype).copy() for x in xs]
        for b in bitsx:
            m = g.random(len(b)) < 0.05
            b[m] = g.choice(P.special_patterns(dtype), size=int(m.sum()))
        xs = [P.from_bits(b, dtype) for b in bitsx]
        outs = C.allreduce(xs, dtype, nthreads=5)
        want = P.bits_of(O.allreduce(xs, dtype), dtype)
        for o in outs:
            got = P.bits_of(o, dtype)
            assert np.all(O.ulp_distance(got, want, dtype) == 0)


@pytest.mark.parametrize("wid", [0, 1, 3])
def test_c_matches_numpy_on_workloads(wid):
    w = W.named()[wid]
    xs = W.generate_all(w)
    want = O.allreduce(xs, w.dtype)
    got = C.allreduce(xs, w.dtype, nthreads=8)
    for g in got:
        assert np.array_equal(P.bits_of(g, w.dtype), P.bits_of(want, w.dtype))


def test_c_thread_count_invariant():
    w = W.ragged_outliers_bf16()
    xs = [W.generate(w, r)[:300_001] for r in range(w.nranks)]
    a = C.allreduce(xs, "bf16", nthreads=1)[0]
    b = C.allreduce(xs, "bf16", nthreads=7)[0]
    assert np.array_equal(a, b)
    assert np.array_equal(a, O.allreduce(xs, "bf16"))
