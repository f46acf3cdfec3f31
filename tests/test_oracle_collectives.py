"""ReduceScatter and AllGather oracles against independent facts (CPU only).

ReduceScatter: integer closed form, the scalar brute force of oracle_pins on
every element, and the hand-derived golden cases placed in a block.
AllGather: element-by-element index arithmetic in plain Python and bitwise
preservation of every pattern (NaN payloads included).  Planted mistakes
(wrong block, reversed rank order, rounding per block boundary, swapped
concatenation order) must be caught.
"""

import numpy as np
import pytest

import oracle_pins as P
from oracle import allreduce as O


def rs_check_integer(rs):
    for dtype in ("fp32", "fp16", "bf16"):
        for R in (1, 2, 3, 8, 16):
            c = 37
            g = P.rng(500 + R)
            ints = [g.integers(-8, 9, size=R * c) for _ in range(R)]
            xs = []
            for v in ints:
                f = v.astype(np.float32)
                xs.append(f if dtype == "fp32" else (f.astype(np.float16) if dtype == "fp16"
                                                     else (f.view(np.uint32) >> 16).astype(np.uint16)))
            outs = rs(xs, dtype)
            total = np.sum(np.stack(ints), axis=0)
            for r in range(R):
                got = [P.scalar_value(b, dtype) for b in P.bits_of(outs[r], dtype)]
                assert got == [float(t) for t in total[r * c:(r + 1) * c]], f"{dtype} R={R} block {r}"


def rs_check_brute(rs):
    for dtype in ("fp32", "fp16", "bf16"):
        for R in (1, 2, 5, 16):
            c = 9
            xs = P.rand_inputs(R, R * c, dtype, seed=600 + R, scale=300.0)
            bitsx = [P.bits_of(x, dtype).copy() for x in xs]
            g = P.rng(601 + R)
            for b in bitsx:
                m = g.random(len(b)) < 0.1
                b[m] = g.choice(P.special_patterns(dtype), size=int(m.sum()))
            xs = [P.from_bits(b, dtype) for b in bitsx]
            outs = rs(xs, dtype)
            for r in range(R):
                ob = P.bits_of(outs[r], dtype)
                for i in range(c):
                    col = [int(b[r * c + i]) for b in bitsx]
                    want = P.brute_force_element(col, dtype)
                    assert P.same_value(ob[i], want, dtype), f"{dtype} R={R} block {r} elem {i}"


def rs_check_hand(rs):
    for dtype, ins, want in P.load_hand_cases():
        R = len(ins)
        # put the hand case at element 3 of the last rank's block, zeros elsewhere
        c = 5
        xs = []
        for v in ins:
            b = np.zeros(R * c, dtype=np.uint32 if dtype == "fp32" else np.uint16)
            b[(R - 1) * c + 3] = v
            xs.append(P.from_bits(b, dtype))
        got = int(P.bits_of(rs(xs, dtype)[R - 1], dtype)[3])
        if want == "nan":
            assert P.decode(got, dtype)[0] == "nan"
        else:
            assert got == int(want, 16), f"{dtype} {ins}"


def ag_check(ag):
    for dtype in ("fp32", "fp16", "bf16"):
        for R in (1, 2, 3, 7, 16):
            c = 11
            g = P.rng(700 + R)
            width = 32 if dtype == "fp32" else 16
            bitsx = [g.integers(0, 2 ** width, size=c, dtype=np.uint64).astype(np.uint32 if width == 32 else np.uint16)
                     for _ in range(R)]  # arbitrary bit patterns
            # signalling NaNs with payloads must come through untouched too
            snan = {"fp32": 0x7F800001, "fp16": 0x7C01, "bf16": 0x7F81}[dtype]
            for b in bitsx:
                b[0] = snan
                b[1] = snan | (1 << (width - 1))
            xs = [P.from_bits(b, dtype) for b in bitsx]
            outs = ag(xs, dtype)
            assert len(outs) == R
            for p in range(R):
                ob = P.bits_of(outs[p], dtype)
                assert len(ob) == R * c
                for r in range(R):
                    for i in range(c):
                        assert int(ob[r * c + i]) == int(bitsx[r][i]), f"{dtype} R={R} out {p} pos {r * c + i}"


def test_reduce_scatter_pins():
    rs_check_integer(O.reduce_scatter)
    rs_check_brute(O.reduce_scatter)
    rs_check_hand(O.reduce_scatter)


def test_reduce_scatter_consistent_with_allreduce():
    xs = P.rand_inputs(8, 8 * 1000, "bf16", seed=3)
    full = O.allreduce(xs, "bf16")
    blocks = O.reduce_scatter(xs, "bf16")
    assert np.array_equal(np.concatenate(blocks), full)


def test_reduce_scatter_rejects_ragged():
    with pytest.raises(ValueError):
        O.reduce_scatter([np.zeros(7, np.float32)] * 2, "fp32")


def test_allgather_pins():
    ag_check(O.allgather)


def m_rs_wrong_block(xs, dtype):
    outs = O.reduce_scatter(xs, dtype)
    return outs[1:] + outs[:1]


def m_rs_reversed(xs, dtype):
    return O.reduce_scatter(xs[::-1], dtype)


def m_rs_round_each_add(xs, dtype):
    R = len(xs)
    c = len(xs[0]) // R
    outs = []
    for r in range(R):
        a = O.round_to(O.to_f32(xs[0][r * c:(r + 1) * c], dtype), dtype)
        for x in xs[1:]:
            a = O.round_to(O.to_f32(a, dtype) + O.to_f32(x[r * c:(r + 1) * c], dtype), dtype)
        outs.append(a)
    return outs


def m_ag_reversed(xs, dtype):
    return O.allgather(xs[::-1], dtype)


def m_ag_through_float(xs, dtype):
    # widening to binary32 and back loses NaN payloads / quiets signalling NaNs
    out = O.allgather(xs, dtype)
    return [O.round_to(O.to_f32(o, dtype), dtype) for o in out]


@pytest.mark.parametrize("mutant", [m_rs_wrong_block, m_rs_reversed, m_rs_round_each_add], ids=lambda m: m.__name__)
def test_rs_mutants_caught(mutant):
    with pytest.raises(AssertionError):
        rs_check_integer(mutant)
        rs_check_brute(mutant)
        rs_check_hand(mutant)


@pytest.mark.parametrize("mutant", [m_ag_reversed, m_ag_through_float], ids=lambda m: m.__name__)
def test_ag_mutants_caught(mutant):
    with pytest.raises(AssertionError):
        ag_check(mutant)
