"""Property tests of the argument validation of mscl_allreduce,
mscl_reduce_scatter and mscl_allgather (host only, no GPU).

Random rank counts, dtypes, algorithms, counts and pointer tables (drawn from
a small pool of addresses so that nulls, misalignment, address-space wrap,
partial overlaps, aliasing and in-place pairs all occur) are checked against
a plain model of the contract in include/mscl.h: checks in the order the
header states them, rank by rank, and the first failing one decides; count 0,
and R = 1 in place, succeed with nothing launched.  A call that passes
validation goes on to look up its channel set, which does not
exist here, so it must end in NOT_INITIALIZED or HIP — never in a validation
status.  No pointer is ever dereferenced: every call stops before a launch.
"""

import ctypes
import random

from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from allreduce_emulated_peer_amd import mscl as M

UINTPTR_MAX = (1 << 64) - 1
SIZE_MAX = (1 << 64) - 1
A = 0x100000000

# addresses: aligned bases a page or two apart (so that buffers of a few KiB
# overlap or not), misaligned neighbours, null, and the top of the space
POOL = [0, A, A + 8, A + 16, A + 0x1000, A + 0x1008, A + 0x2000, A + 0x3000, 2 * A, 2 * A + 0x800,
        UINTPTR_MAX - 0xFFF, UINTPTR_MAX - 15]


def model(ins, outs, count, dtype, R, algo):
    """The status the header promises, or None for 'passes validation'."""
    if R < 1 or R > 16:
        return M.ERR_INVALID_ARGUMENT
    if dtype not in (M.FLOAT32, M.FLOAT16, M.BFLOAT16):
        return M.ERR_INVALID_ARGUMENT
    if algo < 0 or algo > 6:
        return M.ERR_INVALID_ARGUMENT
    e = 4 if dtype == M.FLOAT32 else 2
    if count > SIZE_MAX // e:
        return M.ERR_INVALID_ARGUMENT
    nbytes = count * e
    for r in range(R):
        if ins[r] == 0 or outs[r] == 0:
            return M.ERR_INVALID_ARGUMENT
        if ins[r] % 16 or outs[r] % 16:
            return M.ERR_MISALIGNED
        if UINTPTR_MAX - ins[r] < nbytes or UINTPTR_MAX - outs[r] < nbytes:
            return M.ERR_INVALID_ARGUMENT
    if count == 0:
        return M.SUCCESS

    def overlap(x, y):
        return x < y + nbytes and y < x + nbytes

    for r in range(R):
        for q in range(r + 1, R):
            if overlap(outs[r], outs[q]):
                return M.ERR_INVALID_ARGUMENT
        for p in range(R):
            if p == r and outs[r] == ins[r]:
                continue
            if overlap(outs[r], ins[p]):
                return M.ERR_INVALID_ARGUMENT
    if R == 1 and outs[0] == ins[0]:
        return M.SUCCESS  # the sum of one buffer is already in place: nothing to launch
    return None


@st.composite
def calls(draw):
    R = draw(st.one_of(st.integers(1, 16), st.sampled_from([0, 17])))
    n = max(R, 1)
    ins = draw(st.lists(st.sampled_from(POOL), min_size=n, max_size=n))
    outs = []
    for r in range(n):
        # often in place, often a fresh pool address
        outs.append(ins[r] if draw(st.booleans()) and draw(st.booleans()) else draw(st.sampled_from(POOL)))
    count = draw(st.one_of(st.integers(0, 4096), st.sampled_from([0, 1, 2 ** 61, 2 ** 62, 2 ** 63 - 1])))
    dtype = draw(st.one_of(st.sampled_from([M.FLOAT32, M.FLOAT16, M.BFLOAT16]), st.sampled_from([-1, 3])))
    algo = draw(st.one_of(st.integers(0, 6), st.sampled_from([-1, 7])))
    return ins, outs, count, dtype, R, algo


@settings(max_examples=3000, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(calls())
def test_validation_matches_the_contract(call):
    ins, outs, count, dtype, R, algo = call
    want = model(ins, outs, count, dtype, R, algo)
    got = M.raw_allreduce(ins, outs, count, dtype, R, algo, 0)
    if want is None:
        assert got in (M.ERR_NOT_INITIALIZED, M.ERR_HIP), (got, M.last_error_string())
    else:
        assert got == want, (got, want, M.last_error_string())


def test_the_model_is_not_trivial():
    """The pools reach every outcome (a guard against a model that only ever
    says 'invalid')."""
    g = random.Random(5)
    seen = set()
    for _ in range(20000):
        R = g.randint(1, 16)
        ins = [g.choice(POOL) for _ in range(R)]
        outs = [i if g.random() < 0.3 else g.choice(POOL) for i in ins]
        count = g.choice([0, 1, 64, 4096, 2 ** 62])
        seen.add(model(ins, outs, count, g.choice([0, 1, 2]), R, g.randint(0, 6)))
    assert {None, M.SUCCESS, M.ERR_INVALID_ARGUMENT, M.ERR_MISALIGNED} <= seen


def blocks_model(ins, outs, count, dtype, R, gather):
    """ReduceScatter (gather False: inputs hold R blocks, outputs one) and
    AllGather (gather True: inputs one block, outputs R): element-size
    alignment, and an output may overlap an input only as rank r's own block
    in place (ReduceScatter: outputs[r] == inputs[r] + r * block; AllGather:
    inputs[r] == outputs[r] + r * block)."""
    if R < 1 or R > 16:
        return M.ERR_INVALID_ARGUMENT
    if dtype not in (M.FLOAT32, M.FLOAT16, M.BFLOAT16):
        return M.ERR_INVALID_ARGUMENT
    e = 4 if dtype == M.FLOAT32 else 2
    if count > SIZE_MAX // e // R:
        return M.ERR_INVALID_ARGUMENT
    blk = count * e
    in_len = blk if gather else blk * R
    out_len = blk * R if gather else blk
    for r in range(R):
        if ins[r] == 0 or outs[r] == 0:
            return M.ERR_INVALID_ARGUMENT
        if ins[r] % e or outs[r] % e:
            return M.ERR_MISALIGNED
        if UINTPTR_MAX - ins[r] < in_len or UINTPTR_MAX - outs[r] < out_len:
            return M.ERR_INVALID_ARGUMENT
    if count == 0:
        return M.SUCCESS

    def overlap(x, xl, y, yl):
        return x < y + yl and y < x + xl

    for r in range(R):
        for q in range(r + 1, R):
            if overlap(outs[r], out_len, outs[q], out_len):
                return M.ERR_INVALID_ARGUMENT
        for p in range(R):
            if not overlap(outs[r], out_len, ins[p], in_len):
                continue
            own = p == r and (ins[r] == outs[r] + r * blk if gather else outs[r] == ins[r] + r * blk)
            if not own:
                return M.ERR_INVALID_ARGUMENT
    return None


BLOCK_POOL = [0, A, A + 2, A + 4, A + 16, A + 0x400, A + 0x800, A + 0x1000, A + 0x1800, 2 * A, 2 * A + 6,
              UINTPTR_MAX - 0x7FF]


@st.composite
def block_calls(draw):
    R = draw(st.one_of(st.integers(1, 8), st.sampled_from([0, 17])))
    n = max(R, 1)
    count = draw(st.one_of(st.integers(0, 512), st.sampled_from([0, 1, 2 ** 60, 2 ** 62])))
    dtype = draw(st.one_of(st.sampled_from([M.FLOAT32, M.FLOAT16, M.BFLOAT16]), st.sampled_from([-1, 3])))
    gather = draw(st.booleans())
    e = 4 if dtype == M.FLOAT32 else 2
    ins, outs = [], []
    for r in range(n):
        i = draw(st.sampled_from(BLOCK_POOL))
        if draw(st.integers(0, 3)) == 0 and count < 2 ** 40:  # rank r's own block, in place
            o = i - r * count * e if gather else i + r * count * e
            o = o if 0 <= o <= UINTPTR_MAX else draw(st.sampled_from(BLOCK_POOL))
        else:
            o = draw(st.sampled_from(BLOCK_POOL))
        ins.append(i)
        outs.append(o)
    return ins, outs, count, dtype, R, gather


@settings(max_examples=3000, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(block_calls())
def test_block_validation_matches_the_contract(call):
    ins, outs, count, dtype, R, gather = call
    want = blocks_model(ins, outs, count, dtype, R, gather)
    lib = M.load()
    fn = lib.mscl_allgather if gather else lib.mscl_reduce_scatter
    got = fn(M._ptr_array(ins), M._ptr_array(outs), count, dtype, R, ctypes.c_void_p(None))
    if want is None:
        assert got in (M.ERR_NOT_INITIALIZED, M.ERR_HIP), (got, M.last_error_string())
    else:
        assert got == want, (got, want, M.last_error_string())


def test_the_block_model_is_not_trivial():
    g = random.Random(7)
    seen = {False: set(), True: set()}
    for _ in range(20000):
        R = g.randint(1, 8)
        count = g.choice([0, 1, 8, 64, 512])
        dtype = g.choice([0, 1, 2])
        gather = g.random() < 0.5
        e = 4 if dtype == M.FLOAT32 else 2
        ins = [g.choice(BLOCK_POOL) for _ in range(R)]
        outs = [(i - r * count * e if gather else i + r * count * e) if g.random() < 0.3 and i
                else g.choice(BLOCK_POOL) for r, i in enumerate(ins)]
        seen[gather].add(blocks_model(ins, outs, count, dtype, R, gather))
    for gather in (False, True):
        assert {None, M.SUCCESS, M.ERR_INVALID_ARGUMENT, M.ERR_MISALIGNED} <= seen[gather], (gather, seen[gather])
