"""Property test of mscl_allreduce's argument validation (host only, no GPU).

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
    """The pool and strategy reach every outcome (a guard against a model that
    only ever says 'invalid')."""
    import random

    g = random.Random(5)
    seen = set()
    for _ in range(20000):
        R = g.randint(1, 16)
        ins = [g.choice(POOL) for _ in range(R)]
        outs = [i if g.random() < 0.3 else g.choice(POOL) for i in ins]
        count = g.choice([0, 1, 64, 4096, 2 ** 62])
        seen.add(model(ins, outs, count, g.choice([0, 1, 2]), R, g.randint(0, 6)))
    assert {None, M.SUCCESS, M.ERR_INVALID_ARGUMENT, M.ERR_MISALIGNED} <= seen
