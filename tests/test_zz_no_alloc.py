"""The allocation-free AllReduce (mscl_allreduce_noalloc) against the
allocating entry point (mscl_allreduce), through the C ABI: bit-for-bit equal
outputs on two calls in a row, the second with a smaller input, for every
algorithm that keeps channel state (and the others), out of place and in
place; a rank count with no channel set at all; graph replays."""

import numpy as np
import pytest
import torch

import gpu_helpers as G
import oracle_pins as P
from allreduce_emulated_peer_amd import mscl as M

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    M.load()
    yield


def _ptrs(ts):
    return [t.data_ptr() for t in ts]


def _both(R, n, dtype, algo, in_place, seed):
    """Run the allocating and the allocation-free call on the same inputs;
    return both sets of outputs."""
    xs = P.rand_inputs(R, n, dtype, seed=seed)
    ins_a = [G.to_device(x, dtype) for x in xs]
    ins_b = [t.clone() for t in ins_a]
    outs_a = ins_a if in_place else [G.poison_like(t) for t in ins_a]
    outs_b = ins_b if in_place else [G.poison_like(t) for t in ins_b]
    G.channel(R)
    s = torch.cuda.current_stream().cuda_stream
    M.allreduce(_ptrs(ins_a), _ptrs(outs_a), n, G.CODES[dtype], R, algo, s)
    M.allreduce_noalloc(_ptrs(ins_b), _ptrs(outs_b), n, G.CODES[dtype], R, algo, s)
    torch.cuda.synchronize()
    return outs_a, outs_b


@pytest.mark.parametrize("algo", ["auto", "one_shot", "two_shot", "two_shot_fused", "two_shot_fused_nobarrier",
                                  "two_shot_pertile"])
@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("R,dtype,sizes", [(8, "bf16", (24_000_017, 300_001)), (16, "fp16", (9_000_011, 777)),
                                           (4, "fp32", (3_000_017, 70_001))],
                         ids=["r8_bf16", "r16_fp16", "r4_fp32"])
def test_noalloc_matches_allreduce(algo, in_place, R, dtype, sizes):
    for k, n in enumerate(sizes):  # two calls in a row, the second smaller
        plan = M.channel_plan(G.channel(R), n, G.CODES[dtype], G.ALGOS[algo], in_place=in_place)
        G.note(f"noalloc R={R} {dtype} n={n} {algo} in_place={in_place} uses_barrier={plan.uses_barrier} "
               f"slices={plan.slices}")
        a, b = _both(R, n, dtype, G.ALGOS[algo], in_place, seed=n % 1009 + k)
        G.assert_outputs_equal_each_other(b)
        for r in range(R):
            assert torch.equal(a[r].view(torch.uint8), b[r].view(torch.uint8)), f"output {r} differs (n={n})"


def test_noalloc_needs_no_channel_set():
    """With no channel set for R = 13 in this process (the one the other tests
    made is released first), the allocating entry point refuses and the
    allocation-free one runs and matches the oracle."""
    from oracle import allreduce as O

    R, n, dtype = 13, 1_000_003, "bf16"
    torch.cuda.synchronize()
    cached = G._channels.pop(R, None)
    if cached is not None:
        M.channel_destroy(cached)
    xs = P.rand_inputs(R, n, dtype, seed=13)
    ins = [G.to_device(x, dtype) for x in xs]
    outs = [G.poison_like(t) for t in ins]
    s = torch.cuda.current_stream().cuda_stream
    assert M.raw_allreduce(_ptrs(ins), _ptrs(outs), n, M.BFLOAT16, R, M.ALGO_TWO_SHOT, s) == M.ERR_NOT_INITIALIZED
    for algo in (M.ALGO_TWO_SHOT, M.ALGO_TWO_SHOT_FUSED):
        G.note(f"noalloc R=13 without a channel set, algo {algo}")
        M.allreduce_noalloc(_ptrs(ins), _ptrs(outs), n, M.BFLOAT16, R, algo, s)
        torch.cuda.synchronize()
        G.assert_matches_oracle(outs, O.allreduce(xs, dtype), dtype, f"noalloc R=13 algo {algo}")
    assert M.raw_allreduce_noalloc(_ptrs(ins), _ptrs(outs), n, M.BFLOAT16, R, M.ALGO_TWO_SHOT_PORT, s) == \
        M.ERR_INVALID_ARGUMENT


def test_noalloc_graph_replay():
    """A captured allocation-free two-shot (its scratch clear is a kernel, not a
    memset node) replayed with eager work between replays."""
    R, n, dtype = 8, 4_000_037, "bf16"
    xs = P.rand_inputs(R, n, dtype, seed=77)
    ins = [G.to_device(x, dtype) for x in xs]
    ref = [G.poison_like(t) for t in ins]
    outs = [G.poison_like(t) for t in ins]
    G.channel(R)
    M.allreduce(_ptrs(ins), _ptrs(ref), n, M.BFLOAT16, R, M.ALGO_TWO_SHOT, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        M.allreduce_noalloc(_ptrs(ins), _ptrs(outs), n, M.BFLOAT16, R, M.ALGO_TWO_SHOT, side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        M.allreduce_noalloc(_ptrs(ins), _ptrs(outs), n, M.BFLOAT16, R, M.ALGO_TWO_SHOT,
                            torch.cuda.current_stream().cuda_stream)
    for rep in range(5):
        for o in outs:
            o.zero_()
        small = [G.poison_like(t[:1000]) for t in ins]  # an eager call of another size between replays
        M.allreduce_noalloc(_ptrs([t[:1000] for t in ins]), _ptrs(small), 1000, M.BFLOAT16, R, M.ALGO_TWO_SHOT,
                            torch.cuda.current_stream().cuda_stream)
        G.note(f"noalloc graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for r in range(R):
            assert torch.equal(ref[r].view(torch.uint8), outs[r].view(torch.uint8)), f"replay {rep} output {r}"
    del g
