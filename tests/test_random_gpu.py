"""GPU parity over seeded random calls: rank count, length (log-uniform, any
residue), dtype, algorithm and in-place flag drawn together, so that
combinations no hand-written case names (an odd R with fp16 in place on the
per-tile kernel, a ragged share of a held slice at R = 11, ...) are checked
bit for bit against the oracle too."""

import numpy as np
import pytest
import torch

import gpu_helpers as G
import oracle_pins as P
from oracle import allreduce as O

pytestmark = pytest.mark.gpu

CASES = 600


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    yield


def draw_cases(seed=20261203):
    g = np.random.default_rng(seed)
    algos = list(G.EXPLICIT) + ["auto", "auto"]
    cases = []
    for _ in range(CASES):
        R = int(g.integers(1, 17))
        dtype = ("fp32", "fp16", "bf16")[int(g.integers(0, 3))]
        n = int(np.exp(g.uniform(0.0, np.log(6_000_000)))) + int(g.integers(0, 9))
        algo = algos[int(g.integers(0, len(algos)))]
        in_place = bool(g.integers(0, 2)) and algo != "two_shot_port"
        cases.append((R, n, dtype, algo, in_place))
    return cases


def test_random_calls_match_the_oracle():
    for i, (R, n, dtype, algo, in_place) in enumerate(draw_cases()):
        xs = P.rand_inputs(R, n, dtype, seed=i)
        want = O.allreduce(xs, dtype) if R * n <= (1 << 22) else G.oracle_full(xs, dtype)
        G.note(f"random case {i}: R={R} n={n} {dtype} {algo} in_place={in_place}")
        outs = G.run(xs, dtype, algo, in_place=in_place)
        G.assert_matches_oracle_on_device(outs, want, dtype, f"case {i}: R={R} n={n} {dtype} {algo} in_place={in_place}")
