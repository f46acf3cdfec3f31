"""The channel layer's ordering contracts, checked on the device.

mscl_channel_selftest makes every (rank, slot) workgroup write a mailbox,
signal/wait on the publishing barrier and read the next rank's mailbox, which
a workgroup on another XCD wrote before it signalled, then pass the
write-after-read barrier before the next round overwrites the mailboxes.  A
stale word means the release/acquire pairing across the XCDs' separate L2
caches is broken; a word from the next round means a peer's store overtook
this workgroup's loads across the write-after-read barrier.
"""

import pytest
import torch

import gpu_helpers as G
from allreduce_emulated_peer_amd import mscl as M

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    M.load()
    yield


@pytest.mark.parametrize("R,rounds", [(2, 5000), (3, 5000), (8, 20000), (16, 5000)])
def test_signal_publishes_writes_across_xcds(R, rounds):
    h = G.channel(R)
    G.note(f"channel self-test R={R} rounds={rounds}")
    assert M.channel_selftest(h, rounds) == 0
    assert M.channel_check(h) == M.SUCCESS


def test_selftest_keeps_epochs_for_collectives():
    """The self-test advances the same semaphores; collectives after it still
    line up."""
    import numpy as np

    import oracle_pins as P
    from oracle import allreduce as O

    R = 8
    h = G.channel(R)
    assert M.channel_selftest(h, 100) == 0
    xs = P.rand_inputs(R, 100_003, "bf16", seed=99)
    want = O.allreduce(xs, "bf16")
    for algo in G.EXPLICIT:
        outs = G.run(xs, "bf16", algo)
        G.assert_matches_oracle(outs, want, "bf16", f"after self-test {algo}")
