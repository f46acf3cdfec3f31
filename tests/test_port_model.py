"""CPU model of the port channel's request ring, run under random interleavings.

A plain-Python rendition of the protocol between the posting GPU lanes and the
host proxy: a lane reserves ring index i with an atomic add on `head`, writes
the entry's fields into slot i mod capacity, then writes the sequence word
i + 1 last; the proxy keeps its own `tail`, takes slot tail mod capacity only
once its sequence word equals tail + 1, and then reads the fields.  Each call
posts R*(R-1) requests (R ranks, one lane per peer) and, as in the library,
the next call starts only after the proxy has taken and completed all of them.

Checked over many seeded interleavings and enough calls to wrap the 256-entry
ring several times: every request is taken exactly once, in index order, with
the fields its lane wrote (never a half-written or stale entry).  Planted
mistakes (sequence word written before the fields, a proxy that does not wait
for the sequence word, a sequence word without the +1 offset) must each be
caught.
"""

import random

import pytest

CAPACITY = 256


class Ring:
    def __init__(self):
        self.head = 0
        self.slots = [{"seq": 0, "fields": None} for _ in range(CAPACITY)]


class Protocol:
    """The protocol as built; mutants override single methods."""

    seq_offset = 1

    def post(self, ring, payload):
        idx = ring.head  # atomic fetch-add: one step, no interleaving inside
        ring.head += 1
        yield
        slot = ring.slots[idx % CAPACITY]
        slot["fields"] = ("half", payload)  # a multi-word write is visible part-way
        yield
        slot["fields"] = ("whole", payload)
        yield
        slot["seq"] = idx + self.seq_offset
        yield

    def ready(self, slot, tail):
        return slot["seq"] == tail + 1


class SeqFirst(Protocol):
    def post(self, ring, payload):
        idx = ring.head
        ring.head += 1
        yield
        slot = ring.slots[idx % CAPACITY]
        slot["seq"] = idx + 1
        yield
        slot["fields"] = ("half", payload)
        yield
        slot["fields"] = ("whole", payload)
        yield


class NoSeqCheck(Protocol):
    def ready(self, slot, tail):
        return slot["fields"] is not None


class NoOffset(Protocol):
    seq_offset = 0


def run(protocol, seed, R=8, calls=12):
    rng = random.Random(seed)
    ring = Ring()
    tail = 0
    taken = []
    for call in range(calls):
        posts = [protocol.post(ring, (call, r, p)) for r in range(R) for p in range(R) if p != r]
        live = list(posts)
        expected = len(posts)
        got = 0
        steps = 0
        while got < expected:
            steps += 1
            assert steps < 200_000, "no progress (the proxy waits for an entry that never completes)"
            if live and rng.random() < 0.6:
                g = rng.choice(live)
                try:
                    next(g)
                except StopIteration:
                    live.remove(g)
                continue
            slot = ring.slots[tail % CAPACITY]
            if protocol.ready(slot, tail):
                taken.append((tail, slot["fields"]))
                slot_fields = slot["fields"]
                assert slot_fields is not None and slot_fields[0] == "whole", f"entry {tail} taken half-written"
                assert slot_fields[1][0] == call, f"entry {tail} holds a request of call {slot_fields[1][0]}"
                tail += 1
                got += 1
        for g in live:  # lanes past their last write only have their final step left
            for _ in g:
                pass
    assert [t for t, _ in taken] == list(range(len(taken)))
    payloads = [f[1] for _, f in taken]
    assert len(set(payloads)) == len(payloads) == calls * R * (R - 1)
    return ring


@pytest.mark.parametrize("seed", range(10))
def test_ring_protocol_holds(seed):
    ring = run(Protocol(), seed)
    assert ring.head == 12 * 8 * 7  # wrapped the 256-entry ring more than twice


@pytest.mark.parametrize("R", [1, 2, 16])
def test_ring_protocol_holds_at_other_rank_counts(R):
    run(Protocol(), seed=R, R=R, calls=4)


@pytest.mark.parametrize("mutant", [SeqFirst, NoSeqCheck, NoOffset], ids=lambda m: m.__name__)
def test_planted_ring_mistakes_are_caught(mutant):
    failures = 0
    for seed in range(6):
        try:
            run(mutant(), seed, calls=6)
        except AssertionError:
            failures += 1
    assert failures > 0, f"{mutant.__name__} was never caught"
