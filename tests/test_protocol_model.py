"""CPU model of the channel barrier protocol, run under random interleavings.

A plain-Python rendition of the slot barrier in the device layer: rank r's
slot b signals each peer p by incrementing inbound[p][r][b], waits until its
own inbound[r][p][b] has reached epoch = consumed[r][b] + 1 (compared
wrap-safe, as 32-bit differences), and stores the epoch back.  Each
(rank, slot) "workgroup" is a generator; a seeded scheduler interleaves them
one shared-memory step at a time.  Launches follow one another (a kernel
boundary), with different slot counts and numbers of barriers per workgroup,
as the two-shot (one barrier) and the in-place one-shot (one per tile) do.

Checked: no workgroup leaves barrier k before every peer's same slot has
arrived at barrier k; nothing deadlocks; counters survive any sequence of
launches, including counters that wrap past 2^32; a dropped signal ends in a
bounded timeout that a reset clears.  Planted protocol mistakes (epoch not
stored back, signal sent to the wrong counter, an unsigned instead of a
wrap-safe compare, a missing peer) must each break one of these.
"""

import random

import pytest

MASK = (1 << 32) - 1


class Channel:
    def __init__(self, R, slots, start=0):
        self.R, self.slots = R, slots
        self.inbound = [[[start & MASK] * slots for _ in range(R)] for _ in range(R)]
        self.consumed = [[start & MASK] * slots for _ in range(R)]
        self.timed_out = False

    def reset(self):
        self.__init__(self.R, self.slots)


class Rules:
    """The protocol as built; mutants override single methods."""

    def signal_target(self, rank, peer):  # whose counter a signal to `peer` bumps: inbound[peer][rank]
        return peer, rank

    def reached(self, count, epoch):  # wrap-safe: (int32)(count - epoch) >= 0
        d = (count - epoch) & MASK
        return d < (1 << 31)

    def store_epoch(self, ch, rank, slot, epoch):
        ch.consumed[rank][slot] = epoch

    def peers(self, R, rank):
        return [p for p in range(R) if p != rank]


def workgroup(ch, rules, rank, slot, nbarriers, log, drop_rank=None, spin_budget=10_000):
    for _ in range(nbarriers):
        epoch = (ch.consumed[rank][slot] + 1) & MASK
        yield
        log.append(("arrive", rank, slot, epoch))
        for p in rules.peers(ch.R, rank):
            if rank == drop_rank:
                continue
            a, b = rules.signal_target(rank, p)
            ch.inbound[a][b][slot] = (ch.inbound[a][b][slot] + 1) & MASK
            yield
        for p in rules.peers(ch.R, rank):
            spins = 0
            while not rules.reached(ch.inbound[rank][p][slot], epoch):
                spins += 1
                if spins > spin_budget:
                    ch.timed_out = True
                    break
                yield
        log.append(("leave", rank, slot, epoch))
        rules.store_epoch(ch, rank, slot, epoch)
        yield


def launch(ch, rules, nslots, nbarriers, rng, drop_rank=None, spin_budget=10_000):
    """Run every (rank, slot < nslots) workgroup to completion; return the event log."""
    log = []
    live = [workgroup(ch, rules, r, b, nbarriers, log, drop_rank, spin_budget)
            for b in range(nslots) for r in range(ch.R)]
    steps = 0
    while live:
        g = rng.choice(live)
        try:
            next(g)
        except StopIteration:
            live.remove(g)
        steps += 1
        if steps > 5_000_000:
            raise RuntimeError("scheduler budget exhausted")
    return log


def check_no_early_leave(log, R):
    """A workgroup may leave barrier k of a launch only after every peer's
    same slot has arrived at barrier k (k counted within the launch)."""
    arrived = {}
    seen = {}
    for ev, rank, slot, _epoch in log:
        key = (rank, slot)
        if ev == "arrive":
            arrived[key] = arrived.get(key, 0) + 1
        else:
            k = seen.get(key, 0) + 1
            seen[key] = k
            for p in range(R):
                assert arrived.get((p, slot), 0) >= k, f"rank {rank} slot {slot} left barrier {k} before rank {p}"


def run_scenario(rules, seed, R=4, slots=6, start=0, launches=None):
    rng = random.Random(seed)
    ch = Channel(R, slots, start)
    if launches is None:
        launches = [(rng.randint(1, slots), rng.randint(1, 4)) for _ in range(6)]
    for nslots, nbarriers in launches:
        log = launch(ch, rules, nslots, nbarriers, rng, spin_budget=2_000)
        assert not ch.timed_out, "a wait timed out (deadlock)"
        check_no_early_leave(log, R)
    return ch


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("R", [1, 2, 3, 8])
def test_protocol_holds(seed, R):
    run_scenario(Rules(), seed, R=R, slots=4)


def test_counters_wrap_past_2_to_32():
    run_scenario(Rules(), seed=5, R=3, slots=3, start=MASK - 3, launches=[(3, 3), (2, 4), (3, 2)])


def test_dropped_signal_times_out_then_reset_recovers():
    rng = random.Random(1)
    ch = Channel(3, 2)
    launch(ch, Rules(), 2, 1, rng, drop_rank=1, spin_budget=200)
    assert ch.timed_out
    ch.reset()
    log = launch(ch, Rules(), 2, 2, rng, spin_budget=2_000)
    assert not ch.timed_out
    check_no_early_leave(log, 3)


class NoEpochStore(Rules):
    def store_epoch(self, ch, rank, slot, epoch):
        pass


class WrongCounter(Rules):
    def signal_target(self, rank, peer):
        return rank, peer


class UnsignedCompare(Rules):
    def reached(self, count, epoch):
        return count >= epoch


class MissingPeer(Rules):
    def peers(self, R, rank):
        ps = super().peers(R, rank)
        return ps[:-1] if len(ps) > 1 else ps


@pytest.mark.parametrize("mutant", [NoEpochStore, WrongCounter, MissingPeer], ids=lambda m: m.__name__)
def test_planted_protocol_mistakes_are_caught(mutant):
    failures = 0
    for seed in range(8):
        try:
            run_scenario(mutant(), seed, R=3, slots=3)
        except AssertionError:
            failures += 1
    assert failures > 0, f"{mutant.__name__} was never caught"


def test_unsigned_compare_fails_at_wrap():
    with pytest.raises(AssertionError):
        run_scenario(UnsignedCompare(), seed=5, R=3, slots=3, start=MASK - 3, launches=[(3, 3), (2, 4), (3, 2)])
