"""CPU model of the per-tile semaphore protocol, run under random interleavings.

A plain-Python rendition of the two-shot with per-tile semaphores and a get
(pull) all-gather.  Rank r's slot b is a generator; a seeded scheduler
interleaves all of them one shared-memory step at a time, and launches follow
one another (a kernel boundary) with different chunk geometries (full tiles,
a partial tile owned by one slot, the buffer's partial vector on slot 0),
slot counts and in-place flags, so the monotonic counters carry over from
call to call.

Memory is modelled per item (a tile, the partial tile, the partial vector).
A store is not visible to other workgroups until it completes: completion
happens when the storing workgroup waits for its stores (the model of
`s_waitcnt 0`), at a kernel boundary, or earlier at random, one store at a
time, in any order.

The protocol as built, for rank r, slot b:
- reduce-scatter: for each of the slot's items of chunk r (full tiles b,
  b + B, ..., then the partial tile if this slot owns it, then on slot 0 the
  buffer's partial vector): read the item from every input, store the sum into
  out[r], wait for the store, then add one to progress[r][b];
- all-gather: base = seen[r][p][b] for every peer p; column j: for each peer
  whose slot b has an item j, poll until progress[p][b] - base >= j + 1
  (32-bit wrap-safe), read the item from out[p], store it into out[r]; the
  partial vectors last;
- at the end, seen[r][p][b] = base + the number of items peer p's slot b
  signalled in this call.

Checked: after every launch every output equals the sum of the inputs, item
by item; nothing deadlocks; the counters survive wrapping past 2^32; a dropped
signal ends in a bounded timeout.  Planted mistakes (signalling before the
tile's store completes, not storing `seen` back, a `seen` that leaves out the
partial tile, polling for j instead of j + 1 tiles, an unsigned compare at the
wrap) must each break one of these.
"""

import random

import pytest

MASK = (1 << 32) - 1
POISON = -(10 ** 9)
TIMEOUT_READY = 0x7FFFFFFF


class Channel:
    def __init__(self, R, slots, start=0):
        self.R, self.slots = R, slots
        self.progress = [[start & MASK] * slots for _ in range(R)]
        self.seen = [[[start & MASK] * slots for _ in range(R)] for _ in range(R)]
        self.timed_out = False


def items_of(geo, p, slot, B):
    """Slot `slot`'s items of chunk p, in the order both phases visit them."""
    nfull, partial, tail = geo[p]
    items = [("F", t) for t in range(slot, nfull, B)]
    if partial and nfull % B == slot:
        items.append(("P", nfull))
    if tail and slot == 0:
        items.append(("T", 0))
    return items


def all_items(geo, p, B):
    return [i for b in range(B) for i in items_of(geo, p, b, B)]


class Rules:
    """The protocol as built; mutants override single methods."""

    def finish_tile(self, wg, ch, rank, slot):
        wg.complete_all()
        ch.progress[rank][slot] = (ch.progress[rank][slot] + 1) & MASK

    def reached(self, progress, base, need):  # (int32)((progress - base) - need) >= 0
        return (((progress - base) & MASK) - need) & MASK < (1 << 31)

    def need(self, j):
        return j + 1

    def seen_after(self, base, items):
        return (base + len(items)) & MASK


class Workgroup:
    def __init__(self):
        self.pending = []  # (buffer, key, value) stores not yet complete

    def store(self, buf, key, val):
        self.pending.append((buf, key, val))

    def complete_one(self, rng):
        buf, key, val = self.pending.pop(rng.randrange(len(self.pending)))
        buf[key] = val

    def complete_all(self):
        for buf, key, val in self.pending:
            buf[key] = val
        self.pending.clear()


def wait_tiles(ch, rules, p, slot, base, need, budget):
    spins = 0
    while not rules.reached(ch.progress[p][slot], base, need):
        spins += 1
        if spins > budget:
            ch.timed_out = True
            return TIMEOUT_READY
        yield
    return (ch.progress[p][slot] - base) & MASK


def workgroup(wg, ch, rules, geo, B, ins, outs, rank, slot, drop_rank, budget):
    R = ch.R
    # reduce-scatter into the own output, one signal per item
    for item in items_of(geo, rank, slot, B):
        s = 0
        for p in range(R):
            s += ins[p][(rank, item)]
            yield
        wg.store(outs[rank], (rank, item), s)
        yield
        if rank == drop_rank:
            wg.complete_all()
        else:
            rules.finish_tile(wg, ch, rank, slot)
        yield
    # all-gather by get, column by column
    peers = [(rank + k) % R for k in range(1, R)]
    lists = {p: items_of(geo, p, slot, B) for p in peers}
    nvec = {p: sum(1 for i in lists[p] if i[0] != "T") for p in peers}
    base = {p: ch.seen[rank][p][slot] for p in peers}
    ready = {}
    for p in peers:
        have = (ch.progress[p][slot] - base[p]) & MASK
        ready[p] = have if 0 < have < (1 << 31) else 0
    yield
    for j in range(max(nvec.values(), default=0)):
        for p in peers:
            if j < nvec[p] and j >= ready[p]:
                ready[p] = yield from wait_tiles(ch, rules, p, slot, base[p], rules.need(j), budget)
        got = {}
        for p in peers:
            if j < nvec[p]:
                got[p] = outs[p][(p, lists[p][j])]
                yield
        for p, v in got.items():
            wg.store(outs[rank], (p, lists[p][j]), v)
            yield
    for p in peers:
        if lists[p] and lists[p][-1][0] == "T":
            if ready[p] < nvec[p] + 1:
                yield from wait_tiles(ch, rules, p, slot, base[p], nvec[p] + 1, budget)
            wg.store(outs[rank], (p, lists[p][-1]), outs[p][(p, lists[p][-1])])
            yield
    for p in peers:
        ch.seen[rank][p][slot] = rules.seen_after(base[p], lists[p])


def random_geometry(rng, R):
    """Per chunk: (full tiles, partial tile?, partial vector?) as the host's
    chunking gives them: equal chunks, the last non-empty one shorter and
    holding the buffer's end, later ones empty."""
    c = rng.randint(0, 5)
    pc = rng.random() < 0.5
    k = rng.randint(1, R)
    geo = []
    for p in range(R):
        if p < k - 1:
            geo.append((c, pc, False))
        elif p == k - 1:
            geo.append((rng.randint(0, c), rng.random() < 0.5, rng.random() < 0.5))
        else:
            geo.append((0, False, False))
    return geo


def launch(ch, rules, geo, B, in_place, rng, drop_rank=None, budget=3_000):
    R = ch.R
    keys = [(c, i) for c in range(R) for i in all_items(geo, c, B)]
    ins = [{k: rng.randint(-1000, 1000) for k in keys} for _ in range(R)]
    want = {k: sum(ins[p][k] for p in range(R)) for k in keys}
    outs = ins if in_place else [{k: POISON for k in keys} for _ in range(R)]
    wgs = []
    live = []
    for b in range(B):
        for r in range(R):
            wg = Workgroup()
            wgs.append(wg)
            live.append((wg, workgroup(wg, ch, rules, geo, B, ins, outs, r, b, drop_rank, budget)))
    steps = 0
    while live:
        if rng.random() < 0.3:
            busy = [w for w in wgs if w.pending]
            if busy:
                rng.choice(busy).complete_one(rng)
                continue
        i = rng.randrange(len(live))
        try:
            next(live[i][1])
        except StopIteration:
            live.pop(i)
        steps += 1
        if steps > 2_000_000:
            raise RuntimeError("scheduler budget exhausted")
    for w in wgs:  # the kernel boundary completes every store
        w.complete_all()
    return outs, want


def run_scenario(rules, seed, R=4, slots=4, start=0, launches=8):
    rng = random.Random(seed)
    ch = Channel(R, slots, start)
    for _ in range(launches):
        B = rng.randint(1, slots)
        geo = random_geometry(rng, R)
        in_place = rng.random() < 0.5
        outs, want = launch(ch, rules, geo, B, in_place, rng)
        assert not ch.timed_out, "a wait timed out (deadlock)"
        for q in range(R):
            for k, v in want.items():
                assert outs[q][k] == v, f"rank {q} item {k}: got {outs[q][k]}, want {v} (B={B}, in_place={in_place})"
    return ch


@pytest.mark.parametrize("seed", range(10))
@pytest.mark.parametrize("R", [1, 2, 3, 5])
def test_protocol_holds(seed, R):
    run_scenario(Rules(), seed, R=R, slots=3)


def test_counters_wrap_past_2_to_32():
    for seed in range(4):
        run_scenario(Rules(), seed, R=3, slots=2, start=MASK - 4, launches=6)


def test_dropped_signal_times_out():
    rng = random.Random(3)
    ch = Channel(3, 2)
    geo = [(4, False, False), (4, False, False), (3, True, True)]
    launch(ch, Rules(), geo, 2, False, rng, drop_rank=1, budget=200)
    assert ch.timed_out


class SignalBeforeStoreCompletes(Rules):
    def finish_tile(self, wg, ch, rank, slot):
        ch.progress[rank][slot] = (ch.progress[rank][slot] + 1) & MASK


class SeenNotStored(Rules):
    def seen_after(self, base, items):
        return base


class SeenWithoutPartialTile(Rules):
    def seen_after(self, base, items):
        return (base + sum(1 for i in items if i[0] != "P")) & MASK


class PollOneTileEarly(Rules):
    def need(self, j):
        return j


class UnsignedCompare(Rules):
    def reached(self, progress, base, need):
        return progress >= base + need


def caught(mutant, **kw):
    failures = 0
    for seed in range(12):
        try:
            run_scenario(mutant(), seed, **kw)
        except AssertionError:
            failures += 1
    return failures


@pytest.mark.parametrize("mutant", [SignalBeforeStoreCompletes, SeenNotStored, SeenWithoutPartialTile,
                                    PollOneTileEarly], ids=lambda m: m.__name__)
def test_planted_protocol_mistakes_are_caught(mutant):
    assert caught(mutant, R=3, slots=3) > 0, f"{mutant.__name__} was never caught"


def test_unsigned_compare_fails_at_wrap():
    assert caught(UnsignedCompare, R=3, slots=2, start=MASK - 4, launches=6) > 0
