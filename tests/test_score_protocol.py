"""Interleaving model of the backward scoring pass's LDS ring protocol (CPU).

The scoring kernel (bwd_score_kernel) has one copy wave and eight compute
waves that share an 8-slot LDS ring without a workgroup barrier:

  * the copy wave issues asynchronous copies of item nf into slot nf % 8,
    keeps at most LAG = 3 items in flight, and publishes item m (full[slot] =
    m + 1) only after a vmcnt wait has shown that m's copies landed; before
    it waits for a slot to be released it first lands and publishes
    everything it has issued;
  * compute wave w scores the items of parity w >> 2 in order, waits for
    full[k % 8] == k + 1, reads the slot and releases it (done[slot] += 1);
  * the copy wave reuses a slot for item nf >= 8 only once done[slot] has
    reached 4 * (nf // 8), i.e. the four waves of that parity released the
    slot's previous item.

This module re-states that protocol as small Python agents and runs them
under many random interleavings, with asynchronous copies that land at
random times but in issue order (as vector-memory loads of one wave do).
It checks the properties the kernel relies on: no schedule deadlocks, a
compute wave never reads a slot whose data is not the landed copy of its
item, and no copy overwrites a slot an unfinished wave may still read. With
every wait bounded at 0 polls (the give-up path) every agent still ends.
"""
import random

import pytest

RQ, LAG, NB, NC = 8, 3, 4, 8


class Ring:
    def __init__(self, n_items, bound):
        self.n = n_items
        self.bound = bound
        self.full = [0] * RQ
        self.done = [0] * RQ
        self.data = [None] * RQ       # item whose copy has landed in the slot
        self.inflight = []            # (slot, item) copies issued, in issue order
        self.readers = [set() for _ in range(RQ)]  # waves that may still read the slot
        self.stop = False
        self.violations = []

    def land_one(self):
        slot, item = self.inflight.pop(0)
        if self.readers[slot]:
            self.violations.append(f"copy of item {item} landed in slot {slot} while "
                                   f"waves {sorted(self.readers[slot])} still read it")
        self.data[slot] = item

    def land_until(self, outstanding):
        while len(self.inflight) > outstanding:
            self.land_one()


def wait(ring, ready):
    """Bounded wait as in the kernel: after `bound` unsuccessful polls the
    wave raises `stop`; a raised stop ends every wait."""
    g = 0
    while True:
        if g >= ring.bound:
            ring.stop = True
            return
        if ready():
            return
        if ring.stop:
            return
        g += 1
        yield


def copy_wave(ring):
    marked = 0

    def publish(m):
        ring.full[m % RQ] = m + 1

    for nf in range(ring.n):
        slot = nf % RQ
        if nf >= RQ:
            need = NB * (nf // RQ)
            if ring.done[slot] < need:
                ring.land_until(0)
                while marked < nf:
                    publish(marked)
                    marked += 1
                    yield
                yield from wait(ring, lambda: ring.done[slot] >= need)
        ring.inflight.append((slot, nf))
        yield
        if nf + 1 - marked > LAG:
            ring.land_until(LAG)
            while marked <= nf - LAG:
                publish(marked)
                marked += 1
                yield
    ring.land_until(0)
    while marked < ring.n:
        publish(marked)
        marked += 1
        yield


def compute_wave(ring, w):
    for k in range(w >> 2, ring.n, 2):
        slot = k % RQ
        yield from wait(ring, lambda: ring.full[slot] == k + 1)
        if not ring.stop:
            ring.readers[slot].add(w)
            yield  # the operand reads of the item span several steps
            if ring.data[slot] != k:
                ring.violations.append(f"wave {w} read slot {slot} for item {k} but it "
                                       f"holds item {ring.data[slot]}")
            yield
            ring.readers[slot].discard(w)
        ring.done[slot] += 1
        yield


def run(n_items, seed, bound=1 << 30, max_steps=10 ** 6):
    rng = random.Random(seed)
    ring = Ring(n_items, bound)
    agents = {"copy": copy_wave(ring)}
    for w in range(NC):
        agents[w] = compute_wave(ring, w)
    steps = 0
    while agents:
        # the DMA engine may land the oldest outstanding copy at any time
        if ring.inflight and rng.random() < 0.3:
            ring.land_one()
        name = rng.choice(list(agents))
        try:
            next(agents[name])
        except StopIteration:
            del agents[name]
        steps += 1
        assert steps < max_steps, f"no progress after {max_steps} steps: {sorted(agents, key=str)}"
    return ring


@pytest.mark.parametrize("n_items", [1, 2, 3, 7, 8, 9, 16, 17, 40, 129])
def test_ring_protocol_random_interleavings(n_items):
    for seed in range(60):
        ring = run(n_items, seed)
        assert not ring.violations, ring.violations[:3]
        assert not ring.stop, "a legal schedule reached the wait bound"
        # every item was released by the four waves of its parity
        assert sum(ring.done) == NB * n_items
        assert ring.inflight == []


def test_ring_protocol_gives_up_and_ends():
    """With every wait bounded at zero polls each wave gives up at its first
    wait and still runs to its end (the kernel then reports the give-up)."""
    for n_items in (5, 33):
        for seed in range(10):
            ring = run(n_items, seed, bound=0)
            assert ring.stop
            assert sum(ring.done) == NB * n_items


def test_model_detects_a_missing_release_wait():
    """The model is sharp: a copy wave that skips the release wait for a
    reused slot is caught overwriting data a wave still reads."""
    global copy_wave
    orig = copy_wave

    def eager_copy_wave(ring):
        marked = 0
        for nf in range(ring.n):
            ring.inflight.append((nf % RQ, nf))
            yield
            if nf + 1 - marked > LAG:
                ring.land_until(LAG)
                while marked <= nf - LAG:
                    ring.full[marked % RQ] = marked + 1
                    marked += 1
                    yield
        ring.land_until(0)
        while marked < ring.n:
            ring.full[marked % RQ] = marked + 1
            marked += 1
            yield

    copy_wave = eager_copy_wave
    try:
        found = False
        for seed in range(200):
            try:
                ring = run(40, seed, max_steps=20000)
            except AssertionError:
                found = True  # a wave missed its item for good: no progress
                break
            if ring.violations:
                found = True
                break
        assert found
    finally:
        copy_wave = orig
