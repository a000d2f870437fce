"""CPU emulation of the fused recurrence's LDS hand-over protocol (chunkwise_delta_rule_kda_amd/
csrc/kda_producer.h and the fused compute loop in kda_recurrence_core.h), step by step.

Four producer waves prepare chunks p, p + 4, ... of a run into a ring of NSLOT slots; W
compute waves read every chunk. Counters in LDS replace the workgroup barrier:

* producer, chunk j, slot s = j % NSLOT: wait until done[s] >= W * (j // NSLOT) (all W
  compute waves have read the slot's previous chunk), write the slot, wait for its own
  writes, then ready[s] = j + 1;
* compute wave: wait ready[0] >= 1, read chunk 0, release (done[0] += 1); then for each
  chunk c: wait ready[(c + 1) % NSLOT] >= c + 2 (only if c + 1 < nch), read the next slot
  (unconditionally: past the last chunk the values are unused), compute chunk c, release
  the slot if c + 1 < nch; at the end fin += 1, wait fin >= W, and reuse slot 0 as
  staging (transition runs).

Each wave is a coroutine; a seeded random scheduler interleaves them one shared-memory
step at a time. A read is split into its issue and its completion (the kernel's reads
complete when the wave next waits for its LDS operations), so a producer write that lands
in between is detected. The emulation checks that every read sees the chunk it expects,
that no slot is overwritten while a read of it is pending, that staging never overlaps a
pending read, and that every wave finishes (no deadlock) within a step budget.
"""

import random

import pytest

PRODUCERS = 4


class Deadlock(Exception):
    pass


def emulate(nch, W, nslot, seed, stage=True, max_steps=2_000_000):
    rng = random.Random(seed)
    ready = [0] * nslot
    done = [0] * nslot
    slot_tag = [None] * nslot          # chunk whose data the slot holds
    pending = {}                       # (wave, slot) -> tag seen at issue
    fin = [0]
    staged = [False]
    errors = []

    def producer(pw):
        for j in range(pw, nch, PRODUCERS):
            for _ in range(rng.randint(0, 3)):  # preparation work
                yield
            s = j % nslot
            while done[s] < W * (j // nslot):
                yield
            for (w, ps) in pending:
                if ps == s:
                    errors.append(f"producer {pw} overwrites slot {s} (chunk {j}) while "
                                  f"wave {w} reads it")
            if staged[0]:
                errors.append("producer writes after staging began")
            slot_tag[s] = j
            yield
            ready[s] = j + 1
            yield

    def compute(w):
        def issue(s):
            pending[(w, s)] = slot_tag[s]

        def complete(s, expect):
            tag = pending.pop((w, s))
            if slot_tag[s] != tag:
                errors.append(f"wave {w}: slot {s} changed during a read")
            if expect is not None and tag != expect:
                errors.append(f"wave {w}: slot {s} held chunk {tag}, expected {expect}")

        if nch > 0:
            while ready[0] < 1:
                yield
            issue(0)
            yield
            complete(0, 0)
            done[0] += 1
            yield
            cs = 0
            for c in range(nch):
                ns = (cs + 1) % nslot
                if c + 1 < nch:
                    while ready[ns] < c + 2:
                        yield
                issue(ns)
                yield
                for _ in range(rng.randint(0, 3)):  # the chunk's products
                    yield
                complete(ns, c + 1 if c + 1 < nch else None)
                if c + 1 < nch:
                    done[ns] += 1
                yield
                cs = ns
        if stage:
            fin[0] += 1
            while fin[0] < W:
                yield
            for (ow, ps) in pending:
                if ps == 0:
                    errors.append(f"wave {w} stages into slot 0 while wave {ow} reads it")
            staged[0] = True
            yield

    waves = [producer(p) for p in range(PRODUCERS)] + [compute(w) for w in range(W)]
    live = list(range(len(waves)))
    steps = 0
    while live:
        i = rng.choice(live)
        try:
            next(waves[i])
        except StopIteration:
            live.remove(i)
        steps += 1
        if steps > max_steps:
            raise Deadlock(f"no progress after {steps} steps (nch={nch}, W={W})")
    return errors


@pytest.mark.parametrize("W", [1, 2, 4, 8])
@pytest.mark.parametrize("nch", [0, 1, 2, 3, 4, 5, 6, 7, 11, 47, 130])
def test_protocol_orders_every_read_and_finishes(W, nch):
    nslot = 5 if W == 8 else 6
    for seed in range(4):
        errors = emulate(nch, W, nslot, seed=1000 * W + 10 * nch + seed)
        assert not errors, errors[:5]


def test_counters_catch_a_missing_wait():
    """The emulation detects a broken protocol: without the producers' wait on done[s]
    some seed overwrites a slot that is still being read."""
    found = False
    for seed in range(20):
        errors = emulate_without_slot_wait(nch=40, W=4, nslot=6, seed=seed)
        if errors:
            found = True
            break
    assert found


def emulate_without_slot_wait(nch, W, nslot, seed):
    # The same run with the producers' slot wait removed (only in this emulation).
    rng = random.Random(seed)
    ready = [0] * nslot
    slot_tag = [None] * nslot
    pending = {}
    errors = []

    def producer(pw):
        for j in range(pw, nch, PRODUCERS):
            s = j % nslot
            for (w, ps) in pending:
                if ps == s:
                    errors.append("overwrite during a read")
            slot_tag[s] = j
            yield
            ready[s] = max(ready[s], j + 1)
            yield

    def compute(w):
        for c in range(nch):
            s = c % nslot
            spins = 0
            while ready[s] < c + 1 and spins < 10_000:
                spins += 1
                yield
            pending[(w, s)] = slot_tag[s]
            for _ in range(rng.randint(0, 6)):
                yield
            if slot_tag[s] != pending.pop((w, s)):
                errors.append("slot changed during a read")
            yield

    waves = [producer(p) for p in range(PRODUCERS)] + [compute(w) for w in range(W)]
    live = list(range(len(waves)))
    while live:
        i = rng.choice(live)
        try:
            next(waves[i])
        except StopIteration:
            live.remove(i)
    return errors
