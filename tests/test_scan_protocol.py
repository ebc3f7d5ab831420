"""Host-side model of how the query-path scan's waves agree on their top-k list length (k_scan).

Every step ends with one workgroup barrier.  After it, each thread derives the list length and decides
whether to trim the list; the trim itself holds more barriers, so every wave must take the same
decision.  In the kernel each wave publishes its step-i append count in the LDS slot of parity i & 1,
after the barrier of step i; after the barrier of step i + 1 every thread sums the slots of parity
i & 1.  A slot is thus read only between the barrier that follows its write and the barrier before it
is written again.

The model runs the waves as generators of shared-memory operations and barrier arrivals, interleaved by a
seeded random scheduler (a wave may run any number of operations ahead of the others, up to the next
barrier).  A barrier releases when every wave has arrived; waves arriving at different barrier sites (one
at a trim, another at the next step) are the failure.  The same scheduler must find that failure in the
protocol that read one shared counter, incremented by each wave after scoring, after the step barrier.
"""
import random

import pytest

NWV = 4          # waves of a scan workgroup
TRIM_AT = 100    # list length above which the list is trimmed
KEEP = 40        # length after a trim (the same for every wave: computed together, between barriers)


def wave_fixed(w, appends):
    """The kernel's protocol for wave w; appends[i][w] is what the wave adds in step i."""
    cnt = 0
    steps = len(appends)
    for i in range(steps):
        yield ("bar", "step")
        if i >= 1:
            s = 0
            for w2 in range(NWV):
                s += yield ("read", ("wadd", (i - 1) & 1, w2))
            cnt += s
        yield ("note", cnt)
        if cnt > TRIM_AT:
            yield ("bar", "trim")
            cnt = KEEP
            yield ("bar", "trim-end")
        yield ("write", ("wadd", i & 1, w), appends[i][w])
    yield ("bar", "end")
    last = 0
    for w2 in range(NWV):
        last += yield ("read", ("wadd", (steps - 1) & 1, w2))
    yield ("note", cnt + last)


def wave_shared_counter(w, appends):
    """The earlier protocol: one shared counter, read after the step barrier, added to after scoring."""
    cnt = 0
    for i in range(len(appends)):
        yield ("bar", "step")
        cnt = yield ("read", ("cnt",))
        yield ("note", cnt)
        if cnt > TRIM_AT:
            yield ("bar", "trim")
            if w == 0:
                yield ("write", ("cnt",), KEEP)
            yield ("bar", "trim-end")
        yield ("add", ("cnt",), appends[i][w])
    yield ("bar", "end")


class Desync(Exception):
    pass


def run(program, appends, seed):
    """Interleave the waves; returns each wave's noted values, or raises Desync."""
    rng = random.Random(seed)
    mem = {}
    gens = [program(w, appends) for w in range(NWV)]
    pending = [None] * NWV          # value to send into each generator
    at_bar = [None] * NWV           # barrier site a wave waits at
    done = [False] * NWV
    notes = [[] for _ in range(NWV)]
    while not all(done):
        ready = [w for w in range(NWV) if not done[w] and at_bar[w] is None]
        if not ready:
            sites = {at_bar[w] for w in range(NWV) if not done[w]}
            if len(sites) != 1 or any(done):
                raise Desync(f"waves at barriers {at_bar}, finished {done}")
            for w in range(NWV):
                at_bar[w] = None
            continue
        w = rng.choice(ready)
        # run the chosen wave a random number of operations (but never past a barrier)
        for _ in range(rng.randint(1, 6)):
            try:
                op = gens[w].send(pending[w])
            except StopIteration:
                done[w] = True
                break
            pending[w] = None
            if op[0] == "bar":
                at_bar[w] = op[1]
                break
            if op[0] == "read":
                pending[w] = mem.get(op[1], 0)
            elif op[0] == "write":
                mem[op[1]] = op[2]
            elif op[0] == "add":
                mem[op[1]] = mem.get(op[1], 0) + op[2]
            elif op[0] == "note":
                notes[w].append(op[1])
        if any(done) and not all(done) and any(at_bar[x] is not None for x in range(NWV) if not done[x]):
            raise Desync(f"a wave finished while others wait at barriers {at_bar}")
    return notes


def workload(seed, steps=12):
    rng = random.Random(1000 + seed)
    return [[rng.randint(0, 30) for _ in range(NWV)] for _ in range(steps)]


@pytest.mark.parametrize("seed", range(300))
def test_fixed_protocol_agrees_under_any_schedule(seed):
    appends = workload(seed % 20)
    notes = run(wave_fixed, appends, seed)
    # every wave saw the same list length at every decision and at the end
    assert all(n == notes[0] for n in notes), notes
    # and that length is the true one: replay the step sums without any interleaving
    cnt, expect = 0, []
    for i in range(len(appends)):
        if i >= 1:
            cnt += sum(appends[i - 1])
        expect.append(cnt)
        if cnt > TRIM_AT:
            cnt = KEEP
    expect.append(cnt + sum(appends[-1]))
    assert notes[0] == expect


def test_shared_counter_protocol_is_caught():
    # the model must be able to show the race the parity slots removed
    appends = workload(3)
    failures = 0
    for seed in range(300):
        try:
            notes = run(wave_shared_counter, appends, seed)
        except Desync:
            failures += 1
            continue
        if any(n != notes[0] for n in notes):
            failures += 1
    assert failures > 0
