"""Host-side models of how the scans and the redo plan hand out work (no GPU).

1. Chunk claims (k_scan, k_tscan).  P workers (workgroups or waves) take queue positions: worker i's first
   two are i and P + i, every later one is 2 P + the next value of one shared counter.  k_scan requests
   each claim one chunk ahead (at the start of the chunk before it); k_tscan requests it when it needs
   it.  A worker stops at its first position at or past the queue's length n.  Under any interleaving of
   the counter's increments, every position below n must be processed exactly once, and nothing else.
2. The redo plan's split of the marked queries among the 16 waves of its one workgroup (k_plan_redo):
   wave w, lane l of pass p looks at query p * 1024 + l * 16 + w.  Every query must be looked at by
   exactly one (wave, lane, pass).
"""
import random

import pytest


def run_claims(P, n, seed, ahead):
    """Simulates P workers on a queue of n positions; returns the processed positions in order."""
    rng = random.Random(seed)
    counter = 0
    done = []

    def claim(worker, k):
        nonlocal counter
        if k < 2:
            return k * P + worker
        c = counter
        counter += 1
        return 2 * P + c

    # per worker: (claims made, position being processed or None when stopped, prefetched next position)
    state = {}
    for w in range(P):
        pos = claim(w, 0)
        nxt = claim(w, 1) if ahead and pos < n else None
        state[w] = [1 + (nxt is not None), pos if pos < n else None, nxt]
    live = [w for w in range(P) if state[w][1] is not None]
    while live:
        w = rng.choice(live)   # this worker finishes its chunk now
        st = state[w]
        done.append(st[1])
        if ahead:
            pos = st[2]
            st[2] = None
            if pos < n:
                st[2] = claim(w, st[0])
                st[0] += 1
        else:
            pos = claim(w, st[0])
            st[0] += 1
        if pos < n:
            st[1] = pos
        else:
            st[1] = None
            live.remove(w)
    return done


@pytest.mark.parametrize("ahead", [True, False], ids=["k_scan", "k_tscan"])
@pytest.mark.parametrize("P,n", [(1, 0), (1, 5), (4, 3), (4, 8), (4, 9), (7, 13), (7, 14), (7, 15), (64, 651),
                                 (768, 651), (768, 3072), (4096, 16386), (5, 100)])
def test_every_position_processed_once(P, n, ahead):
    for seed in range(5):
        done = run_claims(P, n, seed, ahead)
        assert sorted(done) == list(range(n)), (P, n, seed)


def test_redo_split_covers_every_query_once():
    NWV, LANES = 16, 64
    for B in (1, 5, 16, 63, 64, 256, 1000, 1024, 1025, 3000):
        seen = []
        for base in range(0, B, NWV * LANES):
            for wv in range(NWV):
                for l in range(LANES):
                    qi = base + l * NWV + wv
                    if qi < B:
                        seen.append(qi)
        assert sorted(seen) == list(range(B)), B
