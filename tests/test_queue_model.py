"""Host-side models of how the scans and the redo plan hand out work (no GPU).

1. Chunk claims (k_scan, k_tscan).  P workers (workgroups or waves) take queue positions: worker i's first
   two are i and P + i, every later one is 2 P + the next value of one shared counter.  k_scan requests
   each claim one chunk ahead (at the start of the chunk before it); k_tscan requests it when it needs
   it.  A worker stops at its first position at or past the queue's length n.  Under any interleaving of
   the counter's increments, every position below n must be processed exactly once, and nothing else.
2. The redo plan's split of the marked queries among the 16 waves of its one workgroup (k_plan_redo):
   wave w, lane l of pass p looks at query p * 1024 + l * 16 + w.  Every query must be looked at by
   exactly one (wave, lane, pass).
3. The query path's cut of a query's stream into chunks (lengths from k_plan_count, ranges from
   k_plan_chunks): the chunks must cover the stream in order, none empty, at most 2048 per query.
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


def _cdiv(a, b):
    return -(-a // b)


def query_chunks(length, ta, cost, tc, max_chunks=2048, tail_div=2):
    """The query path's cut of one query's stream (k_plan_count's lengths, k_plan_chunks' ranges): a
    regular region [0, ta) and a tail region [ta, length) of chunks tail_div times shorter."""
    per = max_chunks // 2 if ta < length else max_chunks
    cl_min = _cdiv(length, per)
    cl = max(_cdiv(tc * length, cost), cl_min)
    cl = min(_cdiv(cl, 64) * 64, length)
    na = _cdiv(ta, cl) if ta > 0 else 0
    nb = 0
    if ta < length:
        clb = max(_cdiv(_cdiv(cl, tail_div), 64) * 64, cl_min)
        nb = _cdiv(length - ta, clb)
    cla = _cdiv(ta, na) if na else 0
    clb2 = _cdiv(length - ta, nb) if nb else 0
    out = []
    for i in range(na + nb):
        if i < na:
            l0 = i * cla
            out.append((l0, min(l0 + cla, ta)))
        else:
            l0 = ta + (i - na) * clb2
            out.append((l0, min(l0 + clb2, length)))
    return out


def test_query_chunks_tile_the_stream():
    """Every query's chunks cover its stream exactly, in order, none empty, at most 2048 of them."""
    rng = random.Random(3)
    for _ in range(3000):
        length = rng.choice([1, 63, 64, 65, 1000, rng.randint(1, 5_000_000)])
        ta = rng.choice([0, length, rng.randint(0, length)])
        cost = length * rng.randint(17, 200)
        tc = rng.choice([16 << 10, rng.randint(1, 1 << 24)])
        ch = query_chunks(length, ta, cost, tc)
        assert 1 <= len(ch) <= 2048
        assert ch[0][0] == 0 and ch[-1][1] == length
        assert all(a < b for a, b in ch), "empty chunk"
        assert all(ch[i][1] == ch[i + 1][0] for i in range(len(ch) - 1))
