"""Pins that tie the CPU oracle to the pages and to mathematics, not to itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError on a mismatch.  They are
run against the real oracle by ``test_oracle.py`` and against deliberately broken builds by
``test_oracle_mutants.py`` (every planted mistake must be rejected by at least one pin).

Sources of truth used here, none of them the oracle's own arithmetic:
  * published splitmix64 outputs for state 0 (Vigna's reference generator; Java's SplittableRandom(0)
    produces the same first value, -2152535657050944081);
  * the hand-worked example in tests/golden/handworked_tiny.txt;
  * numpy library routines for the special case nprobe = nlist (exhaustive filtered int8 MIPS top-k:
    a matrix product and np.lexsort);
  * order invariants of the top-nprobe probe set and of the top-k result;
  * the exact Bloom false-positive probability from the occupancy law (Stirling numbers of the second
    kind), and the no-false-negative property of any Bloom filter;
  * exact rational arithmetic (fractions.Fraction) for dequantisation.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
INT32_MIN = np.iinfo(np.int32).min

# published splitmix64 outputs from state 0
SPLITMIX64_STATE0 = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F, 0xF88BB8A8724C81EC,
                     0x1B39896A51A8749B]


# ------------------------------------------------------------------------------------------------
def exhaustive_topk(items, sigs, queries, masks, k, allowed=None):
    """Library-routine reference: filter with numpy bit operations, score with an int64 matrix
    product, order with np.lexsort (score desc, id asc).  ``allowed`` restricts the candidate ids."""
    B = queries.shape[0]
    ids = np.full((B, k), -1, np.int64)
    sc = np.full((B, k), INT32_MIN, np.int64)
    cnt = np.zeros(B, np.int64)
    X = items.astype(np.int64)
    for b in range(B):
        mb = masks[b] if masks.ndim == 3 else masks[b][None, :]   # [G, W]: eligible under any of them
        ok = np.zeros(sigs.shape[0], bool)
        for m in mb:
            ok |= np.all((sigs & m) == m, axis=1)
        if allowed is not None:
            ok &= allowed[b]
        cand = np.nonzero(ok)[0]
        s = X[cand] @ queries[b].astype(np.int64)
        order = np.lexsort((cand, -s))[:k]
        n = len(order)
        ids[b, :n] = cand[order]
        sc[b, :n] = s[order]
        cnt[b] = n
    return ids, sc, cnt


def small_catalogue(rng, n=3000, d=32, nlist=16, W=1, tie_heavy=False, empty_clusters=0):
    if tie_heavy:
        items = rng.integers(-1, 2, size=(n, d)).astype(np.int8)
        cent = rng.integers(-1, 2, size=(nlist, d)).astype(np.int8)
    else:
        items = rng.integers(-127, 128, size=(n, d)).astype(np.int8)
        cent = rng.integers(-127, 128, size=(nlist, d)).astype(np.int8)
    used = nlist - empty_clusters
    list_of = rng.integers(0, used, size=n).astype(np.int32)
    # signatures with ~25% of bits set so masks of 1-3 bits select a useful fraction
    sigs = np.zeros((n, W), np.uint64)
    for w in range(W):
        bits = rng.random((n, 64)) < 0.45
        sigs[:, w] = (bits.astype(np.uint64) << np.arange(64, dtype=np.uint64)).sum(axis=1, dtype=np.uint64)
    return items, sigs, list_of, cent


def random_masks(rng, B, W, nbits_max=3):
    m = np.zeros((B, W), np.uint64)
    for b in range(B):
        for _ in range(rng.integers(0, nbits_max + 1)):
            w = rng.integers(0, W)
            m[b, w] |= np.uint64(1) << np.uint64(rng.integers(0, 64))
    return m


# ------------------------------------------------------------------------------------------------
def pin_splitmix64(orc):
    out, _ = orc.splitmix64(0, 5)
    assert [int(x) for x in out] == SPLITMIX64_STATE0, "splitmix64 does not reproduce the published sequence"


def _parse_bits(s):
    return int(s, 2)


def load_handworked():
    cent, items, cl, sigs, cases = [], [], [], [], []
    q = None
    with open(os.path.join(GOLDEN, "handworked_tiny.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("centroid"):
                cent.append([int(x) for x in line.split(":")[1].split()])
            elif line.startswith("item"):
                vec, c, s = line.split(":")[1].split("|")
                items.append([int(x) for x in vec.split()])
                cl.append(int(c))
                sigs.append(_parse_bits(s.strip()))
            elif line.startswith("query"):
                q = [int(x) for x in line.split(":")[1].split()]
            elif line.startswith("case"):
                lhs, rhs = line.split("->")
                kv = dict(t.split("=") for t in lhs.split(":")[1].split())
                parts = [p.split() for p in rhs.split("|")]
                ids = [int(x) for x in parts[0][1:]]
                scores = [INT32_MIN if x == "MIN" else int(x) for x in parts[1][1:]]
                fs = [float(x) for x in parts[2][1:]]
                count = int(parts[3][1])
                cases.append(dict(mask=_parse_bits(kv["mask"]), nprobe=int(kv["nprobe"]), k=int(kv["k"]),
                                  ids=ids, scores=scores, fscores=fs, count=count))
    return (np.array(items, np.int8), np.array(sigs, np.uint64)[:, None], np.array(cl, np.int32),
            np.array(cent, np.int8), np.array([q], np.int8), cases)


def pin_handworked(orc):
    items, sigs, cl, cent, q, cases = load_handworked()
    for c in cases:
        masks = np.array([[c["mask"]]], np.uint64)
        ids, sc, fs, cnt, _ = orc.search(items, sigs, cl, cent, 2.0, q, masks, c["nprobe"], c["k"],
                                         query_scales=np.array([4.0], np.float32))
        assert ids[0].tolist() == c["ids"], (c, ids)
        assert sc[0].tolist() == c["scores"], (c, sc)
        assert fs[0].tolist() == c["fscores"], (c, fs)
        assert int(cnt[0]) == c["count"], (c, cnt)


def pin_exhaustive(orc, seed=1, tie_heavy=False, W=1, d=32, k=50):
    """nprobe = nlist reduces the method to exhaustive filtered int8 MIPS top-k."""
    rng = np.random.default_rng(seed)
    items, sigs, cl, cent = small_catalogue(rng, d=d, W=W, tie_heavy=tie_heavy)
    B = 6
    q = (rng.integers(-1, 2, size=(B, d)) if tie_heavy else rng.integers(-127, 128, size=(B, d))).astype(np.int8)
    masks = random_masks(rng, B, W)
    masks[0] = 0  # unfiltered: exact int8 MIPS top-k
    ids, sc, fs, cnt, st = orc.search(items, sigs, cl, cent, 1.0, q, masks, cent.shape[0], k)
    rids, rsc, rcnt = exhaustive_topk(items, sigs, q, masks, k)
    assert np.array_equal(ids, rids), "ids differ from the exhaustive library reference"
    assert np.array_equal(sc.astype(np.int64), rsc), "scores differ from the exhaustive library reference"
    assert np.array_equal(cnt, rcnt)
    assert np.all(st[:, 0] == items.shape[0]), "nprobe = nlist must scan every item"


def pin_probe_set(orc, seed=2):
    """The probe set is the top-nprobe clusters by (score desc, id asc): checked as an order
    invariant against centroid scores computed with numpy."""
    rng = np.random.default_rng(seed)
    for tie_heavy in (False, True):
        nlist, d = 40, 16
        cent = (rng.integers(-1, 2, (nlist, d)) if tie_heavy else rng.integers(-127, 128, (nlist, d))).astype(np.int8)
        for _ in range(5):
            q = (rng.integers(-1, 2, d) if tie_heavy else rng.integers(-127, 128, d)).astype(np.int8)
            for nprobe in (1, 7, nlist):
                probes, scores = orc.coarse(cent, q, nprobe)
                ref = cent.astype(np.int64) @ q.astype(np.int64)
                assert np.array_equal(scores.astype(np.int64), ref), "centroid scores"
                assert len(set(probes.tolist())) == nprobe
                key = [(-int(ref[c]), int(c)) for c in probes]
                assert key == sorted(key), "probes not in (score desc, id asc) order"
                sel = set(probes.tolist())
                rest = [(-int(ref[c]), c) for c in range(nlist) if c not in sel]
                if rest:
                    assert max(key) < min(rest), "a skipped cluster outranks a probed one"


def pin_ivf_restriction(orc, seed=3, W=2):
    """With nprobe < nlist the result is the exhaustive filtered top-k restricted to the items of the
    probed clusters (probe set itself pinned by pin_probe_set)."""
    rng = np.random.default_rng(seed)
    items, sigs, cl, cent = small_catalogue(rng, n=4000, d=32, nlist=24, W=W, empty_clusters=3)
    B, k = 5, 60
    q = rng.integers(-127, 128, (B, 32)).astype(np.int8)
    masks = random_masks(rng, B, W)
    for nprobe in (1, 4, 24):
        ids, sc, fs, cnt, st = orc.search(items, sigs, cl, cent, 1.0, q, masks, nprobe, k)
        allowed = np.zeros((B, items.shape[0]), bool)
        for b in range(B):
            ref = cent.astype(np.int64) @ q[b].astype(np.int64)
            order = np.lexsort((np.arange(24), -ref))[:nprobe]
            allowed[b] = np.isin(cl, order)
            assert st[b, 0] == allowed[b].sum(), "scanned count"
        rids, rsc, rcnt = exhaustive_topk(items, sigs, q, masks, k, allowed)
        assert np.array_equal(ids, rids) and np.array_equal(sc.astype(np.int64), rsc) and np.array_equal(cnt, rcnt)


def pin_mask_groups(orc, seed=12, W=2):
    """Requests of several masks: an item is eligible when it passes any of them.  Against the numpy
    reference (the union of each mask's eligible set), at nprobe = nlist and, restricted to the probed
    clusters, at nprobe < nlist; one group reproduces the one-mask search; a group with every bit set
    matches nothing here (no item has that signature); the order of the groups does not matter."""
    rng = np.random.default_rng(seed)
    items, sigs, cl, cent = small_catalogue(rng, n=4000, d=32, nlist=20, W=W, empty_clusters=2)
    assert not np.any(np.all(sigs == ~np.uint64(0), axis=1))
    B, G, k = 6, 3, 80
    q = rng.integers(-127, 128, (B, 32)).astype(np.int8)
    masks = np.stack([random_masks(rng, B, W, nbits_max=4) for _ in range(G)], axis=1)   # [B, G, W]
    masks[2, 1] = 0          # one group of query 2 makes every item eligible
    ids, sc, fs, cnt, st = orc.search(items, sigs, cl, cent, 1.0, q, masks, 20, k)
    rids, rsc, rcnt = exhaustive_topk(items, sigs, q, masks, k)
    assert np.array_equal(ids, rids) and np.array_equal(sc.astype(np.int64), rsc) and np.array_equal(cnt, rcnt)
    for b in range(B):
        ok = np.zeros(items.shape[0], bool)
        for m in masks[b]:
            ok |= np.all((sigs & m) == m, axis=1)
        assert st[b, 1] == ok.sum(), "eligible count of a several-mask request"
    for nprobe in (1, 5):
        ids, sc, fs, cnt, st = orc.search(items, sigs, cl, cent, 1.0, q, masks, nprobe, k)
        allowed = np.zeros((B, items.shape[0]), bool)
        for b in range(B):
            ref = cent.astype(np.int64) @ q[b].astype(np.int64)
            allowed[b] = np.isin(cl, np.lexsort((np.arange(20), -ref))[:nprobe])
        rids, rsc, rcnt = exhaustive_topk(items, sigs, q, masks, k, allowed)
        assert np.array_equal(ids, rids) and np.array_equal(sc.astype(np.int64), rsc) and np.array_equal(cnt, rcnt)
    one = orc.search(items, sigs, cl, cent, 1.0, q, masks[:, :1, :], 5, k)
    plain = orc.search(items, sigs, cl, cent, 1.0, q, np.ascontiguousarray(masks[:, 0, :]), 5, k)
    assert all(np.array_equal(a, b) for a, b in zip(one, plain))
    padded = np.concatenate([masks, np.full((B, 1, W), ~np.uint64(0))], axis=1)
    with_pad = orc.search(items, sigs, cl, cent, 1.0, q, padded, 5, k)
    base = orc.search(items, sigs, cl, cent, 1.0, q, masks, 5, k)
    assert all(np.array_equal(a, b) for a, b in zip(with_pad, base))
    perm = orc.search(items, sigs, cl, cent, 1.0, q, np.ascontiguousarray(masks[:, ::-1, :]), 5, k)
    assert all(np.array_equal(a, b) for a, b in zip(perm, base))


def pin_padding(orc, seed=4):
    rng = np.random.default_rng(seed)
    items, sigs, cl, cent = small_catalogue(rng, n=200, d=16, nlist=4)
    q = rng.integers(-127, 128, (2, 16)).astype(np.int8)
    masks = np.array([[0], [np.uint64(0xFFFFFFFFFFFFFFFF)]], np.uint64)
    ids, sc, fs, cnt, _ = orc.search(items, sigs, cl, cent, 1.0, q, masks, 4, 300)
    assert cnt[0] == 200 and np.all(ids[0, 200:] == -1) and np.all(sc[0, 200:] == INT32_MIN)
    assert np.all(np.isneginf(fs[0, 200:]))
    assert cnt[1] == 0 and np.all(ids[1] == -1)


def pin_dequant(orc, seed=5):
    """f = S / (item_scale * query_scale) rounded once to float: within one float ulp of the exact
    rational value, and exactly 0 for S = 0."""
    rng = np.random.default_rng(seed)
    for _ in range(2000):
        s = int(rng.integers(-2_064_512, 2_064_513))
        a = float(np.float32(rng.uniform(1.0, 400.0)))
        b = float(np.float32(rng.uniform(1.0, 400.0)))
        f = orc.dequant(s, a, b)
        exact = Fraction(s) / (Fraction(a) * Fraction(b))
        if s == 0:
            assert f == 0.0
            continue
        ulp = abs(float(np.spacing(np.float32(float(exact)))))
        assert abs(Fraction(f) - exact) <= Fraction(ulp), (s, a, b, f, float(exact))
    assert orc.dequant(0, 3.0, 5.0) == 0.0


# ------------------------------------------------------------------------------------------------
def stirling2_row(n):
    """S2(n, j) for j = 0..n by the standard recurrence S2(n,j) = j S2(n-1,j) + S2(n-1,j-1)."""
    row = [1]
    for i in range(1, n + 1):
        new = [0] * (i + 1)
        for j in range(1, i + 1):
            new[j] = j * (row[j] if j < len(row) else 0) + row[j - 1]
        row = new
    return row


def bloom_fp_exact(m, n_tokens, h, absent=1):
    """Exact probability that ``absent`` random tokens (h hashes each) all hit set bits of a signature
    built from n_tokens tokens: occupancy law P(|S|=j) = C(m,j) j! S2(nh,j) / m^(nh)."""
    nh = n_tokens * h
    s2 = stirling2_row(nh)
    tot = Fraction(0)
    for j in range(0, min(m, nh) + 1):
        pj = Fraction(math.comb(m, j) * math.factorial(j) * s2[j], m ** nh)
        tot += pj * Fraction(j, m) ** (h * absent)
    return tot


def pin_bloom(orc, trials=1_000_000, seed=6):
    rng = np.random.default_rng(seed)
    for (W, n_tok, h) in ((1, 3, 2), (2, 5, 3)):
        m = 64 * W
        # occupancy law sanity: sums to one, mean = m (1 - (1 - 1/m)^(nh))
        nh = n_tok * h
        s2 = stirling2_row(nh)
        pj = [Fraction(math.comb(m, j) * math.factorial(j) * s2[j], m ** nh) for j in range(0, min(m, nh) + 1)]
        assert sum(pj) == 1
        mean = sum(j * p for j, p in enumerate(pj))
        assert mean == m * (1 - Fraction(m - 1, m) ** nh)
        fp = float(bloom_fp_exact(m, n_tok, h))
        keys = rng.integers(0, 2**63, size=(trials, n_tok + 1), dtype=np.uint64) * np.uint64(2) + \
            rng.integers(0, 2, size=(trials, n_tok + 1), dtype=np.uint64)
        sig = orc.signatures(keys[:, :n_tok], h, W)
        absent = orc.signatures(keys[:, n_tok:], h, W)
        own = orc.signatures(keys[:, :1], h, W)
        # no false negatives: a mask built from the item's own token always passes
        assert np.all((sig & own) == own)
        rate = float(np.mean(np.all((sig & absent) == absent, axis=1)))
        sigma = math.sqrt(fp * (1 - fp) / trials)
        assert abs(rate - fp) < 4 * sigma, (W, rate, fp, sigma)
        # set-bit count per signature follows the occupancy mean
        pop = np.unpackbits(sig.view(np.uint8), axis=1).sum(axis=1).mean()
        assert abs(pop - float(mean)) < 0.02 * float(mean)


def load_bloom_mapping():
    rows = []
    with open(os.path.join(GOLDEN, "bloom_mapping.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split(":")
            key, h, w = (int(x) for x in lhs.split())
            rows.append((key, h, w, sorted(int(x) for x in rhs.split())))
    return rows


def pin_bloom_mapping(orc):
    """Token -> bit positions, against the hand-derived golden values."""
    for key, h, w, bits in load_bloom_mapping():
        sig = orc.signatures(np.array([[key]], np.uint64), h, w)[0]
        got = sorted(64 * wi + b for wi in range(w) for b in range(64) if (int(sig[wi]) >> b) & 1)
        assert got == bits, (key, h, w, got, bits)


def pin_mask_helper(orc):
    """Mask of a token set equals the OR of single-token signatures; empty mask is all zero."""
    rng = np.random.default_rng(7)
    toks = rng.integers(1, 2**62, size=4, dtype=np.uint64)
    for W, h in ((1, 2), (2, 3)):
        m = orc.mask(toks, h, W)
        singles = orc.signatures(toks[:, None], h, W)
        assert np.array_equal(m, np.bitwise_or.reduce(singles, axis=0))
        assert np.all(orc.mask(toks[:0], h, W) == 0)
        assert np.all(np.unpackbits(singles.view(np.uint8), axis=1).sum(axis=1) <= h)


ALL_PINS = [pin_splitmix64, pin_handworked, pin_exhaustive, pin_probe_set, pin_ivf_restriction, pin_mask_groups,
            pin_padding,
            pin_dequant, pin_bloom, pin_bloom_mapping, pin_mask_helper]
