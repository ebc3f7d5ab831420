"""Host-side models of the large-k path's two algorithms, checked against plain sorting (no GPU).

1. The digit select (k_lk_scan counting passes + k_lk_pick).  The keys are the kernel's 55-bit
   (S + 2^23) << 31 | (2^31 - 1 - id).  A pass counts the keys that share the bits fixed so far by their
   next 11-bit digit, from bit 44 down.  The pick walks 256 threads of 8 bins each from the top bucket down,
   with block-scan prefix counts.  It stops when the digit's bucket is taken whole or the last digit is fixed,
   and it takes every key when the first pass counts at most k.  The collect pass then keeps the keys at or
   above the threshold.  The model must return exactly the k largest keys, after at most 5 passes, for
   random, tie-heavy and wide-id inputs.
2. The register-tiled bitonic network of k_lk_emit.  Each of 1024 threads holds E consecutive keys.
   Strides of E or more exchange with thread t ^ (stride / E) (the same values whether they travel by
   shuffle or LDS); smaller strides exchange in registers.  The model must sort descending for E = 2, 4,
   8, 16 and any fill.
"""
import numpy as np
import pytest

DIGIT, BINS, TOP, PASSES = 11, 2048, 44, 5
THREADS = 1024


def lk_key(score, ident):
    return ((score + (1 << 23)) << 31) | (0x7FFFFFFF - ident)


def digit_select(keys, k):
    """(threshold, passes) as k_lk_scan / k_lk_pick compute them."""
    ka = np.array(keys, dtype=np.uint64)
    prefix, shift, need = 0, TOP, k
    for p in range(1, PASSES + 1):
        hi = ~((1 << (shift + DIGIT)) - 1) & ((1 << 64) - 1)
        m = (ka & np.uint64(hi)) == np.uint64(prefix)
        h = np.bincount(((ka[m] >> np.uint64(shift)) & np.uint64(BINS - 1)).astype(np.int64), minlength=BINS)
        total = int(h.sum())
        if total <= need:
            assert shift == TOP, "only the first pass can count at most k"
            return 0, p
        above_all = 0
        found = None
        for t in range(256):          # thread t: bins 8 (255 - t) .. 8 (255 - t) + 7, higher buckets first
            g = 255 - t
            hb = h[8 * g:8 * g + 8]
            above = above_all
            if above < need <= above + int(hb.sum()):
                for i in range(7, -1, -1):
                    if above + int(hb[i]) >= need:
                        found = (8 * g + i, need - above, int(hb[i]))
                        break
                    above += int(hb[i])
            above_all += int(hb.sum())
        assert found is not None, "exactly one thread holds the k-th key's bucket"
        d, rem, hd = found
        prefix |= d << shift
        if hd == rem or shift == 0:
            return prefix, p
        shift -= DIGIT
        need = rem
    raise AssertionError("not decided after 5 passes")


def _keys(rng, n, kind):
    if kind == "spread":
        s = rng.integers(-4_000_000, 4_000_000, size=n)
    elif kind == "ties":
        s = rng.integers(-3, 4, size=n)
    else:
        s = rng.normal(0, 60000, size=n).astype(np.int64)
    if kind == "wide-ids":
        ids = rng.permutation(np.unique(rng.integers(0, 2 ** 31 - 1, size=2 * n + 2)))[:n]
    else:
        ids = rng.choice(200_000, size=n, replace=False)
    return [lk_key(int(a), int(b)) for a, b in zip(s, ids)]


@pytest.mark.parametrize("kind", ["spread", "ties", "normal", "wide-ids"])
def test_digit_select_takes_exactly_the_k_largest(kind):
    rng = np.random.default_rng({"spread": 1, "ties": 2, "normal": 3, "wide-ids": 4}[kind])
    for _ in range(12):
        n = int(rng.integers(0, 4000))
        keys = _keys(rng, n, kind)
        k = int(rng.integers(1, 5000))
        T, passes = digit_select(keys, k)
        kept = sorted((x for x in keys if x >= T), reverse=True)
        assert kept == sorted(keys, reverse=True)[:k], (kind, n, k)
        assert len(kept) == min(n, k)
        assert passes <= PASSES


def test_key_order_is_score_desc_then_id_asc():
    pairs = [(5, 7), (5, 3), (-2, 0), (4_194_304, 2 ** 31 - 1), (-4_194_304, 0)]
    order = sorted(pairs, key=lambda p: lk_key(*p), reverse=True)
    assert order == sorted(pairs, key=lambda p: (-p[0], p[1]))
    assert all(lk_key(*p) > 0 for p in pairs) and all(lk_key(*p) < 1 << 55 for p in pairs)


def tiled_bitonic(keys, n, E):
    N = E * THREADS
    v = np.zeros(N, np.uint64)
    v[:n] = keys[:n]
    v = v.reshape(THREADS, E)
    tid = np.arange(THREADS)
    size = 2
    while size <= N:
        stride = size >> 1
        while stride >= E:                 # with thread tid ^ (stride / E), element for element
            ts = stride // E
            p = v[tid ^ ts]
            lower = (tid & ts) == 0
            for e in range(E):
                keep_max = lower == (((tid * E + e) & size) == 0)
                v[:, e] = np.where(keep_max, np.maximum(v[:, e], p[:, e]), np.minimum(v[:, e], p[:, e]))
            stride >>= 1
        st = E // 2
        while st >= 1:                     # within the thread
            if st < size:
                for e in range(E):
                    if e & st == 0:
                        desc = ((tid * E + e) & size) == 0
                        x, y = v[:, e].copy(), v[:, e + st].copy()
                        sw = np.where(desc, x < y, x > y)
                        v[:, e], v[:, e + st] = np.where(sw, y, x), np.where(sw, x, y)
            st >>= 1
        size <<= 1
    return v.reshape(-1)


@pytest.mark.parametrize("E", [2, 4, 8, 16])
def test_tiled_bitonic_sorts_descending(E):
    rng = np.random.default_rng(E)
    for n in (0, 1, 7, E * THREADS // 2 + 3, E * THREADS):
        keys = rng.integers(1, 2 ** 55, size=max(n, 1), dtype=np.uint64)
        out = tiled_bitonic(keys, n, E)
        assert np.array_equal(out[:n], np.sort(keys[:n])[::-1])
        assert np.all(out[n:] == 0)
