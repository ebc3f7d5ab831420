"""Searches with k above the fused paths' 2048 (the large-k path: one scan into per-query pools above a
sampled threshold, else a radix select over repeated passes; a collect pass and an LDS sort) against the
CPU oracle, element by element: ids, int32 scores, counts, scan statistics and dequantised scores.  Each
case runs with pools (the default), with every query sent through the passes (thresholds above every
score) and with pools too small to prove k.  Also: the path forced for small k equals the fused paths,
heavy ties, fewer eligible items than k, several masks per query, an updated index, the no-allocation
entry point and a 10M-item catalogue."""
import numpy as np
import pytest

import oracle_pins as P
import synth
from gpu_common import compare, gpu_search, oracle_search, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def svt():
    import torch
    assert torch.cuda.is_available()
    torch.cuda.set_device(0)
    from int8_ivf_ann_amd import svt as m
    m.lib()
    return m


MODES = {"pool": {}, "passes": {"flags": 2}, "overflow": {"pool_keys": 4096}}


def _opts(svt, mode, G=1):
    kw = dict(MODES[mode])
    return svt.make_options("auto", kw.get("pool_keys", 0), kw.get("flags", 0), G)


def _masks(rng, B, W, G, nbits_max=3):
    if G == 1:
        return P.random_masks(rng, B, W, nbits_max)
    return np.stack([P.random_masks(rng, B, W, nbits_max) for _ in range(G)], axis=1)


CASES = [  # d, W, n, nlist, nprobe, k, B, G, scaled
    (16, 1, 20000, 16, 8, 2049, 5, 1, False),
    (64, 2, 60000, 32, 12, 5000, 6, 1, True),
    (128, 2, 50000, 24, 24, 16384, 4, 2, False),   # every cluster probed
    (32, 1, 3000, 8, 3, 16384, 3, 1, False),       # fewer eligible items than k: padding
    (256, 1, 30000, 16, 5, 3000, 4, 3, True),
]


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("case", CASES, ids=[f"d{c[0]}_w{c[1]}_n{c[2]}_p{c[4]}_k{c[5]}_g{c[7]}" for c in CASES])
def test_large_k_matches_oracle(svt, case, mode):
    d, W, n, nlist, nprobe, k, B, G, scaled = case
    rng = np.random.default_rng(500 + d + k)
    items, sigs, list_of, cent = P.small_catalogue(rng, n=n, d=d, nlist=nlist, W=W)
    scale = 127.0 / 4.0
    ix = svt.Index(items, sigs, list_of, cent, scale)
    try:
        q = rng.integers(-127, 128, size=(B, d)).astype(np.int8)
        masks = _masks(rng, B, W, G)
        qs = rng.uniform(20.0, 60.0, size=B).astype(np.float32) if scaled else None
        assert svt.svt_search_path(ix.handle, B, nprobe, k) == "large_k"
        say(f"large-k {mode} d={d} W={W} n={n} nprobe={nprobe}/{nlist} k={k} B={B} G={G}")
        got = gpu_search(ix, q, masks, nprobe, k, query_scales=qs, opts=_opts(svt, mode, G))
        ref = oracle_search(items, sigs, list_of, cent, scale, q, masks, nprobe, k, query_scales=qs)
        compare(got, ref, k, f"large-k {case}")
    finally:
        ix.close()


@pytest.mark.parametrize("k", [1, 100, 2048])
def test_large_k_path_equals_fused_paths(svt, k):
    rng = np.random.default_rng(600 + k)
    d, W, n, nlist, nprobe, B = 64, 2, 40000, 20, 6, 9
    items, sigs, list_of, cent = P.small_catalogue(rng, n=n, d=d, nlist=nlist, W=W)
    ix = svt.Index(items, sigs, list_of, cent, 30.0)
    try:
        q = rng.integers(-127, 128, size=(B, d)).astype(np.int8)
        masks = P.random_masks(rng, B, W)
        assert svt.svt_search_path(ix.handle, B, nprobe, k, svt.make_options("large_k")) == "large_k"
        lk = gpu_search(ix, q, masks, nprobe, k, opts=svt.make_options("large_k"))
        qp = gpu_search(ix, q, masks, nprobe, k, opts=svt.make_options("query"))
        for a, b in zip(lk, qp):
            assert np.array_equal(a, b)
        compare(lk, oracle_search(items, sigs, list_of, cent, 30.0, q, masks, nprobe, k), k, f"large-k path k={k}")
    finally:
        ix.close()


@pytest.mark.parametrize("mode", list(MODES))
def test_large_k_heavy_ties(svt, mode):
    # components in {-1, 0, 1}: a handful of distinct scores, so the selection runs into the id digits
    rng = np.random.default_rng(7)
    d, n, nlist, nprobe, B, k = 16, 30000, 12, 7, 4, 4000
    items, sigs, list_of, cent = P.small_catalogue(rng, n=n, d=d, nlist=nlist, W=1, tie_heavy=True)
    ix = svt.Index(items, sigs, list_of, cent, 1.0)
    try:
        q = rng.integers(-1, 2, size=(B, d)).astype(np.int8)
        masks = np.zeros((B, 1), np.uint64)
        masks[1, 0] = np.uint64(1) << np.uint64(5)
        got = gpu_search(ix, q, masks, nprobe, k, opts=_opts(svt, mode))
        compare(got, oracle_search(items, sigs, list_of, cent, 1.0, q, masks, nprobe, k), k, f"large-k ties {mode}")
    finally:
        ix.close()


@pytest.mark.parametrize("mode", ["pool", "passes"])
def test_large_k_after_updates(svt, mode):
    rng = np.random.default_rng(8)
    d, W, n, nlist, nprobe, B, k = 32, 2, 12000, 10, 4, 5, 6000
    items, sigs, list_of, cent = P.small_catalogue(rng, n=n, d=d, nlist=nlist, W=W)
    ix = svt.Index(items, sigs, list_of, cent, 20.0, id_capacity=14000, slack_min=64)
    try:
        dead = rng.choice(n, size=900, replace=False).astype(np.int64)
        ix.delete(dead)
        new_ids = np.arange(13000, 13300, dtype=np.int64)
        new_rows = rng.integers(-127, 128, size=(300, d)).astype(np.int8)
        new_sigs = sigs[:300].copy()
        new_cl = rng.integers(0, nlist, size=300).astype(np.int32)
        ix.insert(new_ids, new_rows, new_sigs, new_cl)
        keep = np.setdiff1d(np.arange(n), dead)
        ids = np.concatenate([keep, new_ids])
        order = np.argsort(ids)
        ids = ids[order]
        all_items = np.concatenate([items[keep], new_rows])[order]
        all_sigs = np.concatenate([sigs[keep], new_sigs])[order]
        all_cl = np.concatenate([list_of[keep], new_cl])[order]
        q = rng.integers(-127, 128, size=(B, d)).astype(np.int8)
        masks = P.random_masks(rng, B, W)
        got = list(gpu_search(ix, q, masks, nprobe, k, opts=_opts(svt, mode)))
        ref = list(oracle_search(all_items, all_sigs, all_cl, cent, 20.0, q, masks, nprobe, k))
        ref[0] = np.where(ref[0] >= 0, ids[np.maximum(ref[0], 0)], -1)   # oracle rows -> ids
        compare(tuple(got), tuple(ref), k, "large-k updated")
    finally:
        ix.close()


def test_large_k_noalloc(svt):
    import torch
    rng = np.random.default_rng(9)
    d, W, n, nlist, nprobe, B, k = 64, 1, 30000, 16, 5, 3, 9000
    items, sigs, list_of, cent = P.small_catalogue(rng, n=n, d=d, nlist=nlist, W=W)
    ix = svt.Index(items, sigs, list_of, cent, 25.0)
    try:
        q = rng.integers(-127, 128, size=(B, d)).astype(np.int8)
        masks = P.random_masks(rng, B, W)
        q_d = torch.from_numpy(q).cuda()
        m_d = torch.from_numpy(masks.view(np.int64)).cuda()
        outs = svt.svt_search_noalloc(ix.handle, q_d, m_d, nprobe, k)
        torch.cuda.synchronize()
        got = tuple(t.cpu().numpy() for t in outs)
        compare(got, oracle_search(items, sigs, list_of, cent, 25.0, q, masks, nprobe, k), k, "large-k noalloc")
    finally:
        ix.close()


def test_large_k_10m_batch8(svt):
    """The 10M-item catalogue (d = 128, 128-bit signatures), top-16384 of 8 queries, every query
    compared with the oracle."""
    cat = synth.catalogue("10m")
    cfg = cat.cfg
    W, h, nprobe = cfg["sig_words"], cfg["n_hashes"], cfg["nprobe"]
    sigs = svt.svt_bloom_sign(cat.tokens, h, W)
    ix = svt.Index(cat.items, sigs, cat.list_of, cat.centroids, cat.item_scale)
    try:
        B, k = 8, svt.SVT_MAX_K_LARGE
        qs = synth.queries(cat, B, offset=4096)
        masks = np.stack([svt.svt_bloom_mask(qs.required(b), h, W) for b in range(B)])
        say(f"large-k 10m: {cat.n_items} items, nprobe {nprobe}, k {k}, B {B}")
        ref = oracle_search(cat.items, sigs, cat.list_of, cat.centroids, cat.item_scale, qs.queries, masks, nprobe, k)
        for mode in MODES:
            got = gpu_search(ix, qs.queries, masks, nprobe, k, opts=_opts(svt, mode))
            compare(got, ref, k, f"large-k 10m {mode}")
        say(f"large-k 10m: counts {got[3].tolist()}, eligible {got[4][:, 1].tolist()}")
    finally:
        ix.close()


@pytest.mark.parametrize("mode", list(MODES))
def test_large_k_large_batch_tile_pools(svt, mode):
    """Batches of at least 128 queries fill the large-k pools with the tile scan ((score, slot) keys,
    converted to (score, id) keys at the k-th best score); every query compared."""
    rng = np.random.default_rng(42)
    d, W, n, nlist, nprobe, B, k = 64, 2, 60000, 32, 6, 130, 3000
    items, sigs, list_of, cent = P.small_catalogue(rng, n=n, d=d, nlist=nlist, W=W)
    ix = svt.Index(items, sigs, list_of, cent, 30.0)
    try:
        q = rng.integers(-127, 128, size=(B, d)).astype(np.int8)
        masks = P.random_masks(rng, B, W, nbits_max=2)
        assert svt.svt_search_path(ix.handle, B, nprobe, k) == "large_k"
        got = gpu_search(ix, q, masks, nprobe, k, opts=_opts(svt, mode))
        compare(got, oracle_search(items, sigs, list_of, cent, 30.0, q, masks, nprobe, k), k, f"large-k B={B} {mode}")
    finally:
        ix.close()
