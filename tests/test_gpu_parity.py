"""GPU vs CPU oracle, element by element, on small seeded inputs that span several workgroup chunks,
LDS list cuts and ragged tails; plus the degenerate cases of the method."""
import numpy as np
import pytest

import oracle
import oracle_pins as P
import synth
from gpu_common import check_invariants, compare, gpu_search, oracle_search, say
from int8_ivf_ann_amd import svt as svt_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def svt():
    import torch
    assert torch.cuda.is_available()
    torch.cuda.set_device(0)
    from int8_ivf_ann_amd import svt as m
    m.lib()
    return m


# Every case runs on every search path, selected through the search options: query by query (also with
# the merge forced to read every chunk's slot instead of the keys gathered above each query's final
# bound), and the tile path (each probed cluster read once per batch; with nprobe == nlist the MFMA scan
# of the whole catalogue), also with pools of 64 keys (most queries overflow and are redone query by
# query) and with every threshold above any score (every query with an eligible item is redone).
PATHS = {
    "query": dict(path="query"),
    "query-slots": dict(path="query", flags=svt_mod.SVT_OPT_MERGE_FROM_SLOTS),
    "tile": dict(path="tile"),
    "tile-overflow": dict(path="tile", pool_keys=64),
    "tile-redo": dict(path="tile", flags=svt_mod.SVT_OPT_FORCE_REDO),
}


@pytest.fixture(params=list(PATHS))
def opts(request):
    print(f"path {request.param}", flush=True)
    return svt_mod.make_options(**PATHS[request.param])


def _run(svt, opts, items, sigs, list_of, cent, scale, q, masks, nprobe, k, label, query_scales=None,
         invariants=True):
    say(f"case {label}: n={items.shape[0]} d={items.shape[1]} W={sigs.shape[1]} nlist={cent.shape[0]} "
        f"B={q.shape[0]} nprobe={nprobe} k={k}")
    ix = svt.Index(items, sigs, list_of, cent, scale)
    try:
        got = gpu_search(ix, q, masks, nprobe, k, query_scales, opts=opts)
    finally:
        ix.close()
    ref = oracle_search(items, sigs, list_of, cent, scale, q, masks, nprobe, k, query_scales)
    compare(got, ref, k, label)
    if invariants:
        check_invariants(items, sigs, list_of, got, masks, q, k, cent, nprobe)
    return got


def test_tiny_preset(svt, opts):
    cat = synth.catalogue("tiny")
    cfg = cat.cfg
    W, h = cfg["sig_words"], cfg["n_hashes"]
    qs = synth.queries(cat, 4)
    sigs = svt.svt_bloom_sign(cat.tokens, h, W)
    masks = np.stack([svt.svt_bloom_mask(qs.required(b), h, W) for b in range(4)])
    orc = oracle.Oracle()
    assert np.array_equal(sigs, orc.signatures(cat.tokens, h, W))
    assert np.array_equal(masks, orc.masks(qs, h, W))
    _run(svt, opts, cat.items, sigs, cat.list_of, cat.centroids, cat.item_scale, qs.queries, masks, cfg["nprobe"],
         cfg["k"], "tiny")


def test_tiny_preset_more_queries(svt, opts):
    cat = synth.catalogue("tiny")
    cfg = cat.cfg
    W, h = cfg["sig_words"], cfg["n_hashes"]
    qs = synth.queries(cat, 300, offset=1000)
    sigs = svt.svt_bloom_sign(cat.tokens, h, W)
    masks = np.stack([svt.svt_bloom_mask(qs.required(b), h, W) for b in range(300)])
    for nprobe, k in ((1, 1), (8, 100), (64, 2048)):
        _run(svt, opts, cat.items, sigs, cat.list_of, cat.centroids, cat.item_scale, qs.queries, masks, nprobe, k,
             f"tiny300-{nprobe}-{k}")


def test_handworked_example(svt, opts):
    items, sigs, cl, cent, q, cases = P.load_handworked()
    pad = lambda a: np.concatenate([a, np.zeros((a.shape[0], 12), np.int8)], axis=1)  # d 4 -> 16, same dots
    items, cent, q = pad(items), pad(cent), pad(q)
    ix = svt.Index(items, sigs, cl, cent, 2.0)
    try:
        for c in cases:
            masks = np.array([[c["mask"]]], np.uint64)
            ids, sc, fs, cnt, _ = gpu_search(ix, q, masks, c["nprobe"], c["k"], np.array([4.0], np.float32),
                                             opts=opts)
            assert ids[0].tolist() == c["ids"] and sc[0].tolist() == c["scores"] and int(cnt[0]) == c["count"], c
            assert fs[0].tolist() == c["fscores"], c
    finally:
        ix.close()


@pytest.mark.parametrize("d", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("W", [1, 2])
def test_random_shapes(svt, opts, d, W):
    rng = np.random.default_rng(100 + d + W)
    items, sigs, cl, cent = P.small_catalogue(rng, n=7001, d=d, nlist=37, W=W, empty_clusters=4)
    B = 9
    q = rng.integers(-127, 128, (B, d)).astype(np.int8)
    masks = P.random_masks(rng, B, W)
    for nprobe, k in ((1, 1), (5, 37), (37, 300)):
        _run(svt, opts, items, sigs, cl, cent, 3.0, q, masks, nprobe, k, f"rand-d{d}-W{W}-{nprobe}-{k}")


def test_exhaustive_several_query_blocks(svt, opts):
    # nprobe == nlist with 70 queries: three blocks of 32 on the MFMA scan, the last one ragged; 20011
    # items leave a partial last step, and far fewer steps than waves
    rng = np.random.default_rng(31)
    items, sigs, cl, cent = P.small_catalogue(rng, n=20011, d=64, nlist=20, W=2)
    q = rng.integers(-127, 128, (70, 64)).astype(np.int8)
    masks = P.random_masks(rng, 70, 2, nbits_max=2)
    _run(svt, opts, items, sigs, cl, cent, 2.0, q, masks, 20, 100, "exh-70q-k100")
    _run(svt, opts, items, sigs, cl, cent, 2.0, q, masks, 20, 2048, "exh-70q-k2048")


@pytest.mark.parametrize("G", [2, 3, 4])
def test_several_masks_per_query(svt, opts, G):
    # requests of G masks: an item is eligible when it passes any of them (one group of a query makes
    # every item eligible, another query pads its last group with a mask that passes nothing)
    rng = np.random.default_rng(40 + G)
    items, sigs, cl, cent = P.small_catalogue(rng, n=9000, d=64, nlist=30, W=2, empty_clusters=3)
    B = 37
    q = rng.integers(-127, 128, (B, 64)).astype(np.int8)
    masks = np.stack([P.random_masks(rng, B, 2, nbits_max=4) for _ in range(G)], axis=1)
    masks[3, G - 1] = 0
    masks[5, G - 1] = ~np.uint64(0)
    o = svt.make_options(opts.path, opts.pool_keys, opts.flags, G)
    for nprobe, k in ((4, 120), (30, 400)):
        _run(svt, o, items, sigs, cl, cent, 2.0, q, masks, nprobe, k, f"groups{G}-{nprobe}-{k}")


def test_large_k_many_candidates(svt, opts):
    # every query keeps ~40k candidates: LDS lists are cut many times and the merge selects
    rng = np.random.default_rng(7)
    items, sigs, cl, cent = P.small_catalogue(rng, n=120_000, d=64, nlist=8, W=1)
    q = rng.integers(-127, 128, (5, 64)).astype(np.int8)
    masks = np.zeros((5, 1), np.uint64)
    masks[1, 0] = 1
    masks[2, 0] = 0b101
    _run(svt, opts, items, sigs, cl, cent, 1.0, q, masks, 8, 2048, "largek")
    _run(svt, opts, items, sigs, cl, cent, 1.0, q, masks, 3, 2047, "largek-odd")


def test_tie_heavy(svt, opts):
    rng = np.random.default_rng(8)
    items, sigs, cl, cent = P.small_catalogue(rng, n=50_000, d=16, nlist=16, W=2, tie_heavy=True)
    q = rng.integers(-1, 2, (6, 16)).astype(np.int8)
    masks = np.zeros((6, 2), np.uint64)
    _run(svt, opts, items, sigs, cl, cent, 1.0, q, masks, 16, 2048, "ties-all")
    _run(svt, opts, items, sigs, cl, cent, 1.0, q, masks, 3, 500, "ties-ivf")


def test_all_zero_items(svt, opts):
    # every score is 0: the result is the k lowest eligible ids of the probed clusters
    rng = np.random.default_rng(9)
    n, d = 30_000, 32
    items = np.zeros((n, d), np.int8)
    cl = rng.integers(0, 10, n).astype(np.int32)
    cent = rng.integers(-5, 6, (10, d)).astype(np.int8)
    sigs = rng.integers(0, 2**63, (n, 1), dtype=np.uint64)
    q = rng.integers(-127, 128, (3, d)).astype(np.int8)
    masks = np.zeros((3, 1), np.uint64)
    got = _run(svt, opts, items, sigs, cl, cent, 1.0, q, masks, 10, 2048, "zeros")
    assert np.array_equal(got[0][0], np.arange(2048))


def test_empty_and_degenerate(svt, opts):
    rng = np.random.default_rng(10)
    items, sigs, cl, cent = P.small_catalogue(rng, n=3000, d=16, nlist=12, W=1, empty_clusters=6)
    q = rng.integers(-127, 128, (4, 16)).astype(np.int8)
    masks = np.zeros((4, 1), np.uint64)
    masks[1, 0] = np.uint64(0xFFFFFFFFFFFFFFFF)        # nothing eligible
    # query 2 prefers the empty clusters only
    cent[6:] = 100
    cent[:6] = -100
    q[2] = 1
    _run(svt, opts, items, sigs, cl, cent, 1.0, q, masks, 1, 10, "degenerate-1")
    _run(svt, opts, items, sigs, cl, cent, 1.0, q, masks, 6, 10, "degenerate-6")
    # single item, single cluster
    _run(svt, opts, items[:1], sigs[:1], np.zeros(1, np.int32), cent[:1], 1.0, q, masks, 1, 5, "single")


def test_zero_queries(svt, opts):
    import torch
    rng = np.random.default_rng(11)
    items, sigs, cl, cent = P.small_catalogue(rng, n=100, d=16, nlist=4, W=1)
    ix = svt.Index(items, sigs, cl, cent, 1.0)
    q = torch.zeros((0, 16), dtype=torch.int8, device="cuda")
    m = torch.zeros((0, 1), dtype=torch.int64, device="cuda")
    ids, sc, fs, cnt, st = ix.search(q, m, 2, 5, opts=opts)
    torch.cuda.synchronize()
    assert ids.shape == (0, 5)
    ix.close()


def test_query_scales(svt, opts):
    rng = np.random.default_rng(12)
    items, sigs, cl, cent = P.small_catalogue(rng, n=5000, d=32, nlist=8, W=1)
    q = rng.integers(-127, 128, (4, 32)).astype(np.int8)
    masks = P.random_masks(rng, 4, 1)
    qs = np.array([1.0, 0.37, 250.0, 3.5], np.float32)
    _run(svt, opts, items, sigs, cl, cent, 17.25, q, masks, 4, 64, "qscales", query_scales=qs)


def test_batch_composition_invariance(svt, opts):
    """A query's result does not depend on the other queries of its batch."""
    rng = np.random.default_rng(13)
    items, sigs, cl, cent = P.small_catalogue(rng, n=40_000, d=64, nlist=32, W=2)
    B = 40
    q = rng.integers(-127, 128, (B, 64)).astype(np.int8)
    masks = P.random_masks(rng, B, 2)
    ix = svt.Index(items, sigs, cl, cent, 1.0)
    try:
        full = gpu_search(ix, q, masks, 6, 500, opts=opts)
        for b in (0, 17, 39):
            one = gpu_search(ix, q[b:b + 1], masks[b:b + 1], 6, 500, opts=opts)
            for a, c in zip(one, full):
                assert np.array_equal(a[0], c[b])
        again = gpu_search(ix, q, masks, 6, 500, opts=opts)
        for a, c in zip(again, full):
            assert np.array_equal(a, c)
    finally:
        ix.close()


def test_zipf_skewed_cluster(svt, opts):
    rng = np.random.default_rng(14)
    n, d, nlist = 200_000, 32, 64
    items = rng.integers(-127, 128, (n, d)).astype(np.int8)
    p = 1.0 / np.arange(1, nlist + 1) ** 1.5
    cl = rng.choice(nlist, size=n, p=p / p.sum()).astype(np.int32)
    cent = rng.integers(-127, 128, (nlist, d)).astype(np.int8)
    sigs = rng.integers(0, 2**63, (n, 2), dtype=np.uint64)
    q = rng.integers(-127, 128, (12, d)).astype(np.int8)
    q[:6] = cent[0]      # half the queries probe the giant cluster first
    masks = P.random_masks(rng, 12, 2, nbits_max=2)
    _run(svt, opts, items, sigs, cl, cent, 1.0, q, masks, 4, 2048, "zipf")


def test_many_clusters(svt, opts):
    # more clusters than the coarse select keeps in registers: its keys are read from memory instead
    rng = np.random.default_rng(15)
    items, sigs, cl, cent = P.small_catalogue(rng, n=60_000, d=32, nlist=20_000, W=1, empty_clusters=50)
    q = rng.integers(-127, 128, (8, 32)).astype(np.int8)
    masks = P.random_masks(rng, 8, 1, nbits_max=2)
    _run(svt, opts, items, sigs, cl, cent, 0.5, q, masks, 200, 100, "many-clusters")


def test_nprobe_beyond_lds_probe_list(svt, opts):
    # more probes than the select's LDS probe list holds: stream offsets are read from memory instead
    rng = np.random.default_rng(16)
    items, sigs, cl, cent = P.small_catalogue(rng, n=60_000, d=16, nlist=9_000, W=2, empty_clusters=20)
    q = rng.integers(-127, 128, (6, 16)).astype(np.int8)
    masks = P.random_masks(rng, 6, 2, nbits_max=3)
    _run(svt, opts, items, sigs, cl, cent, 1.0, q, masks, 5_000, 300, "many-probes")


@pytest.mark.parametrize("tie_heavy", [False, True])
def test_tile_pool_beyond_lds(svt, tie_heavy):
    """Pools larger than the merge's LDS stage (19456 keys): with 65536-key pools and streams the pool holds
    whole, every eligible item is a candidate, so the pool merge selects in HBM.  With components in
    {-1, 0, 1} the keys at the k-th best score alone exceed LDS (the heavy-ties branch)."""
    rng = np.random.default_rng(77 + tie_heavy)
    d, n, nlist, nprobe, B, k = (16, 60000, 4, 2, 5, 2048) if tie_heavy else (64, 60000, 4, 2, 5, 2048)
    items, sigs, list_of, cent = P.small_catalogue(rng, n=n, d=d, nlist=nlist, W=2, tie_heavy=tie_heavy)
    ix = svt.Index(items, sigs, list_of, cent, 1.0)
    try:
        q = rng.integers(-1, 2, size=(B, d)).astype(np.int8) if tie_heavy else \
            rng.integers(-127, 128, size=(B, d)).astype(np.int8)
        masks = np.zeros((B, 2), np.uint64)
        masks[1, 0] = np.uint64(1) << np.uint64(3)   # about half the items
        opts = svt.make_options("tile", 65536)
        assert svt.svt_search_path(ix.handle, B, nprobe, k, opts) == "tile"
        got = gpu_search(ix, q, masks, nprobe, k, opts=opts)
        assert int(got[4][:, 1].max()) > 19456, "no pool beyond the LDS stage"
        compare(got, oracle_search(items, sigs, list_of, cent, 1.0, q, masks, nprobe, k), k, "pool beyond LDS")
    finally:
        ix.close()
