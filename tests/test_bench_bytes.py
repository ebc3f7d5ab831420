"""The benchmark's algorithmic bytes (bench.algorithmic_bytes), checked on the CPU against a direct count.

The roofline fraction divides these bytes by the scan's time, so they are pinned here: for a batch, every
item of the union of the queries' probe sets costs its signature (8 W bytes), and every such item that at
least one query probing its cluster accepts costs its row (d bytes).  The direct count below takes the probe
sets from the oracle's coarse step and tests each item against each probing query's masks one item at a
time; the eligible-pair count must equal the sum of the oracle's own per-query filter counters.
"""
import numpy as np
import pytest

import bench
import oracle
import synth


def _setup(over, B, G=1, offset=0):
    cat = synth.catalogue("tiny", **over)
    cfg = cat.cfg
    W, h = cfg["sig_words"], cfg["n_hashes"]
    orc = oracle.Oracle()
    sigs = orc.signatures(cat.tokens, h, W)
    qs = synth.queries(cat, B, offset=offset)
    masks = orc.masks(qs, h, W)
    if G > 1:
        # further masks per query: the masks of other queries of the batch (any one passing makes an item eligible)
        masks = np.stack([np.stack([masks[(b + g) % B] for g in range(G)]) for b in range(B)])
    return cat, cfg, sigs, qs, masks, orc


def _direct(cat, sigs, qs, masks, nprobe, orc):
    nlist, d = cat.centroids.shape
    W = sigs.shape[1]
    probed_by = {}
    for b in range(qs.queries.shape[0]):
        probes, _ = orc.coarse(cat.centroids, qs.queries[b], nprobe)
        for c in probes.tolist():
            probed_by.setdefault(c, []).append(b)
    sig_bytes = row_bytes = pairs = 0
    for i in range(cat.n_items):
        c = int(cat.list_of[i])
        if c not in probed_by:
            continue
        sig_bytes += 8 * W
        need = False
        for b in probed_by[c]:
            mb = masks[b] if masks.ndim == 3 else masks[b][None, :]
            if any(all((int(sigs[i, w]) & int(m[w])) == int(m[w]) for w in range(W)) for m in mb):
                pairs += 1
                need = True
        row_bytes += d if need else 0
    return sig_bytes, row_bytes, pairs, len(probed_by)


@pytest.mark.parametrize("B,nprobe,G", [(4, 8, 1), (16, 8, 1), (16, 3, 2), (8, 64, 1)])
def test_algorithmic_bytes_match_direct_count(B, nprobe, G):
    over = dict(n_items=3000, nlist=16)
    cat, cfg, sigs, qs, masks, orc = _setup(over, B, G)
    nlist = cat.centroids.shape[0]
    nprobe = min(nprobe, nlist)
    order = np.argsort(cat.list_of, kind="stable")
    offsets = np.zeros(nlist + 1, np.int64)
    np.cumsum(np.bincount(cat.list_of, minlength=nlist), out=offsets[1:])
    W, d = sigs.shape[1], cat.items.shape[1]
    total, sb, rb, pairs, ncl = bench.algorithmic_bytes(cat, sigs[order], offsets, qs.queries, masks, nprobe, W, d)
    dsb, drb, dpairs, dncl = _direct(cat, sigs, qs, masks, nprobe, orc)
    assert (sb, rb, ncl) == (dsb, drb, dncl)
    assert total == dsb + drb
    assert pairs == dpairs
    # the oracle's filter counters count the same pairs
    st = orc.search(cat.items, sigs, cat.list_of, cat.centroids, cat.item_scale, qs.queries, masks, nprobe, 10)[4]
    assert pairs == int(st[:, 1].sum())
