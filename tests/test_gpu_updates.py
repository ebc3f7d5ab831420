"""In-place index updates (insert, delete, re-sign) against the CPU oracle: after every round of a seeded
stream of updates, searches on every path must return exactly what the oracle returns for the updated
catalogue (the items present, with their current signatures; ids keep their values).  Rejected batches
must leave the index as it was."""
import numpy as np
import pytest

import oracle_pins as P
from gpu_common import compare, gpu_search, oracle_search, say

pytestmark = pytest.mark.gpu

D, W, NLIST = 64, 2, 24
SLACK_MIN, SLACK_FRAC = 8, 0.25


def _sigs(rng, n):
    bits = rng.random((n, W, 64)) < 0.45
    return (bits.astype(np.uint64) << np.arange(64, dtype=np.uint64)).sum(axis=2, dtype=np.uint64)


class Model:
    """The catalogue the index should hold: id -> (row, signature, cluster)."""

    def __init__(self, items, sigs, cl):
        self.rows = {i: items[i] for i in range(items.shape[0])}
        self.sigs = {i: sigs[i].copy() for i in range(items.shape[0])}
        self.cl = {i: int(cl[i]) for i in range(items.shape[0])}
        size = np.bincount(cl, minlength=NLIST)
        self.cap = size + np.maximum(SLACK_MIN, np.ceil(SLACK_FRAC * size)).astype(np.int64)

    def live(self, c):
        return sum(1 for v in self.cl.values() if v == c)

    def arrays(self):
        ids = np.array(sorted(self.rows), np.int64)   # id order: the oracle breaks ties by row index
        items = np.stack([self.rows[i] for i in ids]).astype(np.int8)
        sigs = np.stack([self.sigs[i] for i in ids]).astype(np.uint64)
        cl = np.array([self.cl[i] for i in ids], np.int32)
        return ids, items, sigs, cl


def _check(svt, ix, model, cent, rng, label):
    ids, items, sigs, cl = model.arrays()
    q = rng.integers(-127, 128, (40, D)).astype(np.int8)
    masks = P.random_masks(rng, 40, W, nbits_max=2)
    for path, nprobe, k in (("query", 6, 150), ("tile", 6, 150), ("tile", NLIST, 300), ("query", NLIST, 64)):
        say(f"{label}: path {path} nprobe {nprobe} k {k} ({len(ids)} items)")
        got = gpu_search(ix, q, masks, nprobe, k, opts=svt.make_options(path))
        ref = list(oracle_search(items, sigs, cl, cent, 2.0, q, masks, nprobe, k))
        ref[0] = np.where(ref[0] >= 0, ids[np.clip(ref[0], 0, None)], -1)   # oracle rows -> ids
        compare(got, tuple(ref), k, f"{label} {path} nprobe={nprobe}")


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available()
    torch.cuda.set_device(0)
    from int8_ivf_ann_amd import svt
    return svt


def test_update_stream_matches_oracle(env):
    svt = env
    rng = np.random.default_rng(2024)
    items, sigs, cl, cent = P.small_catalogue(rng, n=6000, d=D, nlist=NLIST, W=W, empty_clusters=2)
    ix = svt.Index(items, sigs, cl, cent, 2.0, id_capacity=12000, slack_min=SLACK_MIN, slack_frac=SLACK_FRAC)
    model = Model(items, sigs, cl)
    try:
        _check(svt, ix, model, cent, rng, "upload")
        next_id = 6000
        for rnd in range(5):
            # deletes
            present = np.array(sorted(model.rows), np.int64)
            dels = rng.choice(present, size=300, replace=False)
            ix.delete(dels)
            for i in dels.tolist():
                del model.rows[i], model.sigs[i], model.cl[i]
            # inserts, within each cluster's free slots (new ids and, from the second update round on, ids deleted before)
            free = {c: int(model.cap[c] - model.live(c)) for c in range(NLIST)}
            new_ids, new_cl = [], []
            reuse = [i for i in range(6000) if i not in model.rows][:50] if rnd >= 2 else []
            for nid in reuse + list(range(next_id, next_id + 400)):
                c = int(rng.integers(0, NLIST))
                if free[c] == 0:
                    continue
                free[c] -= 1
                new_ids.append(nid)
                new_cl.append(c)
            next_id += 400
            rows = rng.integers(-127, 128, (len(new_ids), D)).astype(np.int8)
            nsig = _sigs(rng, len(new_ids))
            ix.insert(np.array(new_ids), rows, nsig, np.array(new_cl))
            for j, nid in enumerate(new_ids):
                model.rows[nid], model.sigs[nid], model.cl[nid] = rows[j], nsig[j], new_cl[j]
            # re-signs
            present = np.array(sorted(model.rows), np.int64)
            rs = rng.choice(present, size=200, replace=False)
            rsig = _sigs(rng, 200)
            ix.resign(rs, rsig)
            for j, i in enumerate(rs.tolist()):
                model.sigs[i] = rsig[j]
            assert ix.n_items == len(model.rows)
            _check(svt, ix, model, cent, rng, f"round {rnd}")
    finally:
        ix.close()


def test_full_cluster_and_rejected_batches(env):
    svt = env
    rng = np.random.default_rng(77)
    items, sigs, cl, cent = P.small_catalogue(rng, n=3000, d=D, nlist=NLIST, W=W)
    ix = svt.Index(items, sigs, cl, cent, 2.0, id_capacity=5000, slack_min=SLACK_MIN, slack_frac=SLACK_FRAC)
    model = Model(items, sigs, cl)
    try:
        # fill cluster 3 to its capacity, then one more insert there is refused
        c = 3
        n_free = int(model.cap[c] - model.live(c))
        new_ids = np.arange(3000, 3000 + n_free)
        rows = rng.integers(-127, 128, (n_free, D)).astype(np.int8)
        nsig = _sigs(rng, n_free)
        ix.insert(new_ids, rows, nsig, np.full(n_free, c))
        for j, nid in enumerate(new_ids.tolist()):
            model.rows[nid], model.sigs[nid], model.cl[nid] = rows[j], nsig[j], c
        bad = [
            ("cluster full", lambda: ix.insert([4000], rows[:1], nsig[:1], [c]), svt.SVT_ENOSPACE),
            ("id present", lambda: ix.insert([5], rows[:1], nsig[:1], [0]), svt.SVT_EINVAL),
            ("id repeated", lambda: ix.insert([4001, 4001], rows[:2], nsig[:2], [0, 1]), svt.SVT_EINVAL),
            ("id out of range", lambda: ix.insert([5000], rows[:1], nsig[:1], [0]), svt.SVT_EINVAL),
            ("cluster out of range", lambda: ix.insert([4002], rows[:1], nsig[:1], [NLIST]), svt.SVT_EINVAL),
            ("reserved signature", lambda: ix.insert([4003], rows[:1], np.full((1, W), ~np.uint64(0)), [0]),
             svt.SVT_EINVAL),
            ("delete absent", lambda: ix.delete([4999]), svt.SVT_EINVAL),
            ("delete repeated", lambda: ix.delete([7, 7]), svt.SVT_EINVAL),
            ("resign absent", lambda: ix.resign([4998], nsig[:1]), svt.SVT_EINVAL),
            ("resign reserved", lambda: ix.resign([8], np.full((1, W), ~np.uint64(0))), svt.SVT_EINVAL),
        ]
        for label, call, code in bad:
            say(f"rejected batch: {label}")
            with pytest.raises(svt.SvtError) as ei:
                call()
            assert f"svt error {code}:" in str(ei.value), (label, str(ei.value))
        # a batch with one bad id changes nothing either: items 10..19 stay
        with pytest.raises(svt.SvtError):
            ix.delete(list(range(10, 20)) + [4999])
        assert ix.n_items == len(model.rows)
        # delete the whole cluster 3, then refill it: the freed slots are used again
        gone = [i for i, v in model.cl.items() if v == c]
        ix.delete(gone)
        for i in gone:
            del model.rows[i], model.sigs[i], model.cl[i]
        _check(svt, ix, model, cent, rng, "cluster 3 emptied")
        refill = np.arange(4100, 4100 + int(model.cap[c]))
        rows2 = rng.integers(-127, 128, (refill.shape[0], D)).astype(np.int8)
        nsig2 = _sigs(rng, refill.shape[0])
        ix.insert(refill, rows2, nsig2, np.full(refill.shape[0], c))
        for j, nid in enumerate(refill.tolist()):
            model.rows[nid], model.sigs[nid], model.cl[nid] = rows2[j], nsig2[j], c
        _check(svt, ix, model, cent, rng, "cluster 3 refilled")
    finally:
        ix.close()


def test_plain_index_refuses_updates(env):
    svt = env
    rng = np.random.default_rng(5)
    items, sigs, cl, cent = P.small_catalogue(rng, n=500, d=D, nlist=4, W=W)
    ix = svt.Index(items, sigs, cl, cent, 1.0)
    try:
        with pytest.raises(svt.SvtError) as ei:
            ix.delete([1])
        assert f"svt error {svt.SVT_ESTATE}:" in str(ei.value)
    finally:
        ix.close()
