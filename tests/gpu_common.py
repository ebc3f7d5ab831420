"""Shared helpers of the GPU parity tests: run one search through the C ABI and through the CPU
oracle on the same seeded inputs and compare element by element.

The bar: ids, int32 scores, counts and scan statistics bit-exact; fscores within 1e-6 relative of
the oracle's (score / (item_scale * query_scale) in double, rounded to float); padding exact.
"""
from __future__ import annotations

import sys

import numpy as np

import oracle

INT32_MIN = np.iinfo(np.int32).min


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_search(ix, queries, masks, nprobe, k, query_scales=None, opts=None):
    import torch
    q = torch.from_numpy(np.ascontiguousarray(queries, np.int8)).cuda()
    m = torch.from_numpy(np.ascontiguousarray(masks, np.uint64).view(np.int64)).cuda()
    qs = None if query_scales is None else torch.from_numpy(np.ascontiguousarray(query_scales, np.float32)).cuda()
    ids, sc, fs, cnt, st = ix.search(q, m, nprobe, k, query_scales=qs, opts=opts)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), sc.cpu().numpy(), fs.cpu().numpy(), cnt.cpu().numpy(), st.cpu().numpy()


def compare(got, ref, k, label=""):
    ids, sc, fs, cnt, st = got
    rids, rsc, rfs, rcnt, rst = ref
    assert np.array_equal(cnt, rcnt), f"{label}: counts differ {cnt[:8]} vs {rcnt[:8]}"
    assert np.array_equal(st, rst), f"{label}: scan statistics differ"
    bad = np.nonzero((ids != rids).any(axis=1) | (sc != rsc).any(axis=1))[0]
    if len(bad):
        b = int(bad[0])
        j = int(np.nonzero((ids[b] != rids[b]) | (sc[b] != rsc[b]))[0][0])
        raise AssertionError(f"{label}: query {b} differs first at rank {j}: gpu ({ids[b, j]}, {sc[b, j]}) "
                             f"oracle ({rids[b, j]}, {rsc[b, j]}); {len(bad)} queries differ")
    valid = rcnt[:, None] > np.arange(k)[None, :]
    assert np.all(np.abs(fs[valid].astype(np.float64) - rfs[valid]) <= 1e-6 * np.abs(rfs[valid].astype(np.float64))), \
        f"{label}: fscores beyond 1e-6 relative"
    assert np.all(np.isneginf(fs[~valid])), f"{label}: fscore padding"
    assert np.all(ids[~valid] == -1) and np.all(sc[~valid] == INT32_MIN), f"{label}: id/score padding"


def check_invariants(items, sigs, list_of, got, masks, queries, k, centroids=None, nprobe=None):
    """Properties that hold at any size: rows sorted by (score desc, id asc), ids unique, every id
    eligible, every score the exact dot product, and (given the centroids) every id in one of the
    query's probed clusters as the oracle's coarse step picks them."""
    ids, sc, fs, cnt, st = got
    orc = oracle.Oracle() if centroids is not None else None
    for b in range(ids.shape[0]):
        n = int(cnt[b])
        i, s = ids[b, :n], sc[b, :n].astype(np.int64)
        assert len(np.unique(i)) == n
        key = list(zip((-s).tolist(), i.tolist()))
        assert key == sorted(key)
        if n:
            mb = masks[b] if masks.ndim == 3 else masks[b][None, :]   # eligible under any of the query's masks
            ok = np.zeros(n, bool)
            for m in mb:
                ok |= np.all((sigs[i] & m) == m, axis=1)
            assert np.all(ok)
            assert np.array_equal(items[i].astype(np.int64) @ queries[b].astype(np.int64), s)
            if orc is not None:
                probes, _ = orc.coarse(centroids, queries[b], nprobe)
                assert np.all(np.isin(list_of[i], probes)), f"query {b}: an id outside the probed clusters"


def oracle_search(items, sigs, list_of, cent, scale, queries, masks, nprobe, k, query_scales=None, threads=8):
    return oracle.Oracle().search(items, sigs, list_of, cent, scale, queries, masks, nprobe, k,
                                  query_scales=query_scales, n_threads=threads)
