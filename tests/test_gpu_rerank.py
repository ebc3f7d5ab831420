"""svt_rerank (gated mixture of experts over the query-candidate interaction, fused with the row fetch and
the final top-k) against the float64 oracle in oracle/rerank.py, on seeded inputs: every supported
dimension, several expert shapes, candidate counts from 0 to the maximum with ragged last tiles,
duplicates, absent ids, an updated index and the candidates of a real search.

The kernel computes in float32, so scores are compared within a bound derived from its arithmetic
(unit roundoff u = 2^-24):
  * the first layer sums d products x V with V = w1 q^ / item_scale (V carries 3 roundings): error at
    most (d + 4) u sum_f |w1 z| + u |b1| per unit;
  * relu is 1-Lipschitz; the weighted sum over the 64 padded units (4 terms per lane, then a 4-level
    tree) and the gate-weighted b2 add at most ~16 u of the magnitudes;
  * a gate logit is 64 lane sums of d/64 products each, added in a 6-level tree, plus the bias: error at
    most (d/64 + 8) u A_e, A_e = sum_f |gate_w q^| + |gate_b|; the softmax turns an error of at most a
    in the logits into a relative error of at most 2 a in every g_e.
Summed: |r_gpu - r| <= u S_abs ((d + 20) + 2 (d/64 + 8) max_e A_e), with S_abs = sum_e g_e (sum_h |w2|
(sum_f |w1 z| + |b1|) + |b2|) from the oracle; the test allows twice that.

Equal float32 keys are ordered by id on the GPU.  The oracle's order is in float64, so where two
candidates' oracle scores lie within the tolerance of each other the GPU may order them either way: the
test checks what is unique (counts, padding, the set above every such near-tie, each score) and that
the rest is a valid ranking (sorted by the GPU's own (score desc, id asc), nothing left out that the
oracle puts clearly above the last one returned).
"""
import ctypes

import numpy as np
import pytest

import oracle_pins as P
from gpu_common import say
import synth
from oracle import rerank as R

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module")
def svt():
    import torch
    assert torch.cuda.is_available()
    torch.cuda.set_device(0)
    from int8_ivf_ann_amd import svt as m
    m.lib()
    return m


def _t(a, dtype=None):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a if dtype is None else a.astype(dtype))).cuda()


def gpu_rerank(ix, queries, cand, net, k_out, query_scales=None):
    import torch
    tnet = {k: _t(v, np.float32) for k, v in net.items()}
    qs = None if query_scales is None else _t(query_scales, np.float32)
    ids, sc, cnt = ix.rerank(_t(queries, np.int8), _t(cand, np.int64), tnet, k_out, query_scales=qs)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), sc.cpu().numpy(), cnt.cpu().numpy()


def tolerance(items, scale, q, qs, ids, net):
    """Per-candidate bound on |r_gpu - r| (see the module docstring)."""
    d = items.shape[1]
    _, s_abs = R.rerank_scores(items, scale, q, qs, ids, net)
    qh = q.astype(np.float64) / float(qs)
    a_max = float(np.max(np.abs(net["gate_w"].astype(np.float64)) @ np.abs(qh) + np.abs(net["gate_b"].astype(np.float64))))
    return 2.0 * U * s_abs * ((d + 20) + 2.0 * (d / 64.0 + 8) * a_max)


def check(items, scale, queries, qs, cand, net, k_out, got, label, present=None):
    """present: ids the index holds (default: every row of items)."""
    ids, sc, cnt = got
    B = queries.shape[0]
    n_rows = items.shape[0]
    # the oracle skips negative ids and ids past its rows; ids the index does not hold are skipped too
    cand_o = np.array(cand, np.int64, copy=True)
    if present is not None:
        keep = np.isin(cand_o, np.asarray(present, np.int64))
        cand_o[~keep] = -1
    cand_o[cand_o >= n_rows] = -1
    rids, rsc, rcnt, _ = R.rerank(items, scale, queries, qs, cand_o, net, k_out)
    assert np.array_equal(cnt, rcnt), f"{label}: counts {cnt[:8]} vs {rcnt[:8]}"
    for b in range(B):
        n = int(rcnt[b])
        assert np.all(ids[b, n:] == -1) and np.all(np.isneginf(sc[b, n:])), f"{label}: padding of query {b}"
        if n == 0:
            continue
        c = cand_o[b][cand_o[b] >= 0]
        q_s = scale if qs is None else float(qs[b])
        r_all, _ = R.rerank_scores(items, scale, queries[b], q_s, c, net)
        tol_all = tolerance(items, scale, queries[b], q_s, c, net)
        g_ids, g_sc = ids[b, :n], sc[b, :n].astype(np.float64)
        # every returned id is a candidate, returned no more often than it was given
        uc, ncand = np.unique(c, return_counts=True)
        ug, ngot = np.unique(g_ids, return_counts=True)
        pos = np.searchsorted(uc, ug)
        assert np.all(pos < len(uc)) and np.all(uc[np.minimum(pos, len(uc) - 1)] == ug), f"{label}: q{b} foreign id"
        assert np.all(ngot <= ncand[pos]), f"{label}: q{b} id returned more often than given"
        # the GPU's own order: (score desc, id asc) over its float32 scores
        for j in range(n - 1):
            assert g_sc[j] > g_sc[j + 1] or (g_sc[j] == g_sc[j + 1] and g_ids[j] <= g_ids[j + 1]), \
                f"{label}: q{b} not sorted at rank {j}"
        # each returned score against the oracle's score of that id
        first = {}
        for i, cid in enumerate(c):
            first.setdefault(int(cid), i)
        oi = np.array([first[int(x)] for x in g_ids])
        err = np.abs(g_sc - r_all[oi])
        assert np.all(err <= tol_all[oi]), \
            f"{label}: q{b} score error {err.max():.3g} above bound {tol_all[oi][np.argmax(err - tol_all[oi])]:.3g}"
        # nothing left out that the oracle puts clearly above a returned one: with |r_gpu - r| <= tol,
        # r_gpu(left) <= r_gpu(chosen) requires r(left) - tol(left) <= r(chosen) + tol(chosen)
        if n < len(c):
            chosen = np.zeros(len(c), bool)
            for cid, m in zip(ug, ngot):
                chosen[np.nonzero(c == cid)[0][:m]] = True
            assert np.max(r_all[~chosen] - tol_all[~chosen]) <= np.min(r_all[chosen] + tol_all[chosen]), \
                f"{label}: q{b} left out a clearly better candidate"
        # where the oracle's neighbours are farther apart than twice the tolerance, the ids agree exactly
        rr = rsc[b, :n]
        gap_ok = np.ones(n, bool)
        tol_r = tol_all[[first[int(x)] for x in rids[b, :n]]]
        gaps = np.diff(rr) * -1.0
        close = gaps <= 2.0 * np.maximum(tol_r[:-1], tol_r[1:])
        gap_ok[:-1] &= ~close
        gap_ok[1:] &= ~close
        if n < len(c):   # the last returned against the best left out
            left = np.ones(len(c), bool)
            left[[first[int(x)] for x in rids[b, :n]]] = False
            if left.any() and rr[-1] - np.max(r_all[left]) <= 2.0 * np.max(tol_all):
                gap_ok[-1] = False
        assert np.array_equal(g_ids[gap_ok], rids[b, :n][gap_ok]), f"{label}: q{b} ids differ away from near-ties"


def _catalogue(rng, n, d, nlist=8):
    items, sigs, list_of, cent = P.small_catalogue(rng, n=n, d=d, nlist=nlist, W=1)
    return items, sigs, list_of, cent


SHAPES = [  # d, E, H, n_cand, k_out, B
    (16, 1, 1, 33, 10, 3),
    (32, 2, 7, 100, 100, 5),
    (64, 4, 16, 1000, 64, 7),
    (128, 8, 8, 4096, 2048, 3),
    (128, 3, 21, 517, 1, 4),
    (256, 2, 32, 1200, 500, 6),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"d{s[0]}_e{s[1]}h{s[2]}_c{s[3]}_k{s[4]}" for s in SHAPES])
@pytest.mark.parametrize("scaled", [False, True])
def test_rerank_matches_oracle(svt, shape, scaled):
    d, E, H, n_cand, k_out, B = shape
    rng = np.random.default_rng(100 + d + E + n_cand + scaled)
    n = 6000
    items, sigs, list_of, cent = _catalogue(rng, n, d)
    scale = 127.0 / 3.0
    ix = svt.Index(items, sigs, list_of, cent, scale)
    try:
        queries = rng.integers(-127, 128, size=(B, d)).astype(np.int8)
        qs = rng.uniform(40.0, 130.0, size=B).astype(np.float32) if scaled else None
        cand = rng.integers(0, n, size=(B, n_cand)).astype(np.int64)
        # some skipped entries: -1 (search padding), past the ids
        cand[rng.random((B, n_cand)) < 0.05] = -1
        cand[rng.random((B, n_cand)) < 0.02] = n + 5
        net = synth.rerank_net(rng, d, E, H)
        say(f"rerank d={d} E={E} H={H} n_cand={n_cand} k_out={k_out} B={B} scaled={scaled}")
        got = gpu_rerank(ix, queries, cand, net, k_out, qs)
        check(items, scale, queries, qs, cand, net, k_out, got, f"d{d} E{E} H{H}")
    finally:
        ix.close()


def test_rerank_ties_duplicates_and_empty(svt):
    import torch
    rng = np.random.default_rng(7)
    d, n = 64, 500
    items, sigs, list_of, cent = _catalogue(rng, n, d)
    items[10] = items[20] = items[30]             # equal rows: equal float32 scores, ordered by id
    scale = 50.0
    ix = svt.Index(items, sigs, list_of, cent, scale)
    try:
        net = synth.rerank_net(rng, d, 2, 8)
        q = rng.integers(-127, 128, size=(4, d)).astype(np.int8)
        cand = np.full((4, 40), -1, np.int64)
        cand[0, :6] = [30, 20, 10, 5, 5, 99]      # ties and a repeated id
        cand[1, :] = -1                            # nothing to score
        cand[2, :3] = [n, n + 1, 10 ** 9]          # only ids past the catalogue
        cand[3, :] = rng.integers(0, n, size=40)
        for k_out in (1, 3, 6, 40):
            ids, sc, cnt = gpu_rerank(ix, q, cand, net, k_out)
            check(items, scale, q, None, cand, net, k_out, (ids, sc, cnt), f"ties k_out={k_out}")
            assert cnt[1] == 0 and cnt[2] == 0
            row = list(ids[0, :cnt[0]])
            t = [x for x in row if x in (10, 20, 30)]
            assert t == sorted(t), f"equal scores not in id order: {row}"
            if t:
                tie = sc[0, [row.index(x) for x in t]]
                assert np.all(tie == tie[0]), "equal rows scored differently"
            if k_out >= 6:   # every candidate returned: the three ties, and id 5 twice
                assert t == [10, 20, 30]
                assert row.count(5) == 2, "a repeated id is returned once per occurrence"
        # zero candidates per query
        out = ix.rerank(_t(q, np.int8), torch.zeros((4, 0), dtype=torch.int64, device="cuda"),
                        {k: _t(v, np.float32) for k, v in net.items()}, 5)
        torch.cuda.synchronize()
        assert np.all(out[0].cpu().numpy() == -1) and np.all(out[2].cpu().numpy() == 0)
    finally:
        ix.close()


def test_rerank_after_updates(svt):
    """Deleted ids are skipped, inserted ids are scored from their new rows."""
    rng = np.random.default_rng(8)
    d, n, nlist = 32, 800, 6
    items, sigs, list_of, cent = _catalogue(rng, n, d, nlist)
    scale = 30.0
    ix = svt.Index(items, sigs, list_of, cent, scale, id_capacity=1200, slack_min=40)
    try:
        dead = np.arange(0, 100, 3, dtype=np.int64)
        ix.delete(dead)
        new_ids = np.arange(1000, 1030, dtype=np.int64)
        new_rows = rng.integers(-127, 128, size=(30, d)).astype(np.int8)
        new_sigs = np.zeros((30, 1), np.uint64)
        ix.insert(new_ids, new_rows, new_sigs, rng.integers(0, nlist, size=30).astype(np.int32))
        full = np.zeros((1200, d), np.int8)
        full[:n] = items
        full[new_ids] = new_rows
        present = np.setdiff1d(np.concatenate([np.arange(n), new_ids]), dead)
        net = synth.rerank_net(rng, d, 4, 4)
        q = rng.integers(-127, 128, size=(5, d)).astype(np.int8)
        cand = np.concatenate([rng.integers(0, 100, size=(5, 40)), rng.integers(1000, 1040, size=(5, 40)),
                               rng.integers(800, 1000, size=(5, 10))], axis=1).astype(np.int64)
        got = gpu_rerank(ix, q, cand, net, 32)
        check(full, scale, q, None, cand, net, 32, got, "updated", present=present)
        assert not np.isin(got[0], dead).any()
    finally:
        ix.close()


def test_rerank_of_search_results(svt):
    """The intended pipeline: the search's ids (with -1 padding) are the candidates."""
    import torch
    rng = np.random.default_rng(9)
    d, n, nlist, B = 128, 20000, 32, 12
    items, sigs, list_of, cent = _catalogue(rng, n, d, nlist)
    scale = 127.0 / 4.0
    ix = svt.Index(items, sigs, list_of, cent, scale)
    try:
        q = rng.integers(-127, 128, size=(B, d)).astype(np.int8)
        masks = P.random_masks(rng, B, 1, nbits_max=4)
        ids, _, _, _, _ = ix.search(_t(q, np.int8), _t(masks.view(np.int64)), 8, 512)
        net = synth.rerank_net(rng, d, 4, 16)
        tnet = {k: _t(v, np.float32) for k, v in net.items()}
        rid, rsc, rcnt = ix.rerank(_t(q, np.int8), ids, tnet, 100)
        torch.cuda.synchronize()
        check(items, scale, q, None, ids.cpu().numpy(), net, 100, (rid.cpu().numpy(), rsc.cpu().numpy(),
                                                                    rcnt.cpu().numpy()), "search->rerank")
    finally:
        ix.close()


def test_rerank_argument_errors(svt):
    import torch
    rng = np.random.default_rng(10)
    d = 32
    items, sigs, list_of, cent = _catalogue(rng, 300, d)
    ix = svt.Index(items, sigs, list_of, cent, 10.0)
    try:
        L = svt.lib()
        q = torch.zeros((2, d), dtype=torch.int8, device="cuda")
        c = torch.zeros((2, 8), dtype=torch.int64, device="cuda")
        oid = torch.empty((2, 8), dtype=torch.int64, device="cuda")
        osc = torch.empty((2, 8), dtype=torch.float32, device="cuda")
        w = torch.zeros(8 * 64 * d, dtype=torch.float32, device="cuda")
        p = w.data_ptr()

        def call(E=2, H=4, n_cand=8, k_out=8, B=2, ptrs=None, qp=q.data_ptr(), cp=c.data_ptr(), ip=oid.data_ptr(),
                 sp=osc.data_ptr()):
            net = svt.svt_rerank_net(E, H, *(ptrs or [p] * 6))
            return L.svt_rerank(ix.handle, B, qp, None, n_cand, cp, ctypes.byref(net), k_out, ip, sp, None, None)

        assert call() == svt.SVT_OK
        torch.cuda.synchronize()
        for kw in ({"E": 0}, {"E": 9}, {"H": 0}, {"E": 4, "H": 17}, {"n_cand": -1}, {"n_cand": 4097},
                   {"k_out": 0}, {"k_out": 2049}, {"B": -1}, {"ptrs": [p, p, 0, p, p, p]}, {"qp": None},
                   {"cp": None}, {"cp": c.data_ptr() + 4}, {"ip": oid.data_ptr() + 4}, {"sp": osc.data_ptr() + 2},
                   {"ptrs": [p, p, p + 2, p, p, p]}):
            assert call(**kw) == svt.SVT_EINVAL, kw
        assert call(B=0, qp=None) == svt.SVT_OK
        assert L.svt_rerank(ix.handle, 2, q.data_ptr(), None, 8, c.data_ptr(), None, 8, oid.data_ptr(),
                            osc.data_ptr(), None, None) == svt.SVT_EINVAL
        with pytest.raises(ValueError, match="shape"):
            ix.rerank(q, c, {"gate_w": torch.zeros((2, d + 1), device="cuda"), "gate_b": torch.zeros(2, device="cuda"),
                             "w1": torch.zeros((2, 3, d), device="cuda"), "b1": torch.zeros((2, 3), device="cuda"),
                             "w2": torch.zeros((2, 3), device="cuda"), "b2": torch.zeros(2, device="cuda")}, 4)
    finally:
        ix.close()


@pytest.mark.parametrize("d,E,H", [(16, 1, 1), (128, 1, 1), (128, 4, 16)])
def test_rerank_is_deterministic(svt, d, E, H):
    """Repeated calls on the same inputs return identical bits (the shared-memory staging of the
    weights has no lost writes: every entry is written once, by one thread), and the first matches the
    oracle."""
    import torch
    rng = np.random.default_rng(11 + d + E)
    n, B, n_cand, k_out = 5000, 96, 300, 40
    items, sigs, list_of, cent = _catalogue(rng, n, d)
    scale = 127.0 / 3.0
    ix = svt.Index(items, sigs, list_of, cent, scale)
    try:
        q = rng.integers(-127, 128, size=(B, d)).astype(np.int8)
        cand = rng.integers(0, n, size=(B, n_cand)).astype(np.int64)
        net = synth.rerank_net(rng, d, E, H)
        net["b1"][:] = np.abs(net["b1"]) + np.float32(0.05)   # positive biases: a lost weight changes scores
        tnet = {k: _t(v, np.float32) for k, v in net.items()}
        q_d, c_d = _t(q, np.int8), _t(cand, np.int64)
        runs = []
        for _ in range(12):
            ids, sc, cnt = ix.rerank(q_d, c_d, tnet, k_out)
            runs.append((ids.clone(), sc.clone(), cnt.clone()))
        torch.cuda.synchronize()
        for ids, sc, cnt in runs[1:]:
            assert torch.equal(ids, runs[0][0]) and torch.equal(sc, runs[0][1]) and torch.equal(cnt, runs[0][2])
        check(items, scale, q, None, cand, net, k_out,
              tuple(t.cpu().numpy() for t in runs[0]), f"deterministic d{d} E{E} H{H}")
    finally:
        ix.close()
