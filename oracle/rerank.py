"""CPU oracle of the fused rerank: a gated mixture of experts over the interaction of a query with each
of its retrieved candidates.

TEST INFRASTRUCTURE ONLY.  Only the test suite and the benchmark's CPU-baseline leg may import this
module.  It shares no code with the GPU library.  Plain numpy in float64, following the definition
step by step.

Sources: "SilverTorch - Index as Model" (Meta engineering post), recommendation-quality section: the
retrieved candidates are re-scored by neural modules (an MLP, a mixture of logits, multi-task heads);
"Meta Andromeda" summary, System section: fetching the candidates' embeddings, their interaction with
the request and the scoring are fused in one kernel.  The pages give no formula; the reading (also the
library's, documented beside its entry point) is:

  q^ = q / query_scale, x^ = x / item_scale                      dequantised int8 vectors
  z = q^ * x^                                                    elementwise interaction, [d]
  g = softmax(gate_w q^ + gate_b)                                expert weights of the query, [E]
  y_e = w2_e . relu(w1_e z + b1_e) + b2_e                        expert e, hidden width H
  r = sum_e g_e y_e                                              the candidate's score

and the result is the k_out best candidates by (r desc, id asc).
"""
from __future__ import annotations

import numpy as np


def rerank_scores(items, item_scale, query, query_scale, ids, net):
    """float64 scores r of the candidates ``ids`` (row ids of ``items``) for one query; also returns
    the magnitude bound S_abs = sum_e g_e (sum_h |w2| (sum_j |w1 z| + |b1|) + |b2|) per candidate."""
    qh = query.astype(np.float64) / float(query_scale)
    xh = items[ids].astype(np.float64) / float(item_scale)
    z = xh * qh[None, :]                                            # [n, d]
    a = net["gate_w"].astype(np.float64) @ qh + net["gate_b"].astype(np.float64)
    g = np.exp(a - a.max())
    g = g / g.sum()                                                 # [E]
    w1 = net["w1"].astype(np.float64)                               # [E, H, d]
    pre = np.einsum("ehd,nd->neh", w1, z) + net["b1"].astype(np.float64)[None]
    h = np.maximum(pre, 0.0)
    w2 = net["w2"].astype(np.float64)                               # [E, H]
    y = (h * w2[None]).sum(axis=2) + net["b2"].astype(np.float64)[None]   # [n, E]
    r = y @ g
    babs = np.einsum("ehd,nd->neh", np.abs(w1), np.abs(z)) + np.abs(net["b1"].astype(np.float64))[None]
    s_abs = ((babs * np.abs(w2)[None]).sum(axis=2) + np.abs(net["b2"].astype(np.float64))[None]) @ g
    return r, s_abs


def rerank(items, item_scale, queries, query_scales, cand_ids, net, k_out):
    """For every query b: its candidates are the non-negative entries of cand_ids[b] that are ids of
    ``items``; returns (ids int64 [B, k_out], scores float64 [B, k_out], counts, bounds) with the
    k_out best by (r desc, id asc), padding -1 / -inf, and each returned score's S_abs."""
    B = queries.shape[0]
    out_ids = np.full((B, k_out), -1, np.int64)
    out_sc = np.full((B, k_out), -np.inf, np.float64)
    out_abs = np.zeros((B, k_out), np.float64)
    cnt = np.zeros(B, np.int64)
    for b in range(B):
        c = np.asarray(cand_ids[b], np.int64)
        c = c[(c >= 0) & (c < items.shape[0])]
        if c.size == 0:
            continue
        qs = item_scale if query_scales is None else query_scales[b]
        r, s_abs = rerank_scores(items, item_scale, queries[b], qs, c, net)
        order = np.lexsort((c, -r))[:k_out]
        n = len(order)
        out_ids[b, :n] = c[order]
        out_sc[b, :n] = r[order]
        out_abs[b, :n] = s_abs[order]
        cnt[b] = n
    return out_ids, out_sc, cnt, out_abs

