"""The rerank oracle against values worked out by hand and closed forms (no GPU).  Each pin would catch a
plausible slip: a missing dequantisation, a transposed expert matrix, a wrong ReLU sign, a dropped bias,
gate weights not normalised, the tie order."""
import math

import numpy as np

import synth
from oracle import rerank as R


def _net(E, H, d):
    z = lambda *s: np.zeros(s, np.float32)
    return {"gate_w": z(E, d), "gate_b": z(E), "w1": z(E, H, d), "b1": z(E, H), "w2": z(E, H), "b2": z(E)}


ITEMS = np.array([[1, 2, 3, 4], [-1, -2, 0, 7], [1, 2, 3, 4]], np.int8)
Q = np.array([[2, -3, 5, 1]], np.int8)


def test_feature_selection_by_hand():
    # one expert, hidden unit h reads feature j_h: w1[0, h] = e_{j_h}; w2 = (1, 2, 4)
    net = _net(1, 3, 4)
    for h, j in enumerate((0, 1, 2)):
        net["w1"][0, h, j] = 1.0
    net["w2"][0] = (1.0, 2.0, 4.0)
    # item_scale 2: x^ = x / 2; query_scale 1: q^ = q
    # item 0: z = (2*0.5, -3*1, 5*1.5) = (1, -3, 7.5)  -> 1*1 + 2*relu(-3) + 4*7.5 = 31
    # item 1: z = (2*-0.5, -3*-1, 5*0) = (-1, 3, 0)    -> relu(-1) + 2*3 + 4*0 = 6
    r, _ = R.rerank_scores(ITEMS, 2.0, Q[0], 1.0, np.array([0, 1]), net)
    assert np.allclose(r, [31.0, 6.0], rtol=0, atol=1e-12)


def test_gate_and_biases_by_hand():
    # two constant experts (w1 = 0): y_e = w2_e * relu(b1_e) + b2_e = (4, 8 + 0.5); gate logits (0, ln 3)
    # from the bias, so g = (1/4, 3/4) and r = 4/4 + 8.5 * 3/4 = 7.375 for every candidate
    net = _net(2, 1, 4)
    net["b1"][:, 0] = (4.0, 8.0)
    net["w2"][:, 0] = 1.0
    net["b2"][:] = (0.0, 0.5)
    net["gate_b"][:] = (0.0, math.log(3.0))
    e1 = math.exp(float(net["gate_b"][1]))   # the weights are float32: ln 3 as stored
    r, _ = R.rerank_scores(ITEMS, 1.0, Q[0], 1.0, np.array([0, 1, 2]), net)
    assert np.allclose(r, (4.0 + 8.5 * e1) / (1.0 + e1), rtol=0, atol=1e-12)
    assert abs(r[0] - 7.375) < 1e-6
    # a gate that reads the query: logit 0 = q^_0 = 2 (query_scale 1), logit 1 = ln 3 + 0
    net["gate_w"][0, 0] = 1.0
    e0 = math.exp(2.0)
    expect = (4.0 * e0 + 8.5 * e1) / (e0 + e1)
    r, _ = R.rerank_scores(ITEMS, 1.0, Q[0], 1.0, np.array([0]), net)
    assert abs(r[0] - expect) < 1e-12


def test_negative_preactivation_is_cut():
    net = _net(1, 1, 4)
    net["w1"][0, 0, 1] = 1.0          # z_1 = q^_1 x^_1 = -3 * 2 = -6 for item 0
    net["b1"][0, 0] = 2.0             # -6 + 2 < 0: cut to 0
    net["w2"][0, 0] = 5.0
    net["b2"][0] = -1.25
    r, _ = R.rerank_scores(ITEMS, 1.0, Q[0], 1.0, np.array([0]), net)
    assert r[0] == -1.25


def test_query_scale_homogeneity():
    # without biases and with a constant gate the score is positively homogeneous in q^
    rng = np.random.default_rng(3)
    net = synth.rerank_net(rng, 4, 3, 5)
    for k in ("gate_w", "b1", "b2"):
        net[k][:] = 0
    r1, _ = R.rerank_scores(ITEMS, 3.0, Q[0], 2.0, np.array([0, 1]), net)
    r2, _ = R.rerank_scores(ITEMS, 3.0, Q[0], 1.0, np.array([0, 1]), net)   # q^ twice as large
    assert np.allclose(r2, 2.0 * r1, rtol=1e-12, atol=0)


def test_order_ties_padding_and_ids():
    # items 0 and 2 are equal rows: equal scores, lower id first; -1 and out-of-range ids are skipped;
    # fewer candidates than k_out pad with -1 / -inf
    net = _net(1, 3, 4)
    for h, j in enumerate((0, 1, 2)):
        net["w1"][0, h, j] = 1.0
    net["w2"][0] = (1.0, 2.0, 4.0)
    cand = np.array([[2, -1, 1, 0, 99]], np.int64)
    ids, sc, cnt, _ = R.rerank(ITEMS, 2.0, Q, np.array([1.0]), cand, net, 5)
    assert cnt[0] == 3
    assert ids[0].tolist() == [0, 2, 1, -1, -1]
    assert np.allclose(sc[0, :3], [31.0, 31.0, 6.0]) and np.all(np.isneginf(sc[0, 3:]))
    ids, sc, cnt, _ = R.rerank(ITEMS, 2.0, Q, None, cand, net, 2)   # query scale = item scale: halved scores
    assert ids[0].tolist() == [0, 2] and cnt[0] == 2


def test_error_bound_is_a_bound():
    # S_abs bounds |r|, with equality when every term is non-negative
    rng = np.random.default_rng(4)
    net = synth.rerank_net(rng, 4, 2, 3)
    r, s_abs = R.rerank_scores(ITEMS, 2.0, Q[0], 1.5, np.array([0, 1, 2]), net)
    assert np.all(np.abs(r) <= s_abs + 1e-12)
    pos = _net(1, 1, 4)
    pos["w1"][0, 0, 0] = 1.0
    pos["w2"][0, 0] = 2.0
    r, s_abs = R.rerank_scores(ITEMS, 2.0, Q[0], 1.0, np.array([0]), pos)
    assert r[0] == s_abs[0] == 2.0
