"""GPU vs oracle on the five workload presets at their full sizes, in the launch configuration the
benchmark times.  The 1M and 10M presets are compared on every query; the 80M presets on a sample
of queries the oracle computes one by one, plus size-independent invariants on every query."""
import time

import numpy as np
import pytest

import oracle
import synth
from gpu_common import check_invariants, compare, gpu_search, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def svt():
    import torch
    assert torch.cuda.is_available()
    torch.cuda.set_device(0)
    from int8_ivf_ann_amd import svt as m
    m.lib()
    return m


class Preset:
    def __init__(self, svt, name):
        t = time.time()
        self.cat = synth.catalogue(name)
        say(f"preset {name}: generated {self.cat.n_items} items in {time.time() - t:.1f}s")
        cfg = self.cat.cfg
        self.cfg, self.W, self.h = cfg, cfg["sig_words"], cfg["n_hashes"]
        t = time.time()
        sigs = svt.svt_bloom_sign(self.cat.tokens, self.h, self.W)
        self.sigs = oracle.Oracle().signatures(self.cat.tokens, self.h, self.W)
        assert np.array_equal(sigs, self.sigs), "library and oracle Bloom signatures differ"
        say(f"preset {name}: signatures agree ({time.time() - t:.1f}s)")
        t = time.time()
        self.ix = svt.Index(self.cat.items, sigs, self.cat.list_of, self.cat.centroids, self.cat.item_scale)
        del sigs
        self.cat.tokens = None
        say(f"preset {name}: uploaded in {time.time() - t:.1f}s")
        self.svt = svt

    def batch(self, B, offset):
        qs = synth.queries(self.cat, B, offset)
        masks = np.stack([self.svt.svt_bloom_mask(qs.required(b), self.h, self.W) for b in range(B)])
        o_masks = oracle.Oracle().masks(qs, self.h, self.W)
        assert np.array_equal(masks, o_masks)
        return qs.queries, masks

    def check(self, B, offset, sample=None, nprobe=None, k=None, label=""):
        nprobe = nprobe or self.cfg["nprobe"]
        k = k or self.cfg["k"]
        q, masks = self.batch(B, offset)
        t = time.time()
        got = gpu_search(self.ix, q, masks, nprobe, k)
        say(f"{label}: B={B} gpu search {1e3 * (time.time() - t):.1f} ms (incl. copies); "
            f"eligible/query median {int(np.median(got[4][:, 1]))}")
        rows = np.arange(B) if sample is None else np.asarray(sample)
        t = time.time()
        ref = oracle.Oracle().search(self.cat.items, self.sigs, self.cat.list_of, self.cat.centroids,
                                     self.cat.item_scale, q[rows], masks[rows], nprobe, k, n_threads=16)
        say(f"{label}: oracle on {len(rows)} queries {time.time() - t:.1f}s")
        compare(tuple(a[rows] for a in got), ref, k, label)
        check_invariants(self.cat.items, self.sigs, self.cat.list_of, got, masks, q, k)
        return got

    def close(self):
        self.ix.close()


@pytest.fixture(scope="module")
def p1m(svt):
    p = Preset(svt, "1m")
    yield p
    p.close()


@pytest.fixture(scope="module")
def p10m(svt):
    p = Preset(svt, "10m")
    yield p
    p.close()


def test_1m_batch1(p1m):
    for off in range(0, 8):
        p1m.check(1, off, label=f"1m-b1-q{off}")


def test_1m_batch8(p1m):
    p1m.check(8, 100, label="1m-b8")


def test_10m_batch64(p10m):
    p10m.check(64, 0, label="10m-b64")


def test_10m_batch64_other(p10m):
    p10m.check(64, 5000, label="10m-b64-2")


def test_10m_batch64_query_path(p10m, monkeypatch):
    """Batches of this size are grouped by default; the query-by-query path at full size too."""
    monkeypatch.setenv("SVT_PATH", "query")
    p10m.check(64, 10_000, label="10m-b64-query-path")
