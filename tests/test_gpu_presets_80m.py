"""The 80M-item IVF preset (d = 128, nlist 16384, nprobe 64, top-2048) at full size, in the launch
configuration the benchmark times: every query of every batch compared with the oracle, on both search
paths, plus the size-independent invariants.  Also at full size: top-16384 on the large-k path (every
query, with pools and with the digit passes), and the benchmark's rerank of 256 queries' top-2048
(32 sampled queries against the float64 oracle)."""
import numpy as np
import pytest

import synth
from gpu_common import say

from test_gpu_presets import Preset, svt  # noqa: F401  (module fixture)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def p80(svt):  # noqa: F811
    p = Preset(svt, "80m")
    yield p
    p.close()


def test_80m_batch256(p80):
    p80.check(256, 0, label="80m-b256")


def test_80m_batch32(p80):
    p80.check(32, 20_000, label="80m-b32")


def test_80m_batch1(p80):
    for off in (40_000, 40_001, 40_002):
        p80.check(1, off, label=f"80m-b1-{off}")


def test_80m_batch4(p80):
    p80.check(4, 50_000, label="80m-b4")


def test_80m_batch32_top16384(p80):
    for flags, what in ((0, "pools"), (2, "passes")):
        p80.check(32, 60_000, k=16384, label=f"80m-b32-k16384-{what}", paths=("auto",), flags=flags)


def test_80m_rerank_of_batch256(p80):
    """The benchmark's rerank leg: the search's top-2048 of batch 0 as candidates, the benchmark's seeded
    4 x 16 net, keep 256."""
    import torch
    from test_gpu_rerank import check as rerank_check
    B, k, k_out = 256, p80.cfg["k"], 256
    q, masks = p80.batch(B, 0)
    q_d = torch.from_numpy(np.ascontiguousarray(q)).cuda()
    m_d = torch.from_numpy(masks.view(np.int64)).cuda()
    ids = p80.ix.search(q_d, m_d, p80.cfg["nprobe"], k)[0]
    net = synth.rerank_net(np.random.default_rng(2024), q.shape[1], 4, 16)
    tnet = {key: torch.from_numpy(v).cuda() for key, v in net.items()}
    r_ids, r_sc, r_cnt = p80.ix.rerank(q_d, ids, tnet, k_out)
    torch.cuda.synchronize()
    sample = np.arange(0, B, 8)
    cand = ids.cpu().numpy()[sample]
    got = (r_ids.cpu().numpy()[sample], r_sc.cpu().numpy()[sample], r_cnt.cpu().numpy()[sample])
    say(f"80m rerank: {int((cand >= 0).sum())} candidates of {len(sample)} sampled queries")
    rerank_check(p80.cat.items, p80.cat.item_scale, q[sample], None, cand, net, k_out, got, "80m rerank")


def test_80m_batch256_top16384(p80):
    p80.check(256, 0, k=16384, label="80m-b256-k16384", paths=("auto",))
