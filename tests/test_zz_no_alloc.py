"""svt_search_noalloc (workspace in the library's static device scratch) against svt_search with a
workspace of the caller's: two calls in a row on each path, the second with a smaller batch, must give
the same ids, scores, counts, statistics and float scores bit for bit; and a search too large for the
scratch is rejected before anything is enqueued."""
import ctypes

import numpy as np
import pytest

import oracle_pins as P
from gpu_common import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available()
    torch.cuda.set_device(0)
    from int8_ivf_ann_amd import svt
    rng = np.random.default_rng(77)
    items, sigs, cl, cent = P.small_catalogue(rng, n=60000, d=64, nlist=48, W=2)
    ix = svt.Index(items, sigs, cl, cent, 3.0)
    yield svt, ix, rng
    ix.close()


def _inputs(rng, B, d=64, W=2):
    import torch
    q = torch.from_numpy(rng.integers(-127, 128, (B, d)).astype(np.int8)).cuda()
    m = torch.from_numpy(P.random_masks(rng, B, W, nbits_max=2).view(np.int64)).cuda()
    qs = torch.from_numpy(rng.uniform(0.5, 4.0, B).astype(np.float32)).cuda()
    return q, m, qs


def _host(outs):
    return [t.cpu().numpy() for t in outs]


# (path, nprobe, k, first batch, second batch); nprobe == nlist takes the exhaustive scan on the tile path
CASES = [
    ("query", 12, 300, 40, 9),
    ("tile", 12, 300, 40, 9),
    ("tile", 48, 200, 33, 5),
    ("auto", 7, 1024, 64, 1),
    ("query", 7, 2048, 3, 1),
]


@pytest.mark.parametrize("path,nprobe,k,b1,b2", CASES)
def test_noalloc_matches_search(env, path, nprobe, k, b1, b2):
    import torch
    svt, ix, rng = env
    opts = svt.make_options(path)
    for B in (b1, b2):
        say(f"noalloc path={path} nprobe={nprobe} k={k} B={B}")
        need = svt.svt_search_workspace_size(ix.handle, B, nprobe, k, opts)
        say(f"  workspace {need} bytes")
        assert need <= svt.SVT_NOALLOC_SCRATCH_BYTES, need
        q, m, qs = _inputs(rng, B)
        ref = ix.search(q, m, nprobe, k, query_scales=qs, opts=opts)
        # outputs start from garbage so that every element is known to be written
        outs = [torch.full_like(t, 5) for t in ref]
        got = svt.svt_search_noalloc(ix.handle, q, m, nprobe, k, query_scales=qs, opts=opts,
                                     out_ids=outs[0], out_scores=outs[1], out_fscores=outs[2],
                                     out_counts=outs[3], out_stats=outs[4])
        torch.cuda.synchronize()
        r, g = _host(ref), _host(got)
        for name, a, b in zip(("ids", "scores", "fscores", "counts", "stats"), r, g):
            assert a.shape == b.shape, name
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{name} differ (B={B})"
        assert int(r[3].sum()) > 0


def test_noalloc_rejects_oversized_search(env):
    import torch
    svt, ix, rng = env
    B, nprobe, k = 8192, 8, 2048
    need = svt.svt_search_workspace_size(ix.handle, B, nprobe, k, None)
    assert need > svt.SVT_NOALLOC_SCRATCH_BYTES
    q, m, _ = _inputs(rng, B)
    ids = torch.full((B, k), 7, dtype=torch.int64, device="cuda")
    sc = torch.full((B, k), 7, dtype=torch.int32, device="cuda")
    L = svt.lib()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = L.svt_search_noalloc(ix.handle, B, p(q), p(m), None, nprobe, k, p(ids), p(sc), None, None, None, None,
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == svt.SVT_EINVAL
    assert "static scratch" in svt.svt_last_error()
    torch.cuda.synchronize()
    assert bool((ids == 7).all()) and bool((sc == 7).all())
