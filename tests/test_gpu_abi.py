"""C-ABI contract on a live index (GPU): every argument error of svt_search and
svt_search_workspace_size is rejected with its documented code before anything is enqueued, and the
caller's outputs are left byte-for-byte as they were."""
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
    rng = np.random.default_rng(21)
    items, sigs, cl, cent = P.small_catalogue(rng, n=5000, d=32, nlist=8, W=2)
    ix = svt.Index(items, sigs, cl, cent, 1.0)
    B, k = 3, 16
    q = torch.from_numpy(rng.integers(-127, 128, (B, 32)).astype(np.int8)).cuda()
    m = torch.zeros((B, 2), dtype=torch.int64, device="cuda")
    outs = dict(ids=torch.full((B, k), 7, dtype=torch.int64, device="cuda"),
                sc=torch.full((B, k), 7, dtype=torch.int32, device="cuda"),
                fs=torch.full((B, k), 7.0, dtype=torch.float32, device="cuda"),
                cnt=torch.full((B,), 7, dtype=torch.int32, device="cuda"),
                st=torch.full((B, 2), 7, dtype=torch.int64, device="cuda"))
    ws = torch.empty((64 << 20,), dtype=torch.uint8, device="cuda")
    yield svt, ix, q, m, outs, ws, B, k
    ix.close()


def _call(svt, ix, q, m, outs, ws, B, nprobe, k, opts=None, ws_bytes=None, ws_off=0, qp=None, off=None, qs=None):
    """off: byte offsets added to output pointers by name (misaligned outputs)."""
    L = svt.lib()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    po = lambda name: ctypes.c_void_p(outs[name].data_ptr() + (off or {}).get(name, 0))
    optp = None if opts is None else ctypes.byref(opts)
    return L.svt_search(ix.handle, B, qp if qp is not None else p(q), p(m), qs, nprobe, k, po("ids"),
                        po("sc"), po("fs"), po("cnt"), po("st"), optp,
                        ctypes.c_void_p(ws.data_ptr() + ws_off),
                        ws.numel() - ws_off if ws_bytes is None else ws_bytes, None)


def _untouched(outs):
    import torch
    torch.cuda.synchronize()
    for name, t in outs.items():
        assert bool((t == 7).all()), f"{name} written on an error"


def test_search_argument_errors(env):
    svt, ix, q, m, outs, ws, B, k = env
    nlist = 8
    cases = [
        ("k = 0", dict(k=0), svt.SVT_EINVAL),
        ("k = SVT_MAX_K_LARGE + 1", dict(k=svt.SVT_MAX_K_LARGE + 1), svt.SVT_EINVAL),
        ("k = 2049 on the query path", dict(k=2049, opts=svt.make_options("query")), svt.SVT_EINVAL),
        ("k = 2049 on the tile path", dict(k=2049, opts=svt.make_options("tile")), svt.SVT_EINVAL),
        ("nprobe = 0", dict(nprobe=0), svt.SVT_EINVAL),
        ("nprobe = nlist + 1", dict(nprobe=nlist + 1), svt.SVT_EINVAL),
        ("n_queries < 0", dict(B=-1), svt.SVT_EINVAL),
        ("workspace too small", dict(ws_bytes=1024), svt.SVT_EINVAL),
        ("workspace misaligned", dict(ws_off=8), svt.SVT_EINVAL),
        ("queries misaligned", dict(qp=ctypes.c_void_p(q.data_ptr() + 1)), svt.SVT_EINVAL),
        ("NULL queries", dict(qp=ctypes.c_void_p(0)), svt.SVT_EINVAL),
        ("out_ids misaligned", dict(off={"ids": 4}), svt.SVT_EINVAL),
        ("out_scores misaligned", dict(off={"sc": 2}), svt.SVT_EINVAL),
        ("out_fscores misaligned", dict(off={"fs": 2}), svt.SVT_EINVAL),
        ("out_counts misaligned", dict(off={"cnt": 1}), svt.SVT_EINVAL),
        ("out_stats misaligned", dict(off={"st": 4}), svt.SVT_EINVAL),
        ("unknown path", dict(opts=svt.make_options(7)), svt.SVT_EINVAL),
        ("negative pool_keys", dict(opts=svt.make_options("tile", -1)), svt.SVT_EINVAL),
        ("unknown flag", dict(opts=svt.make_options("auto", 0, 8)), svt.SVT_EINVAL),
        ("mask_groups = 5", dict(opts=svt.make_options("auto", 0, 0, 5)), svt.SVT_EINVAL),
        ("mask_groups < 0", dict(opts=svt.make_options("tile", 0, 0, -1)), svt.SVT_EINVAL),
    ]
    o = svt.make_options()
    o.reserved[2] = 1
    cases.append(("reserved word", dict(opts=o), svt.SVT_EINVAL))
    for label, kw, code in cases:
        args = dict(B=B, nprobe=4, k=k)
        args.update(kw)
        rc = _call(svt, ix, q, m, outs, ws, args.pop("B"), args.pop("nprobe"), args.pop("k"), **args)
        say(f"{label}: rc {rc} ({svt.svt_last_error()})")
        assert rc == code, label
        assert svt.svt_last_error(), label
        _untouched(outs)


def test_workspace_size_errors(env):
    svt, ix, q, m, outs, ws, B, k = env
    L = svt.lib()
    for args in ((B, 0, k), (B, 9, k), (B, 4, 0), (B, 4, svt.SVT_MAX_K_LARGE + 1), (-1, 4, k), (70000, 4, k)):
        assert L.svt_search_workspace_size(ix.handle, *args, None) == 0, args
        assert svt.svt_last_error()
    assert L.svt_search_workspace_size(ix.handle, B, 4, k, ctypes.byref(svt.make_options(5))) == 0
    # the query path needs no pools: its workspace is smaller than the tile path's
    wq = L.svt_search_workspace_size(ix.handle, 64, 4, 2048, ctypes.byref(svt.make_options("query")))
    wt = L.svt_search_workspace_size(ix.handle, 64, 4, 2048, ctypes.byref(svt.make_options("tile")))
    assert 0 < wq < wt


def test_zero_queries_is_a_no_op(env):
    svt, ix, q, m, outs, ws, B, k = env
    assert _call(svt, ix, q, m, outs, ws, 0, 4, k) == svt.SVT_OK
    _untouched(outs)


def test_valid_call_after_errors(env):
    svt, ix, q, m, outs, ws, B, k = env
    assert _call(svt, ix, q, m, outs, ws, B, 4, k) == svt.SVT_OK
    import torch
    torch.cuda.synchronize()
    assert bool((outs["cnt"] >= 0).all())


def test_free_twice_is_rejected(env):
    svt = env[0]
    rng = np.random.default_rng(22)
    items, sigs, cl, cent = P.small_catalogue(rng, n=100, d=16, nlist=2, W=1)
    h = svt.svt_index_upload(items, sigs, cl, cent, 1.0)
    svt.svt_index_free(h)
    with pytest.raises(svt.SvtError):
        svt.svt_index_free(h)


def test_search_path(env):
    svt, ix, q, m, outs, ws, B, k = env
    nlist = ix.nlist
    assert svt.svt_search_path(ix.handle, 1, 4, k) == "query"
    assert svt.svt_search_path(ix.handle, 32, 4, k) == "query"
    assert svt.svt_search_path(ix.handle, 128, 4, k) == "tile"
    assert svt.svt_search_path(ix.handle, 32, 4, k, svt.make_options("query")) == "query"
    assert svt.svt_search_path(ix.handle, 3, 4, k, svt.make_options("tile")) == "tile"
    assert svt.svt_search_path(ix.handle, 2, nlist, k) == "exhaustive"
    assert svt.svt_search_path(ix.handle, 1, nlist, k, svt.make_options("tile")) == "exhaustive"
    assert svt.svt_search_path(ix.handle, 1, nlist, k) == "query"
    with pytest.raises(svt.SvtError):
        svt.svt_search_path(ix.handle, 1, nlist + 1, k)
