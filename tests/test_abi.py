"""C-ABI library: loads, exports every declared symbol, host-only helpers and argument checks
(no GPU work)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from int8_ivf_ann_amd import svt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(svt.LIB_PATH):
        from int8_ivf_ann_amd import build
        build.build()
    return svt.lib()


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "svt.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(svt_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = declared_symbols()
    assert len(names) >= 10
    assert sorted(svt.EXPORTED) == names
    for n in names:
        assert hasattr(L, n), n


def test_library_is_gfx950_only():
    # the shared object carries a gfx950 code object and no other GPU target
    blob = open(svt.LIB_PATH, "rb").read()
    assert b"gfx950" in blob
    for other in (b"gfx90a", b"gfx942", b"gfx1100"):
        assert other not in blob


def test_bloom_helpers_match_oracle(L):
    orc = oracle.Oracle()
    rng = np.random.default_rng(0)
    toks = rng.integers(1, 2**63, size=(5000, 5), dtype=np.uint64)
    for W, h in ((1, 2), (2, 3), (2, 1), (1, 5)):
        assert np.array_equal(svt.svt_bloom_sign(toks, h, W), orc.signatures(toks, h, W))
        for n in (0, 1, 3):
            assert np.array_equal(svt.svt_bloom_mask(toks[0, :n], h, W), orc.mask(toks[0, :n], h, W))


def test_bloom_mask_argument_errors(L):
    out = np.zeros(2, np.uint64)
    assert L.svt_bloom_mask(None, 1, 2, 1, out.ctypes.data) == svt.SVT_EINVAL
    assert L.svt_bloom_mask(None, 0, 0, 1, out.ctypes.data) == svt.SVT_EINVAL
    assert L.svt_bloom_mask(None, 0, 2, 3, out.ctypes.data) == svt.SVT_EUNSUPPORTED
    assert svt.svt_last_error()


def test_upload_argument_errors(L):
    h = ctypes.c_void_p()
    assert L.svt_index_upload(None, None, ctypes.byref(h)) == svt.SVT_EINVAL
    d = svt.svt_index_desc()
    d.n_items, d.dim, d.sig_words, d.nlist, d.item_scale = 10, 24, 1, 4, 1.0
    assert L.svt_index_upload(ctypes.byref(d), None, ctypes.byref(h)) == svt.SVT_EUNSUPPORTED
    d.dim, d.sig_words = 64, 3
    assert L.svt_index_upload(ctypes.byref(d), None, ctypes.byref(h)) == svt.SVT_EUNSUPPORTED
    d.sig_words, d.nlist = 1, 0
    assert L.svt_index_upload(ctypes.byref(d), None, ctypes.byref(h)) == svt.SVT_EINVAL
    d.nlist = 4
    assert L.svt_index_upload(ctypes.byref(d), None, ctypes.byref(h)) == svt.SVT_EINVAL  # NULL arrays
    assert "NULL" in svt.svt_last_error()


def test_search_rejects_dead_index(L):
    bogus = ctypes.c_void_p(0x1000)
    assert L.svt_search(bogus, 1, None, None, None, 1, 1, None, None, None, None, None, None, 0, None) == svt.SVT_ESTATE
    assert L.svt_search_workspace_size(bogus, 1, 1, 1) == 0
    assert L.svt_index_free(bogus) == svt.SVT_ESTATE
    assert L.svt_index_free(None) == svt.SVT_OK


def test_profile_modes(L):
    # 0 off, 1 every stage, 2 the scan stage only; anything else is rejected
    for mode in (0, 1, 2, 0):
        assert L.svt_profile_enable(mode) == svt.SVT_OK
    assert L.svt_profile_enable(3) == svt.SVT_EINVAL
    assert L.svt_profile_enable(-1) == svt.SVT_EINVAL
    assert L.svt_profile_enable(0) == svt.SVT_OK
    stages, n = svt.svt_profile_read()
    assert n == 0 and list(stages) == ["coarse", "select", "plan", "scan", "fallback", "merge"]
