"""CPU oracle for the fused int8 IVF + Bloom-signature top-k search.

TEST INFRASTRUCTURE ONLY: imported by the test suite, by ``__graft_entry__.smoke()`` and by the
benchmark's CPU-baseline leg, never by the GPU library.  It wraps ``svt_oracle.c`` (plain C, built
by ``oracle/build.py``), which shares no code with the GPU path.

Method followed (see ``svt_oracle.c`` for the step-by-step citations): coarse probe of the int8
centroids (top-nprobe by score, cluster id breaking ties), Bloom conjunctive eligibility test inside
the probed clusters, int8.int8 -> int32 scoring of the survivors, top-k by (score desc, id asc),
dequantisation in double rounded once to float.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_libs = {}


def load(path: Optional[str] = None):
    path = path or LIB_PATH
    if path in _libs:
        return _libs[path]
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() or oracle.build.build()")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.oracle_splitmix64_next.argtypes = [vp]
    lib.oracle_splitmix64_next.restype = ctypes.c_uint64
    lib.oracle_token_bits.argtypes = [ctypes.c_uint64, i32, i32, vp]
    lib.oracle_signatures.argtypes = [vp, i64, i32, i32, i32, vp]
    lib.oracle_mask.argtypes = [vp, i32, i32, i32, vp]
    lib.oracle_coarse.argtypes = [vp, i32, i32, vp, i32, vp, vp]
    lib.oracle_dequant.argtypes = [i32, ctypes.c_float, ctypes.c_float]
    lib.oracle_dequant.restype = ctypes.c_float
    lib.oracle_search_groups.argtypes = [vp, vp, vp, i64, i32, i32, vp, i32, ctypes.c_float, i32, vp, vp, i32, vp,
                                         i32, i32, vp, vp, vp, vp, vp, i32]
    lib.oracle_search_groups.restype = i32
    lib.oracle_search.argtypes = [vp, vp, vp, i64, i32, i32, vp, i32, ctypes.c_float, i32, vp, vp, vp,
                                  i32, i32, vp, vp, vp, vp, vp, i32]
    lib.oracle_search.restype = ctypes.c_int
    _libs[path] = lib
    return lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


class Oracle:
    """Thin ctypes wrapper; ``path`` selects an alternative build (planted-mistake tests)."""

    def __init__(self, path: Optional[str] = None):
        self.lib = load(path)

    def splitmix64(self, state: int, n: int) -> Tuple[np.ndarray, int]:
        st = np.array([state], np.uint64)
        out = np.array([self.lib.oracle_splitmix64_next(_p(st)) for _ in range(n)], np.uint64)
        return out, int(st[0])

    def signatures(self, tokens: np.ndarray, n_hashes: int, sig_words: int) -> np.ndarray:
        tokens = np.ascontiguousarray(tokens, np.uint64)
        n, t = tokens.shape
        out = np.empty((n, sig_words), np.uint64)
        self.lib.oracle_signatures(_p(tokens), n, t, n_hashes, sig_words, _p(out))
        return out

    def mask(self, req_tokens: np.ndarray, n_hashes: int, sig_words: int) -> np.ndarray:
        req = np.ascontiguousarray(req_tokens, np.uint64)
        out = np.empty(sig_words, np.uint64)
        self.lib.oracle_mask(_p(req), len(req), n_hashes, sig_words, _p(out))
        return out

    def masks(self, qs, n_hashes: int, sig_words: int) -> np.ndarray:
        return np.stack([self.mask(qs.required(b), n_hashes, sig_words) for b in range(len(qs.n_req))]) \
            if len(qs.n_req) else np.zeros((0, sig_words), np.uint64)

    def coarse(self, centroids: np.ndarray, q: np.ndarray, nprobe: int) -> Tuple[np.ndarray, np.ndarray]:
        centroids = np.ascontiguousarray(centroids, np.int8)
        q = np.ascontiguousarray(q, np.int8)
        nlist, d = centroids.shape
        probes = np.empty(nprobe, np.int32)
        scores = np.empty(nlist, np.int32)
        self.lib.oracle_coarse(_p(centroids), nlist, d, _p(q), nprobe, _p(probes), _p(scores))
        return probes, scores

    def dequant(self, score: int, item_scale: float, query_scale: float) -> float:
        return float(self.lib.oracle_dequant(int(score), item_scale, query_scale))

    def search(self, items, sigs, list_of, centroids, item_scale, queries, masks, nprobe, k,
               query_scales=None, n_threads: int = 1):
        """Returns (ids int64 [B,k], scores int32 [B,k], fscores f32 [B,k], counts int32 [B],
        stats int64 [B,2] = (items scanned in probed clusters, eligible items scored)).  masks is
        [B, W], or [B, G, W] for requests of G masks (an item is eligible when it passes any)."""
        items = np.ascontiguousarray(items, np.int8)
        sigs = np.ascontiguousarray(sigs, np.uint64)
        list_of = np.ascontiguousarray(list_of, np.int32)
        centroids = np.ascontiguousarray(centroids, np.int8)
        queries = np.ascontiguousarray(queries, np.int8)
        masks = np.ascontiguousarray(masks, np.uint64)
        n, d = items.shape
        w = sigs.shape[1]
        nlist = centroids.shape[0]
        b = queries.shape[0]
        qs = None if query_scales is None else np.ascontiguousarray(query_scales, np.float32)
        ids = np.empty((b, k), np.int64)
        sc = np.empty((b, k), np.int32)
        fs = np.empty((b, k), np.float32)
        cnt = np.empty(b, np.int32)
        st = np.empty((b, 2), np.int64)
        if masks.ndim == 3:
            rc = self.lib.oracle_search_groups(_p(items), _p(sigs), _p(list_of), n, d, w, _p(centroids), nlist,
                                               ctypes.c_float(item_scale), b, _p(queries), _p(masks), masks.shape[1],
                                               _p(qs), nprobe, k, _p(ids), _p(sc), _p(fs), _p(cnt), _p(st), n_threads)
        else:
            rc = self.lib.oracle_search(_p(items), _p(sigs), _p(list_of), n, d, w, _p(centroids), nlist,
                                        ctypes.c_float(item_scale), b, _p(queries), _p(masks), _p(qs), nprobe, k,
                                        _p(ids), _p(sc), _p(fs), _p(cnt), _p(st), n_threads)
        if rc != 0:
            raise ValueError("oracle_search: invalid arguments")
        return ids, sc, fs, cnt, st
