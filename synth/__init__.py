"""Seeded synthetic workloads (inputs only) shared by the CPU oracle and the GPU library.

The catalogue recipes stand in for the production data the SilverTorch pages measure on
("SilverTorch: Index as Model", compute-cost-efficiency section: an 80M-item retrieval workload
served with 64 probes and top-2048).  No production data exists here; each preset is a fixed
recipe (item count, dimension, cluster law, attribute laws, mask sizes) plus a seed.

This module holds none of the search arithmetic: it returns int8 vectors, cluster ids, attribute
token keys and the token keys each query requires.  Bloom signatures and masks are computed from
those keys by each side independently (the library's helper, the oracle's own code).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Dict, List, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")
MAX_ATTRS = 8


class _Params(ctypes.Structure):
    _fields_ = [
        ("seed", ctypes.c_uint64),
        ("n_items", ctypes.c_int64),
        ("dim", ctypes.c_int32),
        ("nlist", ctypes.c_int32),
        ("cluster_zipf", ctypes.c_double),
        ("noise", ctypes.c_double),
        ("n_attrs", ctypes.c_int32),
        ("attr_card", ctypes.c_int32 * MAX_ATTRS),
        ("attr_zipf", ctypes.c_double * MAX_ATTRS),
        ("attr_flag_p", ctypes.c_double * MAX_ATTRS),
        ("mask_min", ctypes.c_int32),
        ("mask_max", ctypes.c_int32),
        ("n_threads", ctypes.c_int32),
    ]


# attribute spec: (name, cardinality, zipf exponent or 0, flag probability or 0)
_ATTR_SMALL = [("language", 20, 1.1, 0.0), ("country", 50, 1.1, 0.0), ("policy", 2, 0.0, 0.9)]
_ATTR_LARGE = [("language", 50, 1.1, 0.0), ("country", 200, 1.1, 0.0), ("policy_a", 2, 0.0, 0.9),
               ("policy_b", 2, 0.0, 0.9), ("policy_c", 2, 0.0, 0.9)]

#: The five workload presets.  ``batches`` lists the query batch sizes the preset is used at.
CONFIGS: Dict[str, dict] = {
    "tiny": dict(index=0, n_items=20_000, dim=64, nlist=64, cluster_zipf=0.0, sig_words=1, n_hashes=2,
                 attrs=_ATTR_SMALL, mask=(1, 3), batches=(4,), nprobe=8, k=100),
    "1m": dict(index=1, n_items=1_000_000, dim=128, nlist=1024, cluster_zipf=0.0, sig_words=2, n_hashes=3,
               attrs=_ATTR_LARGE, mask=(1, 3), batches=(1,), nprobe=32, k=1024),
    "10m": dict(index=2, n_items=10_000_000, dim=128, nlist=4096, cluster_zipf=0.8, sig_words=2, n_hashes=3,
                attrs=_ATTR_LARGE, mask=(2, 4), batches=(64,), nprobe=64, k=2048),
    "80m": dict(index=3, n_items=80_000_000, dim=128, nlist=16384, cluster_zipf=0.8, sig_words=2, n_hashes=3,
                attrs=_ATTR_LARGE, mask=(2, 4), batches=(1, 32, 256), nprobe=64, k=2048),
    "exh": dict(index=4, n_items=80_000_000, dim=64, nlist=16384, cluster_zipf=0.8, sig_words=2, n_hashes=3,
                attrs=_ATTR_LARGE, mask=(2, 4), batches=(32,), nprobe=16384, k=2048),
}
SEED_BASE = 0x5EED0000
NOISE = 0.3


def _lib():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() or synth.build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(_Params)
    vp = ctypes.c_void_p
    lib.synth_centroids.argtypes = [P, vp, vp, vp]
    lib.synth_items_maxabs.argtypes = [P, vp]
    lib.synth_items_maxabs.restype = ctypes.c_double
    lib.synth_items.argtypes = [P, vp, ctypes.c_float, vp, vp, vp]
    lib.synth_queries.argtypes = [P, vp, ctypes.c_float, ctypes.c_int64, ctypes.c_int64, vp, vp, vp, vp, vp]
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_params(name: str, **over) -> Tuple[_Params, dict]:
    """Return the C parameter block and the resolved preset dict (``over`` overrides any key)."""
    cfg = dict(CONFIGS[name])
    cfg.update(over)
    p = _Params()
    p.seed = cfg.get("seed", SEED_BASE + cfg["index"])
    p.n_items = cfg["n_items"]
    p.dim = cfg["dim"]
    p.nlist = cfg["nlist"]
    p.cluster_zipf = cfg["cluster_zipf"]
    p.noise = cfg.get("noise", NOISE)
    attrs = cfg["attrs"]
    p.n_attrs = len(attrs)
    for a, (_, card, z, fp) in enumerate(attrs):
        p.attr_card[a] = card
        p.attr_zipf[a] = z
        p.attr_flag_p[a] = fp
    p.mask_min, p.mask_max = cfg["mask"]
    p.n_threads = cfg.get("n_threads", default_threads())
    if p.dim % 2:
        raise ValueError("dim must be even")
    return p, cfg


@dataclasses.dataclass
class Catalogue:
    name: str
    cfg: dict
    over: dict
    items: np.ndarray          # int8 [N, d]
    list_of: np.ndarray        # int32 [N]
    tokens: np.ndarray         # uint64 [N, n_attrs]
    centroids: np.ndarray      # int8 [nlist, d]
    centroid_scale: float
    item_scale: float
    cent_f: np.ndarray         # float32 [nlist, d] generating directions (query generation)

    @property
    def n_items(self) -> int:
        return int(self.items.shape[0])


@dataclasses.dataclass
class QuerySet:
    queries: np.ndarray        # int8 [B, d]
    cluster: np.ndarray        # int32 [B] generating cluster
    tokens: np.ndarray         # uint64 [B, n_attrs] the query's own attribute tokens
    n_req: np.ndarray          # int32 [B]
    req_tokens: np.ndarray     # uint64 [B, n_attrs], first n_req[b] entries are required

    def required(self, b: int) -> np.ndarray:
        return self.req_tokens[b, : int(self.n_req[b])]


def catalogue(name: str, **over) -> Catalogue:
    """Generate the item catalogue of preset ``name`` (two passes: global max, then quantise)."""
    lib = _lib()
    p, cfg = make_params(name, **over)
    d, nl, n = p.dim, p.nlist, p.n_items
    cent_f = np.empty((nl, d), np.float32)
    cent_q = np.empty((nl, d), np.int8)
    cs = np.zeros(1, np.float32)
    lib.synth_centroids(ctypes.byref(p), _ptr(cent_f), _ptr(cent_q), _ptr(cs))
    mx = lib.synth_items_maxabs(ctypes.byref(p), _ptr(cent_f))
    scale = np.float32(127.0 / mx)
    items = np.empty((n, d), np.int8)
    list_of = np.empty(n, np.int32)
    tokens = np.empty((n, p.n_attrs), np.uint64)
    lib.synth_items(ctypes.byref(p), _ptr(cent_f), ctypes.c_float(scale), _ptr(items), _ptr(list_of), _ptr(tokens))
    return Catalogue(name, cfg, dict(over), items, list_of, tokens, cent_q, float(cs[0]), float(scale), cent_f)


def queries(cat: Catalogue, n: int, offset: int = 0) -> QuerySet:
    """Queries ``offset .. offset+n-1`` of the preset (distinct offsets give distinct batches)."""
    lib = _lib()
    p, _ = make_params(cat.name, **cat.over)
    d, na = p.dim, p.n_attrs
    q = np.empty((n, d), np.int8)
    qc = np.empty(n, np.int32)
    qt = np.empty((n, na), np.uint64)
    nr = np.empty(n, np.int32)
    rt = np.zeros((n, na), np.uint64)
    if n:
        lib.synth_queries(ctypes.byref(p), _ptr(cat.cent_f), ctypes.c_float(cat.item_scale), offset, n,
                          _ptr(q), _ptr(qc), _ptr(qt), _ptr(nr), _ptr(rt))
    return QuerySet(q, qc, qt, nr, rt)


def rerank_net(rng: np.random.Generator, d: int, E: int, H: int, scale: float = 1.0) -> Dict[str, np.ndarray]:
    """Random float32 weights of the rerank's gated mixture of experts (gate_w [E, d], gate_b [E],
    w1 [E, H, d], b1 [E, H], w2 [E, H], b2 [E]): normal draws, fan-in scaled, small biases."""
    f = lambda *s: (rng.standard_normal(s) * scale).astype(np.float32)
    return {"gate_w": f(E, d) / np.float32(np.sqrt(d)), "gate_b": f(E), "w1": f(E, H, d) / np.float32(np.sqrt(d)),
            "b1": f(E, H) * np.float32(0.1), "w2": f(E, H) / np.float32(np.sqrt(H)), "b2": f(E) * np.float32(0.1)}
