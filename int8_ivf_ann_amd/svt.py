"""ctypes binding of the C ABI in include/svt.h (argument marshalling only).

Every step of the search runs in the gfx950 kernels of libsvt.so; this module only converts Python
and torch objects into pointers and sizes.  PyTorch provides device memory and streams.  There is no
fallback: if libsvt.so is missing or fails to load, every entry point raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsvt.so")

SVT_OK, SVT_EINVAL, SVT_ENOMEM, SVT_EDEVICE, SVT_EUNSUPPORTED, SVT_ESTATE, SVT_ENOSPACE = 0, -1, -2, -3, -4, -5, -6
SVT_MAX_K = 2048
SVT_MAX_K_LARGE = 16384
SVT_MAX_SIG_WORDS = 2
SVT_PATH_AUTO, SVT_PATH_QUERY, SVT_PATH_TILE, SVT_PATH_EXHAUSTIVE, SVT_PATH_LARGE_K = 0, 1, 2, 3, 4
SVT_OPT_MERGE_FROM_SLOTS, SVT_OPT_FORCE_REDO = 1, 2
SVT_MAX_MASK_GROUPS = 4
SVT_NOALLOC_SCRATCH_BYTES = 256 << 20
SVT_RERANK_MAX_EXPERTS, SVT_RERANK_MAX_UNITS, SVT_RERANK_MAX_CAND, SVT_RERANK_MAX_OUT = 8, 64, 4096, 2048
_PATHS = {"auto": SVT_PATH_AUTO, "query": SVT_PATH_QUERY, "tile": SVT_PATH_TILE, "large_k": SVT_PATH_LARGE_K}

#: every symbol include/svt.h declares
EXPORTED = ("svt_index_upload", "svt_index_upload_updatable", "svt_index_insert", "svt_index_delete",
            "svt_index_resign", "svt_index_free", "svt_index_info", "svt_search_workspace_size", "svt_search_path",
            "svt_search", "svt_search_noalloc", "svt_rerank", "svt_last_error", "svt_bloom_mask", "svt_bloom_sign", "svt_profile_enable", "svt_profile_read")


class SvtError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"svt error {code}: {msg}")
        self.code = code


class svt_index_desc(ctypes.Structure):
    _fields_ = [
        ("n_items", ctypes.c_int64),
        ("dim", ctypes.c_int32),
        ("sig_words", ctypes.c_int32),
        ("nlist", ctypes.c_int32),
        ("items", ctypes.c_void_p),
        ("sigs", ctypes.c_void_p),
        ("list_of", ctypes.c_void_p),
        ("centroids", ctypes.c_void_p),
        ("item_scale", ctypes.c_float),
    ]


class svt_search_options(ctypes.Structure):
    _fields_ = [
        ("path", ctypes.c_int32),
        ("pool_keys", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("mask_groups", ctypes.c_int32),
        ("reserved", ctypes.c_int32 * 4),
    ]


class svt_rerank_net(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int32), ("hidden", ctypes.c_int32), ("gate_w", ctypes.c_void_p),
                ("gate_b", ctypes.c_void_p), ("w1", ctypes.c_void_p), ("b1", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("b2", ctypes.c_void_p)]


def make_options(path="auto", pool_keys: int = 0, flags: int = 0, mask_groups: int = 0) -> svt_search_options:
    """Search options: path "auto" | "query" | "tile" | "large_k" (or an SVT_PATH_* value), pool_keys (tile path,
    0 = default), flags (OR of SVT_OPT_*), mask_groups (masks per query, 0 or 1: one)."""
    o = svt_search_options()
    o.path = _PATHS[path] if isinstance(path, str) else int(path)
    o.pool_keys = int(pool_keys)
    o.flags = int(flags)
    o.mask_groups = int(mask_groups)
    return o


def _with_groups(opts, G: int):
    """The options to pass for masks of G groups (a copy with mask_groups set; G must agree with it)."""
    if opts is None:
        return make_options(mask_groups=G) if G > 1 else None
    have = max(1, int(opts.mask_groups))
    if have != G:
        raise ValueError(f"masks carry {G} groups per query but the options say mask_groups={opts.mask_groups}")
    return opts


_lib = None


def lib():
    """Load libsvt.so (raises if it is not built: there is no CPU path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.svt_index_upload.argtypes = [ctypes.POINTER(svt_index_desc), vp, ctypes.POINTER(vp)]
    L.svt_index_upload_updatable.argtypes = [ctypes.POINTER(svt_index_desc), i64, i32, ctypes.c_float, vp,
                                             ctypes.POINTER(vp)]
    L.svt_index_insert.argtypes = [vp, i32, vp, vp, vp, vp, vp]
    L.svt_index_delete.argtypes = [vp, i32, vp, vp]
    L.svt_index_resign.argtypes = [vp, i32, vp, vp, vp]
    L.svt_index_free.argtypes = [vp, vp]
    L.svt_index_info.argtypes = [vp, vp, vp, vp, vp]
    L.svt_search_workspace_size.argtypes = [vp, i32, i32, i32, vp]
    L.svt_search_workspace_size.restype = sz
    L.svt_search_path.argtypes = [vp, i32, i32, i32, vp]
    L.svt_search.argtypes = [vp, i32, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.svt_search_noalloc.argtypes = [vp, i32, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    L.svt_rerank.argtypes = [vp, i32, vp, vp, i32, vp, ctypes.POINTER(svt_rerank_net), i32, vp, vp, vp, vp]
    L.svt_last_error.restype = ctypes.c_char_p
    L.svt_bloom_mask.argtypes = [vp, i32, i32, i32, vp]
    L.svt_bloom_sign.argtypes = [vp, i64, i32, i32, i32, vp, i32]
    L.svt_profile_enable.argtypes = [ctypes.c_int]
    L.svt_profile_read.argtypes = [vp, vp, i32, vp, vp]
    for name in EXPORTED:
        if name not in ("svt_search_workspace_size", "svt_last_error"):
            getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def svt_last_error() -> str:
    return lib().svt_last_error().decode()


def _check(rc: int) -> None:
    if rc != SVT_OK:
        raise SvtError(rc, svt_last_error())


def _np_ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _t_ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _opt_ptr(opts):
    return None if opts is None else ctypes.byref(opts)


def _check_tensor(name, t, dtypes, shape, device=None, nullable=False):
    """The C side cannot see dtypes, shapes or strides: a wrong tensor would be read or written out of
    bounds on the device.  Raise ValueError unless t is a contiguous tensor of one of ``dtypes`` with
    exactly ``shape``, on ``device`` (when given)."""
    if t is None:
        if nullable:
            return
        raise ValueError(f"{name}: required")
    if not hasattr(t, "data_ptr") or not hasattr(t, "dtype"):
        raise ValueError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not in {[str(d) for d in dtypes]}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: not contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_cuda:
        raise ValueError(f"{name}: not a device tensor")


# ------------------------------------------------------------------------------------------------
def svt_bloom_mask(token_keys: Sequence[int], n_hashes: int, sig_words: int) -> np.ndarray:
    keys = np.ascontiguousarray(np.asarray(token_keys, dtype=np.uint64))
    out = np.zeros(sig_words, np.uint64)
    _check(lib().svt_bloom_mask(_np_ptr(keys) if keys.size else None, int(keys.size), n_hashes, sig_words,
                                _np_ptr(out)))
    return out


def svt_bloom_sign(token_keys: np.ndarray, n_hashes: int, sig_words: int, n_threads: int = 0) -> np.ndarray:
    keys = np.ascontiguousarray(token_keys, dtype=np.uint64)
    n, t = keys.shape
    out = np.empty((n, sig_words), np.uint64)
    _check(lib().svt_bloom_sign(_np_ptr(keys), n, t, n_hashes, sig_words, _np_ptr(out), n_threads))
    return out


def _desc(items, sigs, list_of, centroids, item_scale):
    items = np.ascontiguousarray(items, np.int8)
    sigs = np.ascontiguousarray(sigs, np.uint64)
    list_of = np.ascontiguousarray(list_of, np.int32)
    centroids = np.ascontiguousarray(centroids, np.int8)
    d = svt_index_desc()
    d.n_items = items.shape[0]
    d.dim = items.shape[1] if items.ndim == 2 else centroids.shape[1]
    d.sig_words = sigs.shape[1] if sigs.ndim == 2 else 1
    d.nlist = centroids.shape[0]
    d.items, d.sigs, d.list_of, d.centroids = (_np_ptr(items), _np_ptr(sigs), _np_ptr(list_of), _np_ptr(centroids))
    d.item_scale = float(item_scale)
    return d, (items, sigs, list_of, centroids)   # the arrays stay alive while d is used


def svt_index_upload(items: np.ndarray, sigs: np.ndarray, list_of: np.ndarray, centroids: np.ndarray,
                     item_scale: float, stream=None) -> ctypes.c_void_p:
    """Host arrays -> device index handle (the current torch device)."""
    d, keep = _desc(items, sigs, list_of, centroids, item_scale)
    h = ctypes.c_void_p()
    _check(lib().svt_index_upload(ctypes.byref(d), _stream_ptr(stream), ctypes.byref(h)))
    return h


def svt_index_upload_updatable(items, sigs, list_of, centroids, item_scale: float, id_capacity: int,
                               slack_min: int = 0, slack_frac: float = 0.0, stream=None) -> ctypes.c_void_p:
    """Host arrays -> an index that takes in-place inserts, deletes and re-signs (free slots per cluster:
    max(slack_min, ceil(slack_frac * size)); later ids in [0, id_capacity))."""
    d, keep = _desc(items, sigs, list_of, centroids, item_scale)
    h = ctypes.c_void_p()
    _check(lib().svt_index_upload_updatable(ctypes.byref(d), int(id_capacity), int(slack_min), float(slack_frac),
                                            _stream_ptr(stream), ctypes.byref(h)))
    return h


def _ids(ids):
    return np.ascontiguousarray(ids, np.int64).reshape(-1)


def svt_index_insert(handle, ids, rows, sigs, list_of, stream=None) -> None:
    """Insert items (host arrays: ids [n], rows [n, dim] int8, sigs [n, W] uint64, list_of [n])."""
    ids = _ids(ids)
    n = ids.shape[0]
    _, dim, W, _ = svt_index_info(handle)
    rows = np.ascontiguousarray(rows, np.int8).reshape(n, dim)
    sigs = np.ascontiguousarray(sigs, np.uint64).reshape(n, W)
    list_of = np.ascontiguousarray(list_of, np.int32).reshape(n)
    _check(lib().svt_index_insert(handle, n, _np_ptr(ids), _np_ptr(rows), _np_ptr(sigs), _np_ptr(list_of),
                                  _stream_ptr(stream)))


def svt_index_delete(handle, ids, stream=None) -> None:
    ids = _ids(ids)
    _check(lib().svt_index_delete(handle, ids.shape[0], _np_ptr(ids), _stream_ptr(stream)))


def svt_index_resign(handle, ids, sigs, stream=None) -> None:
    ids = _ids(ids)
    n = ids.shape[0]
    _, _, W, _ = svt_index_info(handle)
    sigs = np.ascontiguousarray(sigs, np.uint64).reshape(n, W)
    _check(lib().svt_index_resign(handle, n, _np_ptr(ids), _np_ptr(sigs), _stream_ptr(stream)))


def svt_index_free(handle, stream=None) -> None:
    """Free an index after synchronising ``stream`` (the stream its searches ran on)."""
    _check(lib().svt_index_free(handle, _stream_ptr(stream)))


def svt_index_info(handle) -> Tuple[int, int, int, int]:
    n = ctypes.c_int64()
    d, w, nl = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().svt_index_info(handle, ctypes.byref(n), ctypes.byref(d), ctypes.byref(w), ctypes.byref(nl)))
    return n.value, d.value, w.value, nl.value


def svt_search_workspace_size(handle, n_queries: int, nprobe: int, k: int, opts=None) -> int:
    sz = lib().svt_search_workspace_size(handle, n_queries, nprobe, k, _opt_ptr(opts))
    if sz == 0:
        err = svt_last_error()
        if err:
            raise SvtError(SVT_EINVAL, err)
    return int(sz)


def svt_search_path(handle, n_queries: int, nprobe: int, k: int, opts=None) -> str:
    """The path a search of these sizes takes: "query", "tile" or "exhaustive"."""
    rc = lib().svt_search_path(handle, n_queries, nprobe, k, _opt_ptr(opts))
    if rc < 0:
        raise SvtError(rc, svt_last_error())
    return {SVT_PATH_QUERY: "query", SVT_PATH_TILE: "tile", SVT_PATH_EXHAUSTIVE: "exhaustive",
            SVT_PATH_LARGE_K: "large_k"}[rc]


def _search_tensors(handle, queries, masks, k, query_scales, out_ids, out_scores, out_fscores, out_counts,
                    out_stats):
    """Checks the search tensors and allocates the outputs not passed in; returns (B, dev, outputs)."""
    import torch
    n, dim, W, _ = svt_index_info(handle)
    if not hasattr(queries, "shape") or len(queries.shape) != 2:
        raise ValueError("queries: expected a 2-D tensor [B, dim]")
    B = int(queries.shape[0])
    dev = queries.device
    _check_tensor("queries", queries, (torch.int8,), (B, dim))
    if not hasattr(masks, "shape") or len(masks.shape) not in (2, 3):
        raise ValueError("masks: expected a tensor [B, W] or [B, G, W]")
    G = int(masks.shape[1]) if len(masks.shape) == 3 else 1
    if not 1 <= G <= SVT_MAX_MASK_GROUPS:
        raise ValueError(f"masks: {G} groups per query, at most {SVT_MAX_MASK_GROUPS}")
    _check_tensor("masks", masks, (torch.int64, torch.uint64), (B, G, W) if len(masks.shape) == 3 else (B, W), dev)
    _check_tensor("query_scales", query_scales, (torch.float32,), (B,), dev, nullable=True)
    if out_ids is None:
        out_ids = torch.empty((B, k), dtype=torch.int64, device=dev)
    if out_scores is None:
        out_scores = torch.empty((B, k), dtype=torch.int32, device=dev)
    if out_fscores is None:
        out_fscores = torch.empty((B, k), dtype=torch.float32, device=dev)
    if out_counts is None:
        out_counts = torch.empty((B,), dtype=torch.int32, device=dev)
    if out_stats is None:
        out_stats = torch.empty((B, 2), dtype=torch.int64, device=dev)
    _check_tensor("out_ids", out_ids, (torch.int64,), (B, k), dev)
    _check_tensor("out_scores", out_scores, (torch.int32,), (B, k), dev)
    _check_tensor("out_fscores", out_fscores, (torch.float32,), (B, k), dev)
    _check_tensor("out_counts", out_counts, (torch.int32,), (B,), dev)
    _check_tensor("out_stats", out_stats, (torch.int64,), (B, 2), dev)
    return B, dev, G, (out_ids, out_scores, out_fscores, out_counts, out_stats)


def svt_search(handle, queries, masks, nprobe: int, k: int, query_scales=None, out_ids=None, out_scores=None,
               out_fscores=None, out_counts=None, out_stats=None, workspace=None, stream=None, opts=None):
    """queries: int8 [B, d] cuda tensor; masks: uint64 (or int64) [B, W] cuda tensor.
    Returns (ids int64 [B,k], scores int32 [B,k], fscores f32 [B,k], counts int32 [B], stats int64 [B,2]);
    outputs are allocated with torch unless passed in.  Asynchronous on ``stream``.  ``opts``: a
    svt_search_options (see make_options) or None."""
    import torch
    B, dev, G, outs = _search_tensors(handle, queries, masks, k, query_scales, out_ids, out_scores, out_fscores,
                                      out_counts, out_stats)
    opts = _with_groups(opts, G)
    if workspace is None:
        nbytes = svt_search_workspace_size(handle, B, nprobe, k, opts) if B > 0 else 0
        workspace = torch.empty((max(nbytes, 256),), dtype=torch.uint8, device=dev)
    _check_tensor("workspace", workspace, (torch.uint8,), (workspace.numel(),), dev)
    _check(lib().svt_search(handle, B, _t_ptr(queries), _t_ptr(masks), _t_ptr(query_scales), nprobe, k,
                            *[_t_ptr(t) for t in outs], _opt_ptr(opts), _t_ptr(workspace), int(workspace.numel()),
                            _stream_ptr(stream)))
    return outs


def svt_search_noalloc(handle, queries, masks, nprobe: int, k: int, query_scales=None, out_ids=None,
                       out_scores=None, out_fscores=None, out_counts=None, out_stats=None, stream=None, opts=None):
    """svt_search with the library's static scratch as workspace (the C call allocates no device memory;
    outputs not passed in are still allocated here, by torch).  Searches on one GPU must not overlap."""
    B, dev, G, outs = _search_tensors(handle, queries, masks, k, query_scales, out_ids, out_scores, out_fscores,
                                      out_counts, out_stats)
    opts = _with_groups(opts, G)
    _check(lib().svt_search_noalloc(handle, B, _t_ptr(queries), _t_ptr(masks), _t_ptr(query_scales), nprobe, k,
                                    *[_t_ptr(t) for t in outs], _opt_ptr(opts), _stream_ptr(stream)))
    return outs


_NET_KEYS = ("gate_w", "gate_b", "w1", "b1", "w2", "b2")


def svt_rerank(handle, queries, cand_ids, net, k_out: int, query_scales=None, out_ids=None, out_scores=None,
               out_counts=None, stream=None):
    """Re-score each query's candidates with a gated mixture of experts and keep the k_out best.
    queries: int8 [B, d] cuda tensor; cand_ids: int64 [B, n_cand] cuda tensor (e.g. svt_search's ids;
    -1 and ids not in the index are skipped); net: dict of float32 cuda tensors gate_w [E, d],
    gate_b [E], w1 [E, H, d], b1 [E, H], w2 [E, H], b2 [E].  Returns (ids int64 [B, k_out],
    scores float32 [B, k_out], counts int32 [B]); asynchronous on ``stream``."""
    import torch
    n, dim, W, _ = svt_index_info(handle)
    if not hasattr(queries, "shape") or len(queries.shape) != 2:
        raise ValueError("queries: expected a 2-D tensor [B, dim]")
    if not hasattr(cand_ids, "shape") or len(cand_ids.shape) != 2:
        raise ValueError("cand_ids: expected a 2-D tensor [B, n_cand]")
    B, n_cand = int(queries.shape[0]), int(cand_ids.shape[1])
    dev = queries.device
    _check_tensor("queries", queries, (torch.int8,), (B, dim))
    _check_tensor("cand_ids", cand_ids, (torch.int64,), (B, n_cand), dev)
    _check_tensor("query_scales", query_scales, (torch.float32,), (B,), dev, nullable=True)
    if not hasattr(net.get("w1"), "shape") or len(net["w1"].shape) != 3:
        raise ValueError("net['w1']: expected a tensor [E, H, d]")
    E, H = int(net["w1"].shape[0]), int(net["w1"].shape[1])
    shapes = {"gate_w": (E, dim), "gate_b": (E,), "w1": (E, H, dim), "b1": (E, H), "w2": (E, H), "b2": (E,)}
    for key in _NET_KEYS:
        _check_tensor(f"net['{key}']", net.get(key), (torch.float32,), shapes[key], dev)
    if out_ids is None:
        out_ids = torch.empty((B, k_out), dtype=torch.int64, device=dev)
    if out_scores is None:
        out_scores = torch.empty((B, k_out), dtype=torch.float32, device=dev)
    if out_counts is None:
        out_counts = torch.empty((B,), dtype=torch.int32, device=dev)
    _check_tensor("out_ids", out_ids, (torch.int64,), (B, k_out), dev)
    _check_tensor("out_scores", out_scores, (torch.float32,), (B, k_out), dev)
    _check_tensor("out_counts", out_counts, (torch.int32,), (B,), dev)
    cnet = svt_rerank_net(E, H, *[net[key].data_ptr() for key in _NET_KEYS])
    _check(lib().svt_rerank(handle, B, _t_ptr(queries), _t_ptr(query_scales), n_cand, _t_ptr(cand_ids),
                            ctypes.byref(cnet), k_out, _t_ptr(out_ids), _t_ptr(out_scores), _t_ptr(out_counts),
                            _stream_ptr(stream)))
    return out_ids, out_scores, out_counts


def svt_profile_enable(on) -> None:
    """False/0: off; True/1: every stage; 2: the scan stage only (two event records per search)."""
    _check(lib().svt_profile_enable(int(on)))


def svt_profile_read(max_stages: int = 8):
    """Returns ({stage: total ms}, n_searches) over the searches recorded since the last read."""
    ms = (ctypes.c_float * max_stages)()
    names = (ctypes.c_char_p * max_stages)()
    n, ns = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().svt_profile_read(ms, names, max_stages, ctypes.byref(n), ctypes.byref(ns)))
    return {names[i].decode(): float(ms[i]) for i in range(min(n.value, max_stages))}, ns.value


# ------------------------------------------------------------------------------------------------
class Index:
    """Convenience owner of an uploaded index: ``Index(items, sigs, list_of, centroids, scale)``,
    ``search(queries, masks, nprobe, k)`` with torch device tensors, ``close()``."""

    def __init__(self, items, sigs, list_of, centroids, item_scale, stream=None, id_capacity=None, slack_min=0,
                 slack_frac=0.0):
        if id_capacity is None:
            self.handle = svt_index_upload(items, sigs, list_of, centroids, item_scale, stream)
        else:   # updatable
            self.handle = svt_index_upload_updatable(items, sigs, list_of, centroids, item_scale, id_capacity,
                                                     slack_min, slack_frac, stream)
        self.n_items, self.dim, self.sig_words, self.nlist = svt_index_info(self.handle)
        self._ws = None

    def workspace(self, n_queries: int, nprobe: int, k: int, opts=None):
        import torch
        nbytes = max(256, svt_search_workspace_size(self.handle, n_queries, nprobe, k, opts))
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = None
            self._ws = torch.empty((nbytes,), dtype=torch.uint8, device="cuda")
        return self._ws

    def search(self, queries, masks, nprobe: int, k: int, query_scales=None, stream=None, opts=None, **outs):
        B = int(queries.shape[0])
        if hasattr(masks, "shape") and len(masks.shape) == 3:
            opts = _with_groups(opts, int(masks.shape[1]))
        ws = self.workspace(B, nprobe, k, opts) if B > 0 else None
        return svt_search(self.handle, queries, masks, nprobe, k, query_scales=query_scales, workspace=ws,
                          stream=stream, opts=opts, **outs)

    def rerank(self, queries, cand_ids, net, k_out: int, query_scales=None, stream=None, **outs):
        return svt_rerank(self.handle, queries, cand_ids, net, k_out, query_scales=query_scales, stream=stream,
                          **outs)

    def insert(self, ids, rows, sigs, list_of, stream=None):
        svt_index_insert(self.handle, ids, rows, sigs, list_of, stream)
        self.n_items = svt_index_info(self.handle)[0]

    def delete(self, ids, stream=None):
        svt_index_delete(self.handle, ids, stream)
        self.n_items = svt_index_info(self.handle)[0]

    def resign(self, ids, sigs, stream=None):
        svt_index_resign(self.handle, ids, sigs, stream)

    def close(self, stream=None):
        if self.handle is not None:
            svt_index_free(self.handle, stream)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
