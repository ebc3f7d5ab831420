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

SVT_OK, SVT_EINVAL, SVT_ENOMEM, SVT_EDEVICE, SVT_EUNSUPPORTED, SVT_ESTATE = 0, -1, -2, -3, -4, -5
SVT_MAX_K = 2048
SVT_MAX_SIG_WORDS = 2

#: every symbol include/svt.h declares
EXPORTED = ("svt_index_upload", "svt_index_free", "svt_index_info", "svt_search_workspace_size", "svt_search",
            "svt_last_error", "svt_bloom_mask", "svt_bloom_sign", "svt_profile_enable", "svt_profile_read")


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
    L.svt_index_free.argtypes = [vp]
    L.svt_index_info.argtypes = [vp, vp, vp, vp, vp]
    L.svt_search_workspace_size.argtypes = [vp, i32, i32, i32]
    L.svt_search_workspace_size.restype = sz
    L.svt_search.argtypes = [vp, i32, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
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


def svt_index_upload(items: np.ndarray, sigs: np.ndarray, list_of: np.ndarray, centroids: np.ndarray,
                     item_scale: float, stream=None) -> ctypes.c_void_p:
    """Host arrays -> device index handle (the current torch device)."""
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
    h = ctypes.c_void_p()
    _check(lib().svt_index_upload(ctypes.byref(d), _stream_ptr(stream), ctypes.byref(h)))
    return h


def svt_index_free(handle) -> None:
    _check(lib().svt_index_free(handle))


def svt_index_info(handle) -> Tuple[int, int, int, int]:
    n = ctypes.c_int64()
    d, w, nl = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().svt_index_info(handle, ctypes.byref(n), ctypes.byref(d), ctypes.byref(w), ctypes.byref(nl)))
    return n.value, d.value, w.value, nl.value


def svt_search_workspace_size(handle, n_queries: int, nprobe: int, k: int) -> int:
    sz = lib().svt_search_workspace_size(handle, n_queries, nprobe, k)
    if sz == 0 and n_queries >= 0:
        err = svt_last_error()
        if err:
            raise SvtError(SVT_EINVAL, err)
    return int(sz)


def svt_search(handle, queries, masks, nprobe: int, k: int, query_scales=None, out_ids=None, out_scores=None,
               out_fscores=None, out_counts=None, out_stats=None, workspace=None, stream=None):
    """queries: int8 [B, d] cuda tensor; masks: uint64 (or int64) [B, W] cuda tensor.
    Returns (ids int64 [B,k], scores int32 [B,k], fscores f32 [B,k], counts int32 [B], stats int64 [B,2]);
    outputs are allocated with torch unless passed in.  Asynchronous on ``stream``."""
    import torch
    B = int(queries.shape[0])
    dev = queries.device
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
    if workspace is None:
        nbytes = svt_search_workspace_size(handle, B, nprobe, k) if B > 0 else 0
        workspace = torch.empty((max(nbytes, 256),), dtype=torch.uint8, device=dev)
    _check(lib().svt_search(handle, B, _t_ptr(queries), _t_ptr(masks), _t_ptr(query_scales), nprobe, k,
                            _t_ptr(out_ids), _t_ptr(out_scores), _t_ptr(out_fscores), _t_ptr(out_counts),
                            _t_ptr(out_stats), _t_ptr(workspace), int(workspace.numel()), _stream_ptr(stream)))
    return out_ids, out_scores, out_fscores, out_counts, out_stats


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

    def __init__(self, items, sigs, list_of, centroids, item_scale, stream=None):
        self.handle = svt_index_upload(items, sigs, list_of, centroids, item_scale, stream)
        self.n_items, self.dim, self.sig_words, self.nlist = svt_index_info(self.handle)
        self._ws = None

    def workspace(self, n_queries: int, nprobe: int, k: int):
        import torch
        nbytes = max(256, svt_search_workspace_size(self.handle, n_queries, nprobe, k))
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.empty((nbytes,), dtype=torch.uint8, device="cuda")
        return self._ws

    def search(self, queries, masks, nprobe: int, k: int, query_scales=None, stream=None, **outs):
        ws = self.workspace(int(queries.shape[0]), nprobe, k) if int(queries.shape[0]) > 0 else None
        return svt_search(self.handle, queries, masks, nprobe, k, query_scales=query_scales, workspace=ws,
                          stream=stream, **outs)

    def close(self):
        if self.handle is not None:
            svt_index_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
