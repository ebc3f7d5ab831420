"""Fused int8 IVF + Bloom-signature top-k search for AMD MI355X (gfx950).

The search itself runs in hand-written HIP kernels behind the C ABI declared in include/svt.h
(libsvt.so, built in-tree by ``int8_ivf_ann_amd.build``).  ``int8_ivf_ann_amd.svt`` is the thin
ctypes binding with the same entry-point names; PyTorch supplies device memory and streams.
"""
from .svt import (EXPORTED, SVT_EDEVICE, SVT_EINVAL, SVT_ENOMEM, SVT_ENOSPACE, SVT_ESTATE, SVT_EUNSUPPORTED, SVT_MAX_K, SVT_MAX_K_LARGE,
                  SVT_MAX_SIG_WORDS, SVT_MAX_MASK_GROUPS, SVT_OK, SVT_OPT_FORCE_REDO, SVT_OPT_MERGE_FROM_SLOTS, SVT_PATH_AUTO,
                  SVT_PATH_QUERY, SVT_PATH_TILE, SVT_PATH_EXHAUSTIVE, SVT_PATH_LARGE_K, Index, make_options, svt_search_options, SvtError, svt_bloom_mask, svt_bloom_sign, svt_index_free,
                  svt_index_info, svt_index_upload, svt_index_upload_updatable, svt_index_insert, svt_index_delete,
                  svt_index_resign, svt_last_error, svt_profile_enable, svt_profile_read,
                  svt_search, svt_search_noalloc, svt_search_path, svt_search_workspace_size, SVT_NOALLOC_SCRATCH_BYTES,
                  svt_rerank, svt_rerank_net)

__all__ = ["Index", "SvtError", "svt_bloom_mask", "svt_bloom_sign", "svt_index_free", "svt_index_info",
           "svt_index_upload", "svt_index_upload_updatable", "svt_index_insert", "svt_index_delete", "svt_index_resign",
           "svt_last_error", "svt_profile_enable", "svt_profile_read", "svt_search",
           "svt_search_noalloc", "svt_rerank", "svt_rerank_net", "svt_search_path", "svt_search_workspace_size", "SVT_NOALLOC_SCRATCH_BYTES", "EXPORTED", "SVT_OK", "SVT_EINVAL", "SVT_ENOMEM", "SVT_EDEVICE",
           "SVT_EUNSUPPORTED", "SVT_ESTATE", "SVT_ENOSPACE", "SVT_MAX_K", "SVT_MAX_K_LARGE", "SVT_MAX_SIG_WORDS", "SVT_MAX_MASK_GROUPS", "SVT_PATH_AUTO", "SVT_PATH_QUERY",
           "SVT_PATH_TILE", "SVT_PATH_EXHAUSTIVE", "SVT_PATH_LARGE_K", "SVT_OPT_MERGE_FROM_SLOTS", "SVT_OPT_FORCE_REDO", "make_options", "svt_search_options"]
