"""Fused int8 IVF + Bloom-signature top-k search for AMD MI355X (gfx950).

The search itself runs in hand-written HIP kernels behind the C ABI declared in include/svt.h
(libsvt.so, built in-tree by ``int8_ivf_ann_amd.build``).  ``int8_ivf_ann_amd.svt`` is the thin
ctypes binding with the same entry-point names; PyTorch supplies device memory and streams.
"""
from .svt import (EXPORTED, SVT_EDEVICE, SVT_EINVAL, SVT_ENOMEM, SVT_ESTATE, SVT_EUNSUPPORTED, SVT_MAX_K,
                  SVT_MAX_SIG_WORDS, SVT_OK, Index, SvtError, svt_bloom_mask, svt_bloom_sign, svt_index_free,
                  svt_index_info, svt_index_upload, svt_last_error, svt_profile_enable, svt_profile_read,
                  svt_search, svt_search_workspace_size)

__all__ = ["Index", "SvtError", "svt_bloom_mask", "svt_bloom_sign", "svt_index_free", "svt_index_info",
           "svt_index_upload", "svt_last_error", "svt_profile_enable", "svt_profile_read", "svt_search",
           "svt_search_workspace_size", "EXPORTED", "SVT_OK", "SVT_EINVAL", "SVT_ENOMEM", "SVT_EDEVICE",
           "SVT_EUNSUPPORTED", "SVT_ESTATE", "SVT_MAX_K", "SVT_MAX_SIG_WORDS"]
