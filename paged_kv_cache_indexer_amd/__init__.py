"""libdsa for AMD MI355X: one decode step of DSA-style sparse attention in HIP.

The compute path lives in libdsa.so (hand-written gfx950 kernels behind the C ABI of
include/dsa.h); this package only builds and binds it.  There is no CPU fallback:
calling into the library without the built .so raises.
"""
from .api import (  # noqa: F401
    DsaError, Rows, dsa_version, dsa_indexer_scores, dsa_topk, dsa_topk_workspace_size, dsa_indexer_topk_chunks,
    dsa_topk_select_chunks, dsa_topk_union, dsa_plan,
    dsa_gather_kv, dsa_sparse_mla_union_workspace_size, dsa_sparse_mla_decode_union,
    dsa_sparse_mla_workspace_size, dsa_sparse_mla_decode, dsa_sparse_mla_decode_noalloc, dsa_merge_partials, dsa_page_translate, dsa_kv_write,
    DSA_F32, DSA_BF16, DSA_E4M3, DSA_MXFP4, DSA_GATHER_SERVE, DSA_GATHER_INSTALL,
)
from ._lib import LIB_PATH, EXPORTED  # noqa: F401
