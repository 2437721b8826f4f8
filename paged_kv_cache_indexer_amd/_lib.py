"""ctypes declarations of libdsa's C ABI (include/dsa.h)."""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsa.so")

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_HIP, DSA_ERR_WORKSPACE = 0, -1, -2, -3, -4
DSA_F32, DSA_BF16, DSA_E4M3, DSA_MXFP4 = 0, 1, 2, 3
DSA_GATHER_SERVE, DSA_GATHER_INSTALL = 0, 1

STATUS_NAMES = {0: "DSA_OK", -1: "DSA_ERR_INVALID_ARG", -2: "DSA_ERR_UNSUPPORTED", -3: "DSA_ERR_HIP",
                -4: "DSA_ERR_WORKSPACE"}

EXPORTED = ["dsa_version", "dsa_last_error", "dsa_indexer_scores", "dsa_topk_workspace_size", "dsa_topk",
            "dsa_indexer_topk_chunks", "dsa_topk_select_chunks",
            "dsa_topk_union", "dsa_sparse_mla_union_workspace_size", "dsa_sparse_mla_decode_union",
            "dsa_plan", "dsa_gather_kv", "dsa_sparse_mla_workspace_size", "dsa_sparse_mla_decode",
            "dsa_sparse_mla_noalloc_max_workspace", "dsa_sparse_mla_decode_noalloc", "dsa_merge_partials",
            "dsa_page_translate", "dsa_kv_write"]


class dsa_rows_t(ctypes.Structure):
    _fields_ = [
        ("base", ctypes.c_void_p),
        ("num_rows", ctypes.c_int64),
        ("row_bytes", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("page_table", ctypes.c_void_p),
        ("pt_stride", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("req_stride", ctypes.c_int64),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load libdsa.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_indexer_amd.build` "
                           "(or __graft_entry__.build()); libdsa has no CPU fallback")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    prow = ctypes.POINTER(dsa_rows_t)
    sig = {
        "dsa_version": (ctypes.c_int, []),
        "dsa_last_error": (ctypes.c_char_p, []),
        "dsa_indexer_scores": (ctypes.c_int, [vp, ctypes.c_int, vp, prow, ctypes.c_int, vp, vp, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, vp, vp, vp, vp]),
        "dsa_topk_workspace_size": (sz, [ctypes.c_int, ctypes.c_int, ctypes.c_int, i64]),
        "dsa_topk": (ctypes.c_int, [vp, i64, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, sz, vp]),
        "dsa_indexer_topk_chunks": (ctypes.c_int, [vp, ctypes.c_int, vp, prow, ctypes.c_int, vp, vp, ctypes.c_int,
                                                   ctypes.c_int, ctypes.c_int, i64, vp, ctypes.c_int, vp, sz, vp, vp,
                                                   vp]),
        "dsa_topk_select_chunks": (ctypes.c_int, [vp, i64, vp, ctypes.c_int, ctypes.c_int, vp, vp, sz, vp]),
        "dsa_plan": (ctypes.c_int, [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp]),
        "dsa_gather_kv": (ctypes.c_int, [vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, prow, vp, i64,
                                         i32, vp, vp, ctypes.c_int, vp, vp]),
        "dsa_sparse_mla_workspace_size": (sz, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
        "dsa_sparse_mla_decode": (ctypes.c_int, [vp, vp, prow, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_int, ctypes.c_float, vp, ctypes.c_int, vp, vp, sz, vp,
                                                 vp]),
        "dsa_topk_union": (ctypes.c_int, [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp]),
        "dsa_sparse_mla_union_workspace_size": (sz, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
        "dsa_sparse_mla_decode_union": (ctypes.c_int, [vp, vp, vp, vp, prow, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                       ctypes.c_int, ctypes.c_float, vp, ctypes.c_int, vp, vp, sz, vp,
                                                       vp]),
        "dsa_sparse_mla_noalloc_max_workspace": (sz, []),
        "dsa_sparse_mla_decode_noalloc": (ctypes.c_int, [vp, vp, prow, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                         ctypes.c_int, ctypes.c_float, vp, ctypes.c_int, vp, vp, vp]),
        "dsa_merge_partials": (ctypes.c_int, [vp, ctypes.c_int, vp, ctypes.c_int, i64, ctypes.c_int, vp,
                                              ctypes.c_int, vp, vp]),
        "dsa_page_translate": (ctypes.c_int, [vp, i64, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp]),
        "dsa_kv_write": (ctypes.c_int, [vp, vp, ctypes.c_int, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, prow,
                                        prow, ctypes.c_int, vp, vp, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L
