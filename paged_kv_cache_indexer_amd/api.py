"""Thin torch-facing binding of libdsa: argument marshalling only.

Every function has the name of the C entry point it calls and takes device tensors
(torch is used for device memory and streams only); all computation happens in the
HIP kernels.  A non-OK status raises DsaError with the library's error text.
"""
import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import dsa_rows_t, DSA_F32, DSA_BF16, DSA_E4M3, DSA_MXFP4, DSA_GATHER_SERVE, DSA_GATHER_INSTALL  # noqa: F401


class DsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _lib.load().dsa_last_error().decode(errors="replace")
        super().__init__(f"{where}: {_lib.STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def _check(status: int, where: str):
    if status != _lib.DSA_OK:
        raise DsaError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("libdsa needs contiguous tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DSA_F32
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return DSA_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


class Rows:
    """A dsa_rows_t over a tensor of rows (paged when a page table is given)."""

    def __init__(self, base: torch.Tensor, row_bytes: int, page_table: Optional[torch.Tensor] = None,
                 page_size: int = 0, req_stride: int = 0, num_rows: Optional[int] = None,
                 base_ptr: Optional[int] = None):
        self._keep = (base, page_table)
        nbytes = base.numel() * base.element_size()
        self.c = dsa_rows_t()
        self.c.base = base_ptr if base_ptr is not None else base.data_ptr()
        self.c.num_rows = num_rows if num_rows is not None else nbytes // row_bytes
        self.c.row_bytes = row_bytes
        self.c.page_size = page_size
        self.c.page_table = page_table.data_ptr() if page_table is not None else None
        self.c.pt_stride = page_table.shape[-1] if page_table is not None else 0
        self.c.reserved = 0
        self.c.req_stride = req_stride

    def ref(self):
        return ctypes.byref(self.c)


def dsa_version() -> int:
    return _lib.load().dsa_version()


def dsa_indexer_scores(q: torch.Tensor, w: torch.Tensor, keys: Rows, k_scale: Optional[torch.Tensor],
                       seq_lens: torch.Tensor, scores: torch.Tensor, k_dtype: int = DSA_E4M3,
                       err: Optional[torch.Tensor] = None, ready: Optional[torch.cuda.Event] = None, stream=None,
                       q_dtype: Optional[int] = None):
    B, Sq, H, D = q.shape
    qd = _dtype_code(q) if q_dtype is None else q_dtype
    ev = ctypes.c_void_p(ready.cuda_event) if ready is not None else None
    _check(_lib.load().dsa_indexer_scores(_ptr(q), qd, _ptr(w), keys.ref(), k_dtype, _ptr(k_scale), _ptr(seq_lens),
                                          B, Sq, H, D, scores.shape[-1], _ptr(scores), _ptr(err), ev,
                                          _stream(stream)), "dsa_indexer_scores")


def dsa_topk_workspace_size(B: int, Sq: int, k: int, score_stride: int) -> int:
    return _lib.load().dsa_topk_workspace_size(B, Sq, k, score_stride)


def dsa_topk(scores: torch.Tensor, seq_lens: torch.Tensor, idx: torch.Tensor, ws: Optional[torch.Tensor] = None,
             stream=None):
    """ws: workspace tensor of at least dsa_topk_workspace_size(...) bytes (allocated here if None)."""
    B, Sq, k = idx.shape
    if ws is None:
        ws = torch.empty(max(1, dsa_topk_workspace_size(B, Sq, k, scores.shape[-1])), dtype=torch.uint8,
                         device=idx.device)
    ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.load().dsa_topk(_ptr(scores), scores.shape[-1], _ptr(seq_lens), B, Sq, k, _ptr(idx), _ptr(ws),
                                ws_bytes, _stream(stream)), "dsa_topk")


def dsa_indexer_topk_chunks(q: torch.Tensor, w: torch.Tensor, keys: Rows, k_scale: Optional[torch.Tensor],
                            seq_lens: torch.Tensor, scores: torch.Tensor, k: int, ws: torch.Tensor,
                            k_dtype: int = DSA_E4M3, err: Optional[torch.Tensor] = None,
                            ready: Optional[torch.cuda.Event] = None, stream=None, q_dtype: Optional[int] = None):
    """The indexer scan (one query token per request) with the top-k chunk stage in its epilogue:
    writes scores and the chunks' candidates into ws (dsa_topk_workspace_size(B, 1, k, stride) bytes)."""
    B, Sq, H, D = q.shape
    if Sq != 1:
        raise ValueError("dsa_indexer_topk_chunks takes one query token per request")
    qd = _dtype_code(q) if q_dtype is None else q_dtype
    ev = ctypes.c_void_p(ready.cuda_event) if ready is not None else None
    _check(_lib.load().dsa_indexer_topk_chunks(_ptr(q), qd, _ptr(w), keys.ref(), k_dtype, _ptr(k_scale),
                                               _ptr(seq_lens), B, H, D, scores.shape[-1], _ptr(scores), k, _ptr(ws),
                                               ws.numel() * ws.element_size(), _ptr(err), ev, _stream(stream)),
           "dsa_indexer_topk_chunks")


def dsa_topk_select_chunks(scores: torch.Tensor, seq_lens: torch.Tensor, idx: torch.Tensor, ws: torch.Tensor,
                           stream=None):
    """The exact select over the candidates dsa_indexer_topk_chunks left in ws; idx [B, 1, k]."""
    B, Sq, k = idx.shape
    if Sq != 1:
        raise ValueError("dsa_topk_select_chunks takes one query token per request")
    _check(_lib.load().dsa_topk_select_chunks(_ptr(scores), scores.shape[-1], _ptr(seq_lens), B, k, _ptr(idx),
                                              _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "dsa_topk_select_chunks")


def dsa_topk_union(topk: torch.Tensor, uni: torch.Tensor, count: torch.Tensor, uidx: Optional[torch.Tensor] = None,
                   member: Optional[torch.Tensor] = None, err: Optional[torch.Tensor] = None, stream=None):
    """topk [B, Sq, k] -> uni [B, Sq*k], count [B], uidx [B, Sq, k], member [B, Sq, ceil(Sq*k/32)] (int32 views)."""
    B, Sq, k = topk.shape
    _check(_lib.load().dsa_topk_union(_ptr(topk), B, Sq, k, _ptr(uni), _ptr(count), _ptr(uidx), _ptr(member),
                                      _ptr(err), _stream(stream)), "dsa_topk_union")


def dsa_plan(topk: torch.Tensor, pool_ids: torch.Tensor, id_to_slot: torch.Tensor, ptr: torch.Tensor, n_sets: int,
             ways: int, is_hit: torch.Tensor, slot: torch.Tensor, miss_pos: torch.Tensor, miss_slot: torch.Tensor,
             miss_count: torch.Tensor, commit: bool = True, err: Optional[torch.Tensor] = None, stream=None):
    B, Sq, k = topk.shape
    _check(_lib.load().dsa_plan(_ptr(topk), B, Sq, k, _ptr(pool_ids), _ptr(id_to_slot), _ptr(ptr), n_sets, ways,
                                id_to_slot.shape[-1], _ptr(is_hit), _ptr(slot), _ptr(miss_pos), _ptr(miss_slot),
                                _ptr(miss_count), int(commit), _ptr(err), _stream(stream)), "dsa_plan")


def dsa_gather_kv(topk: torch.Tensor, is_hit: Optional[torch.Tensor], slot: Optional[torch.Tensor],
                  src: Optional[Rows], pool: Optional[torch.Tensor], sel: torch.Tensor, mode: int = DSA_GATHER_SERVE,
                  row_bytes: int = 1152, err: Optional[torch.Tensor] = None, stream=None,
                  sel_idx: Optional[torch.Tensor] = None):
    """sel_idx (SERVE, optional): [B, Sq, k] int32 out, t*k + j where a row was served, else -1."""
    B, Sq, k = topk.shape
    pool_rows = 0 if pool is None else (pool.numel() * pool.element_size()) // (B * row_bytes)
    _check(_lib.load().dsa_gather_kv(_ptr(topk), _ptr(is_hit), _ptr(slot), B, Sq, k,
                                     src.ref() if src is not None else None, _ptr(pool), pool_rows, row_bytes,
                                     _ptr(sel), _ptr(sel_idx), mode, _ptr(err), _stream(stream)), "dsa_gather_kv")


def dsa_sparse_mla_workspace_size(B: int, Sq: int, H: int, k: int) -> int:
    return _lib.load().dsa_sparse_mla_workspace_size(B, Sq, H, k)


def dsa_sparse_mla_decode(q: torch.Tensor, idx: torch.Tensor, rows: Rows, scale: float, o: torch.Tensor,
                          lse: torch.Tensor, ws: Optional[torch.Tensor] = None, err: Optional[torch.Tensor] = None,
                          stream=None):
    B, Sq, H, _ = q.shape
    k = idx.shape[-1]
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.load().dsa_sparse_mla_decode(_ptr(q), _ptr(idx), rows.ref(), B, Sq, H, k, float(scale), _ptr(o),
                                             _dtype_code(o), _ptr(lse), _ptr(ws), ws_bytes, _ptr(err),
                                             _stream(stream)), "dsa_sparse_mla_decode")


def dsa_sparse_mla_union_workspace_size(B: int, Sq: int, H: int, U: int) -> int:
    return _lib.load().dsa_sparse_mla_union_workspace_size(B, Sq, H, U)


def dsa_sparse_mla_decode_union(q: torch.Tensor, uni: torch.Tensor, count: Optional[torch.Tensor],
                                member: torch.Tensor, rows: Rows, scale: float, o: torch.Tensor, lse: torch.Tensor,
                                ws: Optional[torch.Tensor] = None, err: Optional[torch.Tensor] = None, stream=None):
    """q [B, Sq, H, 576]; uni [B, U]; member [B, Sq, ceil(U/32)] -> o [B, Sq, H, 512], lse [B, Sq, H]."""
    B, Sq, H, _ = q.shape
    U = uni.shape[-1]
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.load().dsa_sparse_mla_decode_union(_ptr(q), _ptr(uni), _ptr(count), _ptr(member), rows.ref(), B, Sq,
                                                   H, U, float(scale), _ptr(o), _dtype_code(o), _ptr(lse), _ptr(ws),
                                                   ws_bytes, _ptr(err), _stream(stream)),
           "dsa_sparse_mla_decode_union")


def dsa_sparse_mla_decode_noalloc(q: torch.Tensor, idx: torch.Tensor, rows: Rows, scale: float, o: torch.Tensor,
                                  lse: torch.Tensor, err: Optional[torch.Tensor] = None, stream=None):
    """dsa_sparse_mla_decode with the split partials in the library's own scratch array."""
    B, Sq, H, _ = q.shape
    k = idx.shape[-1]
    _check(_lib.load().dsa_sparse_mla_decode_noalloc(_ptr(q), _ptr(idx), rows.ref(), B, Sq, H, k, float(scale),
                                                     _ptr(o), _dtype_code(o), _ptr(lse), _ptr(err), _stream(stream)),
           "dsa_sparse_mla_decode_noalloc")


def dsa_merge_partials(o_parts: torch.Tensor, lse_parts: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                       stream=None):
    """o_parts [R, ..., V] (float32 or bf16), lse_parts [R, ...] float32 -> o [..., V], lse [...]:
    the LSE merge of R partial attention results over disjoint row sets."""
    R, V = o_parts.shape[0], o_parts.shape[-1]
    N = lse_parts[0].numel()
    if o_parts.numel() != R * N * V or o.numel() != N * V or lse.numel() != N:
        raise ValueError("dsa_merge_partials: shapes disagree")
    _check(_lib.load().dsa_merge_partials(_ptr(o_parts), _dtype_code(o_parts), _ptr(lse_parts), R, N, V, _ptr(o),
                                          _dtype_code(o), _ptr(lse), _stream(stream)), "dsa_merge_partials")


def dsa_page_translate(x: torch.Tensor, page_size: int, n_ranks: int, rank: torch.Tensor, local_row: torch.Tensor,
                       err: Optional[torch.Tensor] = None, stream=None):
    _check(_lib.load().dsa_page_translate(_ptr(x), x.numel(), page_size, n_ranks, _ptr(rank), _ptr(local_row),
                                          _ptr(err), _stream(stream)), "dsa_page_translate")


def dsa_kv_write(latent: torch.Tensor, idx_k: torch.Tensor, seq_lens: torch.Tensor, kv: Rows, idx_cache: Rows,
                 idx_scale: torch.Tensor, err: Optional[torch.Tensor] = None, stream=None,
                 cache_dtype: int = DSA_E4M3):
    """Quantise and scatter the new tokens ([B, Sq, 576] latent, [B, Sq, D] keys) into the caches.
    cache_dtype DSA_E4M3: float32 idx_scale per row; DSA_MXFP4: uint8 [rows, D/32] E8M0 scales."""
    B, Sq, D = idx_k.shape
    _check(_lib.load().dsa_kv_write(_ptr(latent), _ptr(idx_k), _dtype_code(idx_k), _ptr(seq_lens), B, Sq, D,
                                    kv.ref(), idx_cache.ref(), cache_dtype, _ptr(idx_scale), _ptr(err),
                                    _stream(stream)),
           "dsa_kv_write")
