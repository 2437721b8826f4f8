"""The C-ABI library loads and exports every entry point include/dsa.h declares; argument
checks that need no device reject bad calls before anything is launched."""
import ctypes
import os
import re
import subprocess

import pytest

import paged_kv_cache_indexer_amd as dsa
from paged_kv_cache_indexer_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared():
    src = open(os.path.join(ROOT, "include", "dsa.h")).read()
    return sorted(set(re.findall(r"^\S[^\n(]*?\b(dsa_\w+)\(", src, re.M)))


def test_header_and_binding_agree():
    assert declared() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    names = {l.split()[-1] for l in out.splitlines() if l.strip()}
    missing = [s for s in declared() if s not in names]
    assert not missing, missing
    L = _lib.load()
    assert L.dsa_version() == 100
    for s in declared():
        assert hasattr(L, s)


def test_invalid_arguments_rejected_without_device():
    L = _lib.load()
    # negative batch, null pointers, k too large: rejected before any HIP call
    assert L.dsa_topk(None, 1, None, -1, 1, 8, None, None, 0, None) == _lib.DSA_ERR_INVALID_ARG
    assert L.dsa_topk(None, 1, None, 2, 1, 8, None, None, 0, None) == _lib.DSA_ERR_INVALID_ARG
    assert L.dsa_topk(ctypes.c_void_p(16), 100, ctypes.c_void_p(16), 2, 1, 9000, ctypes.c_void_p(16), None, 0,
                      None) == _lib.DSA_ERR_UNSUPPORTED
    assert L.dsa_topk(ctypes.c_void_p(16), 100000, ctypes.c_void_p(16), 2, 1, 2048, ctypes.c_void_p(16), None, 0,
                      None) == _lib.DSA_ERR_WORKSPACE
    # wave chunks of 1024 positions: 64 chunks, candidate bound 2k + 18 * 64 = 5248 slots of
    # (key, position), a cut key and a count per chunk
    assert L.dsa_topk_workspace_size(32, 1, 2048, 65536) == 32 * (5248 * 8 + 64 * 8)
    # 300000 positions exceed the wave chunks' 262144: work-group chunks of 8192, 37 of them,
    # bound 2k + 2 * 37 = 4170
    assert L.dsa_topk_workspace_size(2, 1, 2048, 300000) == 2 * (4170 * 8 + 37 * 8)
    # 250048 positions: the slack drops to (8192 - 4096) / 245 - 2 = 14, bound 4096 + 16 * 245 = 8016
    assert L.dsa_topk_workspace_size(66, 1, 2048, 250048) == 66 * (8016 * 8 + 245 * 8)
    assert L.dsa_page_translate(None, 10, 0, 4, None, None, None, None) == _lib.DSA_ERR_INVALID_ARG
    assert L.dsa_plan(None, 1, 1, 8, None, None, None, 4, 2, 10, None, None, None, None, None, 1, None,
                      None) == _lib.DSA_ERR_INVALID_ARG
    assert b"null" in L.dsa_last_error()
    rows = _lib.dsa_rows_t()
    rows.base = 16
    rows.row_bytes = 1000
    assert L.dsa_sparse_mla_decode(ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.byref(rows), 1, 1, 128, 64,
                                   ctypes.c_float(0.1), ctypes.c_void_p(16), _lib.DSA_BF16, ctypes.c_void_p(16),
                                   None, 0, None, None) == _lib.DSA_ERR_INVALID_ARG
    assert L.dsa_gather_kv(ctypes.c_void_p(16), None, None, 1, 1, 4, None, None, 0, 100, ctypes.c_void_p(16), None,
                           0, None, None) == _lib.DSA_ERR_INVALID_ARG
    assert L.dsa_gather_kv(ctypes.c_void_p(16), None, None, 1, 1, 4, None, None, 0, 1152, ctypes.c_void_p(16),
                           ctypes.c_void_p(18), 0, None, None) == _lib.DSA_ERR_INVALID_ARG   # sel_idx misaligned
    kv, ic = _lib.dsa_rows_t(), _lib.dsa_rows_t()
    kv.base, kv.row_bytes, ic.base, ic.row_bytes = 16, 1152, 16, 128
    p = ctypes.c_void_p(16)
    E4, F4 = _lib.DSA_E4M3, _lib.DSA_MXFP4
    assert L.dsa_kv_write(p, p, _lib.DSA_E4M3, p, 1, 1, 128, ctypes.byref(kv), ctypes.byref(ic), E4, p, None,
                          None) == _lib.DSA_ERR_INVALID_ARG          # keys must be bf16 or fp32
    assert L.dsa_kv_write(p, p, _lib.DSA_BF16, p, 1, 1, 130, ctypes.byref(kv), ctypes.byref(ic), E4, p, None,
                          None) == _lib.DSA_ERR_UNSUPPORTED          # D > 128
    assert L.dsa_kv_write(p, p, _lib.DSA_BF16, p, 1, 1, 64, ctypes.byref(kv), ctypes.byref(ic), E4, p, None,
                          None) == _lib.DSA_ERR_INVALID_ARG          # indexer rows must be D bytes
    assert L.dsa_kv_write(p, p, _lib.DSA_BF16, p, 1, 1, 128, ctypes.byref(kv), ctypes.byref(ic), _lib.DSA_BF16, p,
                          None, None) == _lib.DSA_ERR_INVALID_ARG    # the cache is e4m3 or mxfp4
    assert L.dsa_kv_write(p, p, _lib.DSA_BF16, p, 1, 1, 128, ctypes.byref(kv), ctypes.byref(ic), F4, p, None,
                          None) == _lib.DSA_ERR_INVALID_ARG          # mxfp4 rows must be D/2 bytes
    assert L.dsa_kv_write(p, p, _lib.DSA_BF16, p, 1, 1, 48, ctypes.byref(kv), ctypes.byref(ic), F4, p, None,
                          None) == _lib.DSA_ERR_UNSUPPORTED          # mxfp4 needs D % 32 == 0
    assert L.dsa_kv_write(p, p, _lib.DSA_BF16, p, 0, 1, 128, None, None, E4, None, None, None) == _lib.DSA_OK
    # MXFP4 keys: 64-byte rows and a 4-byte aligned block-scale array are required
    k4 = _lib.dsa_rows_t()
    k4.base, k4.row_bytes, k4.num_rows = 16, 64, 64
    assert L.dsa_indexer_scores(p, _lib.DSA_BF16, p, ctypes.byref(k4), _lib.DSA_MXFP4, None, p, 1, 1, 64, 128,
                                64, p, None, None, None) == _lib.DSA_ERR_INVALID_ARG
    assert L.dsa_indexer_scores(p, _lib.DSA_BF16, p, ctypes.byref(k4), _lib.DSA_MXFP4, ctypes.c_void_p(18), p, 1,
                                1, 64, 128, 64, p, None, None, None) == _lib.DSA_ERR_INVALID_ARG
    k4.row_bytes = 128
    assert L.dsa_indexer_scores(p, _lib.DSA_BF16, p, ctypes.byref(k4), _lib.DSA_MXFP4, p, p, 1, 1, 64, 128, 64, p,
                                None, None, None) == _lib.DSA_ERR_INVALID_ARG
    assert L.dsa_indexer_scores(p, _lib.DSA_F32, p, ctypes.byref(k4), _lib.DSA_MXFP4, p, p, 1, 1, 64, 128, 64, p,
                                None, None, None) == _lib.DSA_ERR_UNSUPPORTED
    # empty batches are valid no-ops
    assert L.dsa_topk(None, 1, None, 0, 1, 8, None, None, 0, None) == _lib.DSA_OK


def test_size_products_checked_in_64_bits():
    """Sizes whose products overflow 32 bits are rejected, not wrapped into small values."""
    L = _lib.load()
    p = ctypes.c_void_p(16)
    rows = _lib.dsa_rows_t()
    rows.base, rows.row_bytes, rows.num_rows = 16, 1152, 64
    # 2^20 x 64 query rows x 8 head groups of 16: past the 2^24 pairs one launch covers
    assert L.dsa_sparse_mla_decode(p, p, ctypes.byref(rows), 1 << 20, 64, 128, 2048, ctypes.c_float(0.1), p,
                                   _lib.DSA_BF16, p, None, 0, None, None) == _lib.DSA_ERR_UNSUPPORTED
    assert b"pairs" in L.dsa_last_error()
    # the 64-head kernel keeps row indices as 32-bit in LDS: a row store of 2^31 rows is refused
    big = _lib.dsa_rows_t()
    big.base, big.row_bytes, big.num_rows = 16, 1152, 1 << 31
    assert L.dsa_sparse_mla_decode(p, p, ctypes.byref(big), 1, 1, 128, 2048, ctypes.c_float(0.1), p,
                                   _lib.DSA_BF16, p, None, 0, None, None) == _lib.DSA_ERR_UNSUPPORTED
    assert b"num_rows" in L.dsa_last_error()
    keys = _lib.dsa_rows_t()
    keys.base, keys.row_bytes, keys.num_rows = 16, 128, 64
    # Sq * H = 2^32 wraps to 0 in 32 bits
    assert L.dsa_indexer_scores(p, _lib.DSA_BF16, p, ctypes.byref(keys), _lib.DSA_E4M3, p, p, 1, 1 << 26, 64, 128,
                                64, p, None, None, None) == _lib.DSA_ERR_UNSUPPORTED
    # Sq * k = 2^32 wraps to 0 in 32 bits
    assert L.dsa_plan(p, 1, 1 << 29, 8, p, p, p, 4, 2, 10, p, p, p, p, p, 1, None,
                      None) == _lib.DSA_ERR_UNSUPPORTED


def test_peak_probe_library_exports():
    from paged_kv_cache_indexer_amd import peaks
    out = subprocess.run(["nm", "-D", "--defined-only", peaks.LIB_PATH], capture_output=True, text=True).stdout
    names = {l.split()[-1] for l in out.splitlines() if l.strip()}
    assert {"dsa_peak_stream_read", "dsa_peak_stream_copy", "dsa_peak_mfma"} <= names
    L = peaks.load()
    assert L.dsa_peak_mfma(0, 0, 1, None, None) != 0         # rejected before any launch


def test_indexer_rejects_before_joining_the_load_stream():
    """Unsupported shapes and short key stores are rejected before the stream waits on the
    caller's event: the event passed here is not a valid handle, so a wait would fail."""
    L = _lib.load()
    p = ctypes.c_void_p(16)
    bogus_event = ctypes.c_void_p(0x1000)
    keys = _lib.dsa_rows_t()
    keys.base, keys.row_bytes, keys.num_rows = 16, 128, 16            # fewer than one 32-token tile
    keys.page_table, keys.page_size, keys.pt_stride = 16, 64, 4
    assert L.dsa_indexer_scores(p, _lib.DSA_BF16, p, ctypes.byref(keys), _lib.DSA_E4M3, p, p, 1, 1, 64, 128, 64, p,
                                None, bogus_event, None) == _lib.DSA_ERR_UNSUPPORTED
    assert b"num_rows" in L.dsa_last_error()
    keys.num_rows, keys.page_table, keys.req_stride = 1000, None, 1000  # dense, not whole tiles
    assert L.dsa_indexer_scores(p, _lib.DSA_BF16, p, ctypes.byref(keys), _lib.DSA_E4M3, p, p, 2, 1, 64, 128, 1000,
                                p, None, bogus_event, None) == _lib.DSA_ERR_UNSUPPORTED
    keys.num_rows, keys.req_stride = 1024, 500
    assert L.dsa_indexer_scores(p, _lib.DSA_BF16, p, ctypes.byref(keys), _lib.DSA_E4M3, p, p, 2, 1, 64, 128, 500,
                                p, None, bogus_event, None) == _lib.DSA_ERR_UNSUPPORTED
    keys.req_stride = 512
    # (H / 32, Sq) = (4, 4) has no instantiation
    assert L.dsa_indexer_scores(p, _lib.DSA_BF16, p, ctypes.byref(keys), _lib.DSA_E4M3, p, p, 2, 4, 128, 128, 512,
                                p, None, bogus_event, None) == _lib.DSA_ERR_UNSUPPORTED
    # fp32 path: the batch sits on the grid's y axis
    kf = _lib.dsa_rows_t()
    kf.base, kf.row_bytes, kf.num_rows = 16, 256, 1 << 20
    assert L.dsa_indexer_scores(p, _lib.DSA_F32, p, ctypes.byref(kf), _lib.DSA_F32, None, p, 70000, 1, 4, 64, 64,
                                p, None, bogus_event, None) == _lib.DSA_ERR_UNSUPPORTED


def test_fused_scan_topk_rejects_before_any_device_call():
    """dsa_indexer_topk_chunks / dsa_topk_select_chunks check every argument on the host."""
    L = _lib.load()
    rows = _lib.dsa_rows_t()
    rows.base, rows.row_bytes, rows.num_rows, rows.req_stride = 16, 128, 1 << 20, 65536
    p = ctypes.c_void_p(16)
    ws_need = L.dsa_topk_workspace_size(2, 1, 2048, 65536)

    def fused(q_dtype=_lib.DSA_BF16, k_dtype=_lib.DSA_E4M3, H=64, stride=65536, k=2048, ws_bytes=ws_need):
        return L.dsa_indexer_topk_chunks(p, q_dtype, p, ctypes.byref(rows), k_dtype, None, p, 2, H, 128, stride, p,
                                         k, p, ws_bytes, None, None, None)
    assert fused(k=0) == _lib.DSA_ERR_INVALID_ARG
    assert fused(k=9000) == _lib.DSA_ERR_UNSUPPORTED
    assert fused(q_dtype=_lib.DSA_F32, k_dtype=_lib.DSA_F32) == _lib.DSA_ERR_UNSUPPORTED   # no fp32 grid path
    assert fused(H=96) == _lib.DSA_ERR_UNSUPPORTED
    assert fused(stride=300000, ws_bytes=1 << 30) == _lib.DSA_ERR_UNSUPPORTED   # rows take work-group chunks
    assert b"wave chunks" in L.dsa_last_error()
    assert fused(ws_bytes=ws_need - 8) == _lib.DSA_ERR_WORKSPACE
    assert L.dsa_topk_select_chunks(p, 65536, p, 2, 2048, None, p, ws_need, None) == _lib.DSA_ERR_INVALID_ARG
    assert L.dsa_topk_select_chunks(p, 300000, p, 2, 2048, p, p, 1 << 30, None) == _lib.DSA_ERR_UNSUPPORTED
    assert L.dsa_topk_select_chunks(p, 65536, p, 2, 2048, p, p, ws_need - 8, None) == _lib.DSA_ERR_WORKSPACE


def test_merge_partials_rejects_bad_arguments():
    L = _lib.load()
    p = ctypes.c_void_p(16)
    assert L.dsa_merge_partials(p, _lib.DSA_F32, p, 0, 8, 512, p, _lib.DSA_BF16, p, None) == _lib.DSA_ERR_INVALID_ARG
    assert L.dsa_merge_partials(p, _lib.DSA_F32, p, 4, 8, 500, p, _lib.DSA_BF16, p, None) == _lib.DSA_ERR_INVALID_ARG
    assert L.dsa_merge_partials(p, _lib.DSA_E4M3, p, 4, 8, 512, p, _lib.DSA_BF16, p, None) == _lib.DSA_ERR_INVALID_ARG
    assert L.dsa_merge_partials(ctypes.c_void_p(24), _lib.DSA_F32, p, 4, 8, 512, p, _lib.DSA_BF16, p,
                                None) == _lib.DSA_ERR_INVALID_ARG
    assert L.dsa_merge_partials(None, _lib.DSA_F32, p, 4, 8, 512, p, _lib.DSA_BF16, p, None) == _lib.DSA_ERR_INVALID_ARG
    assert L.dsa_merge_partials(None, _lib.DSA_F32, None, 4, 0, 512, None, _lib.DSA_BF16, None, None) == _lib.DSA_OK
