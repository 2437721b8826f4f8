"""dsa_sparse_mla_decode_noalloc, called through the C ABI, gives exactly the output of
dsa_sparse_mla_decode with a caller workspace: three calls in a row (the row-stream form,
then two split-form calls, each smaller than the one before, while the scratch array keeps
the earlier call's contents), and a call too large for the array is rejected before anything
is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_indexer_amd as dsa
from paged_kv_cache_indexer_amd import _lib
import synth
from tests.dsa_dev import DEV, DevWorkload

pytestmark = pytest.mark.gpu


def _call_noalloc(dw, idx, o, lse):
    L = _lib.load()
    B, Sq, H, _ = dw.mla_q.shape
    st = L.dsa_sparse_mla_decode_noalloc(ctypes.c_void_p(dw.mla_q.data_ptr()), ctypes.c_void_p(idx.data_ptr()),
                                         dw.rows.ref(), B, Sq, H, idx.shape[-1], ctypes.c_float(dw.wl.scale),
                                         ctypes.c_void_p(o.data_ptr()), _lib.DSA_BF16 if o.dtype == torch.bfloat16
                                         else _lib.DSA_F32, ctypes.c_void_p(lse.data_ptr()),
                                         ctypes.c_void_p(dw.err.data_ptr()),
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def test_noalloc_matches_the_workspace_entry_point():
    L = _lib.load()
    assert L.dsa_sparse_mla_noalloc_max_workspace() == 64 << 20
    cases = [(synth.spec(2).scaled(B=66, L=2600), torch.bfloat16),    # row-stream form, 388 partial slots
             (synth.spec(2).scaled(B=16, L=30000), torch.bfloat16),   # 4 splits, bf16 partials
             (synth.spec(3).scaled(B=3, L=9000, mla_heads=64), torch.float32)]   # smaller, fp32 partials
    for cfg, odt in cases:
        wl = synth.make_workload(cfg)
        dw = DevWorkload(wl)
        idx = dw.topk(dw.scores())
        B, Sq, H = wl.B, wl.Sq, wl.mla_q.shape[2]
        assert 0 < dsa.dsa_sparse_mla_workspace_size(B, Sq, H, wl.topk) <= L.dsa_sparse_mla_noalloc_max_workspace()
        want_o, want_l = dw.mla(idx, o_dtype=odt)
        o = torch.full((B, Sq, H, 512), float("nan"), dtype=odt, device=DEV)
        lse = torch.full((B, Sq, H), float("nan"), dtype=torch.float32, device=DEV)
        assert _call_noalloc(dw, idx, o, lse) == _lib.DSA_OK, L.dsa_last_error()
        torch.cuda.synchronize()
        assert int(dw.err) == 0
        assert torch.equal(o.view(torch.uint8), want_o.view(torch.uint8))
        assert torch.equal(lse.view(torch.uint8), want_l.view(torch.uint8))
        assert torch.isfinite(lse).all()


def test_noalloc_rejects_sizes_beyond_the_scratch_array():
    L = _lib.load()
    p = ctypes.c_void_p(16)
    rows = _lib.dsa_rows_t()
    rows.base, rows.row_bytes, rows.num_rows = 16, 1152, 1 << 20
    # 64 requests x 4 query tokens x 128 heads x 2048 rows: 128 MiB of split partials
    B, Sq, H, k = 64, 4, 128, 2048
    assert L.dsa_sparse_mla_workspace_size(B, Sq, H, k) > L.dsa_sparse_mla_noalloc_max_workspace()
    assert L.dsa_sparse_mla_decode_noalloc(p, p, ctypes.byref(rows), B, Sq, H, k, ctypes.c_float(0.1), p,
                                           _lib.DSA_BF16, p, None, None) == _lib.DSA_ERR_UNSUPPORTED
    assert b"scratch" in L.dsa_last_error()
