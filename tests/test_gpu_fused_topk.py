"""The scan with the top-k's chunk stage in its epilogue (dsa_indexer_topk_chunks, then
dsa_topk_select_chunks): scores bit-identical to dsa_indexer_scores, indices bit-identical to
dsa_topk on those scores and to the oracle's select ("Shared-Indexer KV Cache Offload for
GLM-5.2", §2.1: the scores feed the top-2048), over decode workloads with bf16 and fp8
queries, e4m3 and MXFP4 keys, 32 / 64 / 128 heads, and mixed lengths (rows shorter than k,
partial last units)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_indexer_amd as dsa
import synth
from oracle import topk as o_topk
from tests.dsa_dev import DEV, DevWorkload, t_i32

pytestmark = pytest.mark.gpu


def _fused_vs_separate(dw):
    wl = dw.wl
    B, L, k = wl.B, dw.Lmax, wl.topk
    sc_ref = dw.scores()
    idx_ref = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
    dsa.dsa_topk(sc_ref, dw.seq_lens, idx_ref)
    sc = torch.full((B, 1, L), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.full((max(1, dsa.dsa_topk_workspace_size(B, 1, k, L)),), 0x5A, dtype=torch.uint8, device=DEV)
    idx = torch.full((B, 1, k), 7, dtype=torch.int32, device=DEV)
    dsa.dsa_indexer_topk_chunks(dw.idx_q, dw.idx_w, dw.keys, dw.k_scale, dw.seq_lens, sc, k, ws,
                                k_dtype=dw.k_dtype, err=dw.err, q_dtype=dw.q_dtype)
    dsa.dsa_topk_select_chunks(sc, dw.seq_lens, idx, ws)
    torch.cuda.synchronize()
    assert int(dw.err) == 0
    a, b = sc.cpu().numpy(), sc_ref.cpu().numpy()
    for r in range(B):
        n = int(wl.seq_lens[r])
        assert np.array_equal(a[r, 0, :n].view(np.uint32), b[r, 0, :n].view(np.uint32)), r
    got = idx.cpu().numpy()
    assert np.array_equal(got, idx_ref.cpu().numpy())
    for r in range(B):
        n = int(wl.seq_lens[r])
        assert np.array_equal(got[r, 0], o_topk.select(a[r, 0, :n], k)), r
    return got


@pytest.mark.parametrize("case", ["c2_bf16_e4m3", "c2_mxfp4", "fp8_q_h32", "h128", "mixed_lengths"])
def test_fused_scan_topk_matches_separate_calls(case):
    if case == "c2_bf16_e4m3":
        cfg = synth.spec(2).scaled(B=6, L=40000)
    elif case == "c2_mxfp4":
        cfg = synth.spec(2).scaled(B=4, L=33000, idx_k_kind="mxfp4")
    elif case == "fp8_q_h32":
        cfg = synth.spec(3).scaled(B=5, Sq=1, L=26001, idx_heads=32)
    elif case == "h128":
        cfg = synth.spec(2).scaled(B=3, L=17000, idx_heads=128, topk=512)
    else:                                          # mixed lengths: short rows (n <= k), partial units
        cfg = synth.spec(5).scaled(n_short=9, short_lo=1500, short_hi=60000, n_long=1, long_len=200000)
    dw = DevWorkload(synth.make_workload(cfg, with_kv=False), with_kv=False)
    _fused_vs_separate(dw)


def test_fused_scan_topk_rows_the_candidates_cannot_settle():
    """Rows whose answer the chunk candidates cannot prove, so the select goes back to the
    scores the scan wrote: request 0 has a 700-position window of keys that outscore every
    other key (distinct scales, so distinct scores), all inside one 1024-position chunk that
    keeps at most 2 * 32 + 16 candidates; request 1 has an all-zero key cache, so every score
    is +0 and the answer is its first 2048 positions.  Fused and separate calls and the
    oracle's select must agree."""
    wl = synth.make_workload(synth.spec(2).scaled(B=4, L=40000), with_kv=False)
    ps = wl.page_size
    lo, width = 2100, 700
    for j in range(width):
        pos = lo + j
        pg, slot = wl.page_table[0, pos // ps], pos % ps
        wl.idx_k[pg, slot, :] = 0x7E               # e4m3 448 in every dim
        wl.idx_k_scale[pg, slot] = np.float32(1.0 + j / 4096.0)
    wl.idx_k[wl.page_table[1, : -(-int(wl.seq_lens[1]) // ps)]] = 0
    dw = DevWorkload(wl, with_kv=False)
    got = _fused_vs_separate(dw)
    sel0 = got[0, 0]
    # the window's chunk holds far more of the answer than its candidate slots
    assert np.count_nonzero((sel0 >= 2048) & (sel0 < 3072)) >= width > 2 * 32 + 16
    assert np.array_equal(got[1, 0], np.arange(2048, dtype=np.int32))


def test_fused_scan_topk_through_the_decode_step():
    """DecodeStep takes the fused entry points for one query token; its indices equal the
    unfused step's, eager and replayed from a graph."""
    wl = synth.make_workload(synth.spec(2).scaled(B=4, L=12000, mla_heads=16))
    dw = DevWorkload(wl)
    steps = {f: dw.decode_step(2, fused=f) for f in (True, False)}
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for st in steps.values():
            st.run(stream, layer=1)
    torch.cuda.synchronize()
    assert steps[True].fused is True
    assert torch.equal(steps[True].idx, steps[False].idx)
    assert torch.equal(steps[True].o.view(torch.int16), steps[False].o.view(torch.int16))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        steps[True].run(stream, layer=0)
    for _ in range(3):
        steps[True].idx.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            steps[False].run(stream, layer=0)
        torch.cuda.synchronize()
        assert torch.equal(steps[True].idx, steps[False].idx)


def test_fused_entry_rejects_rows_that_take_work_group_chunks():
    """Rows longer than the wave chunks serve (score_stride 300000) are rejected with nothing
    enqueued; the decode step then takes the separate calls."""
    wl = synth.make_workload(synth.spec(2).scaled(B=2, L=3000), with_kv=False)
    dw = DevWorkload(wl, with_kv=False)
    sc = torch.zeros((2, 1, 300000), dtype=torch.float32, device=DEV)
    ws = torch.empty((dsa.dsa_topk_workspace_size(2, 1, 2048, 300000),), dtype=torch.uint8, device=DEV)
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_indexer_topk_chunks(dw.idx_q, dw.idx_w, dw.keys, dw.k_scale, dw.seq_lens, sc, 2048, ws,
                                    k_dtype=dw.k_dtype, q_dtype=dw.q_dtype)
    assert "wave chunks" in str(e.value)
    torch.cuda.synchronize()
    assert int(sc.abs().sum()) == 0
