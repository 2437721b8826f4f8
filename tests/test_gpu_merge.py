"""Merging page-sharded partial attention (HiCache page §1.1: each rank holds and attends over
only its own pages; TokenSpeed audit page "MLA": partials combined by LSE rescaling).

All four ranks' shares of a reduced mixed-length workload run through libdsa one after
another on the one GPU (indexer, top-k over owned tokens, sparse MLA with float32 partial
o); dsa_merge_partials combines them, and the result must equal the oracle's attention over
the union of the four owned selections."""
import numpy as np
import pytest
import torch

import paged_kv_cache_indexer_amd as dsa
import synth
from oracle import mla as o_mla, topk as o_topk
from oracle.step import selected_rows
from tests.dsa_dev import DEV, DevWorkload, bf16_to_f64
from tests.test_gpu_kernels import LSE_MAX, O_MAX, O_MEAN

pytestmark = pytest.mark.gpu


def _rank_shares(cfg):
    parts = []
    for r in range(cfg.n_ranks):
        wl = synth.make_workload(cfg.scaled(rank=r))
        dw = DevWorkload(wl)
        sc = dw.scores()
        idx = dw.topk(sc)
        o, lse = dw.mla(idx, o_dtype=torch.float32)
        torch.cuda.synchronize()
        assert int(dw.err) == 0
        sc_np, idx_np = sc.cpu().numpy(), idx.cpu().numpy()
        for b in range(wl.B):       # each rank's selection is the exact top-k of its own scores
            L = int(wl.seq_lens[b])
            assert np.array_equal(idx_np[b, 0], o_topk.select(sc_np[b, 0, :L], wl.topk)), (r, b)
        parts.append((wl, idx_np, o, lse))
    return parts


def test_four_rank_shares_merge_to_attention_over_the_union():
    cfg = synth.spec(5).scaled(n_short=6, short_lo=3000, short_hi=20000, n_long=1, long_len=60000)
    parts = _rank_shares(cfg)
    wl0 = parts[0][0]
    B, H = wl0.B, wl0.mla_q.shape[2]
    o_parts = torch.stack([p[2] for p in parts])                   # [4, B, 1, H, 512] float32
    lse_parts = torch.stack([p[3] for p in parts])                 # [4, B, 1, H]
    o = torch.empty((B, 1, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, 1, H), dtype=torch.float32, device=DEV)
    dsa.dsa_merge_partials(o_parts, lse_parts, o, lse)
    o32 = torch.empty((B, 1, H, 512), dtype=torch.float32, device=DEV)
    lse32 = torch.empty_like(lse)
    dsa.dsa_merge_partials(o_parts, lse_parts, o32, lse32)
    torch.cuda.synchronize()
    # the GPU merge against the oracle's merge of the same partials (float64)
    po, pl = o_parts.cpu().numpy().astype(np.float64), lse_parts.cpu().numpy().astype(np.float64)
    for b in range(B):
        mo, ml = o_mla.lse_merge([po[r, b, 0] for r in range(4)], [pl[r, b, 0] for r in range(4)])
        assert np.abs(o32[b, 0].cpu().numpy() - mo).max() <= 1e-5 * max(1.0, np.abs(mo).max())
        assert np.abs(lse32[b, 0].cpu().numpy() - ml).max() <= 1e-5 * max(1.0, np.abs(ml).max())
    # the merged result against the oracle's attention over the union of the owned selections
    for b in range(B):
        rows = np.concatenate([selected_rows(wl, b, idx_np[b, 0]) for wl, idx_np, _, _ in parts])
        assert len(rows) == sum(min(wl.topk, int(wl.seq_lens[b])) for wl, _, _, _ in parts)
        o_ref, l_ref = o_mla.sparse_mla(wl0.mla_q[b, 0], rows, wl0.scale)
        d = np.abs(bf16_to_f64(o[b, 0]) - o_ref)
        assert d.max() <= O_MAX and d.mean() <= O_MEAN, (b, d.max(), d.mean())
        assert np.abs(lse[b, 0].cpu().numpy().astype(np.float64) - l_ref).max() <= LSE_MAX, b


@pytest.mark.parametrize("R,V,pdt,odt", [(4, 512, torch.float32, torch.bfloat16), (3, 64, torch.bfloat16,
                                                                                     torch.float32),
                                         (1, 512, torch.float32, torch.float32), (8, 1040, torch.bfloat16,
                                                                                  torch.bfloat16)])
def test_merge_partials_against_the_oracle_merge(R, V, pdt, odt):
    """Random partials, some parts empty (lse = -inf), one row with every part empty."""
    g = torch.Generator().manual_seed(R * 1000 + V)
    N = 77
    o_parts = torch.randn(R, N, V, generator=g).to(pdt)
    lse_parts = (torch.randn(R, N, generator=g) * 6).float()
    lse_parts[0, 5] = float("-inf")
    lse_parts[R - 1, 9] = float("-inf")
    lse_parts[:, 13] = float("-inf")
    o = torch.empty(N, V, dtype=odt, device=DEV)
    lse = torch.empty(N, dtype=torch.float32, device=DEV)
    dsa.dsa_merge_partials(o_parts.to(DEV), lse_parts.to(DEV), o, lse)
    torch.cuda.synchronize()
    po, pl = o_parts.float().numpy().astype(np.float64), lse_parts.numpy().astype(np.float64)
    mo, ml = o_mla.lse_merge([po[r] for r in range(R)], [pl[r] for r in range(R)])
    got_o, got_l = o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    assert np.isneginf(got_l[13]) and (got_o[13] == 0).all()
    fin = np.isfinite(ml)
    assert np.array_equal(np.isfinite(got_l), fin)
    assert np.abs(got_l[fin] - ml[fin]).max() <= 1e-5 * np.abs(ml[fin]).max()
    rel = 2.0 ** -8 if odt == torch.bfloat16 else 1e-5
    assert (np.abs(got_o - mo) <= rel * np.abs(mo) + 1e-5).all()
