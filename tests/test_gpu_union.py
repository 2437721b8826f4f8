"""The union of a request's query selections and attention over it (the de-duplicated
multi-query gather): dsa_topk_union bit for bit against the oracle's union, and
dsa_sparse_mla_decode_union (query tokens packed into the work-group's heads) against the
oracle's attention of every query token over its own selection."""
import numpy as np
import pytest
import torch

import paged_kv_cache_indexer_amd as dsa
import synth
from oracle import gather as o_gather
from oracle.step import decode_request
from tests.dsa_dev import DEV, DevWorkload, bf16_to_f64, t_i32
from tests.test_gpu_kernels import LSE_MAX, O_MAX, O_MEAN

pytestmark = pytest.mark.gpu


def run_union(tk: np.ndarray):
    B, Sq, k = tk.shape
    W = (Sq * k + 31) // 32
    uni = torch.full((B, Sq * k), 7, dtype=torch.int32, device=DEV)
    cnt = torch.empty(B, dtype=torch.int32, device=DEV)
    uidx = torch.full((B, Sq, k), 7, dtype=torch.int32, device=DEV)
    member = torch.full((B, Sq, W), 0x55555555, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    dsa.dsa_topk_union(t_i32(tk), uni, cnt, uidx, member, err=err)
    torch.cuda.synchronize()
    assert int(err) == 0
    return uni.cpu().numpy(), cnt.cpu().numpy(), uidx.cpu().numpy(), member.cpu().numpy().view(np.uint32)


def check_union(tk, uni, cnt, uidx, member):
    B, Sq, k = tk.shape
    for b in range(B):
        U, ui, mem = o_gather.union_select(tk[b])
        n = len(U)
        assert cnt[b] == n and np.array_equal(uni[b, :n], U) and (uni[b, n:] == -1).all(), b
        assert np.array_equal(uidx[b], ui), b
        bits = np.unpackbits(member[b].view(np.uint8), bitorder="little").reshape(Sq, -1)
        assert np.array_equal(bits[:, :n].astype(bool), mem), b
        assert not bits[:, n:].any(), b


def random_selections(rng, B, Sq, k, L, keep):
    out = np.full((B, Sq, k), -1, dtype=np.int32)
    for b in range(B):
        prev = rng.choice(L, size=k, replace=False)
        for t in range(Sq):
            n_valid = k if (b + t) % 3 else k - int(rng.integers(1, max(2, k // 4)))
            kk = min(int(keep * k), n_valid, len(prev))
            kept = rng.choice(prev, size=kk, replace=False)
            fresh = rng.choice(np.setdiff1d(np.arange(L), kept), size=n_valid - kk, replace=False)
            row = np.sort(np.concatenate([kept, fresh]))
            out[b, t, :n_valid] = row
            prev = row
    return out


@pytest.mark.parametrize("B,Sq,k,keep", [(3, 1, 100, 0.0), (4, 2, 256, 0.6), (2, 4, 2048, 0.65), (2, 8, 1024, 0.3),
                                         (3, 4, 33, 1.0), (1, 16, 512, 0.5)])
def test_topk_union_bit_exact(B, Sq, k, keep):
    rng = np.random.default_rng(B * 1000 + Sq * 10 + k)
    tk = random_selections(rng, B, Sq, k, 300000, keep)
    check_union(tk, *run_union(tk))


def test_topk_union_rejects_and_counts():
    tk = np.array([[[5, 3, 9, -1]]], dtype=np.int32)      # a row out of order
    uni = torch.empty((1, 4), dtype=torch.int32, device=DEV)
    cnt = torch.empty(1, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    dsa.dsa_topk_union(t_i32(tk), uni, cnt, err=err)
    torch.cuda.synchronize()
    assert int(err) == 1
    with pytest.raises(dsa.DsaError):
        dsa.dsa_topk_union(torch.zeros((1, 4, 4096), dtype=torch.int32, device=DEV), uni, cnt)


@pytest.mark.parametrize("H", [16, 128])
def test_union_attention_matches_each_query_over_its_own_selection(H):
    """MTP verify with draft-correlated queries (4 query tokens), reduced context: indexer ->
    top-k per query -> union -> packed attention over the union; every (request, query token)
    against the oracle's attention over that query's own selection, and against the per-query
    attention of dsa_sparse_mla_decode."""
    wl = synth.make_workload(synth.spec(3).scaled(B=2, L=20004, mla_heads=H, draft_sigma=0.3))
    dw = DevWorkload(wl)
    idx = dw.topk(dw.scores())
    o_ref_gpu, lse_ref_gpu = dw.mla(idx)
    tk = idx.cpu().numpy()
    uni, cnt, uidx, member = run_union(tk)
    check_union(tk, uni, cnt, uidx, member)
    B, Sq = wl.B, wl.Sq
    U = Sq * wl.topk
    o = torch.empty((B, Sq, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Sq, H), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(1, dsa.dsa_sparse_mla_union_workspace_size(B, Sq, H, U)), dtype=torch.uint8, device=DEV)
    dsa.dsa_sparse_mla_decode_union(dw.mla_q, t_i32(uni), t_i32(cnt), t_i32(member.view(np.int32)), dw.rows,
                                    wl.scale, o, lse, ws=ws, err=dw.err)
    torch.cuda.synchronize()
    assert int(dw.err) == 0
    for b in range(B):
        assert cnt[b] < Sq * wl.topk               # the drafts' selections overlap
        ref = decode_request(wl, b, topk_override=tk[b])
        d = np.abs(bf16_to_f64(o[b]) - ref["o"])
        assert d.max() <= O_MAX and d.mean() <= O_MEAN, (b, d.max(), d.mean())
        assert np.abs(lse[b].cpu().numpy().astype(np.float64) - ref["lse"]).max() <= LSE_MAX, b
        # and against the per-query path on the same selection
        d2 = np.abs(bf16_to_f64(o[b]) - bf16_to_f64(o_ref_gpu[b]))
        assert d2.max() <= O_MAX, b
        assert np.abs((lse[b] - lse_ref_gpu[b]).cpu().numpy()).max() <= LSE_MAX, b


def test_union_attention_skips_entries_past_count():
    """Entries past count[b] are never read: poisoned positions there change nothing."""
    wl = synth.make_workload(synth.spec(3).scaled(B=2, L=9004, mla_heads=16, draft_sigma=0.3))
    dw = DevWorkload(wl)
    tk = dw.topk(dw.scores()).cpu().numpy()
    uni, cnt, uidx, member = run_union(tk)
    B, Sq, H = wl.B, wl.Sq, 16
    U = Sq * wl.topk
    outs = []
    for poison in (False, True):
        u2 = uni.copy()
        if poison:
            for b in range(B):
                u2[b, cnt[b]:] = 123                  # a valid position, wrongly past the count
        o = torch.empty((B, Sq, H, 512), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((B, Sq, H), dtype=torch.float32, device=DEV)
        ws = torch.empty(max(1, dsa.dsa_sparse_mla_union_workspace_size(B, Sq, H, U)), dtype=torch.uint8, device=DEV)
        dsa.dsa_sparse_mla_decode_union(dw.mla_q, t_i32(u2), t_i32(cnt), t_i32(member.view(np.int32)), dw.rows,
                                        wl.scale, o, lse, ws=ws, err=dw.err)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1])


def test_union_serve_over_the_pool_matches_per_entry_serve_and_the_oracle():
    """MTP verify over the device pool (4 query tokens whose selections overlap, 2 layers, 3
    steps): serving the union once per layer gives every query token the attention of the
    oracle over the host rows of its own selection, like serving every entry on its own,
    while fewer rows cross the host link."""
    from synth import gen as sgen
    from oracle import mla as o_mla, plan as o_plan
    from paged_kv_cache_indexer_amd.pipeline import MtpVerifyPoolStep
    from tests.test_gpu_pool_pipeline import _host_rows
    cfg = synth.spec(4).scaled(B=2, L=16384, steps=3, layers=2, id_range=16384)
    traj = sgen.topk_trajectory(cfg)
    hosts = _host_rows(cfg, cfg.layers)
    rows = [r for _, r in hosts]
    Sq, H, k = 4, 32, cfg.topk
    g = torch.Generator().manual_seed(5)
    steps = {u: MtpVerifyPoolStep(cfg.B, Sq, k, H, cfg.n_sets, cfg.ways, cfg.id_range, rows, cfg.scale, union=u)
             for u in (True, False)}
    stream = torch.cuda.Stream()
    state = [o_plan.empty_state(cfg.n_sets, cfg.ways, cfg.id_range) for _ in range(cfg.B)]
    for s in range(cfg.steps):
        tk = sgen.draft_selections(cfg, traj[s], Sq, 0.65, s)
        q = [torch.randn(cfg.B, Sq, H, 576, generator=g).to(torch.bfloat16).to(DEV) for _ in range(cfg.layers)]
        served = {}
        for u, st in steps.items():
            st.run(stream, t_i32(tk), q)
            torch.cuda.synchronize()
            assert int(st.err) == 0
            po = st.plan_out
            if u:
                served[u] = int(po["mc"].sum())                       # distinct misses of the union
            else:
                served[u] = int(((po["is_hit"] == 0) & (t_i32(tk) >= 0)).sum())   # every missing entry
        # the union's distinct misses are the oracle's: the plan over the union is the plan of the step
        want = 0
        for b in range(cfg.B):
            out, state[b] = o_plan.plan_step(tk[b], *state[b], cfg.n_sets, cfg.ways)
            want += out["miss_count"]
        assert served[True] == want <= served[False]
        for l, (h, _) in enumerate(hosts):
            host_np = h.numpy().view(np.uint16)
            for b in range(cfg.B):
                for t in range(Sq):
                    o_ref, l_ref = o_mla.sparse_mla(q[l].view(torch.int16).cpu().numpy().view(np.uint16)[b, t],
                                                    host_np[b * cfg.L + tk[b, t]], cfg.scale)
                    for st in steps.values():
                        d = np.abs(bf16_to_f64(st.o[l][b, t]) - o_ref)
                        assert d.max() <= O_MAX and d.mean() <= O_MEAN, (s, l, b, t)
                        assert np.abs(st.lse[l][b, t].cpu().numpy().astype(np.float64) - l_ref).max() <= LSE_MAX
            # the union buffer holds the host rows of the union
            st = steps[True]
            uni, cnt = st.uni.cpu().numpy()[:, 0], st.count.cpu().numpy()
            sel = st.sel[l].view(torch.int16).cpu().numpy().view(np.uint16)
            for b in range(cfg.B):
                assert np.array_equal(sel[b, :cnt[b]], host_np[b * cfg.L + uni[b, :cnt[b]]])
        print(f"step {s}: host-link rows served, union {served[True]} vs per entry {served[False]}")
    # both committed the same plans, so both pools hold the same rows
    assert torch.equal(steps[True].pids, steps[False].pids)
    for a_, b_ in zip(steps[True].pool, steps[False].pool):
        assert torch.equal(a_, b_)
