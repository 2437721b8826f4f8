"""Parity at the workloads' full sizes, on sampled requests the oracle computes one by one.

Every call goes through the C ABI in the launch configuration the benchmark uses.  The
oracle is run for a few sampled requests of each workload; properties that hold at any
size are checked for all of them.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_indexer_amd as dsa
import synth
from synth import gen as sgen
from oracle import indexer as o_idx, mla as o_mla, paging as o_pg, plan as o_plan, topk as o_topk
from oracle.step import decode_request, selected_rows
from tests.dsa_dev import DecodeStep, DevWorkload, bf16_to_f64, host_device_ptr, t_i32, t_u16_as_bf16, DEV
from tests.test_gpu_kernels import O_MAX, O_MEAN, LSE_MAX, indexer_bound

pytestmark = pytest.mark.gpu


def check_request(wl, b, sc_gpu, idx_gpu, o_gpu, lse_gpu):
    """Scores within the fp32 bound; top-k exact on the GPU's scores and within the error
    band of the oracle's own selection; attention on the GPU's selection within tolerance.
    Returns the number of top-k swaps against the oracle's selection."""
    L = int(wl.seq_lens[b])
    got_idx = idx_gpu[b]
    ref = decode_request(wl, b, topk_override=got_idx)
    swaps = 0
    for t in range(wl.Sq):
        n = o_idx.visible_len(L, wl.Sq, t)
        bound = indexer_bound(wl, b, t, n)
        ref_sc = ref["scores"][t, :n].astype(np.float64)
        gpu_sc = sc_gpu[b, t, :n]
        assert (np.abs(gpu_sc.astype(np.float64) - ref_sc) <= bound).all(), f"b={b} t={t} scores"
        assert np.isneginf(sc_gpu[b, t, n:L]).all()
        # the selection the GPU made is the exact top-k of the scores it computed
        assert np.array_equal(got_idx[t], o_topk.select(gpu_sc, wl.topk)), f"b={b} t={t} top-k"
        # against the oracle's selection: only swaps between entries within the error band of
        # the k-th score
        mine, theirs = set(got_idx[t].tolist()), set(ref["topk"][t].tolist())
        kth = np.sort(ref_sc)[-wl.topk] if n > wl.topk else -np.inf
        pk = int(np.argmin(np.abs(ref_sc - kth))) if n > wl.topk else 0
        for p in mine ^ theirs:
            assert abs(ref_sc[p] - kth) <= bound[p] + bound[pk], f"b={b} t={t} swap at {p} outside the band"
        swaps += len(mine - theirs)
    o = bf16_to_f64(o_gpu[b]) if o_gpu.dtype == torch.bfloat16 else o_gpu[b].cpu().numpy().astype(np.float64)
    d = np.abs(o - ref["o"])
    assert d.max() <= O_MAX and d.mean() <= O_MEAN, f"b={b}: o max {d.max():.3g} mean {d.mean():.3g}"
    lg = lse_gpu[b].cpu().numpy().astype(np.float64)
    assert np.abs(lg - ref["lse"]).max() <= LSE_MAX, f"b={b}: lse"
    return swaps


def check_all_rows(wl, idx):
    """Every selection is ascending, distinct, within the visible range and full."""
    for b in range(wl.B):
        L = int(wl.seq_lens[b])
        for t in range(wl.Sq):
            n = o_idx.visible_len(L, wl.Sq, t)
            row = idx[b, t]
            valid = row[row >= 0]
            assert len(valid) == min(n, wl.topk)
            assert (np.diff(valid) > 0).all() and valid.min() >= 0 and valid.max() < n


def test_decode_b32_ctx65536_full_step():
    """The benchmarked workload (B=32, 64K context, top-2048, 128 heads), as DecodeStep runs it
    (the scan with the top-k chunk stage in its epilogue).  The oracle's scores are computed
    for three sampled requests; for every one of the 32, the selection is the exact top-k of
    the scores the GPU wrote and the attention over it matches the oracle's."""
    wl = synth.make_workload(2)
    dw = DevWorkload(wl)
    step = dw.decode_step()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        step.run(stream)
    torch.cuda.synchronize()
    assert int(dw.err) == 0 and step.fused
    sc, idx = step.scores.cpu().numpy(), step.idx.cpu().numpy()
    check_all_rows(wl, idx)
    assert torch.isfinite(step.lse).all()
    swaps = sum(check_request(wl, b, sc, idx, step.o, step.lse) for b in (0, 13, 31))
    print(f"top-k swaps against the oracle's selection: {swaps}")
    o_all, lse_all = bf16_to_f64(step.o), step.lse.cpu().numpy().astype(np.float64)
    for b in range(wl.B):
        L = int(wl.seq_lens[b])
        assert np.array_equal(idx[b, 0], o_topk.select(sc[b, 0, :L], wl.topk)), b
        o_ref, l_ref = o_mla.sparse_mla(wl.mla_q[b, 0], selected_rows(wl, b, idx[b, 0]), wl.scale)
        d = np.abs(o_all[b, 0] - o_ref)
        assert d.max() <= O_MAX and d.mean() <= O_MEAN, (b, d.max(), d.mean())
        assert np.abs(lse_all[b, 0] - l_ref).max() <= LSE_MAX, b


@pytest.mark.parametrize("cid", [2, 3])
def test_full_step_over_the_fp4_indexer_cache(cid):
    """The decode (B=32, 64K, bf16 queries) and MTP-verify (B=8, 200K, fp8 queries) steps
    with MXFP4 indexer keys instead of e4m3, full size, sampled requests against the oracle."""
    wl = synth.make_workload(synth.spec(cid).scaled(idx_k_kind="mxfp4"), with_kv=True)
    dw = DevWorkload(wl)
    step = dw.decode_step()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        step.run(stream)
    torch.cuda.synchronize()
    assert int(dw.err) == 0
    sc, idx = step.scores.cpu().numpy(), step.idx.cpu().numpy()
    check_all_rows(wl, idx)
    assert torch.isfinite(step.lse).all()
    swaps = sum(check_request(wl, b, sc, idx, step.o, step.lse) for b in ((0, 31) if cid == 2 else (3,)))
    print(f"top-k swaps against the oracle's selection: {swaps}")


def test_mtp_verify_b8_ctx200k_full_step():
    """Four draft queries per request (fp8 queries, causal visibility), full size."""
    wl = synth.make_workload(3)
    dw = DevWorkload(wl)
    step = dw.decode_step()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        step.run(stream)
    torch.cuda.synchronize()
    assert int(dw.err) == 0
    sc, idx = step.scores.cpu().numpy(), step.idx.cpu().numpy()
    check_all_rows(wl, idx)
    swaps = sum(check_request(wl, b, sc, idx, step.o, step.lse) for b in (0, 7))
    print(f"top-k swaps against the oracle's selection: {swaps}")


def test_rank0_share_mixed_lengths_full():
    """Rank 0's share of a page-sharded cache (66 requests, 30K-200K and two 1M contexts).

    Every owned slot's logical id translates to rank 0 and to the physical row the local
    page table names; scores, top-k and fp32 partial attention match on sampled requests.
    """
    wl = synth.make_workload(5)
    N, ps = wl.extra["n_ranks"], wl.page_size
    qids, full = wl.extra["logical_page_ids"], wl.extra["full_lens"]
    xs, want = [], []
    for b in range(wl.B):
        npg = (int(full[b]) + ps - 1) // ps
        for i, j in enumerate(range(0, npg, N)):
            n = min(ps, int(full[b]) - j * ps)
            xs.append(qids[b, j] * ps + np.arange(n))
            want.append(int(wl.page_table[b, i]) * ps + np.arange(n))
    x, want = np.concatenate(xs).astype(np.int64), np.concatenate(want).astype(np.int64)
    rank = torch.empty(len(x), dtype=torch.int32, device=DEV)
    local = torch.empty(len(x), dtype=torch.int64, device=DEV)
    dsa.dsa_page_translate(torch.from_numpy(x).to(DEV), ps, N, rank, local)
    assert (rank.cpu().numpy() == 0).all()
    assert np.array_equal(local.cpu().numpy(), want)
    assert np.array_equal(local.cpu().numpy(), o_pg.owner_local(x, ps, N)[1])

    dw = DevWorkload(wl)
    sc = dw.scores()
    idx = dw.topk(sc)
    o, lse = dw.mla(idx, o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert int(dw.err) == 0
    sc_np, idx_np = sc.cpu().numpy(), idx.cpu().numpy()
    check_all_rows(wl, idx_np)
    longest = int(np.argmax(wl.seq_lens))
    swaps = sum(check_request(wl, b, sc_np, idx_np, o, lse) for b in (0, 40, longest))
    print(f"top-k swaps against the oracle's selection: {swaps}")


def test_pool_group_b16_ctx128k_full_trajectory():
    """The device pool over the 8-step trajectory at full size (16 requests, 128K context,
    1024 sets x 8 ways): plan bit-exact against the oracle at every step, serve bytes equal
    to the host rows (hits from the pool, misses over the host link from pinned memory),
    install leaves every live pool row equal to its host row, and attention over the served
    rows matches."""
    cfg = synth.spec(4)
    wl = synth.make_workload(cfg, with_kv=False)
    traj = wl.extra["traj"]                                  # [steps, B, k]
    B, L, k, S, W = cfg.B, cfg.L, cfg.topk, cfg.n_sets, cfg.ways
    layer = 0
    host = torch.empty((B * L, cfg.kv_dim), dtype=torch.int16, pin_memory=True)
    host_np = host.numpy().view(np.uint16)
    for b in range(B):
        sgen.normal_bf16_rows((cfg.seed, cfg.cid, sgen.T_HOSTKV, layer, b), L, cfg.kv_dim,
                              out=host_np[b * L:(b + 1) * L])
    src = dsa.Rows(host, 1152, req_stride=L, base_ptr=host_device_ptr(host))
    pool = torch.zeros((B, S * W, cfg.kv_dim), dtype=torch.bfloat16, device=DEV)
    pids = torch.full((B, S * W), -1, dtype=torch.int32, device=DEV)
    its = torch.full((B, cfg.id_range), -1, dtype=torch.int32, device=DEV)
    ptr = torch.zeros((B, S), dtype=torch.int32, device=DEV)
    state = [o_plan.empty_state(S, W, cfg.id_range) for _ in range(B)]
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    H = cfg.mla_heads
    hits = []
    for s in range(cfg.steps):
        tk = traj[s][:, None, :]
        tkd = t_i32(tk)
        is_hit = torch.empty((B, 1, k), dtype=torch.uint8, device=DEV)
        slot = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
        mp = torch.empty((B, k), dtype=torch.int32, device=DEV)
        ms = torch.empty((B, k), dtype=torch.int32, device=DEV)
        mc = torch.empty(B, dtype=torch.int32, device=DEV)
        dsa.dsa_plan(tkd, pids, its, ptr, S, W, is_hit, slot, mp, ms, mc, commit=False, err=err)
        sel = torch.empty((B, 1, k, cfg.kv_dim), dtype=torch.bfloat16, device=DEV)
        sel_idx = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
        dsa.dsa_gather_kv(tkd, is_hit, slot, src, pool, sel, dsa.DSA_GATHER_SERVE, err=err, sel_idx=sel_idx)
        q = t_u16_as_bf16(wl.extra["mla_q"][s, layer][:, None])
        o = torch.empty((B, 1, H, 512), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((B, 1, H), dtype=torch.float32, device=DEV)
        ws = torch.empty(max(1, dsa.dsa_sparse_mla_workspace_size(B, 1, H, k)), dtype=torch.uint8, device=DEV)
        dsa.dsa_sparse_mla_decode(q, sel_idx, dsa.Rows(sel, 1152, req_stride=k), cfg.scale, o, lse, ws=ws, err=err)
        # group end: commit the plan, then install the surviving misses
        dsa.dsa_plan(tkd, pids, its, ptr, S, W, is_hit, slot, mp, ms, mc, commit=True, err=err)
        dsa.dsa_gather_kv(tkd, is_hit, slot, None, pool, sel, dsa.DSA_GATHER_INSTALL, err=err)
        torch.cuda.synchronize()
        assert int(err) == 0
        got_sel = sel.view(torch.int16).cpu().numpy().view(np.uint16)
        hit_np, slot_np, mc_np = is_hit.cpu().numpy(), slot.cpu().numpy(), mc.cpu().numpy()
        for b in range(B):
            out, state[b] = o_plan.plan_step(tk[b], *state[b], S, W)
            assert np.array_equal(hit_np[b], out["is_hit"]) and np.array_equal(slot_np[b], out["slot"])
            m = out["miss_count"]
            assert int(mc_np[b]) == m
            assert np.array_equal(mp[b, :m].cpu().numpy(), out["miss_pos"])
            assert np.array_equal(ms[b, :m].cpu().numpy(), out["miss_slot"])
            assert np.array_equal(got_sel[b, 0], host_np[b * L + tk[b, 0]])
        pid_np = pids.cpu().numpy()
        pool_np = pool.view(torch.int16).cpu().numpy().view(np.uint16)
        for b in range(B):
            assert np.array_equal(pid_np[b], state[b][0])
            live = np.nonzero(pid_np[b] >= 0)[0]
            assert np.array_equal(pool_np[b, live], host_np[b * L + pid_np[b, live]])
        b = s % B
        o_ref, l_ref = o_mla.sparse_mla(wl.extra["mla_q"][s, layer, b], host_np[b * L + tk[b, 0]], cfg.scale)
        d = np.abs(bf16_to_f64(o[b, 0]) - o_ref)
        assert d.max() <= O_MAX and d.mean() <= O_MEAN
        assert np.abs(lse[b, 0].cpu().numpy().astype(np.float64) - l_ref).max() <= LSE_MAX
        hits.append(int(hit_np.sum()))
    print("pool hits per step (of %d):" % (B * k), hits)
    assert hits[0] == 0 and min(hits[1:]) > 0


def test_indexer_long_units_flush_scores_mid_unit():
    """8 query tokens x 32 heads over 150K-token caches: units of about 38 tiles against a
    score buffer of 16 tiles per query, so every wave writes its staged scores mid-unit."""
    wl = synth.make_workload(synth.spec(3).scaled(L=150000, Sq=8, idx_heads=32), with_kv=False)
    dw = DevWorkload(wl, with_kv=False)
    sc = dw.scores().cpu().numpy()
    assert int(dw.err) == 0
    for b in (0, 5):
        L = int(wl.seq_lens[b])
        ref = o_idx.scores(wl, b)
        for t in range(wl.Sq):
            n = o_idx.visible_len(L, wl.Sq, t)
            bound = indexer_bound(wl, b, t, n)
            assert (np.abs(sc[b, t, :n].astype(np.float64) - ref[t, :n].astype(np.float64)) <= bound).all(), (b, t)
            assert np.isneginf(sc[b, t, n:L]).all()
