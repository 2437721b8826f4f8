"""The device-pool group of the package's orchestration (PoolGroupStep, MtpDraftSteps) against
the oracle: plans slot for slot (8K and 16K pools), attention over the served rows against
the oracle's attention over the host rows of the selection (padding entries included), and
the auxiliary-stream install bit-identical to the serial order."""
import numpy as np
import pytest
import torch

import paged_kv_cache_indexer_amd as dsa
import synth
from synth import gen as sgen
from oracle import mla as o_mla, plan as o_plan
from tests.dsa_dev import DEV, MtpDraftSteps, PoolGroupStep, bf16_to_f64, host_device_ptr, t_i32
from tests.test_gpu_kernels import LSE_MAX, O_MAX, O_MEAN

pytestmark = pytest.mark.gpu


def _host_rows(cfg, layers):
    out = []
    for l in range(layers):
        h = torch.empty((cfg.B * cfg.L, 576), dtype=torch.int16, pin_memory=True)
        hn = h.numpy().view(np.uint16)
        for b in range(cfg.B):
            sgen.normal_bf16_rows((cfg.seed, cfg.cid, sgen.T_HOSTKV, l, b), cfg.L, 576, out=hn[b * cfg.L:(b + 1) * cfg.L])
        out.append((h, dsa.Rows(h, 1152, req_stride=cfg.L, base_ptr=host_device_ptr(h))))
    return out


def _check_attention_vs_oracle(o, lse, q, host_np, L, b, row, scale):
    """o / lse of request b against the oracle over the host rows of the valid entries of `row`."""
    pos = row[row >= 0]
    o_ref, l_ref = o_mla.sparse_mla(q.view(torch.int16).cpu().numpy().view(np.uint16)[b, 0],
                                    host_np[b * L + pos], scale)
    d = np.abs(bf16_to_f64(o[b, 0]) - o_ref)
    assert d.max() <= O_MAX and d.mean() <= O_MEAN, (b, d.max(), d.mean())
    assert np.abs(lse[b, 0].cpu().numpy().astype(np.float64) - l_ref).max() <= LSE_MAX, b


def _check_plan(pg, po, tk, state, n_sets, ways):
    """Plan outputs of every request against the oracle's plan_step; returns the new states."""
    hit, slot, mp, ms, mc = (po[k].cpu().numpy() for k in ("is_hit", "slot", "mp", "ms", "mc"))
    new = []
    for b in range(tk.shape[0]):
        out, st = o_plan.plan_step(tk[b], *state[b], n_sets, ways)
        assert np.array_equal(hit[b], out["is_hit"]) and np.array_equal(slot[b], out["slot"]), b
        m = out["miss_count"]
        assert int(mc[b]) == m
        assert np.array_equal(mp[b, :m], out["miss_pos"]) and np.array_equal(ms[b, :m], out["miss_slot"]), b
        new.append(st)
    return new


@pytest.mark.parametrize("n_sets,ways", [(1024, 8), (1024, 16)])
def test_aux_stream_install_matches_serial_and_oracle(n_sets, ways):
    cfg = synth.spec(4).scaled(B=4, L=16384, steps=6, layers=2, n_sets=n_sets, ways=ways, id_range=16384)
    traj = sgen.topk_trajectory(cfg)                           # [steps, B, k]
    hosts = _host_rows(cfg, cfg.layers)
    rows = [r for _, r in hosts]
    H = 32
    g = torch.Generator(device="cpu").manual_seed(1)
    qs = [[torch.randn(cfg.B, 1, H, 576, generator=g).to(torch.bfloat16).to(DEV) for _ in range(cfg.layers)]
          for _ in range(cfg.steps)]
    serial = PoolGroupStep(cfg.B, cfg.topk, H, n_sets, ways, cfg.id_range, rows, cfg.scale, aux_install=False)
    aux = PoolGroupStep(cfg.B, cfg.topk, H, n_sets, ways, cfg.id_range, rows, cfg.scale, aux_install=True)
    s_main, a_main = torch.cuda.Stream(), torch.cuda.Stream()
    state = [o_plan.empty_state(n_sets, ways, cfg.id_range) for _ in range(cfg.B)]
    for s in range(cfg.steps):
        tk = traj[s][:, None, :]
        tkd = t_i32(tk)
        serial.run(s_main, tkd, qs[s])
        aux.run(a_main, tkd, qs[s])
        aux.drain(a_main)
        torch.cuda.synchronize()
        state = _check_plan(aux, aux.plan_out[s % 2], tk, state, n_sets, ways)
        for l in range(cfg.layers):
            assert torch.equal(serial.o[l], aux.o[l]) and torch.equal(serial.lse[l], aux.lse[l]), (s, l)
            host_np = hosts[l][0].numpy().view(np.uint16)
            for b in range(cfg.B):
                _check_attention_vs_oracle(aux.o[l], aux.lse[l], qs[s][l], host_np, cfg.L, b, tk[b, 0], cfg.scale)
    assert int(serial.err) == 0 and int(aux.err) == 0
    for l in range(cfg.layers):
        assert torch.equal(serial.pool[l], aux.pool[l])
    assert torch.equal(serial.pids, aux.pids) and torch.equal(serial.its, aux.its) and torch.equal(serial.ptr, aux.ptr)
    pid = aux.pids.cpu().numpy()
    for b in range(cfg.B):
        assert np.array_equal(pid[b], state[b][0])
        assert np.array_equal(aux.ptr[b].cpu().numpy(), state[b][2])
    # every live pool row of every layer holds its host row
    for l, (h, _) in enumerate(hosts):
        pool = aux.pool[l].view(torch.int16).cpu().numpy()
        hn = h.numpy()
        for b in range(cfg.B):
            live = np.nonzero(pid[b] >= 0)[0]
            assert np.array_equal(pool[b, live], hn[b * cfg.L + pid[b, live]])


def test_padded_selection_rows_are_skipped_by_attention():
    """Top-k rows with fewer than k valid positions (a context shorter than k): the padding
    entries are served as zero rows, and attention over the served buffer skips them, so o
    and lse equal the oracle's over the valid rows only."""
    cfg = synth.spec(4).scaled(B=3, L=4096, steps=3, layers=1, n_sets=64, ways=8, id_range=4096)
    k = cfg.topk
    hosts = _host_rows(cfg, 1)
    host_np = hosts[0][0].numpy().view(np.uint16)
    rng = np.random.default_rng(5)
    H = 64
    pg = PoolGroupStep(cfg.B, k, H, cfg.n_sets, cfg.ways, cfg.id_range, [hosts[0][1]], cfg.scale)
    stream = torch.cuda.Stream()
    state = [o_plan.empty_state(cfg.n_sets, cfg.ways, cfg.id_range) for _ in range(cfg.B)]
    for s in range(cfg.steps):
        tk = np.full((cfg.B, 1, k), -1, dtype=np.int32)
        for b, n_valid in enumerate((k, k - 700, 37 + s)):
            tk[b, 0, :n_valid] = np.sort(rng.choice(cfg.L // 2 + 200 * s, size=n_valid, replace=False))
        q = torch.randn(cfg.B, 1, H, 576, generator=torch.Generator().manual_seed(s)).to(torch.bfloat16).to(DEV)
        pg.run(stream, t_i32(tk), [q])
        torch.cuda.synchronize()
        assert int(pg.err) == 0
        state = _check_plan(pg, pg.plan_out[s % 2], tk, state, cfg.n_sets, cfg.ways)
        si = pg.sel_idx[0].cpu().numpy()
        assert np.array_equal(si[:, 0], np.where(tk[:, 0] >= 0, np.arange(k)[None], -1))
        for b in range(cfg.B):
            _check_attention_vs_oracle(pg.o[0], pg.lse[0], q, host_np, cfg.L, b, tk[b, 0], cfg.scale)


def test_mtp_draft_steps_reuse_the_first_selection():
    """Draft steps that reuse the first step's selection buffer attend exactly like draft
    steps that serve the frozen top-k again, leave the same pool, and match the oracle's
    attention of each draft step's queries over the host rows of the frozen selection."""
    cfg = synth.spec(4).scaled(B=4, L=16384, steps=3, layers=2, id_range=16384)
    traj = sgen.topk_trajectory(cfg)
    hosts = _host_rows(cfg, cfg.layers)
    rows = [r for _, r in hosts]
    H, next_n = 32, 4
    g = torch.Generator(device="cpu").manual_seed(2)
    stream = torch.cuda.Stream()
    results = {}
    for reuse in (False, True):
        pg = PoolGroupStep(cfg.B, cfg.topk, H, cfg.n_sets, cfg.ways, cfg.id_range, rows, cfg.scale)
        g.manual_seed(2)
        outs_all, qs_all = [], []
        for s in range(cfg.steps):                       # a few verify steps, each with next_n draft steps
            q_steps = [[torch.randn(cfg.B, 1, H, 576, generator=g).to(torch.bfloat16).to(DEV)
                        for _ in range(cfg.layers)] for _ in range(next_n)]
            tk = t_i32(traj[s][:, None, :])
            outs_all.append(MtpDraftSteps(pg, reuse).run(stream, tk, q_steps))
            qs_all.append(q_steps)
            torch.cuda.synchronize()
        torch.cuda.synchronize()
        assert int(pg.err) == 0
        results[reuse] = (outs_all, [p.clone() for p in pg.pool], pg.pids.clone(), qs_all)
    (o0, p0, i0, _), (o1, p1, i1, qs) = results[False], results[True]
    for s in range(cfg.steps):
        for d in range(next_n):
            for l in range(cfg.layers):
                assert torch.equal(o0[s][d][l][0], o1[s][d][l][0]) and torch.equal(o0[s][d][l][1], o1[s][d][l][1])
                host_np = hosts[l][0].numpy().view(np.uint16)
                b = (s + d + l) % cfg.B
                _check_attention_vs_oracle(o1[s][d][l][0], o1[s][d][l][1], qs[s][d][l], host_np, cfg.L, b,
                                           traj[s][b], cfg.scale)
    assert all(torch.equal(a, b) for a, b in zip(p0, p1)) and torch.equal(i0, i1)
