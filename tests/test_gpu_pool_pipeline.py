"""The device-pool group with each layer's install on an auxiliary stream, overlapped with
that layer's attention, gives exactly the serial result; a 16384-entry pool (1024 sets x 16
ways) plans bit for bit like the oracle."""
import numpy as np
import pytest
import torch

import paged_kv_cache_indexer_amd as dsa
import synth
from synth import gen as sgen
from oracle import plan as o_plan
from tests.dsa_dev import DEV, PoolGroupStep, host_device_ptr, t_i32

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


@pytest.mark.parametrize("n_sets,ways", [(1024, 8), (1024, 16)])
def test_aux_stream_install_matches_serial(n_sets, ways):
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
    hits = np.zeros((cfg.B, cfg.steps), dtype=np.int64)
    for s in range(cfg.steps):
        tk = t_i32(traj[s][:, None, :])
        serial.run(s_main, tk, qs[s])
        aux.run(a_main, tk, qs[s])
        torch.cuda.synchronize()
        for l in range(cfg.layers):
            assert torch.equal(serial.o[l], aux.o[l]) and torch.equal(serial.lse[l], aux.lse[l]), (s, l)
        hits[:, s] = aux.plan_out[s % 2]["is_hit"].sum(dim=(1, 2)).cpu().numpy()
    torch.cuda.synchronize()
    assert int(serial.err) == 0 and int(aux.err) == 0
    for l in range(cfg.layers):
        assert torch.equal(serial.pool[l], aux.pool[l])
    assert torch.equal(serial.pids, aux.pids) and torch.equal(serial.its, aux.its) and torch.equal(serial.ptr, aux.ptr)
    for b in range(cfg.B):
        assert np.array_equal(hits[b], o_plan.fifo_hits(traj[:, b], n_sets, ways, cfg.id_range)), b
    # every live pool row of every layer holds its host row
    pid = aux.pids.cpu().numpy()
    for l, (h, _) in enumerate(hosts):
        pool = aux.pool[l].view(torch.int16).cpu().numpy()
        hn = h.numpy()
        for b in range(cfg.B):
            live = np.nonzero(pid[b] >= 0)[0]
            assert np.array_equal(pool[b, live], hn[b * cfg.L + pid[b, live]])


def test_mtp_draft_steps_reuse_the_first_selection():
    """Draft steps that reuse the first step's selection buffer attend exactly like draft
    steps that serve the frozen top-k again, and leave the same pool."""
    from tests.dsa_dev import MtpDraftSteps
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
        outs_all = []
        for s in range(cfg.steps):                       # a few verify steps, each with next_n draft steps
            q_steps = [[torch.randn(cfg.B, 1, H, 576, generator=g).to(torch.bfloat16).to(DEV)
                        for _ in range(cfg.layers)] for _ in range(next_n)]
            tk = t_i32(traj[s][:, None, :])
            outs_all.append(MtpDraftSteps(pg, reuse).run(stream, tk, q_steps))
            torch.cuda.synchronize()
        torch.cuda.synchronize()
        assert int(pg.err) == 0
        results[reuse] = (outs_all, [p.clone() for p in pg.pool], pg.pids.clone())
    (o0, p0, i0), (o1, p1, i1) = results[False], results[True]
    for s in range(cfg.steps):
        for d in range(next_n):
            for l in range(cfg.layers):
                assert torch.equal(o0[s][d][l][0], o1[s][d][l][0]) and torch.equal(o0[s][d][l][1], o1[s][d][l][1])
    assert all(torch.equal(a, b) for a, b in zip(p0, p1)) and torch.equal(i0, i1)
