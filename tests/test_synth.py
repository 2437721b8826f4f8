"""The seeded generators are deterministic, chunk-independent and shaped as specified."""
import numpy as np

import synth
from synth import gen


def test_deterministic_and_shapes():
    a = synth.make_workload(synth.spec(2).scaled(B=2, L=1000))
    b = synth.make_workload(synth.spec(2).scaled(B=2, L=1000))
    for f in ("idx_q", "idx_w", "idx_k", "idx_k_scale", "mla_q", "kv", "page_table"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    assert a.idx_k.shape == (a.num_pages, 64, 128) and a.idx_k.dtype == np.uint8
    assert a.page_table.shape == (2, 16) and a.num_pages == 32
    assert sorted(a.page_table.reshape(-1)) == list(range(32))
    assert a.kv.shape == (32, 64, 576) and a.mla_q.shape == (2, 1, 128, 576)


def test_host_rows_match_full_host_cache():
    cfg = synth.spec(4).scaled(B=2, L=40000, layers=2)
    full = gen.host_kv(cfg)
    pos = np.array([0, 5, 16383, 16384, 39999, 20000])
    assert np.array_equal(gen.host_kv_rows(cfg, 1, 1, pos), full[1, 1, pos])


def test_sharded_share_structure():
    cfg = synth.spec(5).scaled(n_short=6, short_lo=300, short_hi=2000, n_long=1, long_len=5000)
    w = synth.make_workload(cfg, with_kv=False)
    lens, qids = w.extra["full_lens"], w.extra["logical_page_ids"]
    for b in range(w.B):
        npg = -(-int(lens[b]) // 64)
        assert all(qids[b, j] % 4 == j % 4 for j in range(npg))
        assert w.seq_lens[b] == sum(min(64, int(lens[b]) - j * 64) for j in range(0, npg, 4))
    assert sorted(w.page_table[w.page_table >= 0]) == list(range(w.num_pages))
    ids = qids[qids >= 0]
    assert len(np.unique(ids)) == len(ids)


def test_trajectory_reuse_fraction():
    cfg = synth.spec(4).scaled(B=3)
    tr = gen.topk_trajectory(cfg)
    for b in range(3):
        for s in range(cfg.steps):
            assert len(np.unique(tr[s, b])) == cfg.topk and (np.diff(tr[s, b]) > 0).all()
            if s:
                assert len(np.intersect1d(tr[s, b], tr[s - 1, b])) == 1229


def test_mxfp4_keys_shapes_and_code_ranges():
    a = synth.make_workload(synth.spec(2).scaled(B=2, L=1000, idx_k_kind="mxfp4"), with_kv=False)
    b = synth.make_workload(synth.spec(2).scaled(B=2, L=1000, idx_k_kind="mxfp4"), with_kv=False)
    assert a.idx_k_dtype == "mxfp4"
    assert a.idx_k.shape == (a.num_pages, 64, 64) and a.idx_k.dtype == np.uint8
    assert a.idx_k_scale.shape == (a.num_pages, 64, 4) and a.idx_k_scale.dtype == np.uint8
    assert np.array_equal(a.idx_k, b.idx_k) and np.array_equal(a.idx_k_scale, b.idx_k_scale)
    lo, hi = gen.MXFP4_SCALE_CODES
    assert a.idx_k_scale.min() == lo and a.idx_k_scale.max() == hi
    nib = np.concatenate([a.idx_k.reshape(-1) & 0xF, a.idx_k.reshape(-1) >> 4])
    assert np.bincount(nib, minlength=16).min() > 0.9 * nib.size / 16
