"""Parity of each libdsa entry point with the CPU oracle, through the C ABI, on the GPU.

Bars: bit-exact for integer work (page translation, top-k indices, plans, gathers) and
for indexer scores on the exact fp32 grid; for floating point elsewhere the indexer is
held to |gpu - oracle| <= 2e-5 * sum_h w_h * sigma_s * sum_d |q_hd k_sd| (fp32 dot-product
rounding over ~192 terms), and attention to max-abs 2e-2 / mean-abs 2e-3 on o (bf16) and
max-abs 1e-3 on lse.
"""
import dataclasses

import numpy as np
import pytest
import torch

import paged_kv_cache_indexer_amd as dsa
import synth
from oracle import indexer as o_idx, mla as o_mla, paging as o_pg, plan as o_plan, topk as o_topk
from oracle.step import decode_request, selected_rows
from tests.dsa_dev import DecodeStep, DevWorkload, bf16_to_f64, host_device_ptr, t_i32, t_u16_as_bf16, DEV

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3


def indexer_bound(wl, b, t, n):
    q = o_idx.decode_query(wl.idx_q[b, t], wl.idx_q_dtype)
    k = o_idx.request_keys(wl, b, np.arange(n))
    w = wl.idx_w[b, t].astype(np.float64)
    return 2e-5 * (w @ (np.abs(q) @ np.abs(k).T)) + 1e-30


def check_scores(wl, sc_gpu, exact=False):
    sc = sc_gpu.cpu().numpy()
    for b in range(wl.B):
        ref = o_idx.scores(wl, b)
        L = int(wl.seq_lens[b])
        got = sc[b, :, :L]
        assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"-inf pattern differs (b={b})"
        fin = np.isfinite(ref)
        if exact:
            assert np.array_equal(got[fin], ref[fin]), f"scores not bit-exact (b={b})"
        else:
            for t in range(wl.Sq):
                n = o_idx.visible_len(L, wl.Sq, t)
                bound = indexer_bound(wl, b, t, n)
                err = np.abs(got[t, :n].astype(np.float64) - ref[t, :n].astype(np.float64))
                assert (err <= bound).all(), f"b={b} t={t}: max err/bound {(err / bound).max():.3g}"


def check_attention(o_gpu, lse_gpu, o_ref, lse_ref):
    o = bf16_to_f64(o_gpu)
    d = np.abs(o - o_ref)
    assert d.max() <= O_MAX and d.mean() <= O_MEAN, f"o max {d.max():.3g} mean {d.mean():.3g}"
    lg = lse_gpu.cpu().numpy().astype(np.float64)
    inf = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lg), inf)
    assert np.abs(lg[~inf] - lse_ref[~inf]).max(initial=0) <= LSE_MAX


# ------------------------------------------------------------------ page translation
def test_page_translate_bit_exact():
    rng = np.random.default_rng(0)
    x = np.concatenate([np.arange(5000), rng.integers(0, 1 << 40, 20000), [(1 << 62) + 12345]]).astype(np.int64)
    xd = torch.from_numpy(x).to(DEV)
    for p in (1, 2, 64, 128):
        for N in (1, 2, 3, 4):
            r = torch.empty(len(x), dtype=torch.int32, device=DEV)
            l = torch.empty(len(x), dtype=torch.int64, device=DEV)
            dsa.dsa_page_translate(xd, p, N, r, l)
            rr, ll = o_pg.owner_local(x, p, N)
            assert np.array_equal(r.cpu().numpy(), rr) and np.array_equal(l.cpu().numpy(), ll)
    # negative slots are flagged, not translated
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    xn = torch.tensor([-1, 5, -7], dtype=torch.int64, device=DEV)
    r = torch.empty(3, dtype=torch.int32, device=DEV)
    l = torch.empty(3, dtype=torch.int64, device=DEV)
    dsa.dsa_page_translate(xn, 64, 4, r, l, err=err)
    assert r.tolist() == [-1, 0, -1] and l.tolist() == [-1, 5, -1] and int(err) == 2


# ------------------------------------------------------------------ indexer
def test_indexer_f32_exact_grid_tiny_config():
    wl = synth.make_workload(1, with_kv=False)
    dw = DevWorkload(wl, with_kv=False)
    check_scores(wl, dw.scores(), exact=True)
    assert int(dw.err) == 0


def test_indexer_f32_exact_grid_mtp_ragged():
    wl = synth.make_workload(synth.spec(1).scaled(B=3, L=1000, Sq=4), with_kv=False)
    wl.seq_lens = np.array([1000, 777, 33], dtype=np.int32)
    check_scores(wl, DevWorkload(wl, with_kv=False).scores(), exact=True)


@pytest.mark.parametrize("L", [[1000, 777, 33], [4096, 64, 4095]])
def test_indexer_bf16_e4m3_within_bound(L):
    wl = synth.make_workload(synth.spec(2).scaled(B=3, L=max(L)), with_kv=False)
    wl.seq_lens = np.array(L, dtype=np.int32)
    dw = DevWorkload(wl, with_kv=False)
    check_scores(wl, dw.scores())
    assert int(dw.err) == 0


@pytest.mark.parametrize("cid,B,Sq", [(2, 1024, 1), (3, 300, 4)])
def test_indexer_max_batch_ragged_within_bound(cid, B, Sq):
    """The largest batch one launch takes (1024 requests; 300 with four fp8 queries, which
    fills Sq*H = 256): the per-request unit prefix spans every thread's requests, with
    empty, one-token, tile-edge and page-edge requests among them."""
    L = 700
    wl = synth.make_workload(synth.spec(cid).scaled(B=B, L=L), with_kv=False)
    lens = np.random.default_rng(B).integers(0, L + 1, B).astype(np.int32)
    lens[:9] = [0, 1, 31, 32, 33, 64, 65, L, Sq]
    lens = np.maximum(lens, Sq - 1)                  # the oracle's visibility: seq_len >= Sq - 1
    wl.seq_lens = lens
    dw = DevWorkload(wl, with_kv=False)
    check_scores(wl, dw.scores())
    assert int(dw.err) == 0


@pytest.mark.parametrize("path", ["mfma", "fused", "f32"])
def test_indexer_leaves_positions_past_the_length_untouched_and_reads_a_null_scale_as_one(path):
    """Requests of different lengths in one score array: every entry at or past a request's
    length keeps its sentinel bits (the scan writes only [0, seq_len)), and with k_scale
    NULL the e4m3 keys are scored with sigma = 1 (the oracle with unit scales)."""
    import dataclasses
    if path == "f32":
        wl = synth.make_workload(synth.spec(1).scaled(B=3, L=3000), with_kv=False)
    else:
        wl = synth.make_workload(synth.spec(2).scaled(B=4, L=5000), with_kv=False)
    lens = np.array([5000, 3100, 4097, 2049][:wl.B], dtype=np.int32) if path != "f32" else \
        np.array([3000, 1777, 65], dtype=np.int32)
    wl = dataclasses.replace(wl, seq_lens=lens)
    if path != "f32":
        wl = dataclasses.replace(wl, idx_k_scale=np.ones_like(wl.idx_k_scale))
    dw = DevWorkload(wl, with_kv=False)
    stride = int(lens.max()) + 37
    sentinel = 0x7FC0DEAD
    sc = torch.full((wl.B, wl.Sq, stride), sentinel, dtype=torch.int32, device=DEV).view(torch.float32)
    k_scale = None if path != "f32" else dw.k_scale
    if path == "fused":
        ws = torch.empty((dsa.dsa_topk_workspace_size(wl.B, 1, wl.topk, stride),), dtype=torch.uint8, device=DEV)
        dsa.dsa_indexer_topk_chunks(dw.idx_q, dw.idx_w, dw.keys, k_scale, dw.seq_lens, sc, wl.topk, ws,
                                    k_dtype=dw.k_dtype, err=dw.err, q_dtype=dw.q_dtype)
    else:
        dsa.dsa_indexer_scores(dw.idx_q, dw.idx_w, dw.keys, k_scale, dw.seq_lens, sc, k_dtype=dw.k_dtype,
                               err=dw.err, q_dtype=dw.q_dtype)
    torch.cuda.synchronize()
    assert int(dw.err) == 0
    bits = sc.view(torch.int32).cpu().numpy()
    for b in range(wl.B):
        assert (bits[b, :, int(lens[b]):] == sentinel).all(), b
    check_scores(wl, sc, exact=(path == "f32"))


def test_indexer_length_past_the_score_row_is_clamped():
    """seq_lens[0] = 900 over a 700-wide score row: request 0 scores as a 700-token request,
    counts one error, and nothing is written past the rows (a sentinel row follows them)."""
    wl = synth.make_workload(synth.spec(2).scaled(B=3, L=900), with_kv=False)
    wl.seq_lens = np.array([900, 700, 300], dtype=np.int32)
    dw = DevWorkload(wl, with_kv=False)
    stride = 700
    buf = torch.full((wl.B * wl.Sq + 1, stride), 123.0, dtype=torch.float32, device=DEV)
    sc = buf[:wl.B * wl.Sq].view(wl.B, wl.Sq, stride)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    dsa.dsa_indexer_scores(dw.idx_q, dw.idx_w, dw.keys, dw.k_scale, dw.seq_lens, sc, k_dtype=dw.k_dtype, err=err,
                           q_dtype=dw.q_dtype)
    torch.cuda.synchronize()
    assert int(err.item()) == 1
    assert (buf[-1] == 123.0).all()
    check_scores(dataclasses.replace(wl, seq_lens=np.array([700, 700, 300], dtype=np.int32)), sc)


def test_indexer_e4m3_queries_mtp_within_bound():
    wl = synth.make_workload(synth.spec(3).scaled(B=2, L=1500), with_kv=False)
    wl.seq_lens = np.array([1500, 1031], dtype=np.int32)
    check_scores(wl, DevWorkload(wl, with_kv=False).scores())


@pytest.mark.parametrize("L", [[1000, 777, 33], [4096, 64, 4095]])
def test_indexer_mxfp4_keys_bf16_queries_within_bound(L):
    wl = synth.make_workload(synth.spec(2).scaled(B=3, L=max(L), idx_k_kind="mxfp4"), with_kv=False)
    wl.seq_lens = np.array(L, dtype=np.int32)
    dw = DevWorkload(wl, with_kv=False)
    assert dw.keys.c.row_bytes == 64 and dw.k_dtype == dsa.DSA_MXFP4
    check_scores(wl, dw.scores())
    assert int(dw.err) == 0


def test_indexer_mxfp4_keys_e4m3_queries_mtp_within_bound():
    wl = synth.make_workload(synth.spec(3).scaled(B=2, L=1500, idx_k_kind="mxfp4"), with_kv=False)
    wl.seq_lens = np.array([1500, 1031], dtype=np.int32)
    dw = DevWorkload(wl, with_kv=False)
    check_scores(wl, dw.scores())
    assert int(dw.err) == 0


@pytest.mark.parametrize("qkind,H,Sq", [("bf16", 32, 1), ("e4m3", 64, 1), ("bf16", 128, 2)])
def test_indexer_mxfp4_wide_block_scales(qkind, H, Sq):
    # block scales spread over 2^-27 .. 2^27 and differing inside each token, so a wrong
    # block -> scale mapping or nibble order cannot stay inside the bound
    wl = synth.make_workload(synth.spec(2).scaled(B=2, L=2100, idx_heads=H, Sq=Sq, idx_q_kind=qkind,
                                                  idx_k_kind="mxfp4"), with_kv=False)
    wl.seq_lens = np.array([2100, 1333], dtype=np.int32)
    rng = np.random.default_rng(11)
    wl.idx_k_scale = rng.integers(100, 155, wl.idx_k_scale.shape).astype(np.uint8)
    check_scores(wl, DevWorkload(wl, with_kv=False).scores())


def test_indexer_ready_event_orders_load_before_scan():
    """The scan waits on the load stream's event; without the wait it reads stale keys."""
    wl = synth.make_workload(synth.spec(1).scaled(L=2048), with_kv=False)
    dw = DevWorkload(wl, with_kv=False)
    real = dw.idx_k.clone()
    load = torch.cuda.Stream()
    results = {}
    for join in (True, False):
        dw.idx_k.fill_(1000.0)                          # sentinel: not on the [-4, 4] grid
        torch.cuda.synchronize()
        ev = torch.cuda.Event()
        with torch.cuda.stream(load):
            torch.cuda._sleep(200_000_000)              # a slow host-to-device load
            dw.idx_k.copy_(real, non_blocking=True)
            ev.record(load)
        sc = dw.scores(ready=ev if join else None)
        torch.cuda.synchronize()
        results[join] = sc
    ref = o_idx.scores(wl, 0)
    got = results[True].cpu().numpy()[0]
    assert np.array_equal(got[np.isfinite(ref)], ref[np.isfinite(ref)])
    stale = results[False].cpu().numpy()[0]
    assert not np.array_equal(stale[np.isfinite(ref)], ref[np.isfinite(ref)]), \
        "the unjoined scan should have read the sentinel keys"


# ------------------------------------------------------------------ top-k
def _topk_cases():
    rng = np.random.default_rng(7)
    cases = []
    # many exact ties (small integer grid), a signed-zero row, all equal, n <= k, n = k + 1, long rows
    cases.append((rng.integers(-50, 50, 70000).astype(np.float32), 2048))
    z = np.zeros(5000, np.float32)
    z[rng.random(5000) < 0.5] = -0.0
    z[::97] = 1.0
    cases.append((z, 300))
    cases.append((np.full(9000, 3.25, np.float32), 2048))
    cases.append((rng.standard_normal(100).astype(np.float32), 256))
    cases.append((rng.standard_normal(256).astype(np.float32), 256))
    cases.append((rng.standard_normal(257).astype(np.float32), 256))
    cases.append(((rng.standard_normal(200004) * 1e-3 + 5.0).astype(np.float32), 2048))
    x = rng.standard_normal(65536).astype(np.float32)
    x[rng.integers(0, 65536, 3000)] = np.float32(np.inf)
    cases.append((x, 2048))
    cases.append((-np.abs(rng.standard_normal(40000)).astype(np.float32), 1))
    cases.append((rng.standard_normal(33000).astype(np.float32) * np.float32(1e30), 8192))
    # ascending scores: the whole answer sits in the last chunk, far above its share
    cases.append((np.sort(rng.standard_normal(65536)).astype(np.float32), 2048))
    # one position past a chunk boundary; a large k near the register capacity
    cases.append((rng.standard_normal(8193).astype(np.float32), 4000))
    # more candidates than one work-group holds: the re-select over the row
    cases.append((rng.standard_normal(300000).astype(np.float32), 8192))
    return cases


@pytest.mark.parametrize("case", range(13))
def test_topk_standalone_bit_exact(case):
    s, k = _topk_cases()[case]
    n = len(s)
    sc = torch.from_numpy(s[None, None, :].copy()).to(DEV)
    idx = torch.empty((1, 1, k), dtype=torch.int32, device=DEV)
    dsa.dsa_topk(sc, torch.tensor([n], dtype=torch.int32, device=DEV), idx)
    assert np.array_equal(idx.cpu().numpy()[0, 0], o_topk.select(s, k))


def test_topk_minus_inf_scores_and_lengths_past_the_stride():
    """-inf is an ordinary (lowest) score: a row mostly of -inf takes its finite positions and
    then the lowest -inf positions; a row of -inf only takes its first k positions.  A length
    above the score stride is read as the stride.  Both the wave-chunk rows (stride 9000)
    and the work-group-chunk rows (stride 300000) are checked against the oracle's select."""
    rng = np.random.default_rng(17)
    for stride, k in ((9000, 2048), (300000, 2048)):
        B = 4
        s = rng.standard_normal((B, 1, stride)).astype(np.float32)
        s[0, 0, rng.random(stride) < 0.85] = -np.inf
        s[1, 0, :] = -np.inf
        lens = np.array([stride, stride - 11, stride + 100, stride // 3], dtype=np.int32)
        idx = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
        dsa.dsa_topk(torch.from_numpy(s).to(DEV), t_i32(lens), idx)
        got = idx.cpu().numpy()
        for b in range(B):
            n = min(int(lens[b]), stride)
            assert np.array_equal(got[b, 0], o_topk.select(s[b, 0, :n], k)), (stride, b)


def _long_chunk_rows(stride):
    """Rows of a batch whose 8192-position chunks would take more than 512 work-groups, so
    the chunk stage runs with 16384 positions per chunk."""
    rng = np.random.default_rng(21)
    s = np.zeros((6, 1, stride), dtype=np.float32)
    lens = np.array([stride, 300000, 16385, 2000, 32769, 200004], dtype=np.int32)
    s[0, 0] = rng.standard_normal(stride)
    s[1, 0, :lens[1]] = np.sort(rng.standard_normal(lens[1]))        # answer in the last chunk
    s[2, 0, :lens[2]] = rng.integers(-50, 50, lens[2])                 # ties; one past a boundary
    s[3, 0, :lens[3]] = rng.standard_normal(lens[3])                   # n <= k
    s[4, 0, :lens[4]] = 3.25                                           # all equal
    s[5, 0, :lens[5]] = rng.standard_normal(lens[5]) * 1e-3 + 5.0      # close values
    return s, lens


@pytest.mark.parametrize("k", [2048, 8192])
def test_topk_long_rows_use_16k_chunks_bit_exact(k):
    stride = 1_100_000                                  # 135 chunks of 8192 per row, 6 rows
    assert 6 * -(-stride // 8192) > 512
    s, lens = _long_chunk_rows(stride)
    idx = torch.empty((6, 1, k), dtype=torch.int32, device=DEV)
    dsa.dsa_topk(torch.from_numpy(s).to(DEV), t_i32(lens), idx)
    got = idx.cpu().numpy()
    for b in range(6):
        assert np.array_equal(got[b, 0], o_topk.select(s[b, 0, :lens[b]], k)), b


def test_topk_long_chunk_grid_mtp_rows():
    rng = np.random.default_rng(5)
    B, Sq, Lmax, k = 40, 4, 24600, 512                  # 160 rows x 4 chunks of 8192
    lens = rng.integers(400, Lmax + 1, B).astype(np.int32)
    lens[:3] = [Lmax, 515, 16387]
    s = rng.integers(0, 300, (B, Sq, Lmax)).astype(np.float32)
    idx = torch.empty((B, Sq, k), dtype=torch.int32, device=DEV)
    dsa.dsa_topk(torch.from_numpy(s).to(DEV), t_i32(lens), idx)
    got = idx.cpu().numpy()
    for b in range(B):
        for t in range(Sq):
            n = o_idx.visible_len(lens[b], Sq, t)
            assert np.array_equal(got[b, t], o_topk.select(s[b, t, :n], k)), (b, t)


def test_topk_batched_mtp_rows():
    rng = np.random.default_rng(3)
    B, Sq, Lmax, k = 5, 4, 16390, 512
    lens = np.array([5000, 600, 515, 8195, 16390], dtype=np.int32)
    s = rng.integers(0, 200, (B, Sq, Lmax)).astype(np.float32)
    idx = torch.empty((B, Sq, k), dtype=torch.int32, device=DEV)
    dsa.dsa_topk(torch.from_numpy(s).to(DEV), t_i32(lens), idx)
    got = idx.cpu().numpy()
    for b in range(B):
        for t in range(Sq):
            n = o_idx.visible_len(lens[b], Sq, t)
            assert np.array_equal(got[b, t], o_topk.select(s[b, t, :n], k)), (b, t)


def test_topk_wave_chunks_mixed_rows():
    """Rows on the wave-chunk path at a stride that lowers its slack (250048 positions, as a
    4-way page-sharded share of a 1M context): mixed lengths, a hot window whose 700
    consecutive best scores overflow one chunk's slots (the re-select), a row whose chunks
    are each constant (every search ends on an adjacent bracket), integer ties, and
    close values."""
    rng = np.random.default_rng(31)
    stride, k = 250048, 2048
    lens = np.array([250048, 200000, 65536, 40000, 9000, 2049, 2048, 100, 250048, 131072, 70001, 33000,
                     150000, 250048, 8193, 250047], dtype=np.int32)
    B = len(lens)
    s = np.zeros((B, 1, stride), dtype=np.float32)
    for b in range(B):
        n = lens[b]
        s[b, 0, :n] = rng.standard_normal(n)
    s[2, 0, 30000:30700] = 10.0 + rng.random(700).astype(np.float32)      # hot window inside one chunk
    s[3, 0, :40000] = np.repeat(rng.standard_normal(40), 1000)[:40000]     # constant within each 1000
    s[9, 0, :131072] = rng.integers(-50, 50, 131072)                        # integer ties
    s[10, 0, :70001] = rng.standard_normal(70001) * 1e-3 + 5.0              # close values
    s[12, 0, :150000] = np.abs(rng.standard_normal(150000)) * np.float32(1e30)
    idx = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
    dsa.dsa_topk(torch.from_numpy(s).to(DEV), t_i32(lens), idx)
    got = idx.cpu().numpy()
    for b in range(B):
        assert np.array_equal(got[b, 0], o_topk.select(s[b, 0, :lens[b]], k)), b


# ------------------------------------------------------------------ sparse MLA
@pytest.mark.parametrize("H,k,L", [(128, 2048, 3000), (16, 256, 4096), (64, 300, 700), (128, 100, 100),
                                   (32, 512, 2000), (48, 300, 1000),
                                   (16, 65536, 70000)])          # the largest selection one call takes
def test_mla_against_oracle(H, k, L):
    wl = synth.make_workload(synth.spec(2).scaled(B=2, L=L, mla_heads=H, topk=k))
    rng = np.random.default_rng(H + k)
    idx = np.full((wl.B, 1, k), -1, dtype=np.int32)
    for b in range(wl.B):
        n = min(k, L) - (b * 7 if min(k, L) > 7 else 0)          # some padding rows
        idx[b, 0, :n] = np.sort(rng.choice(L, size=n, replace=False))
    dw = DevWorkload(wl)
    o, lse = dw.mla(t_i32(idx))
    o_ref = np.empty((wl.B, 1, H, 512))
    l_ref = np.empty((wl.B, 1, H))
    for b in range(wl.B):
        o_ref[b, 0], l_ref[b, 0] = o_mla.sparse_mla(wl.mla_q[b, 0], selected_rows(wl, b, idx[b, 0]), wl.scale)
    check_attention(o, lse, o_ref, l_ref)
    assert int(dw.err) == 0


@pytest.mark.parametrize("H,o_dtype", [(80, torch.bfloat16), (192, torch.float32)])
def test_mla_partial_head_blocks_and_query_rows_on_one_xcd(H, o_dtype):
    """64-head work-groups with a partly used last head block (80 heads: its score waves 1-3
    hold no real head) or three head blocks (192), at 8 query rows (every work-group of a
    row and its merge on one XCD), 16 splits of 128 rows each, padded selections."""
    B, k, L = 8, 2048, 3000
    wl = synth.make_workload(synth.spec(2).scaled(B=B, L=L, mla_heads=H, topk=k))
    rng = np.random.default_rng(H)
    idx = np.full((B, 1, k), -1, dtype=np.int32)
    for b in range(B):
        n = k - 37 * b
        idx[b, 0, :n] = np.sort(rng.choice(L, size=n, replace=False))
    dw = DevWorkload(wl)
    o, lse = dw.mla(t_i32(idx), o_dtype=o_dtype)
    o_ref = np.empty((B, 1, H, 512))
    l_ref = np.empty((B, 1, H))
    for b in range(B):
        o_ref[b, 0], l_ref[b, 0] = o_mla.sparse_mla(wl.mla_q[b, 0], selected_rows(wl, b, idx[b, 0]), wl.scale)
    check_attention(o, lse, o_ref, l_ref)
    assert int(dw.err) == 0


@pytest.mark.parametrize("B,k,L", [(2, 32, 500), (129, 100, 300)])
def test_mla_single_split_writes_o_directly(B, k, L):
    """Shapes whose split plan is one split (one tile per row; or 258 work-groups of 64 heads,
    where a second split would add a round): the 64-head kernel writes o and lse itself,
    with no partials and no merge."""
    H = 128
    assert dsa.dsa_sparse_mla_workspace_size(B, 1, H, k) == 0
    wl = synth.make_workload(synth.spec(2).scaled(B=B, L=L, mla_heads=H, topk=k))
    rng = np.random.default_rng(B + k)
    idx = np.full((B, 1, k), -1, dtype=np.int32)
    for b in range(B):
        n = k - (b % 5)
        idx[b, 0, :n] = np.sort(rng.choice(L, size=n, replace=False))
    dw = DevWorkload(wl)
    o, lse = dw.mla(t_i32(idx))
    o_ref = np.empty((B, 1, H, 512))
    l_ref = np.empty((B, 1, H))
    for b in range(B):
        o_ref[b, 0], l_ref[b, 0] = o_mla.sparse_mla(wl.mla_q[b, 0], selected_rows(wl, b, idx[b, 0]), wl.scale)
    check_attention(o, lse, o_ref, l_ref)
    assert int(dw.err) == 0


@pytest.mark.parametrize("cfg,B,H,k,L,o_dtype", [(2, 66, 128, 2048, 2600, torch.bfloat16),
                                                  (2, 50, 128, 2048, 2300, torch.float32),
                                                  (2, 100, 128, 1000, 1500, torch.bfloat16),
                                                  (3, 13, 128, 2048, 2200, torch.bfloat16),
                                                  (2, 70, 80, 1500, 1700, torch.bfloat16),
                                                  (2, 66, 64, 2048, 2100, torch.bfloat16),
                                                  (2, 17, 128, 8192, 9000, torch.bfloat16),
                                                  (2, 17, 256, 2048, 2600, torch.float32)])
def test_mla_row_stream_form_against_oracle(cfg, B, H, k, L, o_dtype):
    """Batches whose split plan would leave a second, partly empty round take the row-stream
    form: each head block's tiles shared evenly by a fixed set of work-groups, a share meeting
    up to two rows.  Every (row, head) against the oracle, padded selections included.  The
    17-row shapes give up to 9 (bf16) and 5 (float32) parts per row, more than the merge
    unrolls: its batched form."""
    from tests.test_mla_addressing import mla_plan
    wl = synth.make_workload(synth.spec(cfg).scaled(B=B, L=L, mla_heads=H, topk=k))
    Sq = wl.Sq
    assert mla_plan(B, Sq, H, k)[2] > 0                   # the row-stream form is the one launched
    rng = np.random.default_rng(B + H + k)
    idx = np.full((B, Sq, k), -1, dtype=np.int32)
    for b in range(B):
        for t in range(Sq):
            n = k - ((b * 3 + t) % 7) * 5
            idx[b, t, :n] = np.sort(rng.choice(L, size=n, replace=False))
    dw = DevWorkload(wl)
    o, lse = dw.mla(t_i32(idx), o_dtype=o_dtype)
    o_ref = np.empty((B, Sq, H, 512))
    l_ref = np.empty((B, Sq, H))
    for b in range(B):
        for t in range(Sq):
            o_ref[b, t], l_ref[b, t] = o_mla.sparse_mla(wl.mla_q[b, t], selected_rows(wl, b, idx[b, t]), wl.scale)
    check_attention(o, lse, o_ref, l_ref)
    assert int(dw.err) == 0


@pytest.mark.parametrize("ps,H", [(16, 128), (128, 128), (64, 32)])
def test_mla_page_sizes_dense_rows_and_unresolvable_entries(ps, H):
    """Pages of 16, 128 and 64 tokens (the last with 32 heads, the two-stream work-group);
    the same rows laid out densely (no page table, one block of L rows per request), which
    must give bit-identical o and lse; and selections holding entries that resolve to no row
    (positions on a page whose table entry is -1, a position past the request's page-table
    row): each is counted once in err_count and left out of the softmax, so o and lse match
    the oracle over the remaining entries."""
    B, k, L = 4, 1024, 3000
    wl = synth.make_workload(synth.spec(2).scaled(B=B, L=L, mla_heads=H, topk=k, page_size=ps))
    rng = np.random.default_rng(ps)
    idx = np.full((B, 1, k), -1, dtype=np.int32)
    for b in range(B):
        n = k - 9 * b
        idx[b, 0, :n] = np.sort(rng.choice(L, size=n, replace=False))
    dw = DevWorkload(wl)
    o, lse = dw.mla(t_i32(idx))
    o_ref = np.empty((B, 1, H, 512))
    l_ref = np.empty((B, 1, H))
    for b in range(B):
        o_ref[b, 0], l_ref[b, 0] = o_mla.sparse_mla(wl.mla_q[b, 0], selected_rows(wl, b, idx[b, 0]), wl.scale)
    check_attention(o, lse, o_ref, l_ref)
    assert int(dw.err) == 0

    dense = np.stack([selected_rows(wl, b, np.arange(L)) for b in range(B)]).reshape(B * L, 576)
    dense_t = t_u16_as_bf16(dense)
    o2, lse2 = dw.mla(t_i32(idx), rows=dsa.Rows(dense_t, 1152, None, 0, req_stride=L))
    torch.cuda.synchronize()
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16)) and torch.equal(lse2, lse)
    assert int(dw.err) == 0

    pt = wl.page_table.copy()
    dead_page = int(idx[0, 0, 40]) // ps                  # request 0: one page marked absent
    pt[0, dead_page] = -1
    bad = idx.copy()
    past = pt.shape[1] * ps + 5                           # request 2: past its page-table row
    bad[2, 0, k - 9 * 2] = past                           # in place of its first padding entry
    pt_t = t_i32(pt)
    o3, lse3 = dw.mla(t_i32(bad), rows=dsa.Rows(dw.kv, 1152, pt_t, ps))
    torch.cuda.synchronize()
    on_dead = (idx[0, 0] >= 0) & (idx[0, 0] // ps == dead_page)
    assert int(dw.err) == int(on_dead.sum()) + 1
    keep = [np.where(on_dead, -1, idx[0, 0])] + [idx[b, 0] for b in range(1, B)]
    for b in range(B):
        o_ref[b, 0], l_ref[b, 0] = o_mla.sparse_mla(wl.mla_q[b, 0], selected_rows(wl, b, keep[b]), wl.scale)
    check_attention(o3, lse3, o_ref, l_ref)


def test_mla_f32_output_and_empty_selection():
    wl = synth.make_workload(synth.spec(2).scaled(B=2, L=500, topk=64))
    idx = np.full((2, 1, 64), -1, dtype=np.int32)
    idx[0, 0, :10] = np.arange(0, 500, 50)
    dw = DevWorkload(wl)
    o, lse = dw.mla(t_i32(idx), o_dtype=torch.float32)
    o_ref, l_ref = o_mla.sparse_mla(wl.mla_q[0, 0], selected_rows(wl, 0, idx[0, 0]), wl.scale)
    check_attention(o[:1], lse[:1], o_ref[None, None], l_ref[None, None])
    assert (o[1].cpu().numpy() == 0).all() and np.isneginf(lse[1].cpu().numpy()).all()


# ------------------------------------------------------------------ end to end, tiny config
def test_tiny_config_end_to_end():
    wl = synth.make_workload(1)
    dw = DevWorkload(wl)
    sc = dw.scores()
    idx = dw.topk(sc)
    o, lse = dw.mla(idx)
    ref = decode_request(wl, 0)
    L = int(wl.seq_lens[0])
    assert np.array_equal(sc.cpu().numpy()[0, :, :L], ref["scores"])
    assert np.array_equal(idx.cpu().numpy()[0], ref["topk"])
    check_attention(o, lse, ref["o"][None], ref["lse"][None])


# ------------------------------------------------------------------ plan
def _run_plan_steps(steps_topk, n_sets, W, id_range, Sq=1):
    """steps_topk: list of int32 [B, Sq, k]; returns per-step GPU and oracle outputs."""
    B = steps_topk[0].shape[0]
    pool = torch.full((B, n_sets * W), -1, dtype=torch.int32, device=DEV)
    its = torch.full((B, id_range), -1, dtype=torch.int32, device=DEV)
    ptr = torch.zeros((B, n_sets), dtype=torch.int32, device=DEV)
    state = [o_plan.empty_state(n_sets, W, id_range) for _ in range(B)]
    for tk in steps_topk:
        k = tk.shape[-1]
        E = tk.shape[1] * k
        is_hit = torch.empty(tk.shape, dtype=torch.uint8, device=DEV)
        slot = torch.empty(tk.shape, dtype=torch.int32, device=DEV)
        mpos = torch.full((B, E), -7, dtype=torch.int32, device=DEV)
        mslot = torch.full((B, E), -7, dtype=torch.int32, device=DEV)
        mcnt = torch.empty(B, dtype=torch.int32, device=DEV)
        dsa.dsa_plan(t_i32(tk), pool, its, ptr, n_sets, W, is_hit, slot, mpos, mslot, mcnt, commit=True)
        for b in range(B):
            out, state[b] = o_plan.plan_step(tk[b], *state[b], n_sets, W)
            m = out["miss_count"]
            assert int(mcnt[b]) == m
            assert np.array_equal(is_hit[b].cpu().numpy(), out["is_hit"])
            assert np.array_equal(slot[b].cpu().numpy(), out["slot"])
            assert np.array_equal(mpos[b, :m].cpu().numpy(), out["miss_pos"])
            assert np.array_equal(mslot[b, :m].cpu().numpy(), out["miss_slot"])
            assert np.array_equal(pool[b].cpu().numpy(), state[b][0])
            assert np.array_equal(its[b].cpu().numpy(), state[b][1])
            assert np.array_equal(ptr[b].cpu().numpy(), state[b][2])


@pytest.mark.parametrize("n_sets,W,k,Sq", [(8, 4, 40, 1), (1, 5, 16, 1), (16, 3, 64, 2), (4, 2, 100, 4)])
def test_plan_small_bit_exact(n_sets, W, k, Sq):
    rng = np.random.default_rng(n_sets * 100 + k)
    id_range, B = 300, 3
    steps = []
    for _ in range(8):
        tk = np.full((B, Sq, k), -1, dtype=np.int32)
        for b in range(B):
            for t in range(Sq):
                n = int(rng.integers(k // 2, k + 1))
                tk[b, t, :n] = np.sort(rng.choice(id_range, size=n, replace=False))
        steps.append(tk)
    _run_plan_steps(steps, n_sets, W, id_range, Sq)


def test_plan_pool_group_trajectory_bit_exact():
    cfg = synth.spec(4).scaled(B=4)
    traj = synth.gen.topk_trajectory(cfg)
    _run_plan_steps([traj[s][:, None, :] for s in range(cfg.steps)], cfg.n_sets, cfg.ways, cfg.id_range)


def test_plan_invalid_ids_and_stored_slots_are_skipped_and_counted():
    """Positions >= id_range and ids whose stored slot lies outside the pool are invalid
    entries: is_hit 0, slot -1, not misses, the metadata untouched for them, one count each
    in err_count.  Everything else equals the oracle's plan of the rows without them."""
    rng = np.random.default_rng(41)
    B, k, n_sets, W, id_range = 2, 40, 8, 4, 300
    first = np.stack([np.sort(rng.choice(id_range, k, replace=False)) for _ in range(B)]).astype(np.int32)
    pool = torch.full((B, n_sets * W), -1, dtype=torch.int32, device=DEV)
    its = torch.full((B, id_range), -1, dtype=torch.int32, device=DEV)
    ptr = torch.zeros((B, n_sets), dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    outs = [torch.empty((B, 1, k), dtype=torch.uint8, device=DEV), torch.empty((B, 1, k), dtype=torch.int32, device=DEV),
            torch.empty((B, k), dtype=torch.int32, device=DEV), torch.empty((B, k), dtype=torch.int32, device=DEV),
            torch.empty(B, dtype=torch.int32, device=DEV)]
    dsa.dsa_plan(t_i32(first[:, None, :]), pool, its, ptr, n_sets, W, *outs, commit=True, err=err)
    torch.cuda.synchronize()
    assert int(err) == 0
    state = [o_plan.plan_step(first[b][None], *o_plan.empty_state(n_sets, W, id_range), n_sets, W)[1]
             for b in range(B)]
    # second step: k - 3 valid ids, then three ids past id_range; one valid id of each row
    # (not pooled) gets a stored slot far outside the pool
    second = np.empty((B, k), dtype=np.int32)
    clean = np.empty((B, k), dtype=np.int32)
    its_np = its.cpu().numpy()
    bad_ids = []
    for b in range(B):
        ids = np.sort(rng.choice(id_range, k - 3, replace=False))
        second[b] = np.concatenate([ids, [id_range, id_range + 7, 5000]])
        u = int(next(x for x in ids if its_np[b, x] == -1))
        bad_ids.append(u)
        its_np[b, u] = 1 << 20
        clean[b] = np.where((second[b] >= id_range) | (second[b] == u), -1, second[b])
    its.copy_(torch.from_numpy(its_np))
    dsa.dsa_plan(t_i32(second[:, None, :]), pool, its, ptr, n_sets, W, *outs, commit=True, err=err)
    torch.cuda.synchronize()
    assert int(err) == B * 4
    is_hit, slot, mpos, mslot, mcnt = (x.cpu().numpy() for x in outs)
    for b in range(B):
        its_b = state[b][1].copy()
        its_b[bad_ids[b]] = 1 << 20
        out, (p_new, i_new, r_new) = o_plan.plan_step(clean[b][None], state[b][0], its_b, state[b][2], n_sets, W)
        m = out["miss_count"]
        assert int(mcnt[b]) == m
        assert np.array_equal(is_hit[b], out["is_hit"]) and np.array_equal(slot[b], out["slot"])
        assert np.array_equal(mpos[b, :m], out["miss_pos"]) and np.array_equal(mslot[b, :m], out["miss_slot"])
        assert np.array_equal(pool[b].cpu().numpy(), p_new)
        assert np.array_equal(its[b].cpu().numpy(), i_new)
        assert np.array_equal(ptr[b].cpu().numpy(), r_new)


def test_gather_unresolvable_positions_and_slots_are_counted():
    """SERVE: a position with no source row gets the zero row, -1 in sel_idx and one count;
    INSTALL: a surviving miss whose slot lies past the pool is skipped and counted, and no
    pool row changes for it."""
    rng = np.random.default_rng(43)
    B, L, k, pool_rows = 2, 500, 16, 8
    full = rng.integers(0, 1 << 16, (B * L, 576), dtype=np.uint16)
    src = dsa.Rows(t_u16_as_bf16(full), 1152, req_stride=L)
    tk = np.stack([np.sort(rng.choice(L, k, replace=False)) for _ in range(B)]).astype(np.int32)
    tk[0, -2:] = [L + 3, L + 90]                          # past request 0's stride
    tk[1, -1] = -1                                        # padding: zero row, not counted
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    sel = torch.full((B, 1, k, 576), 3.0, dtype=torch.bfloat16, device=DEV)
    sel_idx = torch.full((B, 1, k), -9, dtype=torch.int32, device=DEV)
    dsa.dsa_gather_kv(t_i32(tk[:, None, :]), None, None, src, None, sel, dsa.DSA_GATHER_SERVE, err=err,
                      sel_idx=sel_idx)
    torch.cuda.synchronize()
    assert int(err) == 2
    got = sel.view(torch.int16).cpu().numpy().view(np.uint16)
    si = sel_idx.cpu().numpy()
    for b in range(B):
        for j in range(k):
            p = int(tk[b, j])
            if 0 <= p < L:
                assert np.array_equal(got[b, 0, j], full[b * L + p]) and si[b, 0, j] == j
            else:
                assert not got[b, 0, j].any() and si[b, 0, j] == -1
    pool = torch.zeros((B, pool_rows, 576), dtype=torch.bfloat16, device=DEV)
    is_hit = torch.zeros((B, 1, k), dtype=torch.uint8, device=DEV)
    slot_np = np.full((B, 1, k), -1, dtype=np.int32)
    slot_np[0, 0, :3] = [0, pool_rows, 5]                 # the second is past the pool
    slot_np[1, 0, 0] = 2
    dsa.dsa_gather_kv(t_i32(tk[:, None, :]), is_hit, t_i32(slot_np), None, pool, sel, dsa.DSA_GATHER_INSTALL,
                      err=err)
    torch.cuda.synchronize()
    assert int(err) == 3
    pool_np = pool.view(torch.int16).cpu().numpy().view(np.uint16)
    want = np.zeros((B, pool_rows, 576), dtype=np.uint16)
    want[0, 0], want[0, 5], want[1, 2] = full[tk[0, 0]], full[tk[0, 2]], full[L + tk[1, 0]]
    assert np.array_equal(pool_np, want)


# ------------------------------------------------------------------ gather
def test_gather_serve_and_install_bit_exact():
    rng = np.random.default_rng(9)
    B, L, k, n_sets, W = 2, 3000, 256, 32, 4
    full = rng.integers(0, 1 << 16, (B, L, 576), dtype=np.uint16)
    full_d = t_u16_as_bf16(full.reshape(B * L, 576))
    # pinned host copy of the same rows, read over the host link through its device alias
    host = torch.from_numpy(full.reshape(B * L, 576).view(np.int16)).pin_memory()
    prev = np.stack([np.sort(rng.choice(L, k, replace=False)) for _ in range(B)]).astype(np.int32)
    cur = np.stack([np.sort(np.concatenate([rng.choice(prev[b], k // 2, replace=False),
                                            rng.choice(np.setdiff1d(np.arange(L), prev[b]), k // 2,
                                                       replace=False)])) for b in range(B)]).astype(np.int32)
    pool = torch.zeros((B, n_sets * W, 576), dtype=torch.bfloat16, device=DEV)
    pids = torch.full((B, n_sets * W), -1, dtype=torch.int32, device=DEV)
    its = torch.full((B, L), -1, dtype=torch.int32, device=DEV)
    ptr = torch.zeros((B, n_sets), dtype=torch.int32, device=DEV)
    for tk in (prev, cur):
        tkd = t_i32(tk[:, None, :])
        is_hit = torch.empty((B, 1, k), dtype=torch.uint8, device=DEV)
        slot = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
        mp = torch.empty((B, k), dtype=torch.int32, device=DEV)
        ms = torch.empty((B, k), dtype=torch.int32, device=DEV)
        mc = torch.empty(B, dtype=torch.int32, device=DEV)
        dsa.dsa_plan(tkd, pids, its, ptr, n_sets, W, is_hit, slot, mp, ms, mc, commit=True)
        for src in (dsa.Rows(full_d, 1152, req_stride=L),
                    dsa.Rows(host, 1152, req_stride=L, base_ptr=host_device_ptr(host))):
            sel = torch.empty((B, 1, k, 576), dtype=torch.bfloat16, device=DEV)
            dsa.dsa_gather_kv(tkd, is_hit, slot, src, pool, sel, dsa.DSA_GATHER_SERVE)
            torch.cuda.synchronize()
            got = sel.view(torch.int16).cpu().numpy().view(np.uint16)
            for b in range(B):
                assert np.array_equal(got[b, 0], full[b, tk[b]])
        dsa.dsa_gather_kv(tkd, is_hit, slot, None, pool, sel, dsa.DSA_GATHER_INSTALL)
        torch.cuda.synchronize()
        pool_np = pool.view(torch.int16).cpu().numpy().view(np.uint16)
        pid_np = pids.cpu().numpy()
        for b in range(B):
            live = np.nonzero(pid_np[b] >= 0)[0]
            assert np.array_equal(pool_np[b, live], full[b, pid_np[b, live]])
    # the second step had hits: they were served from the pool
    assert int(is_hit.sum()) > 0


@pytest.mark.gpu
def test_decode_step_graph_replay_matches_eager():
    """The whole step captured in a HIP graph gives the eager result on every replay.

    Outputs are overwritten with garbage between replays, and eager work and
    synchronisations run between them; every kernel is deterministic, so the comparison is
    bit-exact.
    """
    wl = synth.make_workload(synth.spec(2).scaled(B=4, L=20000))
    dw = DevWorkload(wl)
    step = dw.decode_step()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        step.run(stream)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (step.scores, step.idx, step.o, step.lse)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step.run(stream)
    for rep in range(4):
        for t in (step.scores, step.idx, step.o, step.lse):
            t.view(torch.uint8).fill_(0x7F + rep)
        other = dw.decode_step()                    # eager work between the replays
        with torch.cuda.stream(stream):
            other.run(stream)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip((step.scores, step.idx, step.o, step.lse), ref):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), f"replay {rep}"
    assert int(dw.err) == 0


@pytest.mark.parametrize("kind", ["grid_f32", "e4m3_scaled", "mxfp4"])
def test_indexer_unresolvable_pages_score_neg_inf_and_count(kind):
    """Page ids past the cache or negative: those tokens score -inf and each counts one
    error; every other score is the oracle's."""
    qk = "grid_f32" if kind == "grid_f32" else "bf16"
    H = 4 if kind == "grid_f32" else 64
    D = 64 if kind == "grid_f32" else 128
    wk = "quarters" if kind == "grid_f32" else "u01_div64"      # quarters keep the fp32 grid exact
    wl = synth.make_workload(synth.spec(2).scaled(B=2, L=1000, idx_heads=H, idx_dim=D, idx_q_kind=qk,
                                                  idx_k_kind=kind, w_kind=wk), with_kv=False)
    wl.seq_lens = np.array([1000, 700], dtype=np.int32)
    ref = [o_idx.scores(wl, b) for b in range(wl.B)]          # oracle on the intact table
    dw = DevWorkload(wl, with_kv=False)
    pt = dw.page_table.clone()
    pt[0, 3] = wl.num_pages + 7                               # past the cache
    pt[1, 10] = -5                                            # negative (page 10 holds 700 - 640 = 60 tokens)
    dw.page_table.copy_(pt)
    got = dw.scores().cpu().numpy()
    bad = {0: range(192, 256), 1: range(640, 700)}
    for b in range(wl.B):
        L = int(wl.seq_lens[b])
        want = ref[b].copy()
        want[:, list(bad[b])] = -np.inf
        g = got[b, :, :L]
        assert np.array_equal(np.isneginf(g), np.isneginf(want)), b
        fin = np.isfinite(want)
        if kind == "grid_f32":
            assert np.array_equal(g[fin], want[fin])
        else:
            for t in range(wl.Sq):
                n = o_idx.visible_len(L, wl.Sq, t)
                bound = indexer_bound(wl, b, t, n)
                ok = fin[t, :n]
                err = np.abs(g[t, :n][ok].astype(np.float64) - want[t, :n][ok].astype(np.float64))
                assert (err <= bound[ok]).all(), f"b={b} t={t}: max err/bound {(err / bound[ok]).max():.3g}"
    assert int(dw.err) == 64 + 60


@pytest.mark.parametrize("kind", ["e4m3_scaled", "mxfp4"])
def test_indexer_dense_key_layout(kind):
    """Keys stored densely per request (no page table, req_stride rows per request, a
    multiple of 32): scores equal the oracle's over the same keys laid out in pages."""
    wl = synth.make_workload(synth.spec(2).scaled(B=3, L=1000, idx_heads=64, idx_k_kind=kind), with_kv=False)
    wl.seq_lens = np.array([1000, 517, 33], dtype=np.int32)
    ref = [o_idx.scores(wl, b) for b in range(wl.B)]
    stride = 1024
    D = wl.idx_k.shape[-1]
    flat_k = wl.idx_k.reshape(-1, D)
    sc_w = wl.idx_k_scale.shape[-1] if kind == "mxfp4" else 1
    flat_s = wl.idx_k_scale.reshape(-1, sc_w)
    dense_k = np.zeros((wl.B * stride, D), dtype=flat_k.dtype)
    dense_s = np.zeros((wl.B * stride, sc_w), dtype=flat_s.dtype)
    for b in range(wl.B):
        rows = o_pg.paged_rows(wl.page_table[b], np.arange(int(wl.seq_lens[b])), wl.page_size)
        dense_k[b * stride:b * stride + len(rows)] = flat_k[rows]
        dense_s[b * stride:b * stride + len(rows)] = flat_s[rows]
    dw = DevWorkload(wl, with_kv=False)
    kd = torch.from_numpy(dense_k).to(DEV)
    sd = torch.from_numpy(dense_s.reshape(-1) if kind != "mxfp4" else dense_s).to(DEV)
    keys = dsa.Rows(kd, D, req_stride=stride)
    sc = torch.full((wl.B, 1, 1000), float("nan"), dtype=torch.float32, device=DEV)
    dsa.dsa_indexer_scores(dw.idx_q, dw.idx_w, keys, sd, dw.seq_lens, sc, k_dtype=dw.k_dtype, err=dw.err,
                           q_dtype=dw.q_dtype)
    got = sc.cpu().numpy()
    assert int(dw.err) == 0
    for b in range(wl.B):
        L = int(wl.seq_lens[b])
        bound = indexer_bound(wl, b, 0, L)
        err = np.abs(got[b, 0, :L].astype(np.float64) - ref[b][0].astype(np.float64))
        assert (err <= bound).all(), b


# every MFMA instantiation: (heads, query tokens) x query dtype x key layout
_SHAPES = [(32, 1), (32, 2), (32, 4), (32, 8), (64, 1), (64, 2), (64, 4), (128, 1), (128, 2)]


@pytest.mark.parametrize("H,Sq", _SHAPES)
@pytest.mark.parametrize("qk", ["bf16", "e4m3"])
@pytest.mark.parametrize("keys", ["e4m3_scaled", "mxfp4"])
def test_indexer_every_mfma_instantiation(H, Sq, qk, keys):
    ps = {1: 64, 2: 32, 4: 128, 8: 32}[Sq]
    wl = synth.make_workload(synth.spec(2).scaled(B=2, L=1300, Sq=Sq, idx_heads=H, idx_q_kind=qk,
                                                  idx_k_kind=keys, page_size=ps, seed=H + Sq), with_kv=False)
    wl.seq_lens = np.array([1300, 97 + Sq], dtype=np.int32)
    dw = DevWorkload(wl, with_kv=False)
    check_scores(wl, dw.scores())
    assert int(dw.err) == 0
