"""dsa_kv_write against the oracle, byte for byte: latent rows, e4m3 or MXFP4 key codes,
scales, untouched rows and the error count."""
import numpy as np
import pytest
import torch

import paged_kv_cache_indexer_amd as dsa
from oracle import formats as of, kvwrite as okw
from tests.dsa_dev import DEV

pytestmark = pytest.mark.gpu


def _tie_row(D):
    """amax = 448 makes sigma exactly 1, so k / sigma = k: the row holds e4m3 midpoints
    (ties), subnormal midpoints, -0.0 and values just past 448's neighbours."""
    pos = of.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    rng = np.random.default_rng(3)
    pick = np.concatenate([mids[:12], mids[rng.choice(np.arange(12, mids.size), D - 16, replace=False)]])
    row = np.concatenate([[448.0, -0.0, -mids[3], -mids[40]], pick]).astype(np.float32)
    assert row.size == D and np.array_equal(row.astype(np.float64), np.concatenate([[448.0, -0.0, -mids[3], -mids[40]], pick]))
    return row


def _fp4_tie_row(D):
    """Blocks scaled by 2^(j-1) holding E2M1 midpoints (ties), values between them, -0.0 and,
    in the fourth block, magnitudes that saturate (7.5 and 6.5 with a shared exponent of 0)."""
    base = [4.0, -0.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 5.5, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5,
            -5.0, 0.1, 0.3, 0.6, 0.9, 1.1, 1.4, 1.6, 1.9, 2.2, 2.8, 3.2, 3.8, 4.5, 5.9, 3.0]
    row = []
    for j in range(D // 32):
        blk = [v * 2.0 ** (j - 1) for v in base]
        if j == 3:
            blk[0], blk[9] = 7.5, -6.5
        row += blk
    return np.array(row, dtype=np.float32)


def _run(seed, B, Sq, D, ps, P, key_dtype, seq_lens, bad=(), separate_tables=False, cache="e4m3"):
    rng = np.random.default_rng(seed)
    n_pages = B * P + 3
    rows = n_pages * ps
    kv_pt = rng.permutation(n_pages)[: B * P].reshape(B, P).astype(np.int32)
    ic_pt = rng.permutation(n_pages)[: B * P].reshape(B, P).astype(np.int32) if separate_tables else kv_pt.copy()
    for b, p in bad:
        kv_pt[b, p] = -1
    lat = rng.integers(0, 65536, (B, Sq, 576), dtype=np.uint16)
    mag = 10.0 ** rng.uniform(-3, 3, (B, Sq, 1))                    # per-token scales over six decades
    keys = (rng.standard_normal((B, Sq, D)) * mag).astype(np.float32)
    keys[0, 0] = 0.0                                                  # zero key
    if B * Sq > 1:
        keys[0, 1 % Sq if Sq > 1 else 0] = 0.0
        keys.reshape(-1, D)[1, :] = 0.0
        keys.reshape(-1, D)[1, 5] = -2.5                              # one nonzero element
    if B * Sq > 2:
        keys.reshape(-1, D)[2] = _tie_row(D) if cache == "e4m3" else _fp4_tie_row(D)
    if key_dtype == torch.bfloat16:
        kbits = torch.from_numpy(keys).to(torch.bfloat16).view(torch.uint16).numpy()
        k_host, k_dev = kbits, torch.from_numpy(keys).to(torch.bfloat16).to(DEV)
    else:
        k_host, k_dev = keys, torch.from_numpy(keys).to(DEV)
    kv0 = rng.integers(0, 65536, (rows, 576), dtype=np.uint16)
    fp4 = cache == "mxfp4"
    ic0 = rng.integers(0, 256, (rows, D // 2 if fp4 else D), dtype=np.uint8)
    is0 = rng.integers(0, 256, (rows, D // 32), dtype=np.uint8) if fp4 else rng.standard_normal(rows).astype(np.float32)
    lens = np.asarray(seq_lens, dtype=np.int32)
    # oracle: the idx cache may use its own table; run the scatter once per cache
    kv_r, _, _, err_kv = okw.kv_write(lat, k_host, lens, kv_pt, ps, kv0, ic0, is0, cache=cache)
    _, ic_r, is_r, err_ic = okw.kv_write(lat, k_host, lens, ic_pt, ps, kv0, ic0, is0, cache=cache)
    # a token skipped in either cache is skipped in both on the device
    skip = []
    for b in range(B):
        for t in range(Sq):
            p = int(lens[b]) - Sq + t
            def row(pt):
                if p < 0 or p // ps >= P or pt[b, p // ps] < 0:
                    return -1
                return int(pt[b, p // ps]) * ps + p % ps
            rk, ri = row(kv_pt), row(ic_pt)
            if rk < 0 or ri < 0:
                skip.append((rk, ri))
    for rk, ri in skip:                                               # restore rows the device leaves alone
        if rk >= 0:
            kv_r[rk] = kv0[rk]
        if ri >= 0:
            ic_r[ri], is_r[ri] = ic0[ri], is0[ri]
    kv_d = torch.from_numpy(kv0.view(np.int16)).to(DEV)
    ic_d = torch.from_numpy(ic0).to(DEV)
    is_d = torch.from_numpy(is0).to(DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    dsa.dsa_kv_write(torch.from_numpy(lat.view(np.int16)).to(DEV), k_dev, torch.from_numpy(lens).to(DEV),
                     dsa.Rows(kv_d, 1152, torch.from_numpy(kv_pt).to(DEV), ps),
                     dsa.Rows(ic_d, D // 2 if fp4 else D, torch.from_numpy(ic_pt).to(DEV), ps), is_d, err,
                     cache_dtype=dsa.DSA_MXFP4 if fp4 else dsa.DSA_E4M3)
    torch.cuda.synchronize()
    assert np.array_equal(kv_d.cpu().numpy().view(np.uint16), kv_r)
    assert np.array_equal(ic_d.cpu().numpy(), ic_r)
    if fp4:
        assert np.array_equal(is_d.cpu().numpy(), is_r)
    else:
        assert np.array_equal(is_d.cpu().numpy().view(np.uint32), is_r.view(np.uint32))
    assert int(err.item()) == len(skip)
    return len(skip)


@pytest.mark.parametrize("key_dtype", [torch.float32, torch.bfloat16])
def test_kv_write_decode_batch(key_dtype):
    assert _run(1, B=32, Sq=1, D=128, ps=64, P=4, key_dtype=key_dtype,
                seq_lens=np.random.default_rng(9).integers(1, 257, 32)) == 0


def test_kv_write_mtp_tokens_ragged_and_invalid():
    # Sq = 4: request 1 is shorter than Sq (negative positions), request 2 lands on an
    # unallocated page, request 3 runs past its page-table row
    n = _run(2, B=5, Sq=4, D=128, ps=16, P=4, key_dtype=torch.float32,
             seq_lens=[40, 2, 33, 70, 64], bad=[(2, 2)], separate_tables=True)
    assert n == 2 + 1 + 4            # request 2 loses only position 32 (page 2)


def test_kv_write_small_key_dim():
    _run(4, B=3, Sq=2, D=64, ps=32, P=2, key_dtype=torch.bfloat16, seq_lens=[10, 64, 33])


@pytest.mark.parametrize("key_dtype", [torch.float32, torch.bfloat16])
def test_kv_write_mxfp4_decode_batch(key_dtype):
    assert _run(5, B=32, Sq=1, D=128, ps=64, P=4, key_dtype=key_dtype,
                seq_lens=np.random.default_rng(8).integers(1, 257, 32), cache="mxfp4") == 0


def test_kv_write_mxfp4_ties_ragged_and_invalid():
    n = _run(6, B=5, Sq=4, D=128, ps=16, P=4, key_dtype=torch.float32,
             seq_lens=[40, 2, 33, 70, 64], bad=[(2, 2)], separate_tables=True, cache="mxfp4")
    assert n == 2 + 1 + 4


def test_kv_write_mxfp4_small_key_dim():
    _run(7, B=3, Sq=2, D=64, ps=32, P=2, key_dtype=torch.bfloat16, seq_lens=[10, 64, 33], cache="mxfp4")


def test_mxfp4_written_keys_are_what_the_indexer_scores():
    """End to end over the FP4 indexer cache: dsa_kv_write quantizes the decode batch's new
    keys into MXFP4 rows, dsa_indexer_scores then reads those rows; the scores match the
    oracle's write followed by the oracle's scores."""
    import synth
    from oracle import indexer as o_idx
    from tests.dsa_dev import DevWorkload
    wl = synth.make_workload(synth.spec(2).scaled(B=3, L=700, idx_k_kind="mxfp4"), with_kv=False)
    wl.seq_lens = np.array([700, 512, 65], dtype=np.int32)
    rng = np.random.default_rng(12)
    new_keys = (rng.standard_normal((wl.B, 1, 128)) * 3).astype(np.float32)
    lat = rng.integers(0, 65536, (wl.B, 1, 576), dtype=np.uint16)
    ic0 = wl.idx_k.reshape(-1, 64)
    is0 = wl.idx_k_scale.reshape(-1, 4)
    kv0 = np.zeros((ic0.shape[0], 576), dtype=np.uint16)
    _, ic_r, is_r, err = okw.kv_write(lat, new_keys, wl.seq_lens, wl.page_table, wl.page_size, kv0, ic0, is0,
                                      cache="mxfp4")
    assert err == 0
    dw = DevWorkload(wl, with_kv=False)
    kv_d = torch.zeros((ic0.shape[0], 576), dtype=torch.int16, device=DEV)
    errd = torch.zeros(1, dtype=torch.int32, device=DEV)
    dsa.dsa_kv_write(torch.from_numpy(lat.view(np.int16)).to(DEV), torch.from_numpy(new_keys).to(DEV),
                     dw.seq_lens, dsa.Rows(kv_d, 1152, dw.page_table, wl.page_size), dw.keys, dw.k_scale, errd,
                     cache_dtype=dsa.DSA_MXFP4)
    sc = dw.scores()
    torch.cuda.synchronize()
    assert int(errd.item()) == 0 and int(dw.err.item()) == 0
    assert np.array_equal(dw.idx_k.cpu().numpy().reshape(-1, 64), ic_r)
    assert np.array_equal(dw.k_scale.cpu().numpy().reshape(-1, 4), is_r)
    wl.idx_k, wl.idx_k_scale = ic_r.reshape(wl.idx_k.shape), is_r.reshape(wl.idx_k_scale.shape)
    got = sc.cpu().numpy()
    for b in range(wl.B):
        L = int(wl.seq_lens[b])
        ref = o_idx.scores(wl, b)
        k = o_idx.request_keys(wl, b, np.arange(L))
        q = o_idx.decode_query(wl.idx_q[b, 0], wl.idx_q_dtype)
        bound = 2e-5 * (wl.idx_w[b, 0].astype(np.float64) @ (np.abs(q) @ np.abs(k).T)) + 1e-30
        assert (np.abs(got[b, 0, :L].astype(np.float64) - ref[0].astype(np.float64)) <= bound).all(), b
