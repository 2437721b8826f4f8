"""Pins for the oracle's sparse MLA: dense attention when every token is selected
(torch SDPA in float64), permutation and single-row cases, and the LSE merge."""
import numpy as np
import torch
import torch.nn.functional as F

import synth
from oracle import formats, gather, mla


def rand_bits(rng, shape):
    return synth.gen.to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def test_all_selected_equals_dense_sdpa():
    rng = np.random.default_rng(0)
    H, n = 16, 333
    q, K = rand_bits(rng, (H, 576)), rand_bits(rng, (n, 576))
    scale = 1 / np.sqrt(576)
    o, lse = mla.sparse_mla(q, K, scale)
    qt = torch.from_numpy(formats.bf16_to_f64(q))[None, :, None, :]        # [1, H, 1, 576]
    Kt = torch.from_numpy(formats.bf16_to_f64(K))[None, None].expand(1, H, n, 576)
    Vt = Kt[..., :512]
    ref = F.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)[0, :, 0]
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-14)
    ref_lse = torch.logsumexp(scale * (qt[0, :, 0] @ Kt[0, 0].T), dim=-1).numpy()
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-13, atol=1e-13)


def test_sparse_selection_equals_dense_on_selected_rows():
    wl = synth.make_workload(synth.spec(1).scaled(L=500))
    from oracle.step import decode_request, selected_rows
    r = decode_request(wl, 0)
    rows = selected_rows(wl, 0, r["topk"][0])
    assert len(rows) == wl.topk
    o, lse = mla.sparse_mla(wl.mla_q[0, 0], rows, wl.scale)
    np.testing.assert_array_equal(o, r["o"][0])
    # k >= L: the selection is every token and attention is dense attention
    wl2 = synth.make_workload(synth.spec(1).scaled(L=200))
    r2 = decode_request(wl2, 0)
    assert list(r2["topk"][0][:200]) == list(range(200))
    allrows = wl2.kv.reshape(-1, 576)[wl2.page_table[0][np.arange(200) // 64] * 64 + np.arange(200) % 64]
    o2, l2 = mla.sparse_mla(wl2.mla_q[0, 0], allrows, wl2.scale)
    np.testing.assert_allclose(r2["o"][0], o2, rtol=1e-12, atol=1e-14)


def test_permutation_and_single_row():
    rng = np.random.default_rng(1)
    q, K = rand_bits(rng, (8, 576)), rand_bits(rng, (50, 576))
    o, lse = mla.sparse_mla(q, K, 0.05)
    o2, lse2 = mla.sparse_mla(q, K[rng.permutation(50)], 0.05)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, rtol=1e-13)
    o1, l1 = mla.sparse_mla(q, K[:1], 0.05)
    Kf, qf = formats.bf16_to_f64(K[0]), formats.bf16_to_f64(q)
    np.testing.assert_allclose(o1, np.broadcast_to(Kf[:512], o1.shape), rtol=1e-15)
    np.testing.assert_allclose(l1, 0.05 * (qf @ Kf), rtol=1e-13)
    oe, le = mla.sparse_mla(q, K[:0], 0.05)
    assert (oe == 0).all() and np.isneginf(le).all()


def test_lse_merge_over_partition_equals_union():
    rng = np.random.default_rng(2)
    q, K = rand_bits(rng, (8, 576)), rand_bits(rng, (200, 576))
    o, lse = mla.sparse_mla(q, K, 0.04)
    cuts = [0, 13, 13, 90, 200]                         # includes an empty part
    parts = [mla.sparse_mla(q, K[a:b], 0.04) for a, b in zip(cuts[:-1], cuts[1:])]
    om, lm = mla.lse_merge([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_allclose(om, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lm, lse, rtol=1e-13)


def test_gather_and_install():
    rng = np.random.default_rng(3)
    full = rng.integers(0, 1 << 16, (100, 576), dtype=np.uint16)
    tk = np.array([3, 7, 99, -1], dtype=np.int64)
    sel = gather.gather_rows(full, tk)
    assert np.array_equal(sel[:3], full[[3, 7, 99]]) and (sel[3] == 0).all()
    pool = np.zeros((8, 576), np.uint16)
    pool2 = gather.install(pool, full, [3, 7, 99], [5, -1, 0])
    assert np.array_equal(pool2[5], full[3]) and np.array_equal(pool2[0], full[99])
    assert (pool2[[1, 2, 3, 4, 6, 7]] == 0).all()
