"""Pins for the oracle's indexer scores.

Each case reduces the score to something fixed independently of the oracle's code:
a library dot product, an exact identity of ReLU, or an invariance of paging.
"""
import dataclasses
import os

import numpy as np
import torch

import synth
from oracle import indexer


def grid_workload(L=300, H=4, D=64, Sq=1, seed=0):
    return synth.make_workload(synth.spec(1).scaled(L=L, idx_heads=H, idx_dim=D, Sq=Sq, seed=seed), with_kv=False)


def keys_dense(wl, b):
    return indexer.request_keys(wl, b, np.arange(wl.seq_lens[b]))


def test_single_head_positive_is_plain_dot():
    wl = grid_workload(H=1)
    wl.idx_q = np.abs(wl.idx_q) + 1
    wl.idx_k = np.abs(wl.idx_k)
    wl.idx_w = np.ones_like(wl.idx_w)
    got = indexer.scores(wl, 0)[0]
    K = keys_dense(wl, 0)
    want = np.array([np.dot(wl.idx_q[0, 0, 0].astype(np.float64), K[s]) for s in range(len(K))])
    assert np.array_equal(got, want.astype(np.float32))


def test_relu_gate_identity():
    # for one head with weight 1: score(q) - score(-q) = q.k and both are >= 0
    wl = grid_workload(H=1)
    wl.idx_w = np.ones_like(wl.idx_w)
    pos = indexer.scores(wl, 0)[0].astype(np.float64)
    neg = dataclasses.replace(wl, idx_q=-wl.idx_q)
    negs = indexer.scores(neg, 0)[0].astype(np.float64)
    K = keys_dense(wl, 0)
    dots = np.array([np.dot(wl.idx_q[0, 0, 0].astype(np.float64), K[s]) for s in range(len(K))])
    assert (pos >= 0).all() and (negs >= 0).all()
    assert np.array_equal(pos - negs, dots)
    assert (dots < 0).any() and (dots > 0).any()


def test_one_hot_head_weights_and_linearity():
    wl = grid_workload(H=4)
    K = keys_dense(wl, 0)
    total = np.zeros(len(K))
    for h in range(4):
        w = np.zeros_like(wl.idx_w)
        w[0, 0, h] = wl.idx_w[0, 0, h]
        one = indexer.scores(dataclasses.replace(wl, idx_w=w), 0)[0].astype(np.float64)
        d = np.array([np.dot(wl.idx_q[0, 0, h].astype(np.float64), K[s]) for s in range(len(K))])
        assert np.array_equal(one, wl.idx_w[0, 0, h] * np.maximum(d, 0))
        total += one
    assert np.array_equal(indexer.scores(wl, 0)[0].astype(np.float64), total)


def test_page_permutation_invariance():
    wl = grid_workload(L=333)
    rng = np.random.default_rng(3)
    perm = rng.permutation(wl.num_pages)              # new physical page of old page i
    k2 = np.empty_like(wl.idx_k)
    k2[perm] = wl.idx_k
    pt2 = wl.page_table.copy()
    ok = pt2 >= 0
    pt2[ok] = perm[pt2[ok]]
    wl2 = dataclasses.replace(wl, idx_k=k2, page_table=pt2)
    assert np.array_equal(indexer.scores(wl, 0), indexer.scores(wl2, 0))


def test_e4m3_scale_is_per_token_and_positive_homogeneous():
    wl = synth.make_workload(synth.spec(2).scaled(B=1, L=200, idx_heads=8), with_kv=False)
    base = indexer.scores(dataclasses.replace(wl, idx_k_scale=np.ones_like(wl.idx_k_scale)), 0)[0]
    got = indexer.scores(wl, 0)[0]
    sig = wl.idx_k_scale.reshape(-1)[indexer.paged_rows(wl.page_table[0], np.arange(200), wl.page_size)]
    # the bf16 x e4m3 products are exact, so the float64 sums differ only by the factor sigma
    np.testing.assert_allclose(got.astype(np.float64), base.astype(np.float64) * sig, rtol=2e-7, atol=0)
    # decoded keys equal torch's float8 decode times sigma
    codes = wl.idx_k.reshape(-1, wl.idx_k.shape[-1])
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref = ref * wl.idx_k_scale.reshape(-1)[:, None].astype(np.float64)
    rows = indexer.paged_rows(wl.page_table[0], np.arange(200), wl.page_size)
    assert np.array_equal(indexer.request_keys(wl, 0, np.arange(200)), ref[rows])


def test_visibility_of_draft_queries():
    wl = grid_workload(L=300, Sq=4)
    sc = indexer.scores(wl, 0)
    for t in range(4):
        n = 300 - 4 + 1 + t                       # history 296 tokens + drafts 0..t
        assert np.isfinite(sc[t, :n]).all()
        assert np.isneginf(sc[t, n:]).all()


def mxfp4_workload(L=200, H=8, seed=0):
    return synth.make_workload(synth.spec(2).scaled(B=1, L=L, idx_heads=H, idx_k_kind="mxfp4", seed=seed),
                               with_kv=False)


def _golden_e2m1():
    path = os.path.join(os.path.dirname(__file__), "golden", "ocp_e2m1_codes.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    return {int(c, 16): float(v) for c, v in rows}


def test_mxfp4_scores_equal_fp32_scores_of_the_decoded_keys():
    # decode every key by hand (nibble loop over the OCP E2M1 table, torch's E8M0 decode),
    # store the values as fp32 keys, and score them on the plain fp32 path
    wl = mxfp4_workload(L=150)
    table = _golden_e2m1()
    packed = wl.idx_k.reshape(-1, 64)
    sc = torch.from_numpy(wl.idx_k_scale.reshape(-1, 4).copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    dec = np.empty((packed.shape[0], 128), dtype=np.float32)
    for r in range(packed.shape[0]):
        for i in range(64):
            byte = int(packed[r, i])
            for half, code in ((0, byte & 0xF), (1, byte >> 4)):
                d = 2 * i + half
                dec[r, d] = table[code] * sc[r, d // 32]
    f32 = dataclasses.replace(wl, idx_k=dec.reshape(wl.num_pages, wl.page_size, 128), idx_k_dtype="f32",
                              idx_k_scale=None)
    assert np.array_equal(indexer.scores(wl, 0), indexer.scores(f32, 0))


def test_mxfp4_block_scale_acts_on_its_own_32_dimensions():
    wl = mxfp4_workload(L=100, H=1)
    wl.idx_w = np.ones_like(wl.idx_w)
    for j in range(4):
        # query: +1 on block j's dimensions only (bf16 1.0 = 0x3F80), so the score is
        # max(0, 2^(e_j - 127) * sum of that block's codes' values)
        q = np.zeros_like(wl.idx_q)
        q[0, 0, 0, 32 * j:32 * j + 32] = 0x3F80
        base = dataclasses.replace(wl, idx_q=q)
        s0 = indexer.scores(base, 0)[0]
        for k in range(4):
            sc = wl.idx_k_scale.copy()
            sc[..., k] += 1
            s1 = indexer.scores(dataclasses.replace(base, idx_k_scale=sc), 0)[0]
            assert np.array_equal(s1, s0 * (2 if k == j else 1)), (j, k)
    assert (s0 > 0).any()


def test_exact_grid_scores_equal_integer_arithmetic():
    """The tiny workload's grid (q, k integers in [-4, 4], w in {1/4, 1/2, 1}): 4 * score is
    the integer sum_h (4 w_h) max(0, sum_d q_hd k_sd), computed here in int64 from the page
    table by hand; the oracle's float32 scores equal it exactly, and so do scores over a
    three-query draft window."""
    for Sq in (1, 3):
        wl = synth.make_workload(synth.spec(1).scaled(Sq=Sq), with_kv=False)
        L, ps = int(wl.seq_lens[0]), wl.page_size
        D = wl.idx_k.shape[-1]
        flat = wl.idx_k.reshape(-1, D)
        K = np.empty((L, D), dtype=np.int64)
        for pos in range(L):
            K[pos] = flat[int(wl.page_table[0, pos // ps]) * ps + pos % ps].astype(np.int64)
        got = indexer.scores(wl, 0)
        for t in range(Sq):
            q = wl.idx_q[0, t].astype(np.int64)                  # [H, D]
            w4 = (wl.idx_w[0, t] * 4).astype(np.int64)
            assert np.array_equal(w4.astype(np.float32) / 4, wl.idx_w[0, t])
            want4 = (np.maximum(K @ q.T, 0) * w4).sum(axis=1)      # [L] int64
            n = L - Sq + 1 + t
            assert np.array_equal(got[t, :n].astype(np.float64) * 4, want4[:n].astype(np.float64))
            assert np.isneginf(got[t, n:]).all()
            assert (want4 > 0).any() and (np.abs(want4[:n]) < 2 ** 24).all()
