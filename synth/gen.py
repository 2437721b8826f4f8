"""Seeded generators for the DSA decode workloads.

Every tensor is drawn from ``numpy.random.default_rng(SeedSequence([seed, cid,
tensor_id, *chunk]))``.  Large tensors are drawn in independently seeded chunks of
rows, so the bytes do not depend on thread count or on how much of a tensor is
materialised.  Results are raw storage arrays:

* bf16  -> ``uint16`` bit patterns (fp32 draw, cast by torch, round-to-nearest-even)
* e4m3  -> ``uint8``  OCP FP8 E4M3FN codes (cast by torch, round-to-nearest-even)
* mxfp4 -> ``uint8``  packed E2M1 codes (two per byte) plus one E8M0 code per 32
  elements, both drawn directly as codes
* fp32 / int32 / int64 as themselves

Paged caches are stored in *physical* page order: one seeded permutation of all
physical pages of the batch, with each request's page-table row taking the next
consecutive chunk of that permutation.  Page-table entries past a request's last
page are -1 and are never dereferenced.

None of the method's arithmetic lives here.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np
import torch

from .configs import WorkloadSpec, spec as _spec

# tensor ids (part of every seed key)
T_PAGEPERM, T_IDXQ, T_IDXW, T_IDXK, T_MLAQ, T_KV, T_LENS, T_LOGPAGE, T_TRAJ, T_HOSTKV, T_POOLQ, T_DRAFT = range(1, 13)

CHUNK_ROWS = 1 << 14
E4M3_MAX = 448.0
_POOL = ThreadPoolExecutor(max_workers=8)


def _ss(*key) -> np.random.SeedSequence:
    return np.random.SeedSequence([int(k) for k in key])


def _rng(*key) -> np.random.Generator:
    return np.random.default_rng(_ss(*key))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def _chunks(n_rows: int):
    for c in range(0, max(1, math.ceil(n_rows / CHUNK_ROWS))):
        lo = c * CHUNK_ROWS
        yield c, lo, min(n_rows, lo + CHUNK_ROWS)


def normal_bf16_rows(key, n_rows: int, width: int, out: Optional[np.ndarray] = None) -> np.ndarray:
    """[n_rows, width] bf16 bits of N(0,1) draws, chunk c seeded by key + (c,)."""
    if out is None:
        out = np.empty((n_rows, width), dtype=np.uint16)

    def work(args):
        c, lo, hi = args
        x = _rng(*key, c).standard_normal((hi - lo, width), dtype=np.float32)
        out[lo:hi] = to_bf16_bits(x)

    list(_POOL.map(work, list(_chunks(n_rows))))
    return out


def scaled_e4m3_rows(key, n_rows: int, width: int):
    """Keys 'N(0,1) scaled to fit' e4m3: per row sigma = max|k|/448, code = e4m3(k/sigma).

    Returns (codes uint8 [n_rows, width], sigma float32 [n_rows]); the dequantised
    key is e4m3(code) * sigma.
    """
    codes = np.empty((n_rows, width), dtype=np.uint8)
    sig = np.empty((n_rows,), dtype=np.float32)

    def work(args):
        c, lo, hi = args
        x = _rng(*key, c).standard_normal((hi - lo, width), dtype=np.float32)
        s = (np.abs(x).max(axis=1) / np.float32(E4M3_MAX)).astype(np.float32)
        s = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
        y = np.clip(x / s[:, None], -E4M3_MAX, E4M3_MAX)
        codes[lo:hi] = to_e4m3_codes(y)
        sig[lo:hi] = s

    list(_POOL.map(work, list(_chunks(n_rows))))
    return codes, sig


MXFP4_SCALE_CODES = (124, 128)     # E8M0 block codes drawn uniformly in this range (2^-3 .. 2^1)


def mxfp4_rows(key, n_rows: int, width: int):
    """MXFP4 keys drawn as codes: uniform random bytes (every E2M1 code equally likely in
    each nibble) and E8M0 block-scale codes uniform in MXFP4_SCALE_CODES.

    Returns (packed uint8 [n_rows, width/2], scales uint8 [n_rows, width/32]).
    """
    assert width % 32 == 0
    packed = np.empty((n_rows, width // 2), dtype=np.uint8)
    scales = np.empty((n_rows, width // 32), dtype=np.uint8)
    lo, hi = MXFP4_SCALE_CODES

    def work(args):
        c, a, b = args
        g = _rng(*key, c)
        packed[a:b] = g.integers(0, 256, (b - a, width // 2), dtype=np.uint8)
        scales[a:b] = g.integers(lo, hi + 1, (b - a, width // 32), dtype=np.uint8)

    list(_POOL.map(work, list(_chunks(n_rows))))
    return packed, scales


@dataclass
class Workload:
    spec: WorkloadSpec
    B: int
    Sq: int
    seq_lens: np.ndarray                 # int32 [B]   cache length (incl. draft tokens)
    page_size: int
    page_table: np.ndarray               # int32 [B, max_pages], -1 past the last page
    num_pages: int
    topk: int
    scale: float
    idx_q: Optional[np.ndarray] = None   # [B,Sq,H,D] f32 | uint16(bf16) | uint8(e4m3)
    idx_q_dtype: str = ""
    idx_w: Optional[np.ndarray] = None   # f32 [B,Sq,H]
    idx_k: Optional[np.ndarray] = None   # [num_pages, ps, D] f32 | uint8(e4m3); [num_pages, ps, D/2] uint8(mxfp4)
    idx_k_dtype: str = ""
    idx_k_scale: Optional[np.ndarray] = None  # f32 [num_pages, ps]; uint8 [num_pages, ps, D/32] (mxfp4); or None
    mla_q: Optional[np.ndarray] = None   # uint16(bf16) [B,Sq,Hm,576]
    kv: Optional[np.ndarray] = None      # uint16(bf16) [num_pages, ps, 576]
    extra: Dict[str, object] = field(default_factory=dict)


def _page_table(cfg: WorkloadSpec, lens: np.ndarray, tid_key=()):
    ps = cfg.page_size
    npg = (lens.astype(np.int64) + ps - 1) // ps
    total = int(npg.sum())
    perm = _rng(cfg.seed, cfg.cid, T_PAGEPERM, *tid_key).permutation(total).astype(np.int32)
    maxp = int(npg.max()) if len(npg) else 0
    pt = np.full((len(lens), maxp), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(npg):
        pt[b, :n] = perm[off:off + n]
        off += int(n)
    return pt, total


def _draft_correlated(cfg: WorkloadSpec, x: np.ndarray) -> np.ndarray:
    """Speculative-decoding drafts follow the token before them: with draft_sigma > 0, query
    t >= 1 of every request is query 0 plus draft_sigma times its own N(0,1) draw (and its
    head weights are pulled towards query 0's likewise, in _indexer_query)."""
    if cfg.draft_sigma <= 0 or x.shape[1] < 2:
        return x
    y = x.copy()
    y[:, 1:] = x[:, :1] + np.float32(cfg.draft_sigma) * x[:, 1:]
    return y


def _indexer_query(cfg: WorkloadSpec, B: int):
    """Indexer queries and head weights (identical on every rank of a sharded cache)."""
    H, D = cfg.idx_heads, cfg.idx_dim
    s, c = cfg.seed, cfg.cid
    out = {}
    if cfg.idx_q_kind == "grid_f32":
        out["idx_q"] = _rng(s, c, T_IDXQ).integers(-4, 5, size=(B, cfg.Sq, H, D)).astype(np.float32)
        out["idx_q_dtype"] = "f32"
    elif cfg.idx_q_kind == "bf16":
        x = _draft_correlated(cfg, _rng(s, c, T_IDXQ).standard_normal((B, cfg.Sq, H, D), dtype=np.float32))
        out["idx_q"] = to_bf16_bits(x)
        out["idx_q_dtype"] = "bf16"
    elif cfg.idx_q_kind == "e4m3":
        x = _draft_correlated(cfg, _rng(s, c, T_IDXQ).standard_normal((B, cfg.Sq, H, D), dtype=np.float32))
        out["idx_q"] = to_e4m3_codes(np.clip(x, -E4M3_MAX, E4M3_MAX))
        out["idx_q_dtype"] = "e4m3"
    else:
        raise ValueError(cfg.idx_q_kind)
    if cfg.w_kind == "quarters":
        out["idx_w"] = _rng(s, c, T_IDXW).choice(
            np.array([0.25, 0.5, 1.0], dtype=np.float32), size=(B, cfg.Sq, H)).astype(np.float32)
    else:
        out["idx_w"] = (_rng(s, c, T_IDXW).random((B, cfg.Sq, H), dtype=np.float32)
                        / np.float32(64.0)).astype(np.float32)
    if cfg.draft_sigma > 0 and cfg.Sq > 1:
        # a draft's head weights follow the token before it the same way (and stay >= 0)
        w = out["idx_w"]
        w[:, 1:] = np.abs(w[:, :1] + np.float32(cfg.draft_sigma) * (w[:, 1:] - w[:, :1]))
    return out


def _indexer_keys(cfg: WorkloadSpec, num_pages: int, key_extra=()):
    """Paged indexer keys [num_pages, ps, D] (+ per-token scale for e4m3, block scales for mxfp4)."""
    D, ps = cfg.idx_dim, cfg.page_size
    s, c = cfg.seed, cfg.cid
    out = {}
    rows = num_pages * ps
    if cfg.idx_k_kind == "grid_f32":
        out["idx_k"] = _rng(s, c, T_IDXK, *key_extra).integers(-4, 5, size=(num_pages, ps, D)).astype(np.float32)
        out["idx_k_dtype"] = "f32"
        out["idx_k_scale"] = None
    elif cfg.idx_k_kind == "mxfp4":
        packed, sc = mxfp4_rows((s, c, T_IDXK) + tuple(key_extra), rows, D)
        out["idx_k"] = packed.reshape(num_pages, ps, D // 2)
        out["idx_k_dtype"] = "mxfp4"
        out["idx_k_scale"] = sc.reshape(num_pages, ps, D // 32)
    else:
        codes, sig = scaled_e4m3_rows((s, c, T_IDXK) + tuple(key_extra), rows, D)
        out["idx_k"] = codes.reshape(num_pages, ps, D)
        out["idx_k_dtype"] = "e4m3"
        out["idx_k_scale"] = sig.reshape(num_pages, ps)
    return out


def _mla_query(cfg: WorkloadSpec, B: int):
    q = normal_bf16_rows((cfg.seed, cfg.cid, T_MLAQ), B * cfg.Sq * cfg.mla_heads, cfg.kv_dim)
    return q.reshape(B, cfg.Sq, cfg.mla_heads, cfg.kv_dim)


def _latent_rows(cfg: WorkloadSpec, num_pages: int, key_extra=()):
    rows = normal_bf16_rows((cfg.seed, cfg.cid, T_KV) + tuple(key_extra), num_pages * cfg.page_size,
                            cfg.kv_dim)
    return rows.reshape(num_pages, cfg.page_size, cfg.kv_dim)


def _fill(w: Workload, cfg: WorkloadSpec, B: int, num_pages: int, with_kv: bool, key_extra=()):
    for k, v in _indexer_query(cfg, B).items():
        setattr(w, k, v)
    for k, v in _indexer_keys(cfg, num_pages, key_extra).items():
        setattr(w, k, v)
    w.mla_q = _mla_query(cfg, B)
    if with_kv:
        w.kv = _latent_rows(cfg, num_pages, key_extra)


def _fixed(cfg: WorkloadSpec, with_kv: bool = True) -> Workload:
    lens = np.full((cfg.B,), cfg.L, dtype=np.int32)
    pt, total = _page_table(cfg, lens)
    w = Workload(spec=cfg, B=cfg.B, Sq=cfg.Sq, seq_lens=lens, page_size=cfg.page_size,
                 page_table=pt, num_pages=total, topk=cfg.topk, scale=cfg.scale)
    _fill(w, cfg, cfg.B, total, with_kv)
    return w


# --------------------------------------------------------------------------------------
# mixed-length batch, one rank's share of a page-sharded cache
# --------------------------------------------------------------------------------------

def mixed_lengths(cfg: WorkloadSpec) -> np.ndarray:
    r = _rng(cfg.seed, cfg.cid, T_LENS)
    u = r.random(cfg.n_short)
    short = np.floor(np.exp(np.log(cfg.short_lo) + u * (np.log(cfg.short_hi) - np.log(cfg.short_lo))))
    short = np.clip(short, cfg.short_lo, cfg.short_hi).astype(np.int64)
    lens = np.concatenate([short, np.full(cfg.n_long, cfg.long_len, dtype=np.int64)])
    return lens.astype(np.int32)


def logical_page_ids(cfg: WorkloadSpec, lens: np.ndarray) -> np.ndarray:
    """Logical page id of page j of request b, with id mod N == j mod N (owner rotation).

    Within each residue class the ids are a seeded shuffle, so every id is used once.
    Returns int64 [B, max_pages], -1 past the last page.
    """
    N, ps = cfg.n_ranks, cfg.page_size
    npg = (lens.astype(np.int64) + ps - 1) // ps
    maxp = int(npg.max())
    q = np.full((len(lens), maxp), -1, dtype=np.int64)
    for r in range(N):
        items = [(b, j) for b in range(len(lens)) for j in range(r, int(npg[b]), N)]
        m = _rng(cfg.seed, cfg.cid, T_LOGPAGE, r).permutation(len(items)).astype(np.int64)
        for (b, j), mm in zip(items, m):
            q[b, j] = mm * N + r
    return q


def _sharded(cfg: WorkloadSpec, with_kv: bool = True) -> Workload:
    N, R, ps = cfg.n_ranks, cfg.rank, cfg.page_size
    lens = mixed_lengths(cfg)
    qids = logical_page_ids(cfg, lens)
    npg = (lens.astype(np.int64) + ps - 1) // ps
    # rank R's local pages: local page index = q // N for every q with q mod N == R
    n_local = int(sum(len(range(R, int(n), N)) for n in npg))
    owned_lens = np.zeros(len(lens), dtype=np.int32)
    maxo = max(len(range(R, int(n), N)) for n in npg)
    pt = np.full((len(lens), max(1, maxo)), -1, dtype=np.int32)
    for b in range(len(lens)):
        js = list(range(R, int(npg[b]), N))
        for i, j in enumerate(js):
            pt[b, i] = int(qids[b, j] // N)
            owned_lens[b] += min(ps, int(lens[b]) - j * ps)
    w = Workload(spec=cfg, B=len(lens), Sq=cfg.Sq, seq_lens=owned_lens, page_size=ps,
                 page_table=pt, num_pages=n_local, topk=cfg.topk, scale=cfg.scale)
    # queries are the same on every rank; the cache share is drawn with the rank in its key
    _fill(w, cfg, len(lens), n_local, with_kv, key_extra=(R,))
    w.extra.update(full_lens=lens, logical_page_ids=qids, n_ranks=N, rank=R)
    return w


# --------------------------------------------------------------------------------------
# device-pool group: synthetic top-k trajectory + host-resident latent rows
# --------------------------------------------------------------------------------------

def _zipf_positions(rng: np.random.Generator, cdf: np.ndarray, L: int, n: int) -> np.ndarray:
    u = rng.random(n)
    r = np.searchsorted(cdf, u, side="right") + 1          # rank in 1..L
    r = np.minimum(r, L)
    return (L - r).astype(np.int64)                        # rank 1 = most recent position


def topk_trajectory(cfg: WorkloadSpec) -> np.ndarray:
    """int32 [steps, B, k]: per step an ascending set of k distinct positions.

    Step 0: k distinct Zipf(a) draws over ranks 1..L (rank r is position L-r).
    Step s: keep round(keep_frac*k) of step s-1's set uniformly without replacement,
    then add Zipf draws that are neither in step s-1's set nor already drawn.
    """
    L, k = cfg.L, cfg.topk
    w = np.arange(1, L + 1, dtype=np.float64) ** (-cfg.zipf_a)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    n_keep = int(round(cfg.keep_frac * k))
    out = np.empty((cfg.steps, cfg.B, k), dtype=np.int32)
    for b in range(cfg.B):
        rng = _rng(cfg.seed, cfg.cid, T_TRAJ, b)
        prev = None
        for s in range(cfg.steps):
            if prev is None:
                chosen, seen = [], set()
                need = k
                excl = set()
            else:
                keep = rng.choice(prev, size=n_keep, replace=False)
                chosen, seen = [int(x) for x in keep], set(int(x) for x in keep)
                excl = set(int(x) for x in prev)
                need = k - n_keep
            got = 0
            while got < need:
                for p in _zipf_positions(rng, cdf, L, 4 * (need - got) + 16):
                    p = int(p)
                    if p in seen or p in excl:
                        continue
                    seen.add(p)
                    chosen.append(p)
                    got += 1
                    if got == need:
                        break
            cur = np.sort(np.array(chosen, dtype=np.int64))
            out[s, b] = cur
            prev = cur
    return out


def draft_selections(cfg: WorkloadSpec, first: np.ndarray, Sq: int, keep: float, step: int) -> np.ndarray:
    """Selections of Sq query tokens for one verify step: token 0 takes `first` [B, k]
    (ascending); token t keeps round(keep * k) positions of token t - 1's selection uniformly
    without replacement and adds Zipf(cfg.zipf_a) draws over the context that are not in it,
    as topk_trajectory does between decode steps.  Returns int32 [B, Sq, k], rows ascending."""
    L, k = cfg.L, cfg.topk
    w = np.arange(1, L + 1, dtype=np.float64) ** (-cfg.zipf_a)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    n_keep = int(round(keep * k))
    out = np.empty((first.shape[0], Sq, k), dtype=np.int32)
    for b in range(first.shape[0]):
        rng = _rng(cfg.seed, cfg.cid, T_DRAFT, step, b)
        prev = np.asarray(first[b], dtype=np.int64)
        out[b, 0] = prev
        for t in range(1, Sq):
            kept = rng.choice(prev, size=n_keep, replace=False)
            seen = set(int(x) for x in prev)
            chosen = [int(x) for x in kept]
            while len(chosen) < k:
                for p in _zipf_positions(rng, cdf, L, 4 * (k - len(chosen)) + 16):
                    p = int(p)
                    if p in seen:
                        continue
                    seen.add(p)
                    chosen.append(p)
                    if len(chosen) == k:
                        break
            prev = np.sort(np.array(chosen, dtype=np.int64))
            out[b, t] = prev
    return out


def _pool_group(cfg: WorkloadSpec, with_kv: bool = True) -> Workload:
    lens = np.full((cfg.B,), cfg.L, dtype=np.int32)
    w = Workload(spec=cfg, B=cfg.B, Sq=1, seq_lens=lens, page_size=cfg.page_size,
                 page_table=np.zeros((cfg.B, 0), np.int32), num_pages=0, topk=cfg.topk,
                 scale=cfg.scale)
    w.extra["traj"] = topk_trajectory(cfg)
    # per (step, layer) MLA queries
    q = normal_bf16_rows((cfg.seed, cfg.cid, T_POOLQ), cfg.steps * cfg.layers * cfg.B * cfg.mla_heads,
                         cfg.kv_dim)
    w.extra["mla_q"] = q.reshape(cfg.steps, cfg.layers, cfg.B, cfg.mla_heads, cfg.kv_dim)
    if with_kv:
        w.extra["host_kv"] = host_kv(cfg)
    w.extra.update(n_sets=cfg.n_sets, ways=cfg.ways, id_range=cfg.id_range,
                   steps=cfg.steps, layers=cfg.layers)
    return w


def host_kv(cfg: WorkloadSpec, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Full latent cache in host memory, layout [layer][request][position][576] bf16."""
    shape = (cfg.layers, cfg.B, cfg.L, cfg.kv_dim)
    if out is None:
        out = np.empty(shape, dtype=np.uint16)
    for l in range(cfg.layers):
        for b in range(cfg.B):
            normal_bf16_rows((cfg.seed, cfg.cid, T_HOSTKV, l, b), cfg.L, cfg.kv_dim, out=out[l, b])
    return out


def host_kv_rows(cfg: WorkloadSpec, layer: int, b: int, positions: np.ndarray) -> np.ndarray:
    """The rows of ``host_kv`` at the given positions, drawing only the chunks they touch."""
    positions = np.asarray(positions, dtype=np.int64)
    res = np.empty((len(positions), cfg.kv_dim), dtype=np.uint16)
    for c in np.unique(positions // CHUNK_ROWS):
        lo = int(c) * CHUNK_ROWS
        hi = min(cfg.L, lo + CHUNK_ROWS)
        x = _rng(cfg.seed, cfg.cid, T_HOSTKV, layer, b, int(c)).standard_normal((hi - lo, cfg.kv_dim),
                                                                               dtype=np.float32)
        rows = to_bf16_bits(x)
        sel = (positions // CHUNK_ROWS) == c
        res[sel] = rows[positions[sel] - lo]
    return res


def make_workload(cfg, with_kv: bool = True) -> Workload:
    """Build the seeded workload of a spec (or a config id)."""
    if isinstance(cfg, int):
        cfg = _spec(cfg)
    if cfg.steps > 0:
        return _pool_group(cfg, with_kv)
    if cfg.lens_kind == "loguniform_plus_long":
        return _sharded(cfg, with_kv)
    return _fixed(cfg, with_kv)
