"""Lightning-Indexer scores for the oracle (test infrastructure only).

[GLM52] §2.1: on the decode path the Lightning Indexer scores every history token
against the current query and keeps the most relevant positions for sparse
attention.  The score used by these workloads is the head-weighted, ReLU-gated
dot product

    score[b,t,s] = sum_h  w[b,t,h] * max(0, sigma_s * sum_d q[b,t,h,d] * c[b,s,d])

where c is the stored key (fp32, or an e4m3 code with per-token scale sigma_s;
sigma = 1 when absent).  The FP4 indexer cache that the TokenSpeed audit page lists
as an option of the DSA backend ("DSA": optional FP4 indexer cache) is not defined
there; it is read here as OCP MXFP4 keys: each block of 32 dimensions is E2M1 codes
times its own E8M0 power of two, decoded exactly, with sigma = 1.  Query t of a request with cache length L and Sq query
tokens sees positions [0, L - Sq + t]; other positions score -inf.  Evaluated in
float64 and rounded once to float32.
"""
import numpy as np

from .formats import bf16_to_f64, e4m3_to_f64, mxfp4_to_f64
from .paging import paged_rows


def decode_query(q, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(q, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f64(q)
    if dtype == "e4m3":
        return e4m3_to_f64(q)
    raise ValueError(dtype)


def request_keys(wl, b: int, positions) -> np.ndarray:
    """Dequantised keys [n, D] (float64) of request b at the given positions."""
    rows = paged_rows(wl.page_table[b], positions, wl.page_size)
    flat = wl.idx_k.reshape(-1, wl.idx_k.shape[-1])[rows]
    if wl.idx_k_dtype == "mxfp4":
        return mxfp4_to_f64(flat, wl.idx_k_scale.reshape(-1, wl.idx_k_scale.shape[-1])[rows])
    k = np.asarray(flat, dtype=np.float32).astype(np.float64) if wl.idx_k_dtype == "f32" else e4m3_to_f64(flat)
    if wl.idx_k_scale is not None:
        k = k * wl.idx_k_scale.reshape(-1)[rows].astype(np.float64)[:, None]
    return k


def visible_len(seq_len: int, Sq: int, t: int) -> int:
    return int(seq_len) - Sq + 1 + t


def scores_request(wl, b: int, t: int, positions=None) -> np.ndarray:
    """Scores of query t of request b over its visible positions (float32, length = visible).

    ``positions`` restricts the evaluation to a subset of visible positions.
    """
    n_vis = visible_len(wl.seq_lens[b], wl.Sq, t)
    pos = np.arange(n_vis) if positions is None else np.asarray(positions, dtype=np.int64)
    q = decode_query(wl.idx_q[b, t], wl.idx_q_dtype)            # [H, D]
    w = np.asarray(wl.idx_w[b, t], dtype=np.float32).astype(np.float64)  # [H]
    out = np.empty(len(pos), dtype=np.float32)
    step = 1 << 15
    for lo in range(0, len(pos), step):
        k = request_keys(wl, b, pos[lo:lo + step])              # [n, D]
        dots = q @ k.T                                          # [H, n]
        out[lo:lo + step] = (w @ np.maximum(dots, 0.0)).astype(np.float32)
    return out


def scores(wl, b: int) -> np.ndarray:
    """All queries of request b: float32 [Sq, L] with -inf at invisible positions."""
    L = int(wl.seq_lens[b])
    res = np.full((wl.Sq, L), -np.inf, dtype=np.float32)
    for t in range(wl.Sq):
        n = visible_len(L, wl.Sq, t)
        res[t, :n] = scores_request(wl, b, t)
    return res
