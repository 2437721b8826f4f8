"""Sparse MLA decode attention for the oracle (test infrastructure only).

[TSA] "MLA (tokenspeed-mla)": one latent row per token, 512 latent + 64 rope
values, is stored once and serves as both key (all 576) and value (the first 512).
[GLM52] §2.1: attention runs only over the selected positions.  Per query head:

    logit_j = scale * <q, K_j>         over the selected rows j
    lse     = ln sum_j exp(logit_j)    (natural log)
    o       = sum_j exp(logit_j - lse) * V_j

computed in float64; an empty selection gives o = 0 and lse = -inf.

[TSA] split-KV decode: partial (o, lse) over disjoint parts of the rows are merged
by LSE rescaling: lse = ln sum_r exp(lse_r), o = sum_r exp(lse_r - lse) * o_r.
"""
import numpy as np

from .formats import bf16_to_f64

V_DIM = 512


def sparse_mla(q_bits: np.ndarray, rows_bits: np.ndarray, scale: float, v_dim: int = V_DIM):
    """q_bits uint16 [H, 576]; rows_bits uint16 [n, 576] (the selected rows).

    Returns (o float64 [H, v_dim], lse float64 [H]).
    """
    q = bf16_to_f64(q_bits)
    H = q.shape[0]
    if len(rows_bits) == 0:
        return np.zeros((H, v_dim)), np.full(H, -np.inf)
    K = bf16_to_f64(rows_bits)
    logits = float(scale) * (q @ K.T)                     # [H, n]
    m = logits.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(logits - m).sum(axis=1))
    p = np.exp(logits - lse[:, None])
    o = p @ K[:, :v_dim]
    return o, lse


def lse_merge(os, lses):
    """Merge partial (o_r [H, V], lse_r [H]) into (o, lse) over the union of their rows."""
    lses = np.stack([np.asarray(l, dtype=np.float64) for l in lses])      # [R, H]
    os = np.stack([np.asarray(o, dtype=np.float64) for o in os])          # [R, H, V]
    m = lses.max(axis=0)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    wsum = np.exp(lses - safe_m).sum(axis=0)
    lse = np.where(np.isfinite(m), safe_m + np.log(np.where(wsum > 0, wsum, 1.0)), -np.inf)
    wts = np.where(np.isfinite(lses), np.exp(lses - np.where(np.isfinite(lse), lse, 0.0)), 0.0)
    o = (wts[:, :, None] * os).sum(axis=0)
    return o, lse
