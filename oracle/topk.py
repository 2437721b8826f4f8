"""Top-k selection for the oracle (test infrastructure only).

[GLM52] §2.1: the indexer keeps the k = 2048 most relevant history positions,
which are the only ones sparse attention reads.  Exact reading used here: among
the visible positions, order by (score descending, position ascending), with -0.0
treated as +0.0, and keep the first k; the result is reported in ascending
position order and padded with -1 when fewer than k positions are visible.
"""
import numpy as np


def select(scores_visible: np.ndarray, k: int) -> np.ndarray:
    """int32 [k]: ascending positions of the k best scores, -1 padded."""
    s = np.asarray(scores_visible, dtype=np.float32)
    assert not np.isnan(s).any()
    s = np.where(s == 0, np.float32(0.0), s)                  # -0.0 -> +0.0
    pos = np.arange(len(s), dtype=np.int64)
    order = np.lexsort((pos, -s.astype(np.float64)))          # score desc, then position asc
    chosen = np.sort(pos[order[:k]])
    out = np.full(k, -1, dtype=np.int32)
    out[:len(chosen)] = chosen
    return out


def select_rows(scores: np.ndarray, vis_lens, k: int) -> np.ndarray:
    """Row-wise ``select`` over a [R, Lmax] score matrix with per-row visible length."""
    return np.stack([select(scores[i, :int(n)], k) for i, n in enumerate(vis_lens)])
