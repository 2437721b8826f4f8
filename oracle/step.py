"""One request's decode step end to end, for the oracle (test infrastructure only).

[GLM52] §2.1 decode path: indexer scores every visible history token, the top-k
positions are kept, their latent rows are gathered, and MLA attention runs over
those rows only ([TSA] "MLA": 576-wide row as K, first 512 as V).
"""
import numpy as np

from . import indexer, topk as topk_mod, mla
from .paging import paged_rows


def selected_rows(wl, b: int, positions) -> np.ndarray:
    """Latent rows (uint16 bf16 bits [n, 576]) of request b at the given positions."""
    pos = np.asarray(positions, dtype=np.int64)
    pos = pos[pos >= 0]
    rows = paged_rows(wl.page_table[b], pos, wl.page_size)
    return wl.kv.reshape(-1, wl.kv.shape[-1])[rows]


def decode_request(wl, b: int, topk_override=None):
    """Returns dict(scores [Sq, L] f32, topk [Sq, k] i32, o [Sq, H, 512] f64, lse [Sq, H] f64).

    ``topk_override`` (int32 [Sq, k]) replaces the oracle's own selection for the
    attention stage, so attention can be compared on identical selections.
    """
    sc = indexer.scores(wl, b)
    L = int(wl.seq_lens[b])
    tk = np.stack([topk_mod.select(sc[t, :indexer.visible_len(L, wl.Sq, t)], wl.topk)
                   for t in range(wl.Sq)])
    use = tk if topk_override is None else np.asarray(topk_override)
    os, ls = [], []
    for t in range(wl.Sq):
        o, l = mla.sparse_mla(wl.mla_q[b, t], selected_rows(wl, b, use[t]), wl.scale)
        os.append(o)
        ls.append(l)
    return {"scores": sc, "topk": tk, "o": np.stack(os), "lse": np.stack(ls)}
