"""Selected-row gather and pool install for the oracle (test infrastructure only).

[GLM52] §2.1: the rows sparse attention needs are scattered over the full cache
and must be gathered together first.  §4.4/§5: the per-layer serve step prepares
exactly those rows, from the device pool on a hit and from the host-resident full
cache on a miss; the install step later writes the surviving misses into their pool
slots.  Whatever the source, the served row of entry j is the full cache's row at
position topk[j]; padding entries (-1) serve a zero row.
"""
import numpy as np


def gather_rows(full_rows: np.ndarray, topk: np.ndarray) -> np.ndarray:
    """sel[..., j, :] = full_rows[topk[..., j]] (zero row where topk is -1)."""
    topk = np.asarray(topk, dtype=np.int64)
    out = np.zeros(topk.shape + full_rows.shape[1:], dtype=full_rows.dtype)
    ok = topk >= 0
    out[ok] = full_rows[topk[ok]]
    return out


def install(pool_rows: np.ndarray, full_rows: np.ndarray, miss_pos, miss_slot) -> np.ndarray:
    """Pool after backfill: pool[slot] = full_rows[pos] for every surviving miss."""
    pool = pool_rows.copy()
    for p, s in zip(np.asarray(miss_pos), np.asarray(miss_slot)):
        if s >= 0:
            pool[s] = full_rows[p]
    return pool


def union_select(topk: np.ndarray):
    """De-duplicated union of one request's selections (test infrastructure only).

    [GLM52] §4.2: the planner works on the de-duplicated, ascending union of the positions
    the query tokens of a step select, so a position several query tokens share is fetched
    once; §5.1: in speculative decoding the draft tokens' selections overlap.  Each query
    then attends over its own positions, which are a subset of the union.

    topk  int [Sq, k] positions (each row ascending, -1 padding)
    Returns (U int64 [n] ascending distinct valid positions,
             uidx int32 [Sq, k] index of each entry's position in U, -1 for padding,
             member bool [Sq, n] member[t, u] iff U[u] is one of query t's positions).
    """
    topk = np.asarray(topk, dtype=np.int64)
    U = np.unique(topk[topk >= 0])
    uidx = np.full(topk.shape, -1, dtype=np.int32)
    ok = topk >= 0
    uidx[ok] = np.searchsorted(U, topk[ok])
    member = np.zeros((topk.shape[0], len(U)), dtype=bool)
    for t in range(topk.shape[0]):
        member[t, uidx[t][uidx[t] >= 0]] = True
    return U, uidx, member
