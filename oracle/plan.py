"""Shared-group cache-pool plan (set-associative FIFO) for the oracle (test infrastructure only).

[GLM52] §3 and §4: a device-resident pool keeps latent rows of recently selected
tokens; per request it is split into n_sets independent sets of W ways.  A token id
maps to exactly one set (set = id mod n_sets here) and may sit in any way of it.
Each set keeps one FIFO pointer that advances once per installed entry; a hit does
not move it, so round-robin replacement is FIFO by install order (§4.3).  The
planner ("DsaPlan", §4.2 and §5) runs once per shared group of 4 layers: per top-k
entry it records whether the row comes from the pool or from the host, and it emits
a compact list of misses for backfill; every layer of the group reuses the plan,
and the pool metadata is advanced once, at the end of the group (§5.1).

Reading of the steps, per request and decode step:
  1. U = ascending de-duplicated union of the valid (>= 0) top-k positions of all
     query tokens.
  2. u is a hit iff id_to_slot[u] != -1.
  3. M = the misses of U, ascending.
  4. For set s let M_s be its misses in ascending order, m_s = |M_s|.  The i-th of
     them (0-based) is installed at way (ptr[s] + i) mod W, slot = s*W + way; it
     survives the step iff i >= m_s - W (later installs to the same way overwrite).
  5. ptr[s] <- (ptr[s] + m_s) mod W.
  6. Commit: for each survivor, clear the evicted occupant's id_to_slot entry, then
     set pool_ids[slot] = u and id_to_slot[u] = slot.
  7. Per top-k entry: is_hit and slot (the hit's slot, the survivor's new slot, or
     -1 for a miss that does not survive, and for -1 padding entries).
Every layer of the group is served from the state before the step (serve runs
before install), so one plan serves all 4 layers.
"""
import numpy as np


def plan_step(topk: np.ndarray, pool_ids: np.ndarray, id_to_slot: np.ndarray, ptr: np.ndarray,
              n_sets: int, ways: int):
    """Plan one decode step for one request.

    topk        int32 [Sq, k]   positions (ascending per row, -1 padded)
    pool_ids    int32 [n_sets*ways]   id held by each slot, -1 if empty
    id_to_slot  int32 [id_range]      slot of each id, -1 if not pooled
    ptr         int32 [n_sets]        FIFO pointer per set
    Returns (outputs dict, new (pool_ids, id_to_slot, ptr)); inputs are not modified.
    """
    topk = np.asarray(topk, dtype=np.int64)
    W = int(ways)
    valid = topk[topk >= 0]
    U = np.unique(valid)                                              # step 1
    id_range = len(id_to_slot)
    assert (U < id_range).all()
    hit_u = id_to_slot[U] != -1                                       # step 2
    M = U[~hit_u]                                                     # step 3
    new_slot_u = np.where(hit_u, id_to_slot[U], -1).astype(np.int64)

    ptr_new = np.array(ptr, dtype=np.int64).copy()
    miss_slot = np.full(len(M), -1, dtype=np.int64)
    sets = M % n_sets
    for s in np.unique(sets):                                          # step 4
        idx = np.nonzero(sets == s)[0]                                 # ascending already
        m_s = len(idx)
        for i, mi in enumerate(idx):
            if i >= m_s - W:
                miss_slot[mi] = int(s) * W + (int(ptr[s]) + i) % W
        ptr_new[s] = (int(ptr[s]) + m_s) % W                           # step 5

    pool_new = np.array(pool_ids, dtype=np.int64).copy()
    its_new = np.array(id_to_slot, dtype=np.int64).copy()
    for u, sl in zip(M, miss_slot):                                    # step 6
        if sl < 0:
            continue
        old = pool_new[sl]
        if old >= 0:
            its_new[old] = -1
        pool_new[sl] = u
        its_new[u] = sl

    new_slot_u[~hit_u] = miss_slot
    pos_in_u = {int(u): i for i, u in enumerate(U)}
    Sq, k = topk.shape
    is_hit = np.zeros((Sq, k), dtype=np.uint8)
    slot = np.full((Sq, k), -1, dtype=np.int32)
    for t in range(Sq):                                                # step 7
        for j in range(k):
            p = int(topk[t, j])
            if p < 0:
                continue
            i = pos_in_u[p]
            is_hit[t, j] = 1 if hit_u[i] else 0
            slot[t, j] = new_slot_u[i]
    out = {
        "is_hit": is_hit,
        "slot": slot,
        "miss_pos": M.astype(np.int32),
        "miss_slot": miss_slot.astype(np.int32),
        "miss_count": int(len(M)),
        "n_unique": int(len(U)),
        "n_hit": int(hit_u.sum()),
    }
    state = (pool_new.astype(np.int32), its_new.astype(np.int32), ptr_new.astype(np.int32))
    return out, state


def empty_state(n_sets: int, ways: int, id_range: int):
    return (np.full(n_sets * ways, -1, np.int32), np.full(id_range, -1, np.int32),
            np.zeros(n_sets, np.int32))


# --------------------------------------------------------------------------------------
# Replacement-policy comparison ([GLM52] §3: an 8192-entry device pool under LRU raises the
# average hit rate on the same top-k trajectory from keeping only the previous step's set;
# §4.3: the set-associative FIFO pool adopted instead).  These run on the CPU only; they
# measure policies on a trajectory and are not part of the device path.

def lru_hits(trajectory: np.ndarray, capacity: int) -> np.ndarray:
    """Hits per step of a fully associative LRU pool of `capacity` ids over one request's
    trajectory [steps, k] (each row ascending, -1 padded).

    Reading, in the plan's two phases: the step's de-duplicated set U is looked up
    against the pool before anything is installed (u is a hit iff pooled before the step);
    the hits are then touched in ascending position, and the misses installed after them in
    ascending position, so they are the most recently used.  The pool keeps the `capacity`
    most recently used ids (|U| <= capacity, so nothing of the current step is evicted).
    """
    last_use = {}
    hits = []
    for s, row in enumerate(np.asarray(trajectory)):
        U = np.unique(row[row >= 0])
        assert len(U) <= capacity
        is_hit = [u in last_use for u in U.tolist()]
        hits.append(sum(is_hit))
        for r, (u, h) in enumerate(zip(U.tolist(), is_hit)):
            last_use[u] = (s, 0 if h else 1, r)
        if len(last_use) > capacity:
            keep = sorted(last_use.items(), key=lambda kv: kv[1])[-capacity:]
            last_use = dict(keep)
    return np.array(hits, dtype=np.int64)


def previous_set_hits(trajectory: np.ndarray) -> np.ndarray:
    """Hits per step when only the previous step's set is kept on the device."""
    prev, hits = set(), []
    for row in np.asarray(trajectory):
        U = set(np.unique(row[row >= 0]).tolist())
        hits.append(len(U & prev))
        prev = U
    return np.array(hits, dtype=np.int64)


def fifo_hits(trajectory: np.ndarray, n_sets: int, ways: int, id_range: int) -> np.ndarray:
    """Hits per step of the set-associative FIFO pool (plan_step) over one request."""
    state = empty_state(n_sets, ways, id_range)
    hits = []
    for row in np.asarray(trajectory):
        out, state = plan_step(row[None, :], *state, n_sets, ways)
        hits.append(out["n_hit"])
    return np.array(hits, dtype=np.int64)
