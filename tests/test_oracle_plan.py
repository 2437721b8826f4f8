"""Pins for the oracle's set-associative FIFO plan.

The reference point is a textbook FIFO cache kept as one deque per set: classify the
step's ids against the contents before the step, then install the misses one at a time
in ascending id order, evicting the oldest entry of a full set.
"""
import collections

import numpy as np
import pytest

import synth
from oracle import plan


def fifo_sim(steps, n_sets, W):
    sets = [collections.deque() for _ in range(n_sets)]
    hits_per_step = []
    for U in steps:
        U = sorted(set(int(u) for u in U))
        before = [set(d) for d in sets]
        hits = {u for u in U if u in before[u % n_sets]}
        for u in U:
            if u in hits:
                continue
            d = sets[u % n_sets]
            if len(d) == W:
                d.popleft()
            d.append(u)
        hits_per_step.append(hits)
    return hits_per_step, sets


def run_plan(steps, n_sets, W, id_range):
    state = plan.empty_state(n_sets, W, id_range)
    outs = []
    for U in steps:
        tk = np.array(sorted(set(int(u) for u in U)), dtype=np.int32)[None, :]
        out, state = plan.plan_step(tk, *state, n_sets, W)
        outs.append((tk[0], out))
    return outs, state


def fifo_order(state, n_sets, W):
    pool_ids, _, ptr = state
    res = []
    for s in range(n_sets):
        ways = [(int(ptr[s]) + i) % W for i in range(W)]
        res.append([int(pool_ids[s * W + w]) for w in ways if pool_ids[s * W + w] >= 0])
    return res


@pytest.mark.parametrize("n_sets,W", [(1, 4), (4, 2), (8, 4), (16, 3)])
def test_matches_deque_fifo(n_sets, W):
    rng = np.random.default_rng(n_sets * 10 + W)
    id_range = 200
    steps = [rng.choice(id_range, size=int(rng.integers(1, 40)), replace=False) for _ in range(12)]
    hits, sets = fifo_sim(steps, n_sets, W)
    outs, state = run_plan(steps, n_sets, W, id_range)
    for (tk, out), h in zip(outs, hits):
        assert {int(u) for u, f in zip(tk, out["is_hit"][0]) if f} == h
        assert out["n_hit"] + out["miss_count"] == out["n_unique"] == len(tk)
    assert fifo_order(state, n_sets, W) == [list(d) for d in sets]


def test_invariants_and_hits_do_not_move_pointer():
    rng = np.random.default_rng(1)
    n_sets, W, id_range = 8, 4, 300
    state = plan.empty_state(n_sets, W, id_range)
    for _ in range(10):
        tk = np.sort(rng.choice(id_range, size=25, replace=False)).astype(np.int32)[None]
        out, new = plan.plan_step(tk, *state, n_sets, W)
        pool_ids, its, ptr = new
        live = np.nonzero(pool_ids >= 0)[0]
        assert np.array_equal(its[pool_ids[live]], live)
        assert (its >= 0).sum() == len(live)
        assert out["n_hit"] + out["miss_count"] == 25
        # replaying only the hits of this step against the new state leaves ptr unchanged
        hits = tk[0][out["is_hit"][0] == 1]
        if len(hits):
            still = hits[new[1][hits] >= 0][None]
            o2, n2 = plan.plan_step(still, *new, n_sets, W)
            assert o2["miss_count"] == 0 and np.array_equal(n2[2], ptr)
        state = new


def test_empty_pool_all_miss_and_repeat_all_hit():
    n_sets, W, id_range = 16, 4, 1000
    rng = np.random.default_rng(2)
    # at most W ids per set so nothing is evicted
    ids = np.sort(np.concatenate([s + n_sets * rng.choice(60, size=3, replace=False) for s in range(n_sets)]))
    tk = ids.astype(np.int32)[None]
    state = plan.empty_state(n_sets, W, id_range)
    out, state = plan.plan_step(tk, *state, n_sets, W)
    assert out["n_hit"] == 0 and out["miss_count"] == len(ids)
    assert (out["slot"] >= 0).all()
    for _ in range(3):
        out, state = plan.plan_step(tk, *state, n_sets, W)
        assert out["n_hit"] == len(ids) and out["miss_count"] == 0


def test_single_set_is_plain_fifo_queue():
    W = 5
    q = collections.deque()
    state = plan.empty_state(1, W, 50)
    rng = np.random.default_rng(4)
    for _ in range(20):
        U = sorted(set(int(x) for x in rng.integers(0, 50, 3)))
        out, state = plan.plan_step(np.array(U, np.int32)[None], *state, 1, W)
        snap = set(q)
        for u in U:
            if u not in snap:
                if len(q) == W:
                    q.popleft()
                q.append(u)
        assert fifo_order(state, 1, W) == [list(q)]


def test_overflowing_set_keeps_last_W_and_advances_pointer():
    W, n_sets = 4, 2
    state = plan.empty_state(n_sets, W, 100)
    ids = np.arange(0, 2 * 7, 2, dtype=np.int32)[None]          # 7 misses, all in set 0
    out, (pool_ids, its, ptr) = plan.plan_step(ids, *state, n_sets, W)
    assert list(out["miss_slot"]) == [-1, -1, -1, 3, 0, 1, 2]     # i-th miss -> way (0+i) mod 4
    assert ptr[0] == 7 % W and ptr[1] == 0
    assert sorted(pool_ids[:4]) == [6, 8, 10, 12]


def test_pool_of_previous_set_reproduces_trajectory_reuse():
    cfg = synth.spec(4).scaled(B=2)
    traj = synth.gen.topk_trajectory(cfg)
    k, id_range = cfg.topk, cfg.id_range
    for b in range(cfg.B):
        for s in range(1, cfg.steps):
            # a pool holding exactly the previous step's set: one set, k ways
            state = plan.empty_state(1, k, id_range)
            _, state = plan.plan_step(traj[s - 1, b][None], *state, 1, k)
            out, _ = plan.plan_step(traj[s, b][None], *state, 1, k)
            assert out["n_hit"] == round(cfg.keep_frac * k) == 1229


def test_multi_query_union_and_padding():
    n_sets, W = 4, 2
    state = plan.empty_state(n_sets, W, 64)
    tk = np.array([[1, 5, 9, -1], [5, 9, 13, 17]], dtype=np.int32)
    out, _ = plan.plan_step(tk, *state, n_sets, W)
    assert out["n_unique"] == 5 and list(out["miss_pos"]) == [1, 5, 9, 13, 17]
    assert out["slot"][0, 3] == -1 and out["is_hit"][0, 3] == 0
    assert out["slot"][0, 1] == out["slot"][1, 0]                # same id -> same decision


# ---------------------------------------------------------------- replacement-policy comparison
def _textbook_lru(traj, capacity):
    """A recency list: per step, look every id up first; move each hit to the back
    (ascending), then append each miss (ascending), dropping the front when over capacity."""
    from collections import OrderedDict
    cache, hits = OrderedDict(), []
    for row in traj:
        U = np.unique(row[row >= 0]).tolist()
        hit = [u for u in U if u in cache]
        for u in hit:
            cache.move_to_end(u)
        for u in U:
            if u not in cache:
                cache[u] = True
                if len(cache) > capacity:
                    cache.popitem(last=False)
        hits.append(len(hit))
    return np.array(hits)


def _random_traj(rng, steps, k, id_range):
    return np.stack([np.sort(rng.choice(id_range, size=k, replace=False)) for _ in range(steps)]).astype(np.int32)


def test_lru_matches_textbook_lru():
    rng = np.random.default_rng(4)
    for cap in (16, 20, 37, 64):
        t = _random_traj(rng, 40, 16, 64)
        assert np.array_equal(plan.lru_hits(t, cap), _textbook_lru(t, cap)), cap


def test_lru_special_cases():
    rng = np.random.default_rng(6)
    t = _random_traj(rng, 25, 12, 50)
    # a pool of exactly k ids holds the previous step's set
    assert np.array_equal(plan.lru_hits(t, 12), plan.previous_set_hits(t))
    # a pool larger than every id hits whatever was seen before
    seen, want = set(), []
    for row in t:
        want.append(len(set(row.tolist()) & seen))
        seen |= set(row.tolist())
    assert np.array_equal(plan.lru_hits(t, 1000), want)
    # one set of enough ways never evicts either
    assert np.array_equal(plan.fifo_hits(t, 1, 64, 64), want)


# ---------------------------------------------------------------- one plan per group of 4 layers
def way_fifo_sim(n_sets, W):
    """A textbook set-associative FIFO cache with explicit ways, for one layer: each set is an
    array of W ways and a pointer to the next way to fill.  A step's ids are looked up against
    the contents before the step; then its misses are installed one at a time, ascending, at
    the pointer's way (evicting whatever sat there), and the pointer moves on.  Returns a
    stepping function giving, per id of the step, its slot for serving: the hit's slot, the
    slot a miss still occupies after the step, or -1 for a miss evicted within the step."""
    ways = [[-1] * W for _ in range(n_sets)]
    ptr = [0] * n_sets

    def step(U):
        U = sorted(set(int(u) for u in U))
        before = {ways[s][w]: s * W + w for s in range(n_sets) for w in range(W) if ways[s][w] >= 0}
        put = {}
        for u in U:
            if u in before:
                continue
            s = u % n_sets
            ways[s][ptr[s]] = u
            put[u] = s * W + ptr[s]
            ptr[s] = (ptr[s] + 1) % W
        after = {ways[s][w]: s * W + w for s in range(n_sets) for w in range(W) if ways[s][w] >= 0}
        res = {}
        for u in U:
            if u in before:
                res[u] = (1, before[u])
            else:
                res[u] = (0, put[u] if after.get(u) == put[u] else -1)
        return res

    return step, ways, ptr


@pytest.mark.parametrize("n_sets,W", [(8, 2), (16, 4), (4, 8)])
def test_group_of_four_layers_shares_one_plan(n_sets, W):
    """[GLM52] §4.1-§4.2: the 4 layers of a group share one top-k, and an id sits in the same
    slot of every layer's pool, so one plan serves the whole group.  Four layers, each with its
    own rows and its own pool kept by its own textbook FIFO (way_fifo_sim), walk a trajectory;
    per step, planning each layer separately from the same pre-step state gives identical
    plans, that plan equals every layer's own simulator slot for slot, serving each layer
    through it returns that layer's rows, and committing it once at the group's end leaves
    the state every layer's simulator holds."""
    rng = np.random.default_rng(n_sets * 100 + W)
    id_range, k, layers = 400, 3 * n_sets, 4
    host = [rng.integers(0, 2 ** 16, size=(id_range, 6), dtype=np.uint16) for _ in range(layers)]
    pools = [np.zeros((n_sets * W, 6), dtype=np.uint16) for _ in range(layers)]
    sims = [way_fifo_sim(n_sets, W) for _ in range(layers)]
    state = plan.empty_state(n_sets, W, id_range)
    prev = None
    for s in range(14):
        if prev is None:
            U = rng.choice(id_range, size=k, replace=False)
        else:                               # about half of the previous set recurs
            keep = rng.choice(prev, size=k // 2, replace=False)
            fresh = rng.choice(np.setdiff1d(np.arange(id_range), prev), size=k - k // 2, replace=False)
            U = np.concatenate([keep, fresh])
        prev = np.sort(U)
        tk = np.concatenate([prev, [-1, -1]]).astype(np.int32)[None]   # two padding entries
        per_layer = [plan.plan_step(tk, *state, n_sets, W) for _ in range(layers)]
        out, new_state = per_layer[0]
        for o2, st2 in per_layer[1:]:
            for key in ("is_hit", "slot", "miss_pos", "miss_slot"):
                assert np.array_equal(o2[key], out[key]), key
            assert all(np.array_equal(a, b) for a, b in zip(st2, new_state))
        for l in range(layers):
            want = sims[l][0](prev)
            for j, u in enumerate(prev):
                assert (int(out["is_hit"][0, j]), int(out["slot"][0, j])) == want[int(u)], (s, l, int(u))
            assert (out["slot"][0, -2:] == -1).all() and (out["is_hit"][0, -2:] == 0).all()
            # serve this layer: hits from its pool, misses from its rows; then install
            served = np.where(out["is_hit"][0, :k, None] == 1, pools[l][np.maximum(out["slot"][0, :k], 0)],
                              host[l][prev])
            assert np.array_equal(served, host[l][prev]), (s, l)
            for u, sl in zip(out["miss_pos"], out["miss_slot"]):
                if sl >= 0:
                    pools[l][sl] = host[l][u]
        state = new_state
        pool_ids, its, ptr = state
        for l in range(layers):
            _, ways, sptr = sims[l]
            assert [pool_ids[sset * W + w] for sset in range(n_sets) for w in range(W)] == \
                [ways[sset][w] for sset in range(n_sets) for w in range(W)]
            assert list(ptr) == sptr
            live = np.nonzero(pool_ids >= 0)[0]
            assert np.array_equal(pools[l][live], host[l][pool_ids[live]])
