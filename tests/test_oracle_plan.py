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
