"""Pins for the oracle's union of the query tokens' selections: set arithmetic on small random
selections, written out with Python sets and sorted lists."""
import numpy as np
import pytest

from oracle import gather


def _selections(rng, Sq, k, L, overlap):
    base = rng.choice(L, size=k, replace=False)
    rows = []
    for t in range(Sq):
        n_valid = k - int(rng.integers(0, 3)) if t % 2 else k          # some rows padded
        keep = rng.choice(base, size=min(int(overlap * k), n_valid), replace=False)
        rest = np.setdiff1d(np.arange(L), keep)
        row = np.sort(np.concatenate([keep, rng.choice(rest, size=n_valid - len(keep), replace=False)]))
        rows.append(np.concatenate([row, np.full(k - n_valid, -1)]))
    return np.stack(rows).astype(np.int32)


@pytest.mark.parametrize("Sq,k,overlap", [(1, 8, 0.0), (2, 16, 0.5), (4, 32, 0.75), (8, 24, 0.0), (4, 40, 1.0)])
def test_union_is_the_sorted_set_of_valid_positions(Sq, k, overlap):
    rng = np.random.default_rng(Sq * 100 + k)
    tk = _selections(rng, Sq, k, 200, overlap)
    U, uidx, member = gather.union_select(tk)
    want = sorted({int(p) for row in tk for p in row if p >= 0})
    assert U.tolist() == want
    for t in range(Sq):
        for j in range(k):
            p = int(tk[t, j])
            assert (uidx[t, j] == -1) if p < 0 else (want[uidx[t, j]] == p)
        assert [want[u] for u in range(len(want)) if member[t, u]] == sorted(int(p) for p in tk[t] if p >= 0)
    # every position of the union belongs to some query; a shared position appears once
    assert member.any(axis=0).all()
    assert len(U) <= sum(int((row >= 0).sum()) for row in tk)


def test_identical_selections_collapse_and_disjoint_ones_add_up():
    rng = np.random.default_rng(3)
    row = np.sort(rng.choice(500, size=32, replace=False)).astype(np.int32)
    U, uidx, member = gather.union_select(np.stack([row] * 4))
    assert np.array_equal(U, row) and member.all() and (uidx == np.arange(32)[None]).all()
    parts = np.sort(rng.choice(500, size=(3 * 16), replace=False)).reshape(3, 16).astype(np.int32)
    U, _, member = gather.union_select(parts)
    assert len(U) == 48 and (member.sum(axis=0) == 1).all()
