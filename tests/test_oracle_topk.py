"""Pins for the oracle's top-k: an independent heap selection, brute force over subsets,
signed-zero and padding cases."""
import heapq
import itertools

import numpy as np
import pytest

from oracle import topk


@pytest.mark.parametrize("seed", range(6))
def test_matches_heapq(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 3000))
    k = int(rng.integers(1, 400))
    s = rng.integers(-20, 20, n).astype(np.float32) * np.float32(0.5)  # many ties
    want = heapq.nlargest(k, ((float(v), -i) for i, v in enumerate(s)))
    want = sorted(-i for _, i in want)
    got = topk.select(s, k)
    assert list(got[:len(want)]) == want
    assert (got[len(want):] == -1).all()


def test_brute_force_tiny():
    rng = np.random.default_rng(11)
    for _ in range(60):
        n = int(rng.integers(1, 8))
        k = int(rng.integers(1, 5))
        s = rng.integers(0, 3, n).astype(np.float32)
        best = None
        for sub in itertools.combinations(range(n), min(k, n)):
            key = (sorted((float(s[i]) for i in sub), reverse=True), [-i for i in sorted(sub)])
            if best is None or key > best[0]:
                best = (key, sub)
        got = topk.select(s, k)
        assert list(got[:min(k, n)]) == sorted(best[1])


def test_signed_zero_ties_and_padding():
    s = np.array([-0.0, 0.0, -0.0, -1.0], dtype=np.float32)
    assert list(topk.select(s, 2)) == [0, 1]
    assert list(topk.select(s, 6)) == [0, 1, 2, 3, -1, -1]
    s = np.array([np.float32(-np.inf), 1.0, np.float32(-np.inf)], dtype=np.float32)
    assert list(topk.select(s, 2)) == [0, 1]
