"""Pins for the page-ownership closed form: brute-force page enumeration and the worked example."""
import os

import numpy as np
import pytest

from oracle import paging

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("p", [1, 2, 4, 64])
@pytest.mark.parametrize("N", [1, 2, 3, 4])
def test_owner_local_brute_force(p, N):
    # Hand pages out round-robin (page q to rank q mod N); each rank numbers its own
    # pages 0, 1, 2, ... in the order it receives them.
    Q = 23
    owner, local_page, count = {}, {}, [0] * N
    for q in range(Q):
        r = q % N
        owner[q] = r
        local_page[q] = count[r]
        count[r] += 1
    x = np.arange(Q * p)
    r, l = paging.owner_local(x, p, N)
    for xi in x:
        q = xi // p
        assert r[xi] == owner[q]
        assert l[xi] == local_page[q] * p + xi % p


def test_owner_local_worked_example():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "hicache_page_ownership.txt"))
            if l.strip() and not l.startswith("#")]
    for name, q, n, want_r, want_page in rows:
        q, n, want_r, want_page = int(q), int(n), int(want_r), int(want_page)
        for p in (1, 64):
            for off in (0, p - 1):
                r, l = paging.owner_local(np.array([q * p + off]), p, n)
                assert r[0] == want_r, name
                assert l[0] == want_page * p + off, name


def test_paged_rows_identity_and_permutation():
    rng = np.random.default_rng(0)
    ps, npages = 8, 13
    perm = rng.permutation(npages)
    pos = np.arange(npages * ps - 3)
    rows = paging.paged_rows(perm, pos, ps)
    assert np.array_equal(rows // ps, perm[pos // ps])
    assert np.array_equal(rows % ps, pos % ps)
    assert len(np.unique(rows)) == len(pos)
    with pytest.raises(AssertionError):
        paging.paged_rows(np.array([0, -1]), np.array([ps]), ps)
