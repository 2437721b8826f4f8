"""Page addressing for the oracle (test infrastructure only).

* Paged cache row of a token: the request's page table maps logical page t//p to
  a physical page; the token sits at offset t mod p inside it (page-table metadata
  kept apart from the physical KV, as the TokenSpeed audit page describes for
  req_to_token_pool vs the KV allocator).
* Page-sharded ownership, [HCCP] §1.1 "Logical radix tree and page ownership": for
  N shard ranks, page size p and logical slot x, the logical page is q = floor(x/p),
  its owner rank is r = q mod N, and the owner stores the token at local row
  l = floor(q/N)*p + (x mod p).  No lookup table is involved.
"""
import numpy as np


def owner_local(x, page_size: int, n_ranks: int):
    """Closed-form owner rank and local row of logical slots x ([HCCP] §1.1)."""
    x = np.asarray(x, dtype=np.int64)
    assert page_size > 0 and n_ranks > 0 and (x >= 0).all()
    q = x // page_size
    r = q % n_ranks
    local = (q // n_ranks) * page_size + (x % page_size)
    return r, local


def paged_rows(page_table_row: np.ndarray, positions, page_size: int) -> np.ndarray:
    """Physical row (page * page_size + offset) of each token position of one request."""
    t = np.asarray(positions, dtype=np.int64)
    pages = np.asarray(page_table_row, dtype=np.int64)[t // page_size]
    assert (pages >= 0).all(), "position past the request's last page"
    return pages * page_size + t % page_size
