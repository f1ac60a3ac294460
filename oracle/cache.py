"""The heterogeneous KV cache layout: a paged classical cache and a
per-request state cache.

Test infrastructure only (see the package docstring).

What the pages define ("DeepSeek-V4技术报告解读，全适配国产算力", 3.2, the
heterogeneous KV cache): the classical cache holds the compressed CSA/HCA
entries in blocks, each block covering 128 raw tokens, several blocks per
request; the state cache is a fixed-size pool, one slot per request, holding
the sliding-window KV (the pages size it at the most recent 4096 tokens) and
the not-yet-compressed tail.

Readings taken:

* A block of 128 raw tokens holds 32 C4A entries (ratio 4) and one C128A
  entry (the page's "one CSA entry" is taken as one block's worth of C4A
  entries).  Entry e of a sequence lives in that sequence's logical block
  e // per_block, slot e % per_block; a block table maps logical blocks to
  physical blocks of a pool.
* The window part of the state cache is a ring: raw position p sits at row
  p % W of the request's slot (W the ring size, at least the window).

These functions only gather: they turn the paged layout back into the
contiguous per-sequence arrays the attention oracles take.
"""
from __future__ import annotations

import numpy as np


def paged_entries(pool, table_row, n: int, per_block: int) -> np.ndarray:
    """Entries 0..n-1 of one sequence from a paged pool.

    pool: [n_pool, per_block, d] (or [n_pool, d] when per_block == 1);
    table_row: that sequence's block table.  Returns [n, d]."""
    pool = np.asarray(pool)
    if per_block == 1 and pool.ndim == 2:
        pool = pool[:, None, :]
    e = np.arange(n)
    blocks = np.asarray(table_row)[e // per_block]
    return pool[blocks, e % per_block]


def ring_rows(ring, positions) -> np.ndarray:
    """Rows of one request's window ring [W, d] at raw positions (p % W)."""
    ring = np.asarray(ring)
    return ring[np.asarray(positions) % ring.shape[0]]
