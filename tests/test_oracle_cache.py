"""Pins of the heterogeneous-cache layout oracle (paged entries, window ring).

Page: "DeepSeek-V4技术报告解读，全适配国产算力" (3.2: classical paged cache,
blocks of 128 raw tokens; per-request state cache with the sliding window).
"""
import numpy as np

from oracle import cache as occ


def test_identity_table_is_the_contiguous_cache():
    g = np.random.default_rng(0)
    cont = g.normal(size=(96, 8))                      # 3 blocks of 32 entries
    pool = cont.reshape(3, 32, 8)
    assert np.array_equal(occ.paged_entries(pool, [0, 1, 2], 96, 32), cont)
    assert np.array_equal(occ.paged_entries(pool, [0, 1, 2], 70, 32), cont[:70])


def test_permuted_pool_and_table_give_the_same_entries():
    g = np.random.default_rng(1)
    cont = g.normal(size=(5 * 32, 4))
    perm = g.permutation(9)[:5]                       # physical blocks 0..8, five in use
    pool = np.zeros((9, 32, 4))
    pool[perm] = cont.reshape(5, 32, 4)
    assert np.array_equal(occ.paged_entries(pool, perm, 160, 32), cont)
    # one entry per block (C128A)
    pool1 = np.zeros((9, 4))
    pool1[perm] = cont[:5]
    assert np.array_equal(occ.paged_entries(pool1, perm, 5, 1), cont[:5])


def test_ring_wraps():
    ring = np.arange(8 * 3).reshape(8, 3)
    # positions 6..13 of a ring of 8: rows 6, 7, 0, 1, ..., 5
    got = occ.ring_rows(ring, range(6, 14))
    assert np.array_equal(got[:, 0], [18, 21, 0, 3, 6, 9, 12, 15])
