"""Pins of the hierarchical-indexer oracles (pool scoring and Top-k inside a
candidate pool).

Page: "DeepSeek Technical Reports" (DeepSeek-V4.1, CSA2: Cross-Layer KV and Index
Reuse; the
hierarchical sparse indexer -- a full indexer pass over the whole context
yields a large candidate pool, and later Reindex layers re-score only inside
that pool with their own query).  The pins tie both functions to the full
indexer and Top-k oracles, which are pinned on their own: a pool holding
every visible entry reproduces the full path, and any pool that contains a
layer's true Top-k set gives back exactly that set.
"""
import numpy as np
import pytest

import synth
from oracle import indexer as oi
from oracle import topk as ot


def _layer(name, B=2, T=5, N=40, q_pos0=150, seed=0):
    q = synth.normal(name + ".q", (B, T, 8, 16), seed=seed).astype(np.float64)
    w = synth.uniform(name + ".w", (B, T, 8), seed=seed).astype(np.float64)
    k = synth.normal(name + ".k", (B, N, 16), seed=seed).astype(np.float64)
    return q, w, k, q_pos0


def _full_pool(B, T, q_pos0, N, P):
    pool = np.full((B, T, P), -1)
    for t in range(T):
        v = min(oi.visible(q_pos0 + t, 4), N)
        pool[:, t, :v] = np.arange(v)
    return pool


def test_pool_of_all_visible_entries_is_the_full_path():
    q, w, k, q0 = _layer("pool.all")
    B, T, N = 2, 5, 40
    pool = _full_pool(B, T, q0, N, P=48)
    full = oi.index_scores(q, w, k, q0, 4)
    ps = oi.pool_scores(q, w, k, pool)
    for t in range(T):
        v = min(oi.visible(q0 + t, 4), N)
        assert np.array_equal(ps[:, t, :v], full[:, t, :v])
        assert np.all(np.isneginf(ps[:, t, v:]))
    sel = ot.pool_select(ps, pool, 7)
    ref = ot.topk_select(full, 7, q0, 4)
    assert np.array_equal(np.sort(sel, axis=-1), np.sort(ref, axis=-1))


@pytest.mark.parametrize("extra", [0, 5, 30])
def test_pool_containing_the_true_topk_gives_it_back(extra):
    """Re-indexing inside any superset of a layer's own Top-k returns that set."""
    q, w, k, q0 = _layer("pool.sup")
    B, T, N, K = 2, 5, 40, 6
    full = oi.index_scores(q, w, k, q0, 4)
    truth = ot.topk_select(full, K, q0, 4)
    rng = np.random.default_rng(7)
    pool = np.full((B, T, K + extra + 3), -1)
    for b in range(B):
        for t in range(T):
            v = min(oi.visible(q0 + t, 4), N)
            others = np.setdiff1d(np.arange(v), truth[b, t])
            add = rng.choice(others, size=min(extra, len(others)), replace=False)
            ids = np.sort(np.concatenate([truth[b, t], add]))
            pool[b, t, :len(ids)] = ids
    sel = ot.pool_select(oi.pool_scores(q, w, k, pool), pool, K)
    assert np.array_equal(np.sort(sel, axis=-1), np.sort(truth, axis=-1))


def test_pool_order_and_empty_slots_do_not_matter():
    """The result is a set over the pool's entries: permuting the slots or
    scattering empty slots among them changes nothing, including the tie rule
    (equal scores go to the lower entry id, not the lower slot)."""
    q, w, k, q0 = _layer("pool.perm")
    B, T, N = 2, 5, 40
    pool = _full_pool(B, T, q0, N, P=48)
    # plant ties: entries 3 and 9 share a key row, so their scores are equal
    k = k.copy()
    k[:, 9] = k[:, 3]
    a = ot.pool_select(oi.pool_scores(q, w, k, pool), pool, 9)
    rng = np.random.default_rng(3)
    perm = pool.copy()
    for b in range(B):
        for t in range(T):
            perm[b, t] = perm[b, t, rng.permutation(48)]
    b_ = ot.pool_select(oi.pool_scores(q, w, k, perm), perm, 9)
    assert np.array_equal(np.sort(a, axis=-1), np.sort(b_, axis=-1))
    # equal scores resolve to the lower entry id
    for bb in range(B):
        for t in range(T):
            s = oi.pool_scores(q, w, k, pool)[bb, t]
            assert s[3] == s[9]


def test_empty_and_out_of_range_slots():
    q, w, k, q0 = _layer("pool.empty")
    pool = np.full((2, 5, 6), -1)
    pool[0, 0, :2] = [4, 40]              # 40 is past N = 40: an empty slot
    ps = oi.pool_scores(q, w, k, pool)
    assert np.isfinite(ps[0, 0, 0]) and np.all(np.isneginf(ps[0, 0, 1:]))
    assert np.all(np.isneginf(ps[1]))
    sel = ot.pool_select(ps, pool, 3, N=40)
    assert list(sel[0, 0]) == [4, -1, -1]
    assert np.all(sel[1] == -1)


def test_pool_scores_are_nonnegative_weighted_relu():
    """Scores of non-empty slots are >= 0 (w >= 0, ReLU) and scale linearly in w."""
    q, w, k, q0 = _layer("pool.lin")
    pool = _full_pool(2, 5, q0, 40, P=40)
    s1 = oi.pool_scores(q, w, k, pool)
    s2 = oi.pool_scores(q, 2.5 * w, k, pool)
    fin = np.isfinite(s1)
    assert np.all(s1[fin] >= 0)
    assert np.allclose(s2[fin], 2.5 * s1[fin], rtol=1e-13)


def test_tie_goes_to_the_lower_entry_id_not_the_earlier_slot():
    q, w, k, q0 = _layer("pool.tie")
    k = k.copy()
    k[:, 9] = k[:, 3]
    pool = np.full((2, 5, 4), -1)
    pool[:, :, 0], pool[:, :, 1] = 9, 3          # the higher id sits in the earlier slot
    ps = oi.pool_scores(q, w, k, pool)
    assert np.array_equal(ps[..., 0], ps[..., 1])
    sel = ot.pool_select(ps, pool, 1)
    assert np.all(sel[..., 0] == 3)
