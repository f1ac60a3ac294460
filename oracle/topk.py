"""Stage 3 oracle: the causal Top-k selector.

Test infrastructure only (see the package docstring).

Definition ("DeepSeek Technical Reports", DSA, the Top-k attention equation;
"DeepSeek V4 结构速览", 核心设计 and Lightning Indexer): each query keeps
the k compressed entries with the highest index scores within its causal
range (k = 512, or 1024 for Pro).

Readings taken:

* The ranking uses the scores as stored (fp32, or BF16 where the scores are
  stored in BF16).  Equal scores are ordered by the lower entry index first,
  and -0.0 equals +0.0.
* Only entries s < V(t) = floor((t + 1) / ratio) are candidates.  When fewer
  than k are visible, all of them are taken and the remaining slots are -1.
* The result is a set: valid indices first, then the -1 padding.  This
  oracle lists the valid indices in rank order.
"""
from __future__ import annotations

import numpy as np

from .indexer import visible


def select_row(scores_row: np.ndarray, n_visible: int, k: int) -> np.ndarray:
    """Top-k of one row over candidates 0..n_visible-1, ties to the lower index."""
    key = np.asarray(scores_row[:n_visible], dtype=np.float64) + 0.0  # -0.0 -> +0.0
    cand = np.arange(n_visible)
    order = np.lexsort((cand, -key))  # last key is primary: score descending, then index
    take = order[:min(k, n_visible)]
    out = np.full(k, -1, dtype=np.int64)
    out[:len(take)] = cand[take]
    return out


def topk_select(scores, k: int, q_pos0: int, ratio: int = 4, rows=None):
    """scores: [B, T, N] stored values.  Returns idx [B, T, k] int64 (-1 padded)."""
    scores = np.asarray(scores)
    B, T, N = scores.shape
    rows = list(range(T)) if rows is None else list(rows)
    out = np.full((B, len(rows), k), -1, dtype=np.int64)
    for b in range(B):
        for r, t in enumerate(rows):
            v = min(visible(q_pos0 + t, ratio), N)
            out[b, r] = select_row(scores[b, t], v, k)
    return out


def pool_select(scores, pool, k: int, N: int | None = None):
    """Top-k inside a candidate pool ("DeepSeek Technical Reports",
    DeepSeek-V4.1, CSA2: Hierarchical Sparse Indexer).

    scores: [B, T, P] stored scores of the pool slots; pool: [B, T, P] entry
    ids (-1, or an id >= N when N is given, = empty).  The candidates of
    row (b, t) are its non-empty slots;
    they are ranked by score, equal scores by the lower entry id (the rule
    of the full Top-k), and the k best entry ids are returned in rank order,
    then -1 padding.  [B, T, k] int64."""
    scores = np.asarray(scores)
    pool = np.asarray(pool)
    B, T, P = pool.shape
    out = np.full((B, T, k), -1, dtype=np.int64)
    for b in range(B):
        for t in range(T):
            ok = (pool[b, t] >= 0) & ((pool[b, t] < N) if N is not None else True)
            ids = pool[b, t][ok].astype(np.int64)
            key = np.asarray(scores[b, t][ok], dtype=np.float64) + 0.0
            order = np.lexsort((ids, -key))
            take = ids[order[:min(k, len(ids))]]
            out[b, t, :len(take)] = take
    return out
