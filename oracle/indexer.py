"""Stage 2 oracle: the lightning indexer.

Test infrastructure only (see the package docstring).

Definition ("DeepSeek Technical Reports", DSA, the lightning-indexer
equation): the score of query token t against key s is the sum over the H_I
indexer heads j of w[t, j] * ReLU(q[t, j] . k[s]).  There is no scale factor
in the equation, so none is applied.  "DeepSeek V4 结构速览" (Lightning
Indexer) adds that the keys come from the same 4-to-1 compressor as the main
KV (one key per C4A entry), that the QK product runs in FP4, that negative
dot products are zeroed by the ReLU before the head-weighted sum, that scores
are stored as BF16, and that only the causal range is scored.

Causal range (a reading; the page's symbol is lost): compressed entry s is
visible to query position t iff its whole block has arrived, s < V(t) =
floor((t + 1) / ratio).  Masked scores are -inf.
"""
from __future__ import annotations

import numpy as np


def visible(t: int, ratio: int) -> int:
    """Number of compressed entries visible to absolute query position t."""
    return (t + 1) // ratio


def index_scores(q, w, k, q_pos0: int, ratio: int = 4, rows=None):
    """q: [B, T, H_I, d_I], w: [B, T, H_I], k: [B, N, d_I] (dequantized values).

    Returns float64 scores [B, T, N] (or [B, len(rows), N] when ``rows`` lists
    the query rows to compute), -inf at masked entries."""
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, T = q.shape[:2]
    N = k.shape[1]
    rows = list(range(T)) if rows is None else list(rows)
    out = np.full((B, len(rows), N), -np.inf)
    for b in range(B):
        for r, t in enumerate(rows):
            v = min(visible(q_pos0 + t, ratio), N)
            if v == 0:
                continue
            dots = q[b, t] @ k[b, :v].T            # [H_I, v]
            out[b, r, :v] = w[b, t] @ np.maximum(dots, 0.0)
    return out


def pool_scores(q, w, k, pool):
    """Scores of a candidate pool ("DeepSeek Technical Reports",
    DeepSeek-V4.1, CSA2: the Hierarchical Sparse Indexer re-scores, with the layer's own query, only
    the entries of a candidate pool found by a full indexer pass).

    q: [B, T, H_I, d_I], w: [B, T, H_I], k: [B, N, d_I], pool: [B, T, P]
    entry ids (-1, or any id outside 0..N-1, marks an empty slot).  Returns
    float64 [B, T, P]: the indexer score of entry pool[b,t,j], -inf for an
    empty slot.  The same equation as ``index_scores``; visibility is the
    pool's business (a pool from a causal Top-P holds visible entries only)."""
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    pool = np.asarray(pool)
    B, T, P = pool.shape
    N = k.shape[1]
    out = np.full((B, T, P), -np.inf)
    for b in range(B):
        for t in range(T):
            ids = pool[b, t]
            ok = (ids >= 0) & (ids < N)
            if not ok.any():
                continue
            dots = q[b, t] @ k[b, ids[ok]].T          # [H_I, n_ok]
            out[b, t, ok] = w[b, t] @ np.maximum(dots, 0.0)
    return out
