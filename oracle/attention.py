"""Stage 4 and 5 oracles: sparse shared-KV MQA, dense attention, HCA with sink.

Test infrastructure only (see the package docstring).

What the pages define:

* CSA ("DeepSeek V4 结构速览", CSA（c4a 路线）; "DeepSeek-V4 技术解读：百万
  Token 上下文的新里程碑", 2.1): 64 query heads of dim 512 attend over one
  shared 512-d latent that is both key and value (K = V, multi-query
  attention).  The set attended is the Top-k selected compressed entries
  concatenated with the sliding-window entries, the last n_w = 128
  uncompressed latents ("DeepSeek Technical Reports", Hybrid Attention).
* HCA ("DeepSeek V4 结构速览", HCA（c128a 路线）): no indexer; dense MQA
  over the window and all compressed C128A entries, with an attention sink.

Readings taken:

* Window of query t: raw positions max(0, t - window + 1) .. t, the query's
  own token included.
* Selected entries and window rows are concatenated with no de-duplication.
* Logits are scale * q . x with scale = 1/sqrt(512) by default; the output is
  sum_x softmax(logits)_x * x.  CSA has no sink.
* The HCA sink is one extra logit z_h per head, not scaled, whose value
  vector is zero: it only adds e^{z_h} to the softmax denominator.
* lse is the natural log of the full softmax denominator (sink included).
* Compressed entry s is visible to t iff s < floor((t + 1) / ratio).
* Top-k slots holding -1 are padding and contribute nothing.
* With rope_dims > 0 the output of query position pos gets inverse RoPE at
  pos on its last rope_dims dimensions (``oracle.rope``); q and the rows are
  taken as given (already rotated by their producers).
"""
from __future__ import annotations

import numpy as np

from . import rope as _rope


def window_rows(t: int, window: int):
    """Absolute raw positions in the sliding window of query position t."""
    return range(max(0, t - window + 1), t + 1)


def _attend(qh: np.ndarray, X: np.ndarray, scale: float):
    """Two-pass softmax attention of queries [H, d] over rows X [n, d] (K = V)."""
    logits = scale * (qh @ X.T)                    # [H, n]
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    s = e.sum(axis=1, keepdims=True)
    o = (e @ X) / s
    lse = (m + np.log(s))[:, 0]
    return o, lse


def sparse_mqa(q, kv_cmp, idx, kv_raw, raw_pos0: int, q_pos0: int, window: int = 128,
               scale: float | None = None, rows=None, rope_dims: int = 0,
               rope_base: float = _rope.DEFAULT_BASE):
    """Attention over Top-k entries concatenated with the window.

    q: [B, T, H, d]; kv_cmp: [B, N, d]; idx: [B, T, k] (-1 = padding);
    kv_raw: [B, n_raw, d] holding raw positions raw_pos0 .. raw_pos0+n_raw-1.
    Returns (o [B, T', H, d], lse [B, T', H]) for the listed rows (all by default)."""
    q = np.asarray(q, dtype=np.float64)
    kv_cmp = np.asarray(kv_cmp, dtype=np.float64)
    kv_raw = np.asarray(kv_raw, dtype=np.float64)
    idx = np.asarray(idx)
    B, T, H, d = q.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    rows = list(range(T)) if rows is None else list(rows)
    o = np.zeros((B, len(rows), H, d))
    lse = np.zeros((B, len(rows), H))
    for b in range(B):
        for r, t in enumerate(rows):
            pos = q_pos0 + t
            sel = [int(s) for s in idx[b, t] if s >= 0]
            win = [u - raw_pos0 for u in window_rows(pos, window)]
            X = np.concatenate([kv_cmp[b, sel], kv_raw[b, win]], axis=0)
            o[b, r], lse[b, r] = _attend(q[b, t], X, scale)
            if rope_dims:
                o[b, r] = _rope.rotate(o[b, r], pos, rope_dims, rope_base, inverse=True)
    return o, lse


def dense_attention(q, kv_cmp, kv_raw, raw_pos0: int, q_pos0: int, ratio: int,
                    window: int = 128, scale: float | None = None, sink=None, rows=None,
                    rope_dims: int = 0, rope_base: float = _rope.DEFAULT_BASE):
    """Masked dense attention over all compressed entries plus the window.

    Written separately from ``sparse_mqa``: one logit matrix over every cache
    row, a boolean visibility mask, and (optionally) a sink column per head.
    sink: [H] logits (unscaled) or None."""
    q = np.asarray(q, dtype=np.float64)
    kv_cmp = np.asarray(kv_cmp, dtype=np.float64)
    kv_raw = np.asarray(kv_raw, dtype=np.float64)
    B, T, H, d = q.shape
    N = kv_cmp.shape[1]
    n_raw = kv_raw.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    rows = list(range(T)) if rows is None else list(rows)
    o = np.zeros((B, len(rows), H, d))
    lse = np.zeros((B, len(rows), H))
    raw_abs = raw_pos0 + np.arange(n_raw)
    for b in range(B):
        allrows = np.concatenate([kv_cmp[b], kv_raw[b]], axis=0)     # [N + n_raw, d]
        for r, t in enumerate(rows):
            pos = q_pos0 + t
            vis_c = np.arange(N) < (pos + 1) // ratio
            vis_w = (raw_abs >= max(0, pos - window + 1)) & (raw_abs <= pos)
            mask = np.concatenate([vis_c, vis_w])
            logits = scale * (q[b, t] @ allrows.T)                     # [H, N + n_raw]
            logits = np.where(mask[None, :], logits, -np.inf)
            if sink is not None:
                z = np.asarray(sink, dtype=np.float64)[:, None]
                logits = np.concatenate([logits, z], axis=1)
                vals = np.concatenate([allrows, np.zeros((1, d))], axis=0)
            else:
                vals = allrows
            m = logits.max(axis=1, keepdims=True)
            e = np.exp(logits - m)
            s = e.sum(axis=1, keepdims=True)
            o[b, r] = (e @ vals) / s
            lse[b, r] = (m + np.log(s))[:, 0]
            if rope_dims:
                o[b, r] = _rope.rotate(o[b, r], pos, rope_dims, rope_base, inverse=True)
    return o, lse


def hca_attention(q, kv_cmp, kv_raw, raw_pos0: int, q_pos0: int, sink, ratio: int = 128,
                  window: int = 128, scale: float | None = None, rows=None, rope_dims: int = 0,
                  rope_base: float = _rope.DEFAULT_BASE):
    """HCA: dense attention over all visible C128A entries and the window, with a sink."""
    return dense_attention(q, kv_cmp, kv_raw, raw_pos0, q_pos0, ratio, window, scale,
                           sink=sink, rows=rows, rope_dims=rope_dims, rope_base=rope_base)
