"""Stage 1 oracle: the C4A / C128A KV compressor.

Test infrastructure only (see the package docstring).

What the pages define ("DeepSeek V4 结构速览", 核心设计 and C4A Compressor;
"DeepSeek-V4技术报告解读，全适配国产算力", 2.1, the compression formula):

* C4A: one compressed entry is a weighted sum of 8 raw tokens at stride 4 --
  the current block of 4 and the previous block of 4, each with its own
  content projection (Ca for the current block, Cb for the previous) and
  weight projection (Za, Zb).  The two blocks' weights are stacked, a
  positional bias B is added, and a softmax is taken over the 8 rows for
  each of the c channels separately.  The contents are stacked the same way
  and summed with those weights.  The result goes through RMSNorm.
* C128A: 128 raw tokens at stride 128, no overlap, one block (Ca, Za), the
  same per-channel softmax pooling and RMSNorm.
* Block 0 has no previous block: its content is zero-filled and its weights
  are set to a value lost in the page's extraction.

Readings taken where the pages are silent or garbled:

* The "a" rows are the current block (raw tokens 4i..4i+3) and the "b" rows
  the previous block (4i-4..4i-1).
* Bias rows 0..3 go with the current block's offsets 0..3 and rows 4..7 with
  the previous block's offsets 0..3; C128A has a [128, c] bias.
* Block 0's missing weights are -inf, so its zero content gets weight 0 and
  entry 0 pools only its own 4 tokens.
* RMSNorm has eps = 1e-6 and weight gamma (ones unless given).
* With rope_dims > 0, partial RoPE (``oracle.rope``) turns the last rope_dims
  channels of each entry after RMSNorm, at the entry's anchor position
  ratio * s + rope_anchor (s the entry's absolute index).
* Trailing tokens that do not complete a block produce no entry.
"""
from __future__ import annotations

import numpy as np

from . import rope as _rope

PREV = 4  # raw tokens in the C4A "previous block"


def _softmax_pool(logits: np.ndarray, contents: np.ndarray):
    """Per-channel softmax over rows, then the weighted sum over rows.

    logits, contents: [rows, c] float64.  Returns (y [c], p [rows, c])."""
    m = logits.max(axis=0)
    e = np.exp(logits - m[None, :])
    p = e / e.sum(axis=0)[None, :]
    y = (p * contents).sum(axis=0)
    return y, p


def _rmsnorm(y: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    return y / np.sqrt(np.mean(y * y) + eps) * gamma


def compress_sequence(Ca, Za, bias, ratio, Cb=None, Zb=None, prev_Cb=None, prev_Zb=None,
                      pos0=0, gamma=None, eps=1e-6, rope_dims=0, rope_base=_rope.DEFAULT_BASE,
                      rope_anchor=0):
    """Compress one sequence's chunk of raw tokens.

    Ca, Za (and Cb, Zb for C4A): [n_tok, c], raw tokens pos0 .. pos0+n_tok-1.
    prev_Cb, prev_Zb: [4, c], the 4 raw tokens before pos0 (C4A, pos0 > 0).
    bias: [8, c] for C4A, [128, c] for C128A.
    Returns (out [n_tok // ratio, c], weights [n_tok // ratio, rows, c])."""
    Ca = np.asarray(Ca, dtype=np.float64)
    Za = np.asarray(Za, dtype=np.float64)
    bias = np.asarray(bias, dtype=np.float64)
    n_tok, c = Ca.shape
    if pos0 % ratio:
        raise ValueError("pos0 must start a block")
    g = np.ones(c) if gamma is None else np.asarray(gamma, dtype=np.float64)
    n_ent = n_tok // ratio
    if ratio == 4:
        Cb = np.asarray(Cb, dtype=np.float64)
        Zb = np.asarray(Zb, dtype=np.float64)
        if pos0 > 0:
            hC = np.asarray(prev_Cb, dtype=np.float64)
            hZ = np.asarray(prev_Zb, dtype=np.float64)
        rows = 2 * ratio
    elif ratio == 128:
        rows = ratio
    else:
        raise ValueError("ratio must be 4 or 128")

    out = np.zeros((n_ent, c))
    weights = np.zeros((n_ent, rows, c))
    for i in range(n_ent):
        cur = slice(ratio * i, ratio * i + ratio)
        L_cur = Za[cur] + bias[:ratio]
        X_cur = Ca[cur]
        if ratio == 4:
            if i >= 1:
                prv = slice(ratio * i - PREV, ratio * i)
                L_prev = Zb[prv] + bias[ratio:]
                X_prev = Cb[prv]
            elif pos0 > 0:
                L_prev = hZ + bias[ratio:]
                X_prev = hC
            else:  # block 0 of the sequence: zero content, weight logit -inf
                L_prev = np.full((PREV, c), -np.inf)
                X_prev = np.zeros((PREV, c))
            L = np.concatenate([L_cur, L_prev], axis=0)
            X = np.concatenate([X_cur, X_prev], axis=0)
        else:
            L, X = L_cur, X_cur
        y, p = _softmax_pool(L, X)
        out[i] = _rmsnorm(y, g, eps)
        if rope_dims:
            at = _rope.entry_position(pos0 // ratio + i, ratio, rope_anchor)
            out[i] = _rope.rotate(out[i], at, rope_dims, rope_base)
        weights[i] = p
    return out, weights


def compress(Ca, Za, bias, ratio, Cb=None, Zb=None, prev_Cb=None, prev_Zb=None, pos0=0,
             gamma=None, eps=1e-6, rope_dims=0, rope_base=_rope.DEFAULT_BASE, rope_anchor=0):
    """Batched form: inputs [B, n_tok, c] (halo [B, 4, c]); returns out [B, n_ent, c]."""
    Ca = np.asarray(Ca)
    outs = []
    for b in range(Ca.shape[0]):
        o, _ = compress_sequence(
            Ca[b], Za[b], bias, ratio,
            None if Cb is None else Cb[b], None if Zb is None else Zb[b],
            None if prev_Cb is None else prev_Cb[b], None if prev_Zb is None else prev_Zb[b],
            pos0=pos0, gamma=gamma, eps=eps, rope_dims=rope_dims, rope_base=rope_base,
            rope_anchor=rope_anchor)
        outs.append(o)
    return np.stack(outs)
