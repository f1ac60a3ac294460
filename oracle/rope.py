"""Partial RoPE and inverse RoPE oracle.

Test infrastructure only (see the package docstring).

What the pages define:

* "DeepSeek Technical Reports" (DeepSeek-V4, Hybrid Attention, CSA): because
  compressed entries stand for several tokens, position needs its own
  treatment, which the report gives in its Partial Rotary Positional
  Embedding section.
* "DeepSeek V4 结构速览" (the CSA operator graph; C4A Compressor; HCA):  The query gets
  RoPE at its position; each compressed entry gets RoPE after its RMSNorm,
  at an anchor position whose symbol is lost in the extraction (one for C4A,
  one for HCA); the attention output has inverse RoPE applied to its last 64
  dimensions.

Readings taken where the pages are silent or garbled:

* The rotary embedding is RoFormer's: the rotated part is the last R
  dimensions (R = 64 on the pages), taken as adjacent pairs (x[2p], x[2p+1])
  of that part, pair p turned by the angle pos * theta_p with
  theta_p = base ** (-2p / R), p = 0 .. R/2 - 1.  The pages give no base; the
  default 10000 is RoFormer's.
* Forward RoPE at position pos maps (x, y) to
  (x cos a - y sin a, x sin a + y cos a), a = pos * theta_p; inverse RoPE at
  pos is forward RoPE at -pos.
* Since K = V, each value row carries the rotation of its own position; the
  inverse RoPE of the output uses the query's position, which leaves in the
  output only the rotation by (row position - query position).
* The anchor of compressed entry s (absolute index, ratio m) is position
  m * s + a for a caller-chosen offset 0 <= a < m (the lost symbol); a = 0,
  the block's first raw token, is the default reading.
"""
from __future__ import annotations

import numpy as np

DEFAULT_BASE = 10000.0


def inv_freq(R: int, base: float = DEFAULT_BASE) -> np.ndarray:
    """theta_p = base ** (-2p / R) for the R/2 pairs, float64."""
    if R % 2:
        raise ValueError("the rotated part has an even number of dimensions")
    return np.asarray(base, dtype=np.float64) ** (-np.arange(0, R, 2, dtype=np.float64) / R)


def rotate(x, pos, R: int, base: float = DEFAULT_BASE, inverse: bool = False) -> np.ndarray:
    """RoPE (or its inverse) on the last R dimensions of x at position(s) pos.

    x: [..., D]; pos: an integer or an integer array that broadcasts against
    x's leading dimensions.  Returns a float64 copy; the first D - R
    dimensions are unchanged."""
    x = np.array(x, dtype=np.float64)
    if R == 0:
        return x
    D = x.shape[-1]
    if R > D:
        raise ValueError("R exceeds the vector width")
    sign = -1.0 if inverse else 1.0
    a = sign * np.asarray(pos, dtype=np.float64)[..., None] * inv_freq(R, base)   # [..., R/2]
    cos, sin = np.cos(a), np.sin(a)
    part = x[..., D - R:]
    ev, od = part[..., 0::2].copy(), part[..., 1::2].copy()
    part[..., 0::2] = ev * cos - od * sin
    part[..., 1::2] = ev * sin + od * cos
    return x


def rotate_rows(x, pos0: int, R: int, base: float = DEFAULT_BASE, inverse: bool = False) -> np.ndarray:
    """x: [B, T, H, D] (or [B, T, D]); row t of every sequence sits at pos0 + t."""
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[1]
    pos = pos0 + np.arange(T)
    shape = [1, T] + [1] * (x.ndim - 3)      # broadcast over B and any head axis
    return rotate(x, pos.reshape(shape), R, base, inverse)


def entry_position(s, ratio: int, anchor: int = 0):
    """Anchor position of compressed entry s (absolute index) of ratio m."""
    if not 0 <= anchor < ratio:
        raise ValueError("the anchor lies inside the entry's block")
    return ratio * np.asarray(s) + anchor
