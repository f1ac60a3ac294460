"""Shared test helpers: host <-> device transfer of seeded inputs and comparison rules.

Tolerances (attention and compressor outputs, indexer scores) are the ones
the workloads state or that follow from the arithmetic; each test names the
one it applies.
"""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda"


def dev(x: np.ndarray, dtype=torch.float32) -> torch.Tensor:
    """Host array -> contiguous device tensor.  Values meant for bf16 must be
    bf16-representable already (synth.round_bf16), so the conversion is exact."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    if t.dtype != dtype:
        t = t.to(dtype)
    return t.to(DEV).contiguous()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))))


def normwise_rel(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


# Tolerances
ATTN_BF16_MAX_ABS = 2e-2        # attention, bf16 I/O (stated for the workloads)
ATTN_NORMWISE = 1e-2            # guard: an all-zero output must not pass
ATTN_F32_MAX_ABS = 1e-4         # attention, fp32 I/O
COMP_F32_MAX_ABS = 1e-4         # compressor, fp32 I/O
COMP_BF16_MAX_ABS = 2e-2        # compressor, bf16 output (outputs are O(1): ~3 bf16 ulps)
INDEX_REL = 1e-3                # indexer scores, fp32 accumulation (stated for the workloads)


def index_close(got, ref, rel=INDEX_REL):
    """|g - o| <= rel*|o| + 1e-5*max_s|o[t,s]| on finite entries; -inf exactly where the oracle has it."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    masked = ~np.isfinite(ref)
    assert np.array_equal(~np.isfinite(got), masked), "masked pattern differs"
    assert np.all(got[masked] == -np.inf)
    r = np.where(masked, 0.0, ref)
    g = np.where(masked, 0.0, got)
    floor = 1e-5 * np.max(np.abs(r), axis=-1, keepdims=True)
    bad = np.abs(g - r) > rel * np.abs(r) + floor
    assert not bad.any(), f"{bad.sum()} scores outside tolerance; worst {np.max(np.abs(g - r) - rel * np.abs(r) - floor)}"
