"""Seeded synthetic inputs for the compressed sparse attention path.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It only *draws and encodes inputs*: random tensors with the
distributions the workloads state, rounding of inputs to bf16, and the fp8 /
MXFP4 encodings the indexer reads.  It contains none of the method's
arithmetic (no pooling, softmax, scoring, selection or attention).

Every tensor is drawn from its own PCG64 stream, keyed by (seed, name), so a
tensor's values do not depend on which other tensors were drawn before it.

Workload shapes follow the DeepSeek-V4 pages: C4A pools 8 tokens at stride 4,
C128A pools 128 at stride 128 ("DeepSeek V4 结构速览", 核心设计); top-k is 512
or 1024; the window is 128 tokens; attention has 64 heads of dim 512 and the
indexer 64 heads of dim 128 (same page, CSA and Lightning Indexer sections).
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field

import numpy as np

# --------------------------------------------------------------------------
# random streams
# --------------------------------------------------------------------------


def rng(name: str, seed: int = 0) -> np.random.Generator:
    """Independent PCG64 stream for one named tensor."""
    key = zlib.crc32(name.encode("utf-8"))
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, key])))


def normal(name: str, shape, var: float = 1.0, seed: int = 0) -> np.ndarray:
    """N(0, var) in float32.  The second parameter of N(.,.) is a variance."""
    g = rng(name, seed)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if var != 1.0:
        x *= np.float32(np.sqrt(var))
    return x


def uniform(name: str, shape, lo: float = 0.0, hi: float = 1.0, seed: int = 0) -> np.ndarray:
    g = rng(name, seed)
    return (g.random(size=shape, dtype=np.float32) * np.float32(hi - lo) + np.float32(lo)).astype(np.float32)


def torch_seed(name: str, seed: int = 0) -> int:
    """Seed for a device-side torch.Generator, for tensors too large to draw on the host."""
    return (seed * 1_000_003 + zlib.crc32(name.encode("utf-8"))) & 0x7FFFFFFF


# --------------------------------------------------------------------------
# input encodings
# --------------------------------------------------------------------------


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-representable."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(b & 0xFFFF):
        raise ValueError("values are not bf16-representable; call round_bf16 first")
    return (b >> 16).astype(np.uint16)


def _e4m3_table() -> np.ndarray:
    """Values of the 127 non-negative finite OCP E4M3 codes (0x00..0x7E)."""
    vals = np.empty(127, dtype=np.float64)
    for code in range(127):
        e = code >> 3
        m = code & 7
        vals[code] = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3 = _e4m3_table()
_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _round_to_table(mag: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the nearest entry of an increasing table; ties go to the even index;
    magnitudes beyond the last entry saturate to it."""
    mag = np.minimum(mag, table[-1])
    hi = np.clip(np.searchsorted(table, mag, side="left"), 1, len(table) - 1)
    lo = hi - 1
    dlo = mag - table[lo]
    dhi = table[hi] - mag
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(mag == table[0], 0, idx)
    return idx


def encode_fp8_e4m3(x: np.ndarray) -> np.ndarray:
    """float -> OCP E4M3 (FN) byte codes, round to nearest even, saturating at 448."""
    x = np.asarray(x, dtype=np.float64)
    idx = _round_to_table(np.abs(x), _E4M3).astype(np.uint8)
    sign = np.where((x < 0) & (idx != 0), np.uint8(0x80), np.uint8(0))
    return (idx | sign).astype(np.uint8)


def quant_fp8_rows(x: np.ndarray):
    """Per-row fp8: scale = amax/448 over the last axis, codes = E4M3(x / scale).

    Returns (codes uint8 with x's shape, scale float32 with x.shape[:-1])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    codes = encode_fp8_e4m3(x.astype(np.float64) / scale[..., None].astype(np.float64))
    return codes, scale


def quant_mxfp4(x: np.ndarray):
    """OCP MX v1.0 MXFP4 along the last axis (a multiple of 32).

    Each block of 32 gets a shared exponent E = floor(log2(amax)) - 2 stored as
    e8m0 (E + 127); elements are x / 2^E rounded to E2M1 (ties to even, clamped
    to +-6).  Two elements per byte: element 2i in the low nibble, 2i+1 in the
    high nibble.  Returns (packed uint8 [..., n/2], scales uint8 [..., n/32])."""
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[-1]
    if n % 32:
        raise ValueError("last axis must be a multiple of 32")
    blocks = x.reshape(*x.shape[:-1], n // 32, 32).astype(np.float64)
    amax = np.abs(blocks).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    e = np.clip(e, -127, 127).astype(np.int32)
    scaled = blocks / np.exp2(e)[..., None]
    idx = _round_to_table(np.abs(scaled), _E2M1).astype(np.uint8)
    sign = np.where((scaled < 0) & (idx != 0), np.uint8(8), np.uint8(0))
    nib = (idx | sign).reshape(*x.shape[:-1], n)
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class Workload:
    """Shapes of one workload.  Positions are absolute and 0-based."""

    name: str
    B: int                 # sequences
    T: int                 # query tokens per sequence
    q_pos0: int            # absolute position of the first query token
    ratio: int             # 4 (C4A / CSA) or 128 (C128A / HCA)
    N: int                 # compressed entries in the cache
    k: int = 0             # top-k (CSA only)
    window: int = 128
    H: int = 64
    d: int = 512
    H_I: int = 64
    d_I: int = 128
    io: str = "bf16"       # attention / compressor I/O type
    qk: str = "bf16"       # indexer QK input type
    score: str = "bf16"    # stored indexer score type
    extra: dict = field(default_factory=dict)

    @property
    def raw_pos0(self) -> int:
        return max(0, self.q_pos0 - self.window + 1)

    @property
    def n_raw(self) -> int:
        return self.q_pos0 + self.T - self.raw_pos0

    @property
    def comp_pos0(self) -> int:
        """First raw token of the compressor's chunk: the block that holds q_pos0."""
        return (self.q_pos0 // self.ratio) * self.ratio

    @property
    def comp_ntok(self) -> int:
        """Raw tokens the compressor pools in this call (whole blocks only)."""
        end = ((self.q_pos0 + self.T) // self.ratio) * self.ratio
        return end - self.comp_pos0


TINY = Workload("tiny_csa_prefill_n256_fp32", B=1, T=256, q_pos0=0, ratio=4, N=64, k=16,
                io="f32", qk="f32", score="f32")
CSA_DECODE = Workload("csa_decode_b32_ctx65536", B=32, T=1, q_pos0=65535, ratio=4, N=16384, k=512)
CSA_PREFILL = Workload("csa_prefill_ctx131072_chunk4096", B=1, T=4096, q_pos0=131072, ratio=4,
                       N=33792, k=512, qk="fp8")
HCA_DECODE = Workload("hca_decode_b16_ctx1048576", B=16, T=1, q_pos0=1048575, ratio=128, N=8192)
HCA_PREFILL = Workload("hca_prefill_ctx1048576_chunk2048", B=1, T=2048, q_pos0=1046528, ratio=128,
                       N=8192)
CSA_1M_DECODE = Workload("csa_decode_b8_ctx1048576_mxfp4", B=8, T=1, q_pos0=1048575, ratio=4,
                         N=262144, k=1024, qk="mxfp4")
# the HCA layer that sits beside the CSA decode layer in a decode step
HCA_DECODE_64K = Workload("hca_decode_b32_ctx65536", B=32, T=1, q_pos0=65535, ratio=128, N=512)

WORKLOADS = {w.name: w for w in (TINY, CSA_DECODE, CSA_PREFILL, HCA_DECODE, HCA_PREFILL,
                                 CSA_1M_DECODE, HCA_DECODE_64K)}


def compressor_inputs(prefix: str, B: int, n_tok: int, c: int, ratio: int, pos0: int,
                      dtype: str = "f32", seed: int = 0) -> dict:
    """Ca, Za (and Cb, Zb, the 4-token halo for C4A) ~ N(0,1); bias ~ N(0, 0.1).

    Shapes are [B, n_tok, c]; the halo is [B, 4, c] and only present when the
    chunk does not start at position 0."""
    out = {}
    names = ["Ca", "Za"] + (["Cb", "Zb"] if ratio == 4 else [])
    for nm in names:
        out[nm] = normal(f"{prefix}.{nm}", (B, n_tok, c), seed=seed)
    if ratio == 4 and pos0 > 0:
        out["prev_Cb"] = normal(f"{prefix}.prev_Cb", (B, 4, c), seed=seed)
        out["prev_Zb"] = normal(f"{prefix}.prev_Zb", (B, 4, c), seed=seed)
    nb = 2 * ratio if ratio == 4 else ratio
    out["bias"] = normal(f"{prefix}.bias", (nb, c), var=0.1, seed=seed)
    if dtype == "bf16":
        for nm in list(out):
            if nm != "bias":
                out[nm] = round_bf16(out[nm])
    return out


# --------------------------------------------------------------------------
# device-side draws for tensors too large to draw on the host
# --------------------------------------------------------------------------


def device_normal(name: str, shape, dtype=None, device="cuda", var: float = 1.0, seed: int = 0):
    """N(0, var) drawn by torch on the device from a seeded generator, then
    cast (round to nearest even) to ``dtype``.  Deterministic for a given
    (seed, name, shape) on a given torch version."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(torch_seed(name, seed))
    x = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32)
    if var != 1.0:
        x.mul_(float(np.sqrt(var)))
    return x if dtype is None else x.to(dtype)


def device_uniform(name: str, shape, device="cuda", seed: int = 0):
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(torch_seed(name, seed))
    return torch.rand(tuple(shape), generator=gen, device=device, dtype=torch.float32)


def random_topk_indices(name: str, B: int, T: int, k: int, visible, seed: int = 0) -> np.ndarray:
    """A seeded stand-in for Top-k output: for each (b, t) a random set of
    min(k, visible[t]) distinct entries of [0, visible[t]) in ascending order,
    then -1 padding.  ``visible`` is a length-T sequence."""
    g = rng(name, seed)
    out = np.full((B, T, k), -1, dtype=np.int32)
    for b in range(B):
        for t in range(T):
            v = int(visible[t])
            n = min(k, v)
            if n == 0:
                continue
            if v <= 4 * n:
                sel = np.sort(g.permutation(v)[:n])
            else:
                sel = np.sort(g.choice(v, size=n, replace=False))
            out[b, t, :n] = sel
    return out


# --------------------------------------------------------------------------
# the same input encodings in torch, for tensors drawn on the device
# --------------------------------------------------------------------------


def _torch_round_to_table(mag, table):
    """torch form of _round_to_table (float64 magnitudes, increasing float64 table)."""
    import torch

    mag = torch.minimum(mag, table[-1])
    flat = mag.reshape(-1).contiguous()
    hi = torch.searchsorted(table, flat, right=False).clamp(1, table.numel() - 1)
    lo = hi - 1
    dlo = flat - table[lo]
    dhi = table[hi] - flat
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    idx = torch.where(pick_hi, hi, lo)
    idx = torch.where(flat == table[0], torch.zeros_like(idx), idx)
    return idx.reshape(mag.shape)


def device_quant_fp8_rows(x):
    """quant_fp8_rows for a torch tensor (any device): per row of the last axis
    scale = amax / 448 in float32 (1 for an all-zero row), codes = E4M3(x / scale)
    with the quotient in float64, nearest even, saturating.  Bit-identical to
    quant_fp8_rows.  Returns (codes uint8, scale float32)."""
    import torch

    x = x.to(torch.float32)
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / torch.tensor(448.0, dtype=torch.float32, device=x.device),
                        torch.ones_like(amax))
    v = x.to(torch.float64) / scale.to(torch.float64)[..., None]
    table = torch.from_numpy(_E4M3).to(x.device)
    idx = _torch_round_to_table(v.abs(), table).to(torch.uint8)
    sign = ((v < 0) & (idx != 0)).to(torch.uint8) * 0x80
    return (idx | sign).contiguous(), scale.contiguous()


def device_quant_mxfp4(x):
    """quant_mxfp4 for a torch tensor (any device): per block of 32 along the
    last axis E = floor(log2 amax) - 2 (read off frexp, exact; -127 for an
    all-zero block; clipped to [-127, 127]), elements x / 2^E to E2M1, nearest
    even, clamped to 6, even element in the low nibble.  Bit-identical to
    quant_mxfp4.  Returns (packed uint8 [..., n/2], scales uint8 [..., n/32])."""
    import torch

    n = x.shape[-1]
    if n % 32:
        raise ValueError("last axis must be a multiple of 32")
    blocks = x.to(torch.float32).to(torch.float64).reshape(*x.shape[:-1], n // 32, 32)
    amax = blocks.abs().amax(dim=-1)
    _, ex = torch.frexp(amax)                      # amax = m 2^ex, m in [0.5, 1)
    e = torch.where(amax > 0, ex.to(torch.int64) - 3, torch.full_like(ex, -127, dtype=torch.int64))
    e = e.clamp(-127, 127)
    scaled = blocks / torch.exp2(e.to(torch.float64))[..., None]
    table = torch.from_numpy(_E2M1).to(x.device)
    idx = _torch_round_to_table(scaled.abs(), table).to(torch.uint8)
    sign = ((scaled < 0) & (idx != 0)).to(torch.uint8) * 8
    nib = (idx | sign).reshape(*x.shape[:-1], n)
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).contiguous()
    return packed, (e + 127).to(torch.uint8).contiguous()
