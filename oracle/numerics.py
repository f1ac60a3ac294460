"""Exact decoding of the quantized indexer inputs, bf16 score storage, and the
fp8 row quantizer of quantize-on-write.

Test infrastructure only (see the package docstring).

The pages state the indexer's QK path runs in FP4 and its scores are stored
as BF16 ("DeepSeek V4 结构速览", Lightning Indexer); the fp8 variant follows
the V3.2-style indexer.  The formats are the OCP ones:

* E4M3 (FN): 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent field 0
  is subnormal (m/8 * 2^-6); 0x7F / 0xFF are NaN; largest finite 448.
* E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* E8M0: an unsigned power of two, 2^(e - 127); 0xFF is NaN.
* MXFP4 (OCP MX v1.0): blocks of 32 E2M1 elements sharing one E8M0 scale;
  two elements per byte, the even element in the low nibble.
"""
from __future__ import annotations

import numpy as np


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """E4M3 byte codes -> float64 values (bit-field decoding)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    v = np.where(e == 0, sub, normal)
    v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    return sign * v


def decode_e2m1(nibbles: np.ndarray) -> np.ndarray:
    """4-bit E2M1 codes -> float64 values (bit-field decoding)."""
    n = np.asarray(nibbles, dtype=np.uint8).astype(np.int64)
    sign = np.where(n & 0x8, -1.0, 1.0)
    e = (n >> 1) & 0x3
    m = (n & 0x1).astype(np.float64)
    v = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e.astype(np.float64) - 1.0))
    return sign * v


def decode_e8m0(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def dequant_fp8_rows(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """x = E4M3(code) * row_scale, the scale shared along the last axis."""
    return decode_e4m3(codes) * np.asarray(scale, dtype=np.float64)[..., None]


def dequant_mxfp4(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Unpack [..., n/2] bytes and [..., n/32] E8M0 scales to float64 [..., n]."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = p & 0x0F
    hi = p >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(*p.shape[:-1], p.shape[-1] * 2)
    vals = decode_e2m1(nib)
    n = vals.shape[-1]
    blocks = vals.reshape(*vals.shape[:-1], n // 32, 32)
    blocks = blocks * decode_e8m0(scales)[..., None]
    return blocks.reshape(vals.shape)


def store_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 -> nearest bfloat16 (ties to even), as float64.

    This is how a score computed in fp32 is stored in BF16.  +-inf stay
    infinite; the rounding is written out on the float32 bit pattern."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    finite = np.isfinite(f)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    r = np.where(finite, r, f.view(np.uint32))
    return r.view(np.float32).astype(np.float64)


def encode_e4m3(x: np.ndarray) -> np.ndarray:
    """Values -> E4M3 byte codes: the nearest finite E4M3 value, ties to the
    code with an even mantissa (round to nearest even), magnitudes past 448
    to 448 (saturation); the sign is kept, so -0.0 -> 0x80.  A brute-force
    search over the 126 finite non-negative codes."""
    x = np.asarray(x, dtype=np.float64)
    codes = np.arange(0x7F, dtype=np.uint8)               # 0x00 .. 0x7E: every finite non-negative code
    vals = decode_e4m3(codes)
    a = np.abs(x)[..., None]
    d = np.abs(a - vals)
    best = d.min(axis=-1, keepdims=True)
    tie_ok = d == best
    # among equally near codes take the one with an even mantissa (bit 0 clear)
    even = (codes & 1) == 0
    pick = np.where(tie_ok & even, 0, np.where(tie_ok, 1, 2))
    idx = np.argmin(pick, axis=-1)
    out = codes[idx]
    return np.where(np.signbit(x), out | 0x80, out).astype(np.uint8)


def quant_fp8_rows_f32(y: np.ndarray):
    """Quantize-on-write of rows to fp8 ("DeepSeek-V4 技术报告解读" / "DeepSeek V4
    结构速览": the indexer keys are kept in low precision): per row of the last
    axis, scale = amax / 448 and code = E4M3(y / scale), every step in fp32
    (the precision the writing kernel decides in); an all-zero row gets scale
    1.  Returns (codes uint8 like y, scale float32 like y.shape[:-1])."""
    y = np.asarray(y, dtype=np.float32)
    amax = np.abs(y).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    v = (y / scale[..., None]).astype(np.float32)
    return encode_e4m3(v), scale


def encode_e2m1(v: np.ndarray) -> np.ndarray:
    """Values -> E2M1 nibbles: the nearest of the 8 magnitudes, ties to the
    code with an even mantissa, magnitudes past 6 to 6; a value that rounds
    to 0 is written +0 (code 0).  Brute force over the table."""
    v = np.asarray(v, dtype=np.float64)
    codes = np.arange(8, dtype=np.uint8)
    mags = decode_e2m1(codes)
    d = np.abs(np.abs(v)[..., None] - mags)
    best = d.min(axis=-1, keepdims=True)
    tie = d == best
    pick = np.where(tie & ((codes & 1) == 0), 0, np.where(tie, 1, 2))
    code = codes[np.argmin(pick, axis=-1)]
    return np.where((v < 0) & (code != 0), code | 8, code).astype(np.uint8)


def quant_mxfp4_rows_f32(y: np.ndarray):
    """Quantize-on-write of rows to MXFP4 (OCP MX v1.0; "DeepSeek V4 结构速览",
    CSA operator graph: the indexer scores in FP4): per block of 32 elements of
    the last axis, the shared exponent E = floor(log2(amax)) - 2 (E + 127 as
    E8M0, clipped to [0, 254]; 0 for an all-zero block), elements y / 2^E
    (exact) as E2M1, two per byte with element 2i in the low nibble.
    Returns (packed uint8 [..., n/2], scales uint8 [..., n/32])."""
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    n = y.shape[-1]
    blocks = y.reshape(*y.shape[:-1], n // 32, 32)
    amax = np.abs(blocks).max(axis=-1)
    _, ex = np.frexp(amax)                       # amax = m 2^ex with m in [0.5, 1): floor(log2) = ex - 1
    E = np.where(amax > 0, ex - 1 - 2, -127)
    E = np.clip(E, -127, 127).astype(np.int64)
    nib = encode_e2m1(blocks * np.exp2(-E)[..., None]).reshape(*y.shape[:-1], n)
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return packed, (E + 127).astype(np.uint8)
