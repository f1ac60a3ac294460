"""Pins of the indexer and Top-k oracles, and of the quantized-input decoders.

Pages: "DeepSeek Technical Reports" (DSA: the indexer and Top-k equations);
"DeepSeek V4 结构速览" (Lightning Indexer: ReLU, head-weighted sum, BF16
scores, causal range, top-512).
"""
import json
import os

import numpy as np
import pytest
import torch

import synth
from oracle import indexer as oi
from oracle import numerics as on
from oracle import topk as ot

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _qwk(B=2, T=12, N=5, H=4, d=8, seed=1):
    q = synth.normal("q", (B, T, H, d), seed=seed).astype(np.float64)
    w = synth.uniform("w", (B, T, H), seed=seed).astype(np.float64)
    k = synth.normal("k", (B, N, d), seed=seed).astype(np.float64)
    return q, w, k


# ---------------------------------------------------------------- decoders


def test_ocp_code_points():
    with open(os.path.join(GOLDEN, "ocp_codes.json")) as f:
        g = json.load(f)
    for code, v in g["e4m3"]:
        got = on.decode_e4m3(np.array([int(code, 16)], dtype=np.uint8))[0]
        assert got == v and np.signbit(got) == np.signbit(v), (code, got, v)
    for code in g["e4m3_nan"]:
        assert np.isnan(on.decode_e4m3(np.array([int(code, 16)], dtype=np.uint8))[0])
    for code, v in g["e2m1"]:
        got = on.decode_e2m1(np.array([code], dtype=np.uint8))[0]
        assert got == v and np.signbit(got) == np.signbit(v)
    for code, v in g["e8m0"]:
        assert on.decode_e8m0(np.array([code], dtype=np.uint8))[0] == v
    assert np.isnan(on.decode_e8m0(np.array([g["e8m0_nan"]], dtype=np.uint8))[0])


def test_fp8_encode_decode_is_nearest():
    """The input encoder picks a nearest E4M3 value; decoding gives it back."""
    x = synth.normal("x", (4000,), seed=5).astype(np.float64) * 60
    codes = synth.encode_fp8_e4m3(x)
    dec = on.decode_e4m3(codes)
    allv = on.decode_e4m3(np.arange(256, dtype=np.uint8))
    allv = allv[np.isfinite(allv)]
    best = np.min(np.abs(np.clip(x, -448, 448)[:, None] - allv[None, :]), axis=1)
    np.testing.assert_allclose(np.abs(np.clip(x, -448, 448) - dec), best, rtol=0, atol=1e-12)


def test_mxfp4_encode_decode_within_half_step():
    x = synth.normal("x", (6, 128), seed=6)
    packed, sc = synth.quant_mxfp4(x)
    assert packed.shape == (6, 64) and sc.shape == (6, 4)
    dec = on.dequant_mxfp4(packed, sc)
    blocks = x.reshape(6, 4, 32).astype(np.float64)
    scale = on.decode_e8m0(sc)
    # largest element lands in [4, 8) * scale before clamping at 6
    amax = np.abs(blocks).max(axis=-1)
    assert np.all((amax / scale >= 4) & (amax / scale < 8))
    err = np.abs(dec.reshape(6, 4, 32) - blocks) / scale[..., None]
    # E2M1 spacing is at most 2 below 6; clamping loses at most 2 more
    assert np.all(err <= 2.0 + 1e-12)
    assert np.all(err[np.abs(blocks) / scale[..., None] < 4] <= 0.5 + 1e-12)


def test_mxfp4_nibble_order():
    """Element 0 of a block sits in the low nibble of byte 0."""
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 4.0     # amax 4 -> E = 0, code 6
    x[0, 1] = -1.0    # code 0b1010
    packed, sc = synth.quant_mxfp4(x)
    assert sc[0, 0] == 127
    assert packed[0, 0] == (0x6 | (0xA << 4))


def test_store_bf16_rounding():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -np.inf, np.inf, 0.0, 3.0e38])
    got = on.store_bf16(vals)
    assert got[0] == 1.0
    assert got[1] == 1.0                 # tie -> even
    assert got[2] == 1.0 + 2 ** -7       # above half -> up
    assert got[3] == -np.inf and got[4] == np.inf and got[5] == 0.0
    assert got[6] == np.float64(np.float32(3.0e38)) or np.isfinite(got[6])


# ---------------------------------------------------------------- indexer


def test_visible_counts():
    assert [oi.visible(t, 4) for t in range(9)] == [0, 0, 0, 1, 1, 1, 1, 2, 2]
    assert oi.visible(127, 128) == 1 and oi.visible(126, 128) == 0
    assert oi.visible(65535, 4) == 16384 and oi.visible(1048575, 128) == 8192


def test_scores_nonnegative_for_nonnegative_weights():
    q, w, k = _qwk(T=40, N=10)
    s = oi.index_scores(q, w, k, q_pos0=0, ratio=4)
    fin = np.isfinite(s)
    assert np.all(s[fin] >= 0)
    assert fin.sum() > 0


def test_mask_is_exactly_the_causal_range():
    q, w, k = _qwk(T=40, N=10)
    s = oi.index_scores(q, w, k, q_pos0=0, ratio=4)
    for t in range(40):
        v = min(oi.visible(t, 4), 10)
        assert np.all(np.isfinite(s[:, t, :v])) and np.all(s[:, t, v:] == -np.inf)


def test_single_head_unit_weight_is_relu_of_gemm():
    """H_I = 1, w = 1: scores are ReLU(q k^T), a plain matrix product (torch, CPU)."""
    q, _, k = _qwk(T=6, N=7, H=1, d=16)
    w = np.ones((2, 6, 1))
    s = oi.index_scores(q, w, k, q_pos0=100, ratio=4)
    ref = torch.relu(torch.from_numpy(q[:, :, 0]) @ torch.from_numpy(k).transpose(1, 2)).numpy()
    np.testing.assert_allclose(s, ref, rtol=1e-13, atol=1e-13)


def test_scores_linear_in_weights():
    q, w, k = _qwk(T=8, N=6)
    w2 = synth.uniform("w2", w.shape, seed=9).astype(np.float64)
    a = oi.index_scores(q, w, k, 50, 4)
    b = oi.index_scores(q, w2, k, 50, 4)
    c = oi.index_scores(q, w + 2.0 * w2, k, 50, 4)
    np.testing.assert_allclose(c, a + 2.0 * b, rtol=1e-12, atol=1e-12)


def test_bruteforce_loops_tiny():
    q, w, k = _qwk(B=1, T=9, N=3, H=3, d=5)
    s = oi.index_scores(q, w, k, q_pos0=2, ratio=4)
    for t in range(9):
        for sidx in range(3):
            if sidx >= (2 + t + 1) // 4:
                assert s[0, t, sidx] == -np.inf
                continue
            tot = 0.0
            for j in range(3):
                dot = sum(q[0, t, j, e] * k[0, sidx, e] for e in range(5))
                tot += w[0, t, j] * (dot if dot > 0 else 0.0)
            assert abs(s[0, t, sidx] - tot) < 1e-12


def test_negative_dot_products_are_dropped_not_negated():
    """Flipping the sign of a key changes which heads contribute (ReLU, not |.|)."""
    q, w, k = _qwk(B=1, T=1, N=1, H=6, d=4)
    a = oi.index_scores(q, w, k, 3, 4)[0, 0, 0]
    b = oi.index_scores(q, w, -k, 3, 4)[0, 0, 0]
    dots = q[0, 0] @ k[0, 0]
    np.testing.assert_allclose(a - b, w[0, 0] @ dots, rtol=1e-12)


# ---------------------------------------------------------------- top-k


def _bruteforce(row, v, k):
    cands = sorted(range(v), key=lambda s: (-(row[s] + 0.0), s))
    take = cands[:k]
    return take + [-1] * (k - len(take))


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_full_sort_with_ties(seed):
    g = np.random.default_rng(seed)
    T, N, k = 30, 40, 7
    scores = g.integers(0, 5, size=(1, T, N)).astype(np.float64)   # many ties
    idx = ot.topk_select(scores, k, q_pos0=90, ratio=4)
    for t in range(T):
        v = min((90 + t + 1) // 4, N)
        assert list(idx[0, t]) == _bruteforce(scores[0, t], v, k)


def test_topk_all_equal_gives_first_k():
    s = np.full((1, 1, 100), 0.25)
    assert list(ot.topk_select(s, 10, q_pos0=399, ratio=4)[0, 0]) == list(range(10))


def test_topk_fewer_visible_than_k_pads():
    s = synth.normal("s", (1, 12, 8), seed=2).astype(np.float64)
    idx = ot.topk_select(s, 5, q_pos0=0, ratio=4)
    for t in range(12):
        v = (t + 1) // 4
        row = idx[0, t]
        if v < 5:
            assert sorted(row[:v]) == list(range(v)) and np.all(row[v:] == -1)


def test_topk_monotone_rows():
    dec = np.arange(50, 0, -1, dtype=np.float64)[None, None]
    inc = np.arange(50, dtype=np.float64)[None, None]
    assert list(ot.topk_select(dec, 6, q_pos0=199, ratio=4)[0, 0]) == list(range(6))
    assert sorted(ot.topk_select(inc, 6, q_pos0=199, ratio=4)[0, 0]) == list(range(44, 50))


def test_topk_signed_zero_is_a_tie():
    s = np.array([[[-0.0, 0.0, -0.0, 0.0]]])
    assert list(ot.topk_select(s, 2, q_pos0=15, ratio=4)[0, 0]) == [0, 1]
