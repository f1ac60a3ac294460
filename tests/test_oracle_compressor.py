"""Pins of the compressor oracle against what the pages and the mathematics fix.

Page: "DeepSeek V4 结构速览", C4A Compressor and 核心设计; compression formula
of "DeepSeek-V4技术报告解读，全适配国产算力", section 2.1.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import compressor as oc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(name, shape, seed=3):
    return synth.normal(name, shape, seed=seed).astype(np.float64)


def _norm_rows(y, eps):
    return y / np.sqrt((y * y).mean(axis=-1, keepdims=True) + eps)


@pytest.mark.parametrize("pos0", [0, 8])
def test_weights_sum_to_one_per_channel(pos0):
    n, c = 32, 16
    Ca, Za, Cb, Zb = (_rand(nm, (n, c)) for nm in ("Ca", "Za", "Cb", "Zb"))
    hC, hZ = _rand("hC", (4, c)), _rand("hZ", (4, c))
    bias = _rand("bias", (8, c)) * 0.3
    _, p = oc.compress_sequence(Ca, Za, bias, 4, Cb, Zb, hC, hZ, pos0=pos0)
    assert p.shape == (8, 8, c)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-12
    assert np.all(p >= 0)
    if pos0 == 0:   # block 0 has no previous block: its 4 padded rows get weight 0
        assert np.all(p[0, 4:] == 0.0)
        assert np.all(p[1:, 4:] > 0.0)
    else:
        assert np.all(p[:, 4:] > 0.0)


def test_c128a_weights_sum_to_one():
    n, c = 256, 8
    _, p = oc.compress_sequence(_rand("Ca", (n, c)), _rand("Za", (n, c)), _rand("b", (128, c)), 128)
    assert p.shape == (2, 128, c)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-12


@pytest.mark.parametrize("ratio", [4, 128])
def test_constant_content_gives_rmsnorm_of_it(ratio):
    """Same vector v in every token: pooling returns v whatever the weights."""
    n, c, eps = 2 * ratio, 24, 1e-6
    v = _rand("v", (c,))
    C = np.tile(v, (n, 1))
    Z = _rand("Z", (n, c)) * 3
    bias = _rand("b", (2 * ratio if ratio == 4 else ratio, c))
    gamma = _rand("g", (c,))
    out, _ = oc.compress_sequence(C, Z, bias, ratio, C, -Z, pos0=0, gamma=gamma, eps=eps)
    expect = v / math.sqrt(float(np.mean(v * v)) + eps) * gamma
    np.testing.assert_allclose(out, np.tile(expect, (n // ratio, 1)), rtol=1e-13, atol=1e-13)


def test_zero_logits_is_average_pooling_c4a():
    """Z = B = 0 and Ca = Cb = X: entry i >= 1 is the mean of X[4i-4 : 4i+4]
    (torch avg_pool1d, kernel 8, stride 4); entry 0 the mean of X[0:4]."""
    n, c, eps = 64, 32, 1e-6
    X = _rand("X", (n, c))
    Z = np.zeros((n, c))
    out, _ = oc.compress_sequence(X, Z, np.zeros((8, c)), 4, X, Z, pos0=0, eps=eps)
    xt = torch.from_numpy(X.T[None])                       # [1, c, n]
    pool8 = torch.nn.functional.avg_pool1d(xt, 8, 4)[0].numpy().T   # entries 1..
    pool4 = torch.nn.functional.avg_pool1d(xt, 4, 4)[0].numpy().T
    np.testing.assert_allclose(out[1:], _norm_rows(pool8, eps), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out[0], _norm_rows(pool4[0], eps), rtol=1e-12, atol=1e-12)


def test_zero_logits_is_average_pooling_c128a():
    n, c, eps = 384, 16, 1e-6
    X = _rand("X", (n, c))
    out, _ = oc.compress_sequence(X, np.zeros((n, c)), np.zeros((128, c)), 128, eps=eps)
    pool = torch.nn.functional.avg_pool1d(torch.from_numpy(X.T[None]), 128, 128)[0].numpy().T
    np.testing.assert_allclose(out, _norm_rows(pool, eps), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("r", [0, 1, 2, 3])
def test_large_logit_picks_one_token_from_the_right_block(r):
    """A +60 logit on current-block offset r picks Ca[4i+r]; a +60 bias on row
    4+r picks Cb[4i-4+r].  Fixes which projection is the current block and the
    bias row order."""
    n, c, eps = 32, 8, 0.0
    Ca, Cb = _rand("Ca", (n, c)), _rand("Cb", (n, c))
    Z = np.zeros((n, c))
    Za = Z.copy()
    Za[r::4] = 60.0
    out, _ = oc.compress_sequence(Ca, Za, np.zeros((8, c)), 4, Cb, Z, pos0=0, eps=eps)
    np.testing.assert_allclose(out, _norm_rows(Ca[r::4], eps), rtol=1e-12, atol=1e-12)
    bias = np.zeros((8, c))
    bias[4 + r] = 60.0
    out, _ = oc.compress_sequence(Ca, Z, bias, 4, Cb, Z, pos0=0, eps=eps)
    prev = Cb[np.arange(1, n // 4) * 4 - 4 + r]
    np.testing.assert_allclose(out[1:], _norm_rows(prev, eps), rtol=1e-12, atol=1e-12)
    # entry 0 has no previous block: the bias on padded rows changes nothing
    np.testing.assert_allclose(out[0], _norm_rows(Ca[0:4].mean(axis=0), eps), rtol=1e-12)


def test_rmsnorm_unit_mean_square():
    n, c = 64, 64
    out, _ = oc.compress_sequence(_rand("Ca", (n, c)), _rand("Za", (n, c)), _rand("b", (8, c)), 4,
                                  _rand("Cb", (n, c)), _rand("Zb", (n, c)), pos0=0, eps=0.0)
    np.testing.assert_allclose((out * out).mean(axis=1), 1.0, rtol=1e-13)


def test_causality_of_entries():
    """Changing raw tokens >= 4(i+1) leaves entries 0..i unchanged, bit for bit."""
    n, c = 64, 16
    arrs = {nm: _rand(nm, (n, c)) for nm in ("Ca", "Za", "Cb", "Zb")}
    bias = _rand("b", (8, c))
    base, _ = oc.compress_sequence(arrs["Ca"], arrs["Za"], bias, 4, arrs["Cb"], arrs["Zb"])
    for i in (0, 5, 14):
        pert = {k: v.copy() for k, v in arrs.items()}
        for v in pert.values():
            v[4 * (i + 1):] += 7.0
        out, _ = oc.compress_sequence(pert["Ca"], pert["Za"], bias, 4, pert["Cb"], pert["Zb"])
        assert np.array_equal(out[:i + 1], base[:i + 1])
        assert not np.array_equal(out[i + 1:], base[i + 1:])


def test_chunk_with_halo_matches_whole_sequence():
    """A chunk starting at pos0 = 24 with the 4-token halo gives the same entries
    as compressing the whole sequence from 0."""
    n, c = 64, 16
    arrs = {nm: _rand(nm, (n, c)) for nm in ("Ca", "Za", "Cb", "Zb")}
    bias = _rand("b", (8, c))
    whole, _ = oc.compress_sequence(arrs["Ca"], arrs["Za"], bias, 4, arrs["Cb"], arrs["Zb"])
    p0 = 24
    part, _ = oc.compress_sequence(arrs["Ca"][p0:], arrs["Za"][p0:], bias, 4, arrs["Cb"][p0:],
                                   arrs["Zb"][p0:], arrs["Cb"][p0 - 4:p0], arrs["Zb"][p0 - 4:p0],
                                   pos0=p0)
    np.testing.assert_array_equal(part, whole[p0 // 4:])


def test_ragged_tail_produces_no_entry():
    n, c = 30, 8
    out, _ = oc.compress_sequence(_rand("Ca", (n, c)), _rand("Za", (n, c)), _rand("b", (8, c)), 4,
                                  _rand("Cb", (n, c)), _rand("Zb", (n, c)))
    assert out.shape == (7, c)


def test_golden_worked_example():
    with open(os.path.join(GOLDEN, "compressor_worked_example.json")) as f:
        g = json.load(f)

    def val(x):
        return math.log(float(x[2:])) if isinstance(x, str) else float(x)

    arr = {k: np.array([[val(x) for x in row] for row in g[k]]) for k in ("Ca", "Za", "Cb", "Zb", "bias")}
    out, _ = oc.compress_sequence(arr["Ca"], arr["Za"], arr["bias"], g["ratio"], arr["Cb"], arr["Zb"],
                                  pos0=0, eps=g["eps"])
    np.testing.assert_allclose(out, np.array(g["expected_out"]), rtol=1e-14, atol=1e-14)
