"""Pins of the attention oracles (sparse shared-KV MQA, dense, HCA with sink).

Pages: "DeepSeek V4 结构速览" (CSA and HCA sections: K = V MQA, window,
sink); "DeepSeek-V4 技术解读：百万 Token 上下文的新里程碑" (2.1, shared-KV MQA);
"DeepSeek Technical Reports" (DSA: attention over the Top-k entries; HCA:
every history region keeps a compressed entry).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import attention as oa
from oracle import indexer as oi


def _case(B=1, T=6, N=12, H=4, d=16, q_pos0=40, window=8, seed=0):
    q = synth.normal("q", (B, T, H, d), seed=seed).astype(np.float64)
    kv = synth.normal("kv", (B, N, d), seed=seed).astype(np.float64)
    raw_pos0 = max(0, q_pos0 - window + 1)
    n_raw = q_pos0 + T - raw_pos0
    raw = synth.normal("raw", (B, n_raw, d), seed=seed).astype(np.float64)
    return q, kv, raw, raw_pos0


def _all_visible_idx(B, T, q_pos0, ratio, k):
    idx = np.full((B, T, k), -1)
    for t in range(T):
        v = oi.visible(q_pos0 + t, ratio)
        idx[:, t, :v] = np.arange(v)
    return idx


def test_sparse_with_all_entries_equals_dense():
    B, T, q_pos0, window = 2, 7, 40, 8
    q, kv, raw, rp0 = _case(B=B, T=T, q_pos0=q_pos0, window=window)
    idx = _all_visible_idx(B, T, q_pos0, 4, k=16)
    o1, l1 = oa.sparse_mqa(q, kv, idx, raw, rp0, q_pos0, window)
    o2, l2 = oa.dense_attention(q, kv, raw, rp0, q_pos0, 4, window)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=1e-12, atol=1e-12)


def test_first_token_attends_only_to_itself():
    q, kv, raw, rp0 = _case(T=1, q_pos0=0)
    idx = np.full((1, 1, 4), -1)
    o, lse = oa.sparse_mqa(q, kv, idx, raw, rp0, 0, 8)
    np.testing.assert_array_equal(o[0, 0], np.tile(raw[0, 0], (4, 1)))


def test_zero_query_gives_mean_of_set():
    q, kv, raw, rp0 = _case(T=2, q_pos0=40, window=8)
    q[:] = 0
    idx = np.array([[[3, 1, 7, -1], [0, 2, -1, -1]]])
    o, lse = oa.sparse_mqa(q, kv, idx, raw, rp0, 40, 8)
    X0 = np.concatenate([kv[0, [3, 1, 7]], raw[0, 40 - 7 - rp0:40 - rp0 + 1]])
    np.testing.assert_allclose(o[0, 0], np.tile(X0.mean(axis=0), (4, 1)), rtol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.log(len(X0)), rtol=1e-13)


def test_planted_needle_dominates():
    q, kv, raw, rp0 = _case(T=1, q_pos0=40, window=8, d=16)
    kv[0, 5] = 0
    kv[0, 5, :] = 3.0 * q[0, 0, 0] / np.linalg.norm(q[0, 0, 0]) * 8
    idx = np.array([[[5, 1, 2, -1]]])
    o, _ = oa.sparse_mqa(q, kv, idx, raw, rp0, 40, 8, scale=1.0)
    np.testing.assert_allclose(o[0, 0, 0], kv[0, 5], rtol=1e-6, atol=1e-6)


def test_output_in_convex_hull_and_permutation_invariant():
    q, kv, raw, rp0 = _case(T=3, q_pos0=44, window=8)
    idx = np.array([[[9, 2, 4, 0], [1, 3, -1, 5], [8, 6, 7, -1]]])
    o, lse = oa.sparse_mqa(q, kv, idx, raw, rp0, 44, 8)
    perm = idx[:, :, ::-1].copy()
    o2, lse2 = oa.sparse_mqa(q, kv, perm, raw, rp0, 44, 8)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=1e-12)
    for t in range(3):
        sel = [s for s in idx[0, t] if s >= 0]
        X = np.concatenate([kv[0, sel], raw[0, 44 + t - 7 - rp0:44 + t - rp0 + 1]])
        assert np.all(o[0, t] <= X.max(axis=0) + 1e-12)
        assert np.all(o[0, t] >= X.min(axis=0) - 1e-12)


def test_window_rows_are_concatenated_not_deduplicated():
    """A compressed entry equal to a window row counts twice in the softmax."""
    q, kv, raw, rp0 = _case(T=1, q_pos0=40, window=8)
    q[:] = 0
    kv[0, 0] = raw[0, -1]
    idx = np.array([[[0, -1]]])
    o, _ = oa.sparse_mqa(q, kv, idx, raw, rp0, 40, 8)
    X = np.concatenate([kv[0, [0]], raw[0]])
    np.testing.assert_allclose(o[0, 0, 0], X.mean(axis=0), rtol=1e-13)


@pytest.mark.parametrize("ratio", [4, 128])
def test_dense_equals_torch_sdpa(ratio):
    """Dense masked attention equals torch's scaled_dot_product_attention
    (CPU, float64) with K = V and an explicit boolean mask."""
    B, T, H, d, window = 1, 5, 4, 16, 8
    q_pos0 = 300 if ratio == 128 else 40
    N = (q_pos0 + T) // ratio + 1
    q, kv, raw, rp0 = _case(B=B, T=T, N=N, H=H, d=d, q_pos0=q_pos0, window=window)
    o, _ = oa.dense_attention(q, kv, raw, rp0, q_pos0, ratio, window)
    allrows = torch.from_numpy(np.concatenate([kv[0], raw[0]]))
    mask = torch.zeros(T, N + raw.shape[1], dtype=torch.bool)
    for t in range(T):
        pos = q_pos0 + t
        mask[t, :(pos + 1) // ratio] = True
        for u in range(max(0, pos - window + 1), pos + 1):
            mask[t, N + u - rp0] = True
    for h in range(H):
        qt = torch.from_numpy(q[0, :, h])[None, None]       # [1,1,T,d]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, allrows[None, None], allrows[None, None], attn_mask=mask[None, None])
        np.testing.assert_allclose(o[0, :, h], ref[0, 0].numpy(), rtol=1e-12, atol=1e-12)


def test_sink_closed_form():
    """With a sink z_h: o_sink = o * sigmoid(lse - z_h), lse_sink = logaddexp(lse, z_h)."""
    q, kv, raw, rp0 = _case(T=3, N=4, q_pos0=300, window=8, H=4)
    sink = synth.normal("sink", (4,), seed=1).astype(np.float64)
    o, lse = oa.dense_attention(q, kv, raw, rp0, 300, 128, 8)
    os_, lses = oa.hca_attention(q, kv, raw, rp0, 300, sink, ratio=128, window=8)
    sig = 1.0 / (1.0 + np.exp(-(lse - sink[None, None, :])))
    np.testing.assert_allclose(os_, o * sig[..., None], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lses, np.logaddexp(lse, sink[None, None, :]), rtol=1e-13)


def test_sink_limits():
    q, kv, raw, rp0 = _case(T=2, N=4, q_pos0=300, window=8, H=4)
    o, _ = oa.dense_attention(q, kv, raw, rp0, 300, 128, 8)
    o_ninf, _ = oa.hca_attention(q, kv, raw, rp0, 300, np.full(4, -np.inf), ratio=128, window=8)
    np.testing.assert_allclose(o_ninf, o, rtol=1e-14, atol=1e-15)
    o_big, _ = oa.hca_attention(q, kv, raw, rp0, 300, np.full(4, 800.0), ratio=128, window=8)
    assert np.max(np.abs(o_big)) < 1e-300


@pytest.mark.parametrize("ratio", [4, 128])
def test_entries_and_window_cover_the_whole_history(ratio):
    """Visible entries' raw spans together with the window cover [0, t] exactly:
    no causal gap, no future token."""
    window = 128
    for t in list(range(0, 700)) + [65535, 1048575]:
        v = oi.visible(t, ratio)
        covered_entries = v * ratio          # entries cover raw [0, v*ratio)
        assert covered_entries <= t + 1      # nothing from the future
        w0 = max(0, t - window + 1)
        assert w0 <= covered_entries         # no gap between entries and window
