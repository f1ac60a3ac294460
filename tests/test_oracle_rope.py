"""Pins of the partial-RoPE oracle and of its use in the compressor and
attention oracles.

Pages: "DeepSeek Technical Reports" (DeepSeek-V4, Hybrid Attention, CSA:
position handled by partial RoPE) and "DeepSeek V4 结构速览" (the compressor's RMSNorm + RoPE at an anchor position; inverse RoPE on the
last 64 output dimensions).  The rotation convention (adjacent pairs of the
last R dimensions, theta_p = base^(-2p/R)) is RoFormer's, a reading; the pins
below fix it by closed forms, and fix the way the three uses fit together by
the property the construction exists for: attention logits and outputs that
depend on positions only through differences.
"""
import math

import numpy as np
import pytest

import synth
from oracle import attention as oa
from oracle import compressor as oc
from oracle import rope as orp


def test_closed_form_values():
    """Hand-computed rotations: pair 0 turns by pos radians; with R = 4 and
    base 100, pair 1 turns by pos / 10."""
    got = orp.rotate([1.0, 0.0], 1, R=2)
    assert np.allclose(got, [math.cos(1.0), math.sin(1.0)], rtol=0, atol=1e-15)
    got = orp.rotate([0.0, 0.0, 0.0, 1.0], 5, R=4, base=100.0)
    assert np.allclose(got, [0.0, 0.0, -math.sin(0.5), math.cos(0.5)], rtol=0, atol=1e-15)
    # only the last R dims move: a 6-d vector with R = 2
    got = orp.rotate([7.0, -3.0, 2.0, 5.0, 0.0, 2.0], 3, R=2)
    assert np.allclose(got, [7.0, -3.0, 2.0, 5.0, -2.0 * math.sin(3.0), 2.0 * math.cos(3.0)], atol=1e-15)
    # the inverse turns the other way
    got = orp.rotate([1.0, 0.0], 2, R=2, inverse=True)
    assert np.allclose(got, [math.cos(2.0), -math.sin(2.0)], atol=1e-15)


def test_frequencies_closed_form():
    f = orp.inv_freq(8, 10000.0)
    assert np.allclose(f, [1.0, 0.1, 0.01, 0.001], rtol=1e-14)


def test_pair_norms_kept_and_inverse():
    x = synth.normal("rope.x", (5, 3, 512)).astype(np.float64)
    pos = np.array([0, 1, 4095, 65535, 1048575])[:, None]
    y = orp.rotate(x, pos, 64)
    assert np.array_equal(y[..., :448], x[..., :448])
    n0 = x[..., 448:].reshape(5, 3, 32, 2)
    n1 = y[..., 448:].reshape(5, 3, 32, 2)
    assert np.allclose(np.hypot(n0[..., 0], n0[..., 1]), np.hypot(n1[..., 0], n1[..., 1]), rtol=1e-13)
    back = orp.rotate(y, pos, 64, inverse=True)
    assert np.allclose(back, x, rtol=0, atol=1e-12)
    # position 0 is the identity
    assert np.array_equal(orp.rotate(x, 0, 64), x)


def test_composition_and_relative_logits():
    """R(a) R(b) = R(a + b), and <R(m) q, R(n) k> depends on m - n only."""
    q = synth.normal("rope.q", (512,)).astype(np.float64)
    k = synth.normal("rope.k", (512,)).astype(np.float64)
    assert np.allclose(orp.rotate(orp.rotate(q, 300, 64), 77, 64), orp.rotate(q, 377, 64), atol=1e-12)
    for m, n in [(10, 3), (70000, 69993), (1048575, 1048568)]:
        lhs = orp.rotate(q, m, 64) @ orp.rotate(k, n, 64)
        rhs = orp.rotate(q, m - n, 64) @ k
        assert abs(lhs - rhs) < 1e-9 * (abs(rhs) + 1.0), (m, n)


def test_rotate_rows_positions():
    x = synth.normal("rope.rows", (2, 5, 3, 16)).astype(np.float64)
    y = orp.rotate_rows(x, 40, 8)
    for t in range(5):
        assert np.allclose(y[:, t], orp.rotate(x[:, t], 40 + t, 8), atol=1e-14)


def test_compressor_rope_at_anchor():
    """Entry s of a chunk gets RoPE at ratio * s + anchor after RMSNorm."""
    B, n_tok, c, pos0 = 1, 16, 128, 32
    inp = synth.compressor_inputs("rope.cmp", B, n_tok, c, 4, pos0)
    base = oc.compress(inp["Ca"], inp["Za"], inp["bias"], 4, inp["Cb"], inp["Zb"], inp["prev_Cb"],
                       inp["prev_Zb"], pos0=pos0)
    for anchor in (0, 3):
        got = oc.compress(inp["Ca"], inp["Za"], inp["bias"], 4, inp["Cb"], inp["Zb"], inp["prev_Cb"],
                          inp["prev_Zb"], pos0=pos0, rope_dims=64, rope_anchor=anchor)
        for i in range(n_tok // 4):
            exp = orp.rotate(base[0, i], 4 * (pos0 // 4 + i) + anchor, 64)
            assert np.allclose(got[0, i], exp, atol=1e-14)
    with pytest.raises(ValueError):
        orp.entry_position(3, 4, 4)


def test_single_row_output_is_the_unrotated_value():
    """A query that sees one row only (its own token, window 1): the softmax
    weight is 1, so the output is that row; rotated at the query's position
    and inverse-rotated at the same position, the value comes back exactly
    as it was before RoPE -- fixing the inverse's sign and position."""
    q = synth.normal("rope.q1", (1, 1, 4, 32)).astype(np.float64)
    v = synth.normal("rope.v1", (1, 1, 32)).astype(np.float64)
    pos = 1000
    vr = orp.rotate(v, pos, 16)
    qr = orp.rotate(q, pos, 16)
    idx = np.full((1, 1, 4), -1)
    o, _ = oa.sparse_mqa(qr, np.zeros((1, 1, 32)), idx, vr, pos, pos, window=1, rope_dims=16)
    assert np.allclose(o[0, 0], np.broadcast_to(v[0, 0], (4, 32)), atol=1e-12)
    o2, _ = oa.dense_attention(qr, np.zeros((1, 0, 32)), vr, pos, pos, 4, window=1, rope_dims=16)
    assert np.allclose(o2[0, 0], np.broadcast_to(v[0, 0], (4, 32)), atol=1e-12)


@pytest.mark.parametrize("ratio", [4, 128])
def test_layer_output_is_shift_invariant(ratio):
    """The whole layer with RoPE -- q at its position, window rows at theirs,
    compressed entries at their anchors, inverse RoPE on the output -- gives
    the same output when every position moves by a multiple of the ratio:
    the construction leaves only position differences.  A wrong sign, pair
    layout or position in any of the three uses breaks this."""
    c, H, T, n_blk, window = 64, 4, 3, 6, 8
    n_tok = n_blk * ratio
    inp = synth.compressor_inputs(f"rope.layer{ratio}", 1, n_tok, c, ratio, 0)
    raw = synth.normal(f"rope.raw{ratio}", (1, n_tok + T, c)).astype(np.float64)
    q = synth.normal(f"rope.lq{ratio}", (1, T, H, c)).astype(np.float64)
    outs = []
    for shift in (0, 5 * ratio, 1 << 16):
        pos0 = shift                      # the chunk of raw tokens starts here
        kw = dict(rope_dims=32, rope_anchor=ratio - 1)
        if ratio == 4:
            # a block before the chunk with no weight: the same pooling as block 0
            pz = np.full((1, 4, c), -np.inf) if pos0 else None
            pc = np.zeros((1, 4, c)) if pos0 else None
            ent = oc.compress(inp["Ca"], inp["Za"], inp["bias"], 4, inp["Cb"], inp["Zb"], pc, pz,
                              pos0=pos0, **kw)
        else:
            ent = oc.compress(inp["Ca"], inp["Za"], inp["bias"], 128, pos0=pos0, **kw)
        q_pos0 = pos0 + n_tok
        kv_raw = orp.rotate_rows(raw, pos0, 32)
        qr = orp.rotate_rows(q, q_pos0, 32)
        # the cache holds this chunk's entries at their absolute indices; the
        # queries select exactly those
        N = (pos0 + n_tok) // ratio
        cache = np.zeros((1, N, c))
        cache[0, pos0 // ratio:] = ent[0]
        idx = np.broadcast_to(np.arange(pos0 // ratio, N), (1, T, n_blk))
        o, _ = oa.sparse_mqa(qr, cache, idx, kv_raw, pos0, q_pos0, window, rope_dims=32)
        outs.append(o)
    for o in outs[1:]:
        assert np.allclose(o, outs[0], rtol=0, atol=1e-10)
    # and without the inverse RoPE the outputs do move with the shift
    assert not np.allclose(orp.rotate_rows(outs[0], n_tok, 32), orp.rotate_rows(outs[1], 5 * ratio + n_tok, 32))


def test_dense_with_rope_equals_sparse_with_all_entries():
    """The dense (HCA) oracle applies the same inverse RoPE as the sparse one."""
    B, T, N, H, d, q_pos0, window = 1, 5, 12, 4, 32, 40, 8
    q = synth.normal("rope.dq", (B, T, H, d)).astype(np.float64)
    kv = synth.normal("rope.dkv", (B, N, d)).astype(np.float64)
    rp0 = q_pos0 - window + 1
    raw = synth.normal("rope.draw", (B, q_pos0 + T - rp0, d)).astype(np.float64)
    idx = np.full((B, T, N), -1)
    for t in range(T):
        v = (q_pos0 + t + 1) // 4
        idx[:, t, :v] = np.arange(v)
    o1, l1 = oa.sparse_mqa(q, kv, idx, raw, rp0, q_pos0, window, rope_dims=16, rope_base=500.0)
    o2, l2 = oa.dense_attention(q, kv, raw, rp0, q_pos0, 4, window, rope_dims=16, rope_base=500.0)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12)
    assert np.allclose(l1, l2, rtol=1e-12, atol=1e-12)
    o0, _ = oa.sparse_mqa(q, kv, idx, raw, rp0, q_pos0, window)
    assert np.array_equal(o1[..., :16], o0[..., :16])
    assert not np.allclose(o1[..., 16:], o0[..., 16:])
