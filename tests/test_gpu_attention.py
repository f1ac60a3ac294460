"""GPU parity of sparse_mqa_attn (stage 4) and hca_attn (stage 5) against the
oracle, through the C ABI.

Pages: "DeepSeek V4 结构速览" (CSA and HCA sections); "DeepSeek-V4 技术解读：百万
Token 上下文的新里程碑" (2.1).  Tolerances: bf16 I/O 2e-2 max-abs (stated for the
workloads) plus a normwise-relative guard of 1e-2 so that an all-zero output
cannot pass; fp32 I/O 1e-4 max-abs.  Large caches are drawn on the device from
seeded generators; the oracle reads the same bytes (the rows it needs are
copied back).
"""
import numpy as np
import pytest
import torch

import long_context_sparse_compress_amd as csa
import synth
from oracle import attention as oa
from helpers import (ATTN_BF16_MAX_ABS, ATTN_F32_MAX_ABS, ATTN_NORMWISE, dev, host, max_abs,
                     normwise_rel)

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _visible(q_pos0, T, ratio, N):
    return [min((q_pos0 + t + 1) // ratio, N) for t in range(T)]


def _sparse_ref(q, kv, idx, raw, raw_pos0, q_pos0, b, t, window=128, lse=False):
    """Oracle for one (b, t): compact the selected rows, keep the bytes."""
    sel = idx[b, t]
    valid = sel[sel >= 0]
    kv_rows = host(kv[b, torch.as_tensor(valid, device=kv.device, dtype=torch.long)]) if len(valid) else \
        np.zeros((0, 512), np.float32)
    pos = q_pos0 + t
    w0 = max(0, pos - window + 1)
    rw = host(raw[b, w0 - raw_pos0:pos - raw_pos0 + 1])
    qq = host(q[b, t])[None, None]
    cidx = np.arange(len(valid))[None, None]
    o, l = oa.sparse_mqa(qq, kv_rows[None], cidx, rw[None], w0, pos, window)
    return (o[0, 0], l[0, 0]) if lse else o[0, 0]


def _dense_ref(q, kv, raw, raw_pos0, q_pos0, b, t, ratio, sink, window=128):
    pos = q_pos0 + t
    V = (pos + 1) // ratio
    w0 = max(0, pos - window + 1)
    rw = host(raw[b, w0 - raw_pos0:pos - raw_pos0 + 1])
    kvh = host(kv[b, :V])
    qq = host(q[b, t])[None, None]
    o, l = oa.dense_attention(qq, kvh[None], rw[None], w0, pos, ratio, window,
                              sink=None if sink is None else host(sink))
    return o[0, 0], l[0, 0]


def _assert_bf16(got, ref):
    assert max_abs(got, ref) < ATTN_BF16_MAX_ABS
    assert normwise_rel(got, ref) < ATTN_NORMWISE


def _sparse_case(name, B, T, N, k, q_pos0, dtype=BF, window=128):
    raw_pos0 = max(0, q_pos0 - window + 1)
    n_raw = q_pos0 + T - raw_pos0
    q = synth.device_normal(name + ".q", (B, T, 64, 512), dtype)
    kv = synth.device_normal(name + ".kv", (B, N, 512), dtype)
    raw = synth.device_normal(name + ".raw", (B, n_raw, 512), dtype)
    idx = synth.random_topk_indices(name + ".idx", B, T, k, _visible(q_pos0, T, 4, N))
    return q, kv, raw, idx, raw_pos0


def test_tiny_prefill_fp32():
    """256 queries, 64 entries, k = 16, fp32 I/O: every row checked."""
    q, kv, raw, idx, rp0 = _sparse_case("at.tiny", 1, 256, 64, 16, 0, torch.float32)
    out = csa.sparse_mqa_attn(q, kv, dev(idx, torch.int32), raw, q_pos0=0, raw_pos0=rp0)
    torch.cuda.synchronize()
    ref, _ = oa.sparse_mqa(host(q), host(kv), idx, host(raw), rp0, 0, 128)
    assert max_abs(host(out), ref) < ATTN_F32_MAX_ABS


def test_csa_decode_bf16():
    """Batch 32 at 65,536 context: 512 of 16,384 entries + 128 window rows."""
    B, N, k, q0 = 32, 16384, 512, 65535
    q, kv, raw, idx, rp0 = _sparse_case("at.dec", B, 1, N, k, q0)
    out, lse = csa.sparse_mqa_attn(q, kv, dev(idx, torch.int32), raw, q_pos0=q0, raw_pos0=rp0,
                                   return_lse=True)
    torch.cuda.synchronize()
    got, gl = host(out), host(lse)
    for b in range(B):
        r, rl = _sparse_ref(q, kv, idx, raw, rp0, q0, b, 0, lse=True)
        _assert_bf16(got[b, 0], r)
        assert max_abs(gl[b, 0], rl) < 1e-3


def test_csa_prefill_bf16_sampled():
    """4,096 queries at 131,072 context (33,792 entries, k = 512); sampled rows."""
    T, N, k, q0 = 4096, 33792, 512, 131072
    q, kv, raw, idx, rp0 = _sparse_case("at.pf", 1, T, N, k, q0)
    out = csa.sparse_mqa_attn(q, kv, dev(idx, torch.int32), raw, q_pos0=q0, raw_pos0=rp0)
    torch.cuda.synchronize()
    got = host(out)
    for t in [0, 1, 127, 128, 2047, 4094, 4095]:
        _assert_bf16(got[0, t], _sparse_ref(q, kv, idx, raw, rp0, q0, 0, t))


def test_csa_1m_decode_bf16():
    """Batch 8 at 1M context: 1,024 of 262,144 entries + 128 window rows."""
    B, N, k, q0 = 8, 262144, 1024, 1048575
    q, kv, raw, idx, rp0 = _sparse_case("at.1m", B, 1, N, k, q0)
    out = csa.sparse_mqa_attn(q, kv, dev(idx, torch.int32), raw, q_pos0=q0, raw_pos0=rp0)
    torch.cuda.synchronize()
    got = host(out)
    for b in range(B):
        _assert_bf16(got[b, 0], _sparse_ref(q, kv, idx, raw, rp0, q0, b, 0))


def _hca_case(name, B, T, N, q_pos0, window=128, dtype=BF):
    raw_pos0 = max(0, q_pos0 - window + 1)
    n_raw = q_pos0 + T - raw_pos0
    q = synth.device_normal(name + ".q", (B, T, 64, 512), dtype)
    kv = synth.device_normal(name + ".kv", (B, N, 512), dtype)
    raw = synth.device_normal(name + ".raw", (B, n_raw, 512), dtype)
    sink = synth.device_normal(name + ".sink", (64,))
    return q, kv, raw, sink, raw_pos0


def test_hca_decode_bf16():
    """Batch 16 at 1,048,576 context: 8,192 C128A entries + 128 window rows, sink."""
    B, N, q0 = 16, 8192, 1048575
    q, kv, raw, sink, rp0 = _hca_case("at.hdec", B, 1, N, q0)
    out, lse = csa.hca_attn(q, kv, raw, q_pos0=q0, raw_pos0=rp0, sink=sink, return_lse=True)
    torch.cuda.synchronize()
    got, gl = host(out), host(lse)
    for b in [0, 7, 15]:
        r, rl = _dense_ref(q, kv, raw, rp0, q0, b, 0, 128, sink)
        _assert_bf16(got[b, 0], r)
        assert max_abs(gl[b, 0], rl) < 1e-3


def test_hca_prefill_bf16_sampled():
    """The last 2,048 tokens of a 1,048,576 context (V runs 8,176 -> 8,192), sink."""
    T, N, q0 = 2048, 8192, 1046528
    q, kv, raw, sink, rp0 = _hca_case("at.hpf", 1, T, N, q0)
    out = csa.hca_attn(q, kv, raw, q_pos0=q0, raw_pos0=rp0, sink=sink)
    torch.cuda.synchronize()
    got = host(out)
    for t in [0, 126, 127, 1000, 2047]:
        r, _ = _dense_ref(q, kv, raw, rp0, q0, 0, t, 128, sink)
        _assert_bf16(got[0, t], r)


def test_sparse_with_all_entries_equals_dense():
    """k >= visible entries: sparse attention equals the dense form (ratio 4, no
    sink), on the GPU and against the oracle."""
    B, T, N, q0 = 2, 9, 40, 150
    q, kv, raw, _, rp0 = _hca_case("at.eq", B, T, N, q0)
    vis = _visible(q0, T, 4, N)
    idx = np.full((B, T, 48), -1, np.int32)
    for t in range(T):
        idx[:, t, :vis[t]] = np.arange(vis[t])
    a = csa.sparse_mqa_attn(q, kv, dev(idx, torch.int32), raw, q_pos0=q0, raw_pos0=rp0)
    d = csa.hca_attn(q, kv, raw, q_pos0=q0, raw_pos0=rp0, ratio=4, sink=None)
    torch.cuda.synchronize()
    # the two lists tile differently (padding slots), so rounding differs; the
    # outputs agree to the bf16 attention tolerance
    _assert_bf16(host(a), host(d))
    for t in range(T):
        r, _ = _dense_ref(q, kv, raw, rp0, q0, 1, t, 4, None)
        _assert_bf16(host(d)[1, t], r)


def test_planted_needle():
    """A cache row aligned with every head's query dominates: |o| = O(1), so the
    2e-2 bound is meaningful."""
    B, N, k, q0 = 4, 4096, 512, 4 * 4096 - 1
    q, kv, raw, idx, rp0 = _sparse_case("at.needle", B, 1, N, k, q0)
    qm = q[:, 0].float().mean(dim=1)                    # [B, 512]
    needle = (qm / qm.norm(dim=1, keepdim=True) * 60.0).to(BF)
    for b in range(B):
        kv[b, int(idx[b, 0, 7])] = needle[b]
    out = csa.sparse_mqa_attn(q, kv, dev(idx, torch.int32), raw, q_pos0=q0, raw_pos0=rp0)
    torch.cuda.synchronize()
    got = host(out)
    for b in range(B):
        r = _sparse_ref(q, kv, idx, raw, rp0, q0, b, 0)
        big = np.abs(r).max()
        assert big > 1.0
        # bf16 output rounding alone is ~2^-9 |o|: the 2e-2 bound scales with |o|
        assert max_abs(got[b, 0], r) < ATTN_BF16_MAX_ABS * max(1.0, big)
        assert normwise_rel(got[b, 0], r) < ATTN_NORMWISE


@pytest.mark.parametrize("q0,T,N,k,window", [
    (0, 3, 1, 4, 128),       # first tokens: window only, all slots padding
    (37, 7, 12, 8, 16),      # short window, ragged T, partly padded slots
    (5000, 5, 1300, 300, 128),
])
def test_edge_cases_bf16(q0, T, N, k, window):
    q, kv, raw, idx, rp0 = _sparse_case(f"at.edge{q0}", 2, T, N, k, q0, window=window)
    out = csa.sparse_mqa_attn(q, kv, dev(idx, torch.int32), raw, q_pos0=q0, raw_pos0=rp0, window=window)
    torch.cuda.synchronize()
    got = host(out)
    for b in range(2):
        for t in range(T):
            _assert_bf16(got[b, t], _sparse_ref(q, kv, idx, raw, rp0, q0, b, t, window=window))
    if q0 == 0:   # t = 0 attends to its own raw row only
        assert np.array_equal(got[:, 0], np.broadcast_to(host(raw)[:, 0][:, None, :], got[:, 0].shape))


def test_fp32_dense_with_sink():
    q, kv, raw, sink, rp0 = _hca_case("at.f32h", 1, 5, 6, 700, dtype=torch.float32)
    out, lse = csa.hca_attn(q, kv, raw, q_pos0=700, raw_pos0=rp0, sink=sink, return_lse=True)
    torch.cuda.synchronize()
    ref, rl = oa.hca_attention(host(q), host(kv), host(raw), rp0, 700, host(sink), ratio=128)
    assert max_abs(host(out), ref) < ATTN_F32_MAX_ABS
    assert max_abs(host(lse), rl) < 1e-4


def test_causality_prefill():
    """Changing raw rows after position p leaves the outputs of queries <= p bit-identical."""
    T, N, q0 = 64, 400, 1000
    q, kv, raw, sink, rp0 = _hca_case("at.caus", 1, T, N, q0)
    a = csa.hca_attn(q, kv, raw, q_pos0=q0, raw_pos0=rp0, ratio=4, sink=sink).clone()
    raw2 = raw.clone()
    raw2[:, (q0 + 32) - rp0:] += 3.0
    b = csa.hca_attn(q, kv, raw2, q_pos0=q0, raw_pos0=rp0, ratio=4, sink=sink)
    torch.cuda.synchronize()
    assert torch.equal(a[:, :32], b[:, :32])
    assert not torch.equal(a[:, 32:], b[:, 32:])


def test_deterministic_split_decode():
    q, kv, raw, sink, rp0 = _hca_case("at.det", 4, 1, 8192, 1048575)
    a = csa.hca_attn(q, kv, raw, q_pos0=1048575, raw_pos0=rp0, sink=sink).clone()
    b = csa.hca_attn(q, kv, raw, q_pos0=1048575, raw_pos0=rp0, sink=sink)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_batch_invariant_csa_decode_bits():
    """Batch-invariant mode ("DeepSeek-V4 技术解读：百万 Token 上下文的新里程碑",
    3.3): a decode query gives the same bits alone, in a small batch (one
    workgroup per head block) and in a batch of 300 (one workgroup per query),
    and matches the oracle."""
    B, N, k, q0 = 300, 2048, 512, 8191
    q, kv, raw, idx, rp0 = _sparse_case("at.bi", B, 1, N, k, q0)
    di = dev(idx, torch.int32)
    big, lse = csa.sparse_mqa_attn(q, kv, di, raw, q_pos0=q0, raw_pos0=rp0, batch_invariant=True,
                                   return_lse=True)
    for pick in ([0, 77, 299], [150]):
        s = torch.as_tensor(pick, device="cuda")
        small, sl = csa.sparse_mqa_attn(q[s].contiguous(), kv[s].contiguous(), di[s].contiguous(),
                                        raw[s].contiguous(), q_pos0=q0, raw_pos0=rp0,
                                        batch_invariant=True, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(small, big[s]), pick
        assert torch.equal(sl, lse[s]), pick
    got = host(big)
    for b in [0, 150, 299]:
        _assert_bf16(got[b, 0], _sparse_ref(q, kv, idx, raw, rp0, q0, b, 0))


def test_batch_invariant_prefill_query_equals_decode():
    """A query of a 512-token prefill chunk and the same query decoded alone
    give the same bits in batch-invariant mode (CSA, and HCA with sink)."""
    T, N, k, q0 = 512, 4096, 512, 16384
    q, kv, raw, idx, rp0 = _sparse_case("at.bip", 1, T, N, k, q0)
    di = dev(idx, torch.int32)
    chunk = csa.sparse_mqa_attn(q, kv, di, raw, q_pos0=q0, raw_pos0=rp0, batch_invariant=True)
    Nh = (q0 + T) // 128
    hq, hkv, hraw, sink, hrp0 = _hca_case("at.bih", 1, T, Nh, q0)
    hchunk = csa.hca_attn(hq, hkv, hraw, q_pos0=q0, raw_pos0=hrp0, sink=sink, batch_invariant=True)
    for t in [0, 1, 127, 300, 511]:
        one = csa.sparse_mqa_attn(q[:, t:t + 1].contiguous(), kv, di[:, t:t + 1].contiguous(), raw,
                                  q_pos0=q0 + t, raw_pos0=rp0, batch_invariant=True)
        hone = csa.hca_attn(hq[:, t:t + 1].contiguous(), hkv, hraw, q_pos0=q0 + t, raw_pos0=hrp0,
                            sink=sink, batch_invariant=True)
        torch.cuda.synchronize()
        assert torch.equal(one[:, 0], chunk[:, t]), t
        assert torch.equal(hone[:, 0], hchunk[:, t]), t
    got, hgot = host(chunk), host(hchunk)
    for t in [0, 511]:
        _assert_bf16(got[0, t], _sparse_ref(q, kv, idx, raw, rp0, q0, 0, t))
        r, _ = _dense_ref(hq, hkv, hraw, hrp0, q0, 0, t, 128, sink)
        _assert_bf16(hgot[0, t], r)


def test_batch_invariant_hca_decode_matches_oracle():
    """HCA decode with sink in batch-invariant mode: a batch of 16 at 1M
    context (one workgroup per head block) against the oracle."""
    B, N, q0 = 16, 8192, 1048575
    q, kv, raw, sink, rp0 = _hca_case("at.hdec", B, 1, N, q0)
    out, lse = csa.hca_attn(q, kv, raw, q_pos0=q0, raw_pos0=rp0, sink=sink, return_lse=True,
                            batch_invariant=True)
    torch.cuda.synchronize()
    got, gl = host(out), host(lse)
    for b in [0, 15]:
        r, rl = _dense_ref(q, kv, raw, rp0, q0, b, 0, 128, sink)
        _assert_bf16(got[b, 0], r)
        assert max_abs(gl[b, 0], rl) < 1e-3


def _scramble(idx, N, name, dup=True, far=False):
    """Any slot order, -1 anywhere, repeated entries and (far) ids >= N: the
    forms include/csa.h allows for idx.  Returns (scrambled, the same with ids
    >= N written as -1)."""
    g = synth.rng(name)
    out = idx.copy()
    B, T, k = out.shape
    for b in range(B):
        for t in range(T):
            row = out[b, t]
            valid = row[row >= 0]
            n = len(valid)
            slots = g.permutation(k)
            new = np.full(k, -1, dtype=np.int32)
            new[slots[:n]] = valid                      # shuffled, -1 in between
            if dup and n >= 4:
                free = slots[n:]
                for j in range(min(3, len(free))):      # a few entries twice
                    new[free[j]] = valid[g.integers(n)]
            if n >= 2:
                new[slots[0]] = -1                      # a hole where an entry was
            if far and k - n > 4:
                new[slots[-1]] = N + int(g.integers(1000))
                new[slots[-2]] = 2 ** 30
            out[b, t] = new
    as_pad = np.where(out >= N, -1, out).astype(np.int32)
    return out.astype(np.int32), as_pad


@pytest.mark.parametrize("B,T,N,k,q0", [
    (32, 1, 16384, 512, 65535),      # split decode + combine
    (2, 40, 4096, 512, 16383 - 39),  # one workgroup per query (prefill shape)
    (3, 1, 300, 512, 1199),          # fewer entries than k: most slots empty
])
def test_sparse_idx_any_order_padding_duplicates(B, T, N, k, q0):
    name = f"at.scr.{B}.{T}.{N}"
    q, kv, raw, idx, rp0 = _sparse_case(name, B, T, N, k, q0)
    scr, pad = _scramble(idx, N, name + ".s", far=True)
    out = csa.sparse_mqa_attn(q, kv, dev(scr, torch.int32), raw, q_pos0=q0, raw_pos0=rp0)
    out_pad = csa.sparse_mqa_attn(q, kv, dev(pad, torch.int32), raw, q_pos0=q0, raw_pos0=rp0)
    torch.cuda.synchronize()
    got, got_pad = host(out), host(out_pad)
    # ids >= N are padding exactly as -1 is
    assert np.array_equal(got, got_pad)
    for b in range(B):
        for t in sorted({0, T // 2, T - 1}):
            _assert_bf16(got[b, t], _sparse_ref(q, kv, pad, raw, rp0, q0, b, t))


def test_sparse_idx_whole_tiles_of_padding():
    """Slot runs of 32 and 64 -1s (whole row tiles) between valid slots, split decode."""
    B, N, k, q0 = 16, 16384, 512, 65535
    q, kv, raw, idx, rp0 = _sparse_case("at.holes", B, 1, N, k, q0)
    g = synth.rng("at.holes.s")
    scr = np.full_like(idx, -1)
    for b in range(B):
        valid = idx[b, 0][idx[b, 0] >= 0][:320]
        pos = np.concatenate([np.arange(0, 32), np.arange(96, 192), np.arange(256, 448)])   # 320 slots
        scr[b, 0, pos] = g.permutation(valid)
    out = csa.sparse_mqa_attn(q, kv, dev(scr, torch.int32), raw, q_pos0=q0, raw_pos0=rp0)
    torch.cuda.synchronize()
    got = host(out)
    for b in range(B):
        _assert_bf16(got[b, 0], _sparse_ref(q, kv, scr, raw, rp0, q0, b, 0))


@pytest.mark.parametrize("T,bi", [(1, False), (1, True), (40, False)])
def test_growing_logits_force_rescales(T, bi):
    """Rows whose logits climb from tile to tile by steps both below and above
    the kernel's rescale threshold (a factor 2^8), so the running reference
    maximum both stays put and moves after O has accumulated: split decode,
    batch-invariant and a multi-query chunk against the oracle."""
    B, N, k = 2, 2048, 640
    q0 = 4 * N - T
    q, kv, raw, idx, rp0 = _sparse_case(f"at.grow{T}{bi}", B, T, N, k, q0)
    rng = np.random.default_rng(7)
    u = q[:, :, :].float().mean(dim=(1, 2))                       # [B, 512]
    u = u / u.norm(dim=1, keepdim=True)
    for b in range(B):
        # entry order of query 0's list: tile i (32 slots) gets rows along u
        # with a per-tile level climbing by 0 to ~14 log2 units a tile
        sel = idx[b, 0]
        level = np.cumsum(rng.uniform(0.0, 80.0, size=k // 32))
        lv = np.repeat(level, 32) + rng.normal(0.0, 4.0, size=k)
        rows = torch.as_tensor(lv, dtype=torch.float32, device=kv.device)[:, None] * u[b][None, :]
        for p in range(k):
            if sel[p] >= 0:
                kv[b, int(sel[p])] = (rows[p] + 0.1 * kv[b, int(sel[p])].float()).to(BF)
    out = csa.sparse_mqa_attn(q, kv, dev(idx, torch.int32), raw, q_pos0=q0, raw_pos0=rp0,
                              batch_invariant=bi)
    torch.cuda.synchronize()
    got = host(out)
    for b in range(B):
        for t in sorted({0, T // 2, T - 1}):
            r = _sparse_ref(q, kv, idx, raw, rp0, q0, b, t)
            big = np.abs(r).max()
            assert max_abs(got[b, t], r) < ATTN_BF16_MAX_ABS * max(1.0, big)
            assert normwise_rel(got[b, t], r) < ATTN_NORMWISE


@pytest.mark.parametrize("T", [1, 3])
def test_growing_logits_force_rescales_dense(T):
    """Dense HCA rows (with sink) whose logits climb from tile to tile by steps
    on both sides of the rescale threshold: the two-tile-group split decode
    (T = 1, 8,320 rows) and a short chunk, against the oracle."""
    B, N = 2, 8192
    q0 = 128 * N - T
    q, kv, raw, sink, rp0 = _hca_case(f"at.hgrow{T}", B, T, N, q0)
    rng = np.random.default_rng(11)
    u = q.float().mean(dim=(1, 2))
    u = u / u.norm(dim=1, keepdim=True)
    level = np.repeat(np.cumsum(rng.uniform(0.0, 80.0, size=N // 32)), 32) + rng.normal(0.0, 4.0, size=N)
    lv = torch.as_tensor(level, dtype=torch.float32, device=kv.device)
    for b in range(B):
        kv[b] = (lv[:, None] * u[b][None, :] + 0.1 * kv[b].float()).to(BF)
    out = csa.hca_attn(q, kv, raw, q_pos0=q0, raw_pos0=rp0, sink=sink)
    torch.cuda.synchronize()
    got = host(out)
    for b in range(B):
        for t in sorted({0, T - 1}):
            r, _ = _dense_ref(q, kv, raw, rp0, q0, b, t, 128, sink)
            big = np.abs(r).max()
            assert max_abs(got[b, t], r) < ATTN_BF16_MAX_ABS * max(1.0, big)
            assert normwise_rel(got[b, t], r) < ATTN_NORMWISE
