"""GPU parity of the hierarchical sparse indexer (lightning_index_pool,
topk_select_pool) against the oracle, through the C ABI.

Page: "DeepSeek Technical Reports" (DeepSeek-V4.1, CSA2: a full indexer pass yields a candidate
pool; Reindex layers re-score only the pool with their own query).
Tolerances as for lightning_index: fp32 scores 1e-3 relative (plus a floor of
1e-5 of the row's largest score), bf16 scores within one bf16 ulp of the
oracle's score rounded to bf16; Top-k inside the pool reads the same score
tensor on both sides and must give identical entries.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_compress_amd as csa
import synth
from oracle import indexer as oi
from oracle import numerics as on
from oracle import topk as ot
from helpers import dev, host, index_close

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _bf16_close(got, ref64):
    ref = on.store_bf16(ref64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin)
    assert np.all(got[~fin] == -np.inf)
    a = np.maximum(np.abs(ref[fin]), 2.0 ** -126)
    ulp = np.exp2(np.floor(np.log2(a)) - 7)
    assert np.all(np.abs(got[fin] - ref[fin]) <= ulp * 1.0001)


def _layer(prefix, B, T, N):
    q = synth.round_bf16(synth.normal(prefix + ".q", (B, T, 64, 128), var=1.0 / 128))
    w = synth.uniform(prefix + ".w", (B, T, 64))
    k = synth.round_bf16(synth.normal(prefix + ".k", (B, N, 128)))
    return q, w, k


def _vis(q_pos0, T, N):
    return [min((q_pos0 + t + 1) // 4, N) for t in range(T)]


def _scores(q, w, k, pool, score_dtype):
    s = csa.lightning_index_pool(dev(q, BF), dev(w), dev(k, BF), dev(pool, torch.int32), score_dtype=score_dtype)
    torch.cuda.synchronize()
    return s


def test_tiny_pool_fp32_all_rows():
    B, T, N, q0, P = 2, 3, 300, 1000, 200
    q, w, k = _layer("pl.tiny", B, T, N)
    pool = synth.random_topk_indices("pl.tiny.pool", B, T, P, _vis(q0, T, N))
    got = host(_scores(q, w, k, pool, torch.float32))
    index_close(got, oi.pool_scores(q, w, k, pool))


@pytest.mark.parametrize("P", [37, 64, 300])
def test_empty_and_out_of_range_slots(P):
    """Ragged pools with -1 slots, ids past N and a row with no entry at all:
    those slots score -inf and read no key."""
    B, T, N = 2, 2, 64
    q, w, k = _layer(f"pl.edge{P}", B, T, N)
    pool = np.full((B, T, P), -1, dtype=np.int32)
    pool[0, 0, :min(P, 30)] = np.arange(min(P, 30)) * 2
    pool[0, 1, :3] = [5, N, N + 1000]          # two slots past the cache
    pool[1, 0, ::2] = np.arange((P + 1) // 2) % N
    # pool[1, 1] stays empty
    for sd in (torch.float32, BF):
        got = host(_scores(q, w, k, pool, sd))
        ref = oi.pool_scores(q, w, k, pool)
        if sd == torch.float32:
            index_close(got, ref)
        else:
            _bf16_close(got, ref)
    assert np.all(np.isneginf(got[1, 1]))


def _full_then_pool(prefix, B, T, N, q0, P):
    """The Full layer on the GPU: lightning_index over every key, topk_select
    with k = P -> the pool (ascending ids, then -1)."""
    q, w, k = _layer(prefix + ".full", B, T, N)
    s = csa.lightning_index(dev(q, BF), dev(w), dev(k, BF), q_pos0=q0, ratio=4, score_dtype=BF)
    pool = csa.topk_select(s, P, q_pos0=q0, ratio=4)
    torch.cuda.synchronize()
    return k, pool


def test_decode_reindex_layer_bf16():
    """Batch 32 at 65,536 context: a Full layer picks a 2,048-entry pool from
    16,384 keys, a Reindex layer (its own q and w) scores the pool and takes
    its top 512 inside it."""
    B, T, N, q0, P, K = 32, 1, 16384, 65535, 2048, 512
    k, pool = _full_then_pool("pl.dec", B, T, N, q0, P)
    q2, w2, _ = _layer("pl.dec.re", B, T, 1)
    s = csa.lightning_index_pool(dev(q2, BF), dev(w2), dev(k, BF), pool, score_dtype=BF)
    idx = csa.topk_select_pool(s, pool, K, N=N)
    torch.cuda.synchronize()
    hp, hs, hi = host(pool).astype(np.int64), host(s), host(idx)
    _bf16_close(hs, oi.pool_scores(q2, w2, k, hp))
    ref = ot.pool_select(hs, hp, K, N=N)
    assert np.array_equal(hi, _ascending(ref))      # ascending entry ids (the pool is ascending)


def test_prefill_reindex_sampled_rows():
    """A 4,096-token chunk after 131,072 tokens (33,792 entries), pools of
    2,048: scores on sampled rows against the oracle, Top-k on every row."""
    B, T, N, q0, P, K = 1, 4096, 33792, 131072, 2048, 512
    q, w, k = _layer("pl.pf", B, T, N)
    pool = synth.random_topk_indices("pl.pf.pool", B, T, P, _vis(q0, T, N))
    dpool = dev(pool, torch.int32)
    s = csa.lightning_index_pool(dev(q, BF), dev(w), dev(k, BF), dpool, score_dtype=torch.float32)
    idx = csa.topk_select_pool(s, dpool, K, N=N)
    torch.cuda.synchronize()
    hs, hi = host(s), host(idx)
    rows = [0, 1, 255, 2048, 4094, 4095]
    index_close(hs[:, rows], oi.pool_scores(q[:, rows], w[:, rows], k, pool[:, rows]))
    assert np.array_equal(hi, _ascending(ot.pool_select(hs, pool, K, N=N)))


@pytest.mark.parametrize("P,score,K", [
    (2048, "bf16", 512),   # register selection
    (2048, "f32", 512),    # LDS selection
    (37, "bf16", 16),      # a row length that is not a multiple of 8: LDS selection
    (100, "bf16", 512),    # fewer slots than k: every entry, then -1
    (16384, "bf16", 2048), # the largest pool
])
def test_topk_select_pool_matches_oracle(P, score, K):
    """The same score tensor on both sides; pools with empty slots and ids
    past N at their end (ascending ids, then the empty slots)."""
    B, T, N = 3, 2, 40000
    g = np.random.default_rng(P)
    pool = np.full((B, T, P), -1, dtype=np.int32)
    scores = np.full((B, T, P), -np.inf, dtype=np.float32)
    for b in range(B):
        for t in range(T):
            n = P - (b * 7 + t * 3) % max(1, P // 4)        # some rows end in empty slots
            ids = np.sort(g.choice(N, size=n, replace=False)).astype(np.int32)
            if b == 2 and t == 1 and n > 2:
                ids[-2:] = [N, N + 9]                       # past the cache: empty slots
            pool[b, t, :n] = ids
            # coarse scores: many ties, broken by the lower entry id
            scores[b, t, :n] = np.round(g.random(n) * 64) / 64
            scores[b, t, :n][ids >= N] = -np.inf
    tdt = BF if score == "bf16" else torch.float32
    ds = dev(scores, tdt)
    idx = csa.topk_select_pool(ds, dev(pool, torch.int32), K, N=N)
    torch.cuda.synchronize()
    ref = ot.pool_select(host(ds), pool, K, N=N)
    assert np.array_equal(host(idx), _ascending(ref))


def _ascending(ref):
    """Oracle rank order -> the GPU's layout: ascending ids, then -1."""
    out = np.full_like(ref, -1)
    for idx in np.ndindex(ref.shape[:-1]):
        v = np.sort(ref[idx][ref[idx] >= 0])
        out[idx][:len(v)] = v
    return out


def test_pool_of_every_visible_entry_matches_the_full_indexer():
    """A pool listing every visible entry: the same scores as lightning_index
    (up to summation order) and the same selection as topk_select."""
    B, T, N, q0, K = 4, 3, 4096, 16380, 256
    q, w, k = _layer("pl.eq", B, T, N)
    vis = _vis(q0, T, N)
    pool = np.full((B, T, N), -1, dtype=np.int32)
    for t in range(T):
        pool[:, t, :vis[t]] = np.arange(vis[t])
    dq, dw, dk = dev(q, BF), dev(w), dev(k, BF)
    full = csa.lightning_index(dq, dw, dk, q_pos0=q0, ratio=4, score_dtype=torch.float32)
    ps = csa.lightning_index_pool(dq, dw, dk, dev(pool, torch.int32), score_dtype=torch.float32)
    torch.cuda.synchronize()
    index_close(host(ps), host(full))
    # selection on the full path's own scores, viewed as a pool
    idx_full = csa.topk_select(full, K, q_pos0=q0, ratio=4)
    idx_pool = csa.topk_select_pool(full, dev(pool, torch.int32), K, N=N)
    torch.cuda.synchronize()
    assert torch.equal(idx_full, idx_pool)


def test_long_runs_with_a_ragged_pool():
    """Enough queries for the long-run kernel (eight chunks of 64 slots per
    wave) with a pool of 300 slots: the last chunks are partly or wholly past
    the pool, and some rows end in empty slots."""
    B, T, N, q0, P = 1, 1100, 400, 5000, 300
    q, w, k = _layer("pl.long", B, T, N)
    pool = synth.random_topk_indices("pl.long.pool", B, T, P, [min(N, 250 + t % 200) for t in range(T)])
    got = host(_scores(q, w, k, pool, torch.float32))
    rows = [0, 1, 63, 64, 500, 1099]
    index_close(got[:, rows], oi.pool_scores(q[:, rows], w[:, rows], k, pool[:, rows]))


# ---------------------------------------------------------------- low-precision pools
# "DeepSeek V4 结构速览" (Lightning Indexer: the QK path runs in low precision,
# FP4 in the Pro model): a Reindex layer scores its pool from the same key
# cache the Full layer read, so it takes the cache's precision.  The oracle
# scores the decoded q and keys (the quantization is the input's, not the
# method's); tolerances as for the full indexer.


def _quant_layer(prefix, B, T, N, fmt):
    """q, k drawn N(0, 1) then encoded; returns device tensors and the decoded
    fp64 copies the oracle reads."""
    q = synth.normal(prefix + ".q", (B, T, 64, 128))
    w = synth.uniform(prefix + ".w", (B, T, 64))
    k = synth.normal(prefix + ".k", (B, N, 128))
    if fmt == "fp8":
        qc, qs = synth.quant_fp8_rows(q)
        kc, ks = synth.quant_fp8_rows(k)
        qd, kd = on.dequant_fp8_rows(qc, qs), on.dequant_fp8_rows(kc, ks)
        dq = dict(q=dev(qc, torch.uint8), q_scale=dev(qs), k=dev(kc, torch.uint8), k_scale=dev(ks),
                  qk_dtype=csa.FP8_E4M3)
    else:
        qc, qs = synth.quant_mxfp4(q)
        kc, ks = synth.quant_mxfp4(k)
        qd, kd = on.dequant_mxfp4(qc, qs), on.dequant_mxfp4(kc, ks)
        dq = dict(q=dev(qc, torch.uint8), q_scale=dev(qs, torch.uint8), k=dev(kc, torch.uint8),
                  k_scale=dev(ks, torch.uint8), qk_dtype=csa.MXFP4)
    return dq, w, qd, kd


def _quant_scores(dq, w, pool, sd):
    s = csa.lightning_index_pool(dq["q"], dev(w), dq["k"], dev(pool, torch.int32), qk_dtype=dq["qk_dtype"],
                                 q_scale=dq["q_scale"], k_scale=dq["k_scale"], score_dtype=sd)
    torch.cuda.synchronize()
    return host(s)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_quantized_pool_all_rows(fmt):
    """Ragged pools (empty slots at the end of rows, an empty row, ids past
    N) over fp8 / MXFP4 keys, fp32 and bf16 scores."""
    B, T, N, q0, P = 2, 3, 3000, 11000, 600
    dq, w, qd, kd = _quant_layer(f"pl.q.{fmt}", B, T, N, fmt)
    pool = synth.random_topk_indices(f"pl.q.{fmt}.pool", B, T, P, [min(N, 500 + 200 * t) for t in range(T)])
    pool[1, 2, :] = -1
    pool[0, 1, 3:5] = [N, N + 77]
    ref = oi.pool_scores(qd, w, kd, pool)
    index_close(_quant_scores(dq, w, pool, torch.float32), ref)
    _bf16_close(_quant_scores(dq, w, pool, BF), ref)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_quantized_pool_long_runs(fmt):
    """The long-run kernel (eight chunks per wave) over quantized keys, sampled rows."""
    B, T, N, P = 1, 1100, 5000, 700
    dq, w, qd, kd = _quant_layer(f"pl.ql.{fmt}", B, T, N, fmt)
    pool = synth.random_topk_indices(f"pl.ql.{fmt}.pool", B, T, P, [min(N, 400 + t) for t in range(T)])
    got = _quant_scores(dq, w, pool, torch.float32)
    rows = [0, 1, 63, 64, 700, 1099]
    index_close(got[:, rows], oi.pool_scores(qd[:, rows], w[:, rows], kd, pool[:, rows]))


def test_pro_decode_reindex_mxfp4():
    """The Pro decode shape: batch 8 at 1,048,576 context (262,144 C4A
    entries), MXFP4 keys, a 2,048-entry pool per query, top-1024 inside it.
    Keys are drawn and encoded on the device; the oracle reads back the
    pooled rows."""
    B, N, P, K = 8, 262144, 2048, 1024
    kp, ks = synth.device_quant_mxfp4(synth.device_normal("pl.pro.k", (B, N, 128)))
    q = synth.normal("pl.pro.q", (B, 1, 64, 128))
    qc, qs = synth.quant_mxfp4(q)
    w = synth.uniform("pl.pro.w", (B, 1, 64))
    pool = synth.random_topk_indices("pl.pro.pool", B, 1, P, [N] * B)
    dpool = dev(pool, torch.int32)
    s = csa.lightning_index_pool(dev(qc, torch.uint8), dev(w), kp, dpool, qk_dtype=csa.MXFP4,
                                 q_scale=dev(qs, torch.uint8), k_scale=ks, score_dtype=BF)
    idx = csa.topk_select_pool(s, dpool, K, N=N)
    torch.cuda.synchronize()
    hs, hi = host(s), host(idx)
    qd = on.dequant_mxfp4(qc, qs)
    for b in range(B):
        ids = pool[b, 0][pool[b, 0] >= 0].astype(np.int64)
        sel = torch.as_tensor(ids, device="cuda")
        kd = on.dequant_mxfp4(host(kp[b][sel]), host(ks[b][sel]))      # the pooled rows, in pool order
        local = np.full((1, 1, P), -1, dtype=np.int64)
        local[0, 0, :len(ids)] = np.arange(len(ids))
        _bf16_close(hs[b:b + 1], oi.pool_scores(qd[b:b + 1], w[b:b + 1], kd[None], local))
    assert np.array_equal(hi, _ascending(ot.pool_select(hs, pool, K, N=N)))
