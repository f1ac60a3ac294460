"""GPU parity at the 1M-context Pro decode size: batch 8 at 1,048,576 tokens of
context, 262,144 C4A entries per sequence, MXFP4 indexer q and keys (drawn
N(0, 1) and quantized), bf16 scores, top-1024, sparse MQA over 64 x 512 heads
with a 128-token window.

Pages: "DeepSeek V4 结构速览" (核心设计: k = 1024 for Pro; Lightning Indexer: the
QK path in FP4, scores stored BF16; the C4A compressor at decode), "DeepSeek
Technical Reports" (DSA: the indexer and Top-k equations).

* The indexer over all 8 x 262,144 keys, checked on two whole sequences (the
  first and the last, every key run including the last one) against the
  oracle on the same bytes: bf16 scores within one bf16 ulp of the oracle's
  score rounded to bf16, fp32 scores within 1e-3 relative.
* The whole chain for one sequence at that size: the decode step's compressor
  writes the new block's 512-d latent (bf16) and its 128-d key (quantized on
  write to MXFP4) into cache slot 262,143; the MXFP4 indexer scores all
  262,144 keys; Top-1024; sparse MQA.  The oracle runs the same chain on its
  own: its compressor output (fp64, and its own MXFP4 encoding of the key),
  its scores rounded to bf16, its Top-k, its attention.  Selected sets must be
  equal in size and may differ only in entries whose oracle score lies within
  1e-3 relative or one bf16 ulp of the k-th oracle score (the chained rule for
  bf16-stored scores); attention is compared on the selection the GPU made
  once that selection has been checked to be one of the oracle's valid ones.

Large tensors are drawn on the device from seeded generators; the oracle reads
back the bytes it needs before any kernel runs.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_compress_amd as csa
import synth
from oracle import attention as oa
from oracle import compressor as oc
from oracle import indexer as oi
from oracle import numerics as on
from oracle import topk as ot
from helpers import ATTN_BF16_MAX_ABS, ATTN_NORMWISE, dev, host, index_close, max_abs, normwise_rel

pytestmark = pytest.mark.gpu
BF = torch.bfloat16
B, N, K, CTX = 8, 262144, 1024, 1048576
T_POS = CTX - 1                 # the query token completes the last block
RAW0 = T_POS - 127


def _bf16_ulp(v):
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def _bf16_close(got, ref64):
    ref = on.store_bf16(ref64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin)
    d = np.abs(got[fin] - ref[fin])
    assert np.all(d <= _bf16_ulp(ref[fin]) * 1.0001), f"max diff {d.max()}"


def _mxfp4_keys(name, nseq):
    """N(0, 1) keys drawn on the device, then MXFP4-encoded there."""
    x = synth.device_normal(name, (nseq, N, 128))
    kp, ks = synth.device_quant_mxfp4(x)
    del x
    return kp, ks


def test_mxfp4_indexer_full_size_two_sequences():
    kp, ks = _mxfp4_keys("pro.ix.k", B)
    q = synth.device_normal("pro.ix.q", (B, 1, 64, 128))
    qp, qs = synth.device_quant_mxfp4(q)
    w = synth.device_uniform("pro.ix.w", (B, 1, 64))
    check = [0, B - 1]
    host_in = {b: (host(qp[b]), host(qs[b]), host(kp[b]), host(ks[b])) for b in check}
    wh = host(w)
    s16 = csa.lightning_index(qp, w, kp, q_pos0=T_POS, qk_dtype=csa.MXFP4, q_scale=qs, k_scale=ks,
                              score_dtype=BF)
    s32 = csa.lightning_index(qp, w, kp, q_pos0=T_POS, qk_dtype=csa.MXFP4, q_scale=qs, k_scale=ks,
                              score_dtype=torch.float32)
    torch.cuda.synchronize()
    for b in check:
        qpb, qsb, kpb, ksb = host_in[b]
        qd = on.dequant_mxfp4(qpb, qsb)[None]          # [1, 1, 64, 128]
        kd = on.dequant_mxfp4(kpb, ksb)[None]          # [1, N, 128]
        ref = oi.index_scores(qd, wh[b][None], kd, T_POS, 4)
        _bf16_close(host(s16[b])[None], ref)
        index_close(host(s32[b])[None], ref)


def _band_ok(sc_stored, kth, s):
    return abs(sc_stored[s] - kth) <= max(1e-3 * abs(kth), _bf16_ulp(kth))


def test_pro_decode_chain_one_sequence():
    nb = 1
    pos4 = T_POS - 3                                  # the block the query completes
    # ---- inputs (seeded); host copies for the oracle are taken before any kernel runs
    kv = synth.device_normal("pro.ch.kv", (nb, N, 512), BF)
    kp, ks = _mxfp4_keys("pro.ch.k", nb)
    kv_h = kv.cpu()                                   # bf16 on the host
    kp_h, ks_h = host(kp), host(ks)
    c4 = {nm: synth.round_bf16(synth.normal(f"pro.ch.c4.{nm}", (nb, 4, 512)))
          for nm in ("Ca", "Za", "Cb", "Zb", "pCb", "pZb")}
    c4k = {nm: synth.round_bf16(synth.normal(f"pro.ch.c4k.{nm}", (nb, 4, 128)))
           for nm in ("Ca", "Za", "Cb", "Zb", "pCb", "pZb")}
    b4 = synth.normal("pro.ch.b4", (8, 512), var=0.1)
    b4k = synth.normal("pro.ch.b4k", (8, 128), var=0.1)
    qi = synth.normal("pro.ch.qi", (nb, 1, 64, 128))
    qp, qs = synth.quant_mxfp4(qi)
    w = synth.uniform("pro.ch.w", (nb, 1, 64))
    q = synth.round_bf16(synth.normal("pro.ch.q", (nb, 1, 64, 512)))
    raw = synth.round_bf16(synth.normal("pro.ch.raw", (nb, 128, 512)))

    # ---- GPU chain
    d4 = {k2: dev(v, BF) for k2, v in c4.items()}
    d4k = {k2: dev(v, BF) for k2, v in c4k.items()}
    csa.csa_compress_batch([
        dict(ratio=4, Ca=d4["Ca"], Za=d4["Za"], bias=dev(b4), Cb=d4["Cb"], Zb=d4["Zb"], prev_Cb=d4["pCb"],
             prev_Zb=d4["pZb"], pos0=pos4, out=kv, cache_entry0=N - 1),
        dict(ratio=4, Ca=d4k["Ca"], Za=d4k["Za"], bias=dev(b4k), Cb=d4k["Cb"], Zb=d4k["Zb"], prev_Cb=d4k["pCb"],
             prev_Zb=d4k["pZb"], pos0=pos4, out=kp, out_scale=ks, cache_entry0=N - 1)])
    scores = csa.lightning_index(dev(qp, torch.uint8), dev(w), kp, q_pos0=T_POS, qk_dtype=csa.MXFP4,
                                 q_scale=dev(qs, torch.uint8), k_scale=ks, score_dtype=BF)
    idx = csa.topk_select(scores, K, q_pos0=T_POS)
    out = csa.sparse_mqa_attn(dev(q, BF), kv, idx, dev(raw, BF), q_pos0=T_POS, raw_pos0=RAW0)
    torch.cuda.synchronize()
    g_kv_last = host(kv[0, N - 1])
    g_kp_last, g_ks_last = host(kp[0, N - 1]), host(ks[0, N - 1])
    g_scores, g_idx, g_out = host(scores)[0, 0], host(idx)[0, 0], host(out)[0, 0]

    # ---- oracle chain (its own compressor, encoding, scores, Top-k and attention)
    ent, _ = oc.compress_sequence(c4["Ca"][0], c4["Za"][0], b4, 4, c4["Cb"][0], c4["Zb"][0], c4["pCb"][0],
                                  c4["pZb"][0], pos0=pos4)
    key, _ = oc.compress_sequence(c4k["Ca"][0], c4k["Za"][0], b4k, 4, c4k["Cb"][0], c4k["Zb"][0], c4k["pCb"][0],
                                  c4k["pZb"][0], pos0=pos4)
    o_kp, o_ks = on.quant_mxfp4_rows_f32(key[0])
    keys_o = on.dequant_mxfp4(kp_h[0], ks_h[0])
    keys_o[N - 1] = on.dequant_mxfp4(o_kp, o_ks)
    sc = oi.index_scores(on.dequant_mxfp4(qp, qs), w, keys_o[None], T_POS, 4)
    stored = on.store_bf16(sc)
    o_idx = ot.topk_select(stored, K, T_POS, 4)[0, 0]

    # compressor outputs: the latent at the bf16 bound, the key's decoded values
    # within half an E2M1 step of the oracle's (plus the fp32 compressor bound)
    assert max_abs(g_kv_last, ent[0]) < 2e-2
    dec = on.dequant_mxfp4(g_kp_last, g_ks_last)
    s = np.repeat(on.decode_e8m0(g_ks_last), 32)
    a = np.abs(key[0] / s)
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    assert np.all((np.abs(dec - key[0]) <= 0.5 * step * s * (1 + 1e-6) + 1e-4) | (a > 6))

    # scores: every key the host drew, within one bf16 ulp; the new key's score
    # agrees too when both sides encoded it to the same bytes
    same_key = np.array_equal(g_kp_last, o_kp) and np.array_equal(g_ks_last, o_ks)
    upto = N if same_key else N - 1
    _bf16_close(g_scores[None, None, :upto], sc[:, :, :upto])

    # Top-k: equal sizes; differences only inside the tie band of the k-th score
    st = stored[0, 0]
    kth = np.sort(st)[::-1][K - 1]
    gs = set(int(v) for v in g_idx if v >= 0)
    os_ = set(int(v) for v in o_idx if v >= 0)
    assert len(gs) == len(os_) == K
    for e in gs ^ os_:
        assert _band_ok(st, kth, e), f"entry {e} differs outside the tie band"

    # attention over the GPU's selection (checked valid above), the oracle's rows:
    # the host copy of the cache, and the oracle's own entry for slot N - 1
    sel = sorted(gs)
    rows = kv_h[0, torch.as_tensor([e for e in sel if e != N - 1], dtype=torch.long)].float().numpy()
    rows = rows.astype(np.float64)
    if N - 1 in gs:
        rows = np.concatenate([rows, ent[0][None]], axis=0)
    ref, _ = oa.sparse_mqa(q, rows[None], np.arange(len(sel))[None, None], raw, RAW0, T_POS, 128)
    assert max_abs(g_out, ref[0, 0]) < ATTN_BF16_MAX_ABS
    assert normwise_rel(g_out, ref[0, 0]) < ATTN_NORMWISE


def test_mxfp4_paged_indexer_equals_contiguous_full_size():
    """The paged MXFP4 indexer over the same 8 x 262,144 keys laid out in
    shuffled 32-entry pages gives the contiguous indexer's scores bit for bit
    (same kernel shape; paging only moves each tile's base row)."""
    kp, ks = _mxfp4_keys("pro.pg.k", B)
    q = synth.device_normal("pro.pg.q", (B, 1, 64, 128))
    qp, qs = synth.device_quant_mxfp4(q)
    w = synth.device_uniform("pro.pg.w", (B, 1, 64))
    per_seq = N // 32
    g = np.random.default_rng(5)
    perm = torch.as_tensor(g.permutation(B * per_seq), dtype=torch.int64, device="cuda")
    pool = torch.empty(B * per_seq, 32, 64, dtype=torch.uint8, device="cuda")
    spool = torch.empty(B * per_seq, 32, 4, dtype=torch.uint8, device="cuda")
    pool[perm] = kp.reshape(B * per_seq, 32, 64)
    spool[perm] = ks.reshape(B * per_seq, 32, 4)
    table = perm.reshape(B, per_seq).to(torch.int32)
    seq_pos = torch.full((B,), T_POS, dtype=torch.int64, device="cuda")
    ref = csa.lightning_index(qp, w, kp, q_pos0=T_POS, qk_dtype=csa.MXFP4, q_scale=qs, k_scale=ks, score_dtype=BF)
    got = csa.lightning_index_paged(qp[:, 0], w[:, 0], pool, table, seq_pos, qk_dtype=csa.MXFP4, q_scale=qs[:, 0],
                                    k_scale=spool, score_dtype=BF)
    torch.cuda.synchronize()
    assert torch.equal(got, ref[:, 0])
