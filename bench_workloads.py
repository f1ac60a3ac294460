"""Workloads of bench.py: inputs, stages, algorithmic work and CPU-oracle samples.

Every workload is one pass of its stages ("a step") over synthetic inputs
resident in HBM.  Large caches exist in ``copies`` seeded copies and step i
runs on copy i % copies, so the bytes a decode step streams (keys, selected
rows) come from HBM and not from the 256 MB Infinity Cache left warm by the
previous step.  Each stage is a list of library calls with the algorithmic
bytes and FLOPs of one launch (unique bytes only) and the roofline that
bounds it: "hbm", or the MFMA dtype ("bf16", "fp8", "mxfp4").

The five configurations of the method (one GPU):

  csa_1m_decode   8 sequences at 1,048,576 tokens of context (Pro): the C4A
                  compressor writes the new block's 512-d latent (bf16) and its
                  128-d key quantized on write to MXFP4 inside the MXFP4
                  indexer's launch (lightning_index_compressed), which scores
                  all 262,144 keys; top-1024; sparse MQA over 1,024 entries +
                  128 window rows
  csa_decode      32 sequences at 65,536 context: C4A compress (latent + bf16
                  key), the bf16 indexer over 16,384 keys, top-512, sparse MQA
  csa_prefill     a 4,096-token chunk after 131,072 tokens: C4A compress of the
                  chunk (latent bf16 + key quantized on write to fp8 into the
                  key cache), the fp8 indexer over 4,096 x 33,792, top-512,
                  sparse MQA
  hca_decode      16 sequences at 1,048,576 context: C128A compress of the last
                  block, dense MQA with sink over 8,192 entries + window
  hca_prefill     the last 2,048 tokens of a 1,048,576 context: C128A compress of
                  the chunk (16 entries), dense MQA with sink

Other workloads (``bench.py --workload NAME``): csa_hca_decode (a CSA and an
HCA layer decode step at 65,536 context, with the --keys / --rope /
--batch-invariant variants), c128a_1m, csa_reindex_decode,
csa_reindex_prefill, csa_paged_decode, hbm_copy (the counter calibration), hbm_read (a plain
streaming read, the attainable read bandwidth).

The CPU baseline of each configuration runs the oracle (NumPy fp64, test
infrastructure) over a bounded sample of the same step: whole query tokens
through every stage, inputs copied to the host before the clock starts.
"""
from __future__ import annotations

import os
import time

import numpy as np

HBM = 8000.0
PEAK = {"bf16": 2500.0, "fp8": 5000.0, "mxfp4": 10100.0}


class Work:
    """A workload: stages (name, fn(copy), alg bytes, alg flops, bound) run in order."""

    def __init__(self, key, label, queries, copies, info, dominant, unit="query-tokens/s", units=None):
        self.key, self.label, self.queries, self.copies = key, label, queries, copies
        self.info, self.dominant, self.unit = info, dominant, unit
        self.units = queries if units is None else units      # units of `unit` per step
        self.stages = []
        self.cpu = None                                        # callable(budget_s) -> dict

    def add(self, name, fn, nbytes, flops, bound):
        self.stages.append((name, fn, int(nbytes), int(flops), bound))


def _ws(torch, csa, op, B, T, N, k):
    return torch.empty(max(16, csa.workspace_bytes(op, B, T, N, k)), dtype=torch.uint8, device="cuda")


def cpu_info():
    """Host threads the oracle's BLAS uses, and the machine they run on."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"cores": int(min(threads, aff)), "blas_threads": int(threads), "cpu_count": os.cpu_count(),
            "affinity": aff, "cpu_model": model}


def _baseline(done, seconds, sample, unit="query-tokens/s", value=None):
    rec = {"value": round(done / seconds if value is None else value, 3), "unit": unit, "kind": "oracle",
           "sample": sample}
    rec.update(cpu_info())
    return rec


def _h(t):
    return t.float().cpu().numpy()


# ---------------------------------------------------------------- decode CSA layers


def _c4_inputs(dn, bf, tag, B, c):
    return {nm: dn(f"{tag}.{nm}", (B, 4, c), bf) for nm in ("Ca", "Za", "Cb", "Zb", "pCb", "pZb")}


def _c4_job(c4, bias, pos0, out, entry, out_scale=None):
    j = dict(ratio=4, Ca=c4["Ca"], Za=c4["Za"], bias=bias, Cb=c4["Cb"], Zb=c4["Zb"], prev_Cb=c4["pCb"],
             prev_Zb=c4["pZb"], pos0=pos0, out=out, cache_entry0=entry)
    if out_scale is not None:
        j["out_scale"] = out_scale
    return j


def _c4_decode_bytes(B, c, key_bytes=None):
    """One C4A entry per sequence from a 4-token block: the current block's Ca,
    Za and the previous block's Cb, Zb (16 rows of c bf16), the fp32 bias, one
    entry written (c bf16, or the encoded key's bytes)."""
    out = c * 2 if key_bytes is None else key_bytes
    return B * (16 * c * 2 + out) + 8 * c * 4


def csa_1m_decode(torch, csa, synth, copies=4, fuse=True):
    """Config 5: CSA decode at 1,048,576 context, batch 8, MXFP4 indexer, top-1024.
    fuse: the compressor writes run inside the indexer's launch
    (lightning_index_compressed); else a compressor launch, then the indexer."""
    bf = torch.bfloat16
    dn = synth.device_normal
    B, N, k, t = 8, 262144, 1024, 1048575
    raw0, pos4 = t - 127, t - 3
    kv, kp, ks = [], [], []
    for r in range(copies):
        kv.append(dn(f"m.kv.{r}", (B, N, 512), bf))
        x = dn(f"m.keys.{r}", (B, N, 128))
        a, s = synth.device_quant_mxfp4(x)        # N(0, 1) keys, then MXFP4 (the configuration's recipe)
        del x
        kp.append(a)
        ks.append(s)
    c4 = _c4_inputs(dn, bf, "m.c4", B, 512)
    c4k = _c4_inputs(dn, bf, "m.c4k", B, 128)
    b4, b4k = dn("m.b4", (8, 512), var=0.1), dn("m.b4k", (8, 128), var=0.1)
    qp, qs = synth.device_quant_mxfp4(dn("m.qi", (B, 1, 64, 128)))
    w = synth.device_uniform("m.w", (B, 1, 64))
    q = dn("m.q", (B, 1, 64, 512), bf)
    raw = dn("m.raw", (B, 128, 512), bf)
    scores = torch.empty(B, 1, N, dtype=bf, device="cuda")
    idx = torch.empty(B, 1, k, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    ws_t = _ws(torch, csa, csa.OP_TOPK, B, 1, N, k)
    ws_a = _ws(torch, csa, csa.OP_SPARSE_ATTN, B, 1, N, k)
    wk = Work("csa_1m_decode" if fuse else "csa_1m_decode_separate",
              "csa_1m_decode: CSA decode at 1,048,576 context (Pro): C4A compress (latent bf16 + key quantized on "
              "write to MXFP4) " + ("inside the MXFP4 indexer's launch" if fuse else "in its own launch, then the "
                                   "MXFP4 indexer") + " over 262,144 keys, top-1024, sparse MQA",
              B, copies, dict(batch=B, context=t + 1, c4a_entries=N, topk=k, window=128, heads=64, head_dim=512,
                              index_heads=64, index_dim=128, index_qk="mxfp4", scores="bf16",
                              cache_copies_rotated=copies),
              "lightning_index")
    def jobs(r):
        return [_c4_job(c4, b4, pos4, kv[r], N - 1), _c4_job(c4k, b4k, pos4, kp[r], N - 1, ks[r])]

    c_bytes = _c4_decode_bytes(B, 512) + _c4_decode_bytes(B, 128, 64 + 4)
    i_bytes, i_flops = B * N * 68 + B * 64 * 68 + B * 64 * 4 + B * N * 2, B * N * 64 * 128 * 2
    if fuse:
        wk.dominant = "compress_index"
        wk.add("compress_index", lambda r: csa.lightning_index_compressed(
            qp, w, kp[r], jobs(r), e_new=N - 1, q_pos0=t, qk_dtype=csa.MXFP4, q_scale=qs, k_scale=ks[r],
            scores=scores, N=N), c_bytes + i_bytes, i_flops, "hbm")
    else:
        wk.add("compress_c4a_kv_keys", lambda r: csa.csa_compress_batch(jobs(r)), c_bytes, 0, "hbm")
        wk.add("lightning_index", lambda r: csa.lightning_index(qp, w, kp[r], q_pos0=t, qk_dtype=csa.MXFP4,
                                                                q_scale=qs, k_scale=ks[r], scores=scores, N=N),
               i_bytes, i_flops, "hbm")
    wk.add("topk_select", lambda r: csa.topk_select(scores, k, q_pos0=t, idx=idx, workspace=ws_t),
           B * N * 2 + B * k * 4, 0, "hbm")
    wk.add("sparse_mqa_attn", lambda r: csa.sparse_mqa_attn(q, kv[r], idx, raw, q_pos0=t, raw_pos0=raw0, out=out,
                                                            workspace=ws_a),
           B * ((k + 128) * 1024 + k * 4 + 2 * 64 * 512 * 2), B * (k + 128) * 64 * 512 * 4, "hbm")

    def cpu(budget):
        from oracle import attention as oa, compressor as oc, indexer as oi, numerics as on, topk as ot
        seqs = [0, 1]
        hs = {b: dict(kp=_h(kp[0][b]).astype(np.uint8), ks=_h(ks[0][b]).astype(np.uint8), kv=kv[0][b].cpu(),
                      c4={n: _h(v[b]) for n, v in c4.items()}, c4k={n: _h(v[b]) for n, v in c4k.items()},
                      qp=_h(qp[b]).astype(np.uint8), qs=_h(qs[b]).astype(np.uint8), w=_h(w[b]), q=_h(q[b]),
                      raw=_h(raw[b])) for b in seqs}
        hb4, hb4k = _h(b4), _h(b4k)
        done, t0 = 0, time.perf_counter()
        while True:
            s = hs[seqs[done % len(seqs)]]
            c, ck = s["c4"], s["c4k"]
            ent, _ = oc.compress_sequence(c["Ca"], c["Za"], hb4, 4, c["Cb"], c["Zb"], c["pCb"], c["pZb"], pos0=pos4)
            key, _ = oc.compress_sequence(ck["Ca"], ck["Za"], hb4k, 4, ck["Cb"], ck["Zb"], ck["pCb"], ck["pZb"],
                                          pos0=pos4)
            kcode, kscale = on.quant_mxfp4_rows_f32(key[0])
            keys = on.dequant_mxfp4(s["kp"], s["ks"])
            keys[N - 1] = on.dequant_mxfp4(kcode, kscale)
            sc = oi.index_scores(on.dequant_mxfp4(s["qp"], s["qs"])[None], s["w"][None], keys[None], t, 4)
            sel = ot.topk_select(on.store_bf16(sc), k, t, 4)[0, 0]
            sel = sel[sel >= 0]
            rows = s["kv"][torch.as_tensor(np.where(sel == N - 1, 0, sel), dtype=torch.long)].float().numpy()
            rows = rows.astype(np.float64)
            rows[sel == N - 1] = ent[0]
            oa.sparse_mqa(s["q"][None], rows[None], np.arange(len(sel))[None, None], s["raw"][None], raw0, t, 128)
            done += 1
            el = time.perf_counter() - t0
            if el >= budget:
                break
        return _baseline(done, el, f"{done} query tokens (sequences 0 and 1 cycled), each through the whole step: "
                                   f"both C4A compressors and the key's MXFP4 encoding, the indexer over {N} keys, "
                                   f"top-{k}, sparse MQA; {el:.1f} s")

    wk.cpu = cpu
    return wk


def csa_decode(torch, csa, synth, copies=4, fuse=True):
    """Config 2: CSA decode at 65,536 context, batch 32, bf16 indexer, top-512.
    fuse: the key write inside the indexer's launch (lightning_index_compressed)
    and the latent write in spare workgroups of Top-k's (topk_select_compressed);
    else one compressor launch for both."""
    bf = torch.bfloat16
    dn = synth.device_normal
    B, N, k, t = 32, 16384, 512, 65535
    raw0, pos4 = t - 127, t - 3
    kv = [dn(f"d.kv.{r}", (B, N, 512), bf) for r in range(copies)]
    keys = [dn(f"d.keys.{r}", (B, N, 128), bf) for r in range(copies)]
    c4 = _c4_inputs(dn, bf, "d.c4", B, 512)
    c4k = _c4_inputs(dn, bf, "d.c4k", B, 128)
    b4, b4k = dn("d.b4", (8, 512), var=0.1), dn("d.b4k", (8, 128), var=0.1)
    qi = dn("d.qi", (B, 1, 64, 128), bf, var=1.0 / 128)
    w = synth.device_uniform("d.w", (B, 1, 64))
    q = dn("d.q", (B, 1, 64, 512), bf)
    raw = dn("d.raw", (B, 128, 512), bf)
    scores = torch.empty(B, 1, N, dtype=bf, device="cuda")
    idx = torch.empty(B, 1, k, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    ws_t = _ws(torch, csa, csa.OP_TOPK, B, 1, N, k)
    ws_a = _ws(torch, csa, csa.OP_SPARSE_ATTN, B, 1, N, k)
    wk = Work("csa_decode", "csa_decode: CSA decode at 65,536 context, batch 32: C4A compress (latent + bf16 key), "
              "bf16 indexer over 16,384 keys, top-512, sparse MQA",
              B, copies, dict(batch=B, context=t + 1, c4a_entries=N, topk=k, window=128, heads=64, head_dim=512,
                              index_heads=64, index_dim=128, index_qk="bf16", scores="bf16",
                              cache_copies_rotated=copies),
              "lightning_index")
    c_lat, c_key = _c4_decode_bytes(B, 512), _c4_decode_bytes(B, 128)
    i_bytes, i_flops = B * N * 256 + B * 64 * 128 * 2 + B * 64 * 4 + B * N * 2, B * N * 64 * 128 * 2
    t_bytes = B * N * 2 + B * k * 4
    if fuse:
        wk.dominant = "compress_index"
        wk.label = wk.label.replace("C4A compress (latent + bf16 key), bf16 indexer",
                                    "C4A compress (bf16 key inside the bf16 indexer's launch, latent inside "
                                    "Top-k's), bf16 indexer")
        wk.add("compress_index", lambda r: csa.lightning_index_compressed(
            qi, w, keys[r], [_c4_job(c4k, b4k, pos4, keys[r], N - 1)], e_new=N - 1, q_pos0=t, scores=scores),
            c_key + i_bytes, i_flops, "hbm")
        wk.add("compress_topk", lambda r: csa.topk_select_compressed(
            scores, k, [_c4_job(c4, b4, pos4, kv[r], N - 1)], q_pos0=t, idx=idx, workspace=ws_t),
            c_lat + t_bytes, 0, "hbm")
    else:
        wk.add("compress_c4a_kv_keys", lambda r: csa.csa_compress_batch([
            _c4_job(c4, b4, pos4, kv[r], N - 1), _c4_job(c4k, b4k, pos4, keys[r], N - 1)]), c_lat + c_key, 0, "hbm")
        wk.add("lightning_index", lambda r: csa.lightning_index(qi, w, keys[r], q_pos0=t, scores=scores),
               i_bytes, i_flops, "hbm")
        wk.add("topk_select", lambda r: csa.topk_select(scores, k, q_pos0=t, idx=idx, workspace=ws_t), t_bytes, 0,
               "hbm")
    wk.add("sparse_mqa_attn", lambda r: csa.sparse_mqa_attn(q, kv[r], idx, raw, q_pos0=t, raw_pos0=raw0, out=out,
                                                            workspace=ws_a),
           B * ((k + 128) * 1024 + k * 4 + 2 * 64 * 512 * 2), B * (k + 128) * 64 * 512 * 4, "hbm")

    def cpu(budget):
        from oracle import attention as oa, compressor as oc, indexer as oi, numerics as on, topk as ot
        seqs = [0, 1, 2, 3]
        hs = {b: dict(keys=_h(keys[0][b]), kv=kv[0][b].cpu(), c4={n: _h(v[b]) for n, v in c4.items()},
                      c4k={n: _h(v[b]) for n, v in c4k.items()}, qi=_h(qi[b]), w=_h(w[b]), q=_h(q[b]),
                      raw=_h(raw[b])) for b in seqs}
        hb4, hb4k = _h(b4), _h(b4k)
        done, t0 = 0, time.perf_counter()
        while True:
            s = hs[seqs[done % len(seqs)]]
            c, ck = s["c4"], s["c4k"]
            ent, _ = oc.compress_sequence(c["Ca"], c["Za"], hb4, 4, c["Cb"], c["Zb"], c["pCb"], c["pZb"], pos0=pos4)
            key, _ = oc.compress_sequence(ck["Ca"], ck["Za"], hb4k, 4, ck["Cb"], ck["Zb"], ck["pCb"], ck["pZb"],
                                          pos0=pos4)
            kk = s["keys"].astype(np.float64)
            kk[N - 1] = key[0]
            sc = oi.index_scores(s["qi"][None], s["w"][None], kk[None], t, 4)
            sel = ot.topk_select(on.store_bf16(sc), k, t, 4)[0, 0]
            sel = sel[sel >= 0]
            rows = s["kv"][torch.as_tensor(np.where(sel == N - 1, 0, sel), dtype=torch.long)].float().numpy()
            rows = rows.astype(np.float64)
            rows[sel == N - 1] = ent[0]
            oa.sparse_mqa(s["q"][None], rows[None], np.arange(len(sel))[None, None], s["raw"][None], raw0, t, 128)
            done += 1
            el = time.perf_counter() - t0
            if el >= budget:
                break
        return _baseline(done, el, f"{done} query tokens (sequences 0..3 cycled), each through the whole step: both "
                                   f"C4A compressors, the indexer over {N} bf16 keys, top-{k}, sparse MQA; {el:.1f} s")

    wk.cpu = cpu
    return wk


# ---------------------------------------------------------------- prefill CSA layer


def csa_decode_separate(torch, csa, synth, copies=4):
    """The CSA decode at 65,536 context with both compressor writes in a launch of
    their own (A/B against the configuration's fused launches)."""
    wk = csa_decode(torch, csa, synth, copies=copies, fuse=False)
    wk.key = "csa_decode_separate"
    return wk


def csa_prefill(torch, csa, synth, copies=1):
    """Config 3: a 4,096-token chunk after 131,072 tokens of context, fp8 indexer."""
    bf = torch.bfloat16
    dn = synth.device_normal
    T, N, k, q0 = 4096, 33792, 512, 131072
    raw0 = q0 - 127
    E0 = q0 // 4                                   # first entry of the chunk
    c = {nm: dn(f"p.{nm}", (1, T, 512), bf) for nm in ("Ca", "Za", "Cb", "Zb")}
    ck = {nm: dn(f"p.k{nm}", (1, T, 128), bf) for nm in ("Ca", "Za", "Cb", "Zb")}
    h = {nm: dn(f"p.h{nm}", (1, 4, 512), bf) for nm in ("Cb", "Zb")}
    hk = {nm: dn(f"p.hk{nm}", (1, 4, 128), bf) for nm in ("Cb", "Zb")}
    b4, b4k = dn("p.b4", (8, 512), var=0.1), dn("p.b4k", (8, 128), var=0.1)
    kv = dn("p.kv", (1, N, 512), bf)
    kc, ks = synth.device_quant_fp8_rows(dn("p.ki", (1, N, 128)))     # the cache's fp8 keys + row scales
    qc, qs = synth.device_quant_fp8_rows(dn("p.qi", (1, T, 64, 128)))
    w = synth.device_uniform("p.w", (1, T, 64))
    q = dn("p.q", (1, T, 64, 512), bf)
    raw = dn("p.raw", (1, q0 + T - raw0, 512), bf)
    scores = torch.empty(1, T, N, dtype=bf, device="cuda")
    idx = torch.empty(1, T, k, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    n_vis = sum(min((q0 + tt + 1) // 4, N) for tt in range(T))
    wk = Work("csa_prefill", "csa_prefill: a 4,096-token chunk after 131,072 tokens: C4A compress of the chunk "
              "(latent bf16 + key quantized on write to fp8), fp8 indexer over 4,096 x 33,792, top-512, sparse MQA",
              T, copies, dict(batch=1, context=q0, chunk=T, c4a_entries=N, topk=k, window=128, heads=64,
                              head_dim=512, index_qk="fp8_e4m3", scores="bf16"),
              "lightning_index")
    wk.add("compress_c4a_kv_keys", lambda r: csa.csa_compress_batch([
        dict(ratio=4, Ca=c["Ca"], Za=c["Za"], bias=b4, Cb=c["Cb"], Zb=c["Zb"], prev_Cb=h["Cb"], prev_Zb=h["Zb"],
             pos0=q0, out=kv, cache_entry0=E0),
        dict(ratio=4, Ca=ck["Ca"], Za=ck["Za"], bias=b4k, Cb=ck["Cb"], Zb=ck["Zb"], prev_Cb=hk["Cb"],
             prev_Zb=hk["Zb"], pos0=q0, out=kc, out_scale=ks, cache_entry0=E0)]),
        T * 4 * (512 + 128) * 2 + T // 4 * (512 * 2 + 128 + 4) + 8 * (512 + 128) * 4, 0, "hbm")
    wk.add("lightning_index", lambda r: csa.lightning_index(qc, w, kc, q_pos0=q0, qk_dtype=csa.FP8_E4M3,
                                                            q_scale=qs, k_scale=ks, scores=scores),
           T * 64 * 132 + N * 132 + T * N * 2, n_vis * 64 * 128 * 2, "fp8")
    wk.add("topk_select", lambda r: csa.topk_select(scores, k, q_pos0=q0, idx=idx), T * N * 2 + T * k * 4, 0, "hbm")
    wk.add("sparse_mqa_attn", lambda r: csa.sparse_mqa_attn(q, kv, idx, raw, q_pos0=q0, raw_pos0=raw0, out=out),
           T * (k * 4 + 2 * 64 * 512 * 2) + (N + raw.shape[1]) * 1024, T * (k + 128) * 64 * 512 * 4, "bf16")

    def cpu(budget):
        from oracle import attention as oa, compressor as oc, indexer as oi, numerics as on, topk as ot
        hc = {n: _h(v[0]) for n, v in c.items()}
        hck = {n: _h(v[0]) for n, v in ck.items()}
        hh = {n: _h(v[0]) for n, v in h.items()}
        hhk = {n: _h(v[0]) for n, v in hk.items()}
        hkc, hks = _h(kc[0]).astype(np.uint8), _h(ks[0])
        hqc, hqs, hw = _h(qc[0]).astype(np.uint8), _h(qs[0]), _h(w[0])
        hkv, hq, hraw = kv[0].cpu(), q[0], _h(raw[0])
        hb4, hb4k = _h(b4), _h(b4k)
        t0 = time.perf_counter()
        # once per chunk: both compressors, the keys' fp8 encoding, the key cache decoded
        ent, _ = oc.compress_sequence(hc["Ca"], hc["Za"], hb4, 4, hc["Cb"], hc["Zb"], hh["Cb"], hh["Zb"], pos0=q0)
        key, _ = oc.compress_sequence(hck["Ca"], hck["Za"], hb4k, 4, hck["Cb"], hck["Zb"], hhk["Cb"], hhk["Zb"],
                                      pos0=q0)
        kcodes, kscales = on.quant_fp8_rows_f32(key)
        keys = on.dequant_fp8_rows(hkc, hks)
        keys[E0:] = on.dequant_fp8_rows(kcodes, kscales)
        t_chunk = time.perf_counter() - t0
        g = np.random.default_rng(0)
        order = g.permutation(T)
        done = 0
        t1 = time.perf_counter()
        while True:
            tt = int(order[done % T])
            qd = on.dequant_fp8_rows(hqc[tt], hqs[tt])
            sc = oi.index_scores(qd[None, None], hw[tt][None, None], keys[None], q0 + tt, 4)
            sel = ot.topk_select(on.store_bf16(sc), k, q0 + tt, 4)[0, 0]
            sel = sel[sel >= 0]
            new = sel >= E0
            rows = hkv[torch.as_tensor(np.where(new, 0, sel), dtype=torch.long)].float().numpy().astype(np.float64)
            rows[new] = ent[sel[new] - E0]
            qq = _h(hq[tt])[None, None]
            w0 = q0 + tt - 127
            oa.sparse_mqa(qq, rows[None], np.arange(len(sel))[None, None], hraw[None, w0 - raw0:q0 + tt + 1 - raw0],
                          w0, q0 + tt, 128)
            done += 1
            el = time.perf_counter() - t1
            if el + t_chunk >= budget:
                break
        # the chunk's one-off work is charged to the sampled rows pro rata
        seconds = el + t_chunk * done / T
        return _baseline(done, seconds, f"{done} of the chunk's {T} query rows (seeded order), each through the "
                                        f"indexer over its visible fp8 keys, top-{k} and sparse MQA, plus "
                                        f"{done}/{T} of the chunk's compressor and key-encoding time "
                                        f"({t_chunk:.1f} s for the whole chunk); {el:.1f} s of rows")

    wk.cpu = cpu
    return wk


# ---------------------------------------------------------------- HCA layer


def _hca(torch, csa, synth, decode, copies, fuse=True):
    bf = torch.bfloat16
    dn = synth.device_normal
    B, T = (16, 1) if decode else (1, 2048)
    N = 8192
    q0 = 1048575 if decode else 1046528
    raw0 = q0 - 127
    cpos = q0 + 1 - 128 if decode else q0
    ntok = 128 if decode else T
    tag = "hd" if decode else "hp"
    kv = [dn(f"{tag}.kv.{r}", (B, N, 512), bf) for r in range(copies)]
    c = {nm: dn(f"{tag}.{nm}", (B, ntok, 512), bf) for nm in ("Ca", "Za")}
    b128 = dn(f"{tag}.b", (128, 512), var=0.1)
    q = dn(f"{tag}.q", (B, T, 64, 512), bf)
    raw = dn(f"{tag}.raw", (B, q0 + T - raw0, 512), bf)
    sink = dn(f"{tag}.sink", (64,))
    out = torch.empty_like(q)
    ws = _ws(torch, csa, csa.OP_HCA_ATTN, B, T, N, 0)
    wsc = _ws(torch, csa, csa.OP_COMPRESS, B, ntok, 512, 128)
    rows = sum(min((q0 + tt + 1) // 128, N) + 128 for tt in range(T))
    if decode:
        wk = Work("hca_decode", "hca_decode: HCA decode at 1,048,576 context, batch 16: C128A compress of the last "
                  "block, dense MQA with sink over 8,192 entries + 128 window rows", B, copies,
                  dict(batch=B, context=q0 + 1, c128a_entries=N, window=128, heads=64, head_dim=512,
                       cache_copies_rotated=copies), "hca_attn")
    else:
        wk = Work("hca_prefill", "hca_prefill: the last 2,048 tokens of a 1,048,576 context: C128A compress of the "
                  "chunk, dense MQA with sink over 8,176..8,192 entries + window", T, copies,
                  dict(batch=1, context=1048576, chunk=T, c128a_entries=N, window=128, heads=64, head_dim=512),
                  "hca_attn")
    c_bytes = B * ntok * 512 * 4 + B * ntok // 128 * 1024 + 128 * 512 * 4
    a_bytes = (B * rows * 1024 if decode else (N + raw.shape[1]) * 1024) + B * T * 2 * 64 * 512 * 2
    a_flops = B * rows * 64 * 512 * 4
    if decode and fuse:
        # the C128A write inside the attention's launch (hca_attn_compressed)
        wk.dominant = "compress_attn"
        wk.label = wk.label.replace("C128A compress of the last block, dense MQA",
                                    "C128A compress of the last block inside the dense MQA's launch")
        job = lambda r: dict(ratio=128, Ca=c["Ca"], Za=c["Za"], bias=b128, pos0=cpos, out=kv[r],
                             cache_entry0=cpos // 128)
        wk.add("compress_attn", lambda r: csa.hca_attn_compressed(q, kv[r], raw, job(r), e_new=cpos // 128,
                                                                  q_pos0=q0, raw_pos0=raw0, sink=sink, out=out,
                                                                  workspace=ws),
               c_bytes + a_bytes, a_flops, "hbm")
    else:
        wk.add("compress_c128a_kv", lambda r: csa.csa_compress(128, c["Ca"], c["Za"], b128, pos0=cpos, out=kv[r],
                                                               cache_entry0=cpos // 128, workspace=wsc),
               c_bytes, 0, "hbm")
        wk.add("hca_attn", lambda r: csa.hca_attn(q, kv[r], raw, q_pos0=q0, raw_pos0=raw0, sink=sink, out=out,
                                                  workspace=ws),
               a_bytes, a_flops, "hbm" if decode else "bf16")

    def cpu(budget):
        from oracle import attention as oa, compressor as oc
        seqs = [0, 1] if decode else [0]
        hs = {b: dict(kv=_h(kv[0][b]), Ca=_h(c["Ca"][b]), Za=_h(c["Za"][b]), raw=_h(raw[b])) for b in seqs}
        hb, hsink = _h(b128), _h(sink)
        E0 = cpos // 128
        if decode:
            done, t0 = 0, time.perf_counter()
            while True:
                b = seqs[done % len(seqs)]
                s = hs[b]
                ent, _ = oc.compress_sequence(s["Ca"], s["Za"], hb, 128, pos0=cpos)
                kvh = s["kv"].astype(np.float64)
                kvh[E0] = ent[0]
                oa.hca_attention(_h(q[b])[None], kvh[None], s["raw"][None], raw0, q0, hsink, ratio=128)
                done += 1
                el = time.perf_counter() - t0
                if el >= budget:
                    break
            return _baseline(done, el, f"{done} query tokens (sequences 0 and 1 cycled), each through the C128A "
                                       f"compressor of its block and dense attention with sink over {N} entries + "
                                       f"128 window rows; {el:.1f} s")
        s = hs[0]
        t0 = time.perf_counter()
        ent, _ = oc.compress_sequence(s["Ca"], s["Za"], hb, 128, pos0=cpos)
        kvh = s["kv"].astype(np.float64)
        kvh[E0:E0 + ent.shape[0]] = ent
        t_chunk = time.perf_counter() - t0
        order = np.random.default_rng(0).permutation(T)
        hq = q[0]
        done, t1 = 0, time.perf_counter()
        while True:
            tt = int(order[done % T])
            oa.hca_attention(_h(hq[tt:tt + 1])[None], kvh[None], s["raw"][None], raw0, q0 + tt, hsink, ratio=128)
            done += 1
            el = time.perf_counter() - t1
            if el + t_chunk >= budget:
                break
        seconds = el + t_chunk * done / T
        return _baseline(done, seconds, f"{done} of the chunk's {T} query rows (seeded order), each through dense "
                                        f"attention with sink over its visible entries + window, plus {done}/{T} of "
                                        f"the chunk's C128A compressor time ({t_chunk:.2f} s); {el:.1f} s of rows")

    wk.cpu = cpu
    return wk


def hca_decode(torch, csa, synth, copies=4):
    """Config 4, decode: batch 16 at 1,048,576 context."""
    return _hca(torch, csa, synth, True, copies)


def hca_decode_separate(torch, csa, synth, copies=4):
    """The HCA decode with the C128A write in launches of its own (A/B against the
    configuration's single launch)."""
    wk = _hca(torch, csa, synth, True, copies, fuse=False)
    wk.key = "hca_decode_separate"
    return wk


def hca_prefill(torch, csa, synth, copies=1):
    """Config 4, prefill: a 2,048-token chunk at the end of a 1,048,576 context."""
    return _hca(torch, csa, synth, False, copies)


CONFIGS = {"csa_1m_decode": csa_1m_decode, "csa_decode": csa_decode, "csa_prefill": csa_prefill,
           "hca_decode": hca_decode, "hca_prefill": hca_prefill}
# the headline first, then the other configurations in the order the method lists them
DEFAULT_ORDER = ["csa_1m_decode", "csa_decode", "csa_prefill", "hca_decode", "hca_prefill"]


# ---------------------------------------------------------------- other workloads


def _quant_fp8_pair(torch, synth, x):
    return synth.device_quant_fp8_rows(x)


def csa_hca_decode(torch, csa, synth, copies=4, keys="bf16", rope=0, batch_invariant=False):
    """A decode step of one CSA layer and one HCA layer for 32 sequences at 65,536
    context (16,384 C4A and 512 C128A entries); index keys bf16, or quantized on
    write to fp8 / MXFP4 (--keys); partial RoPE fused into the compressors and
    the attention epilogues (--rope); batch-invariant attention."""
    bf = torch.bfloat16
    dn = synth.device_normal
    B, ctx, k = 32, 65536, 512
    N4, N128 = ctx // 4, ctx // 128
    t, raw0, pos4 = ctx - 1, ctx - 128, ctx - 4
    kv = [dn(f"b.kv.{r}", (B, N4, 512), bf) for r in range(copies)]
    kvh = [dn(f"b.kvh.{r}", (B, N128, 512), bf) for r in range(copies)]
    kb = [dn(f"b.keys.{r}", (B, N4, 128), bf) for r in range(copies)]
    qi = dn("b.qi", (B, 1, 64, 128), bf, var=1.0 / 128)
    if keys == "fp8":
        pairs = [synth.device_quant_fp8_rows(x) for x in kb]
        qq = synth.device_quant_fp8_rows(qi)
        qk, kbytes = csa.FP8_E4M3, 132
    elif keys == "fp4":
        pairs = [synth.device_quant_mxfp4(x) for x in kb]
        qq = synth.device_quant_mxfp4(qi)
        qk, kbytes = csa.MXFP4, 68
    else:
        pairs, qq, qk, kbytes = None, None, csa.BF16, 256
    c4 = _c4_inputs(dn, bf, "b.c4", B, 512)
    c4k = _c4_inputs(dn, bf, "b.c4k", B, 128)
    b4, b4k = dn("b.bias4", (8, 512), var=0.1), dn("b.bias4k", (8, 128), var=0.1)
    c128 = {nm: dn(f"b.c128.{nm}", (B, 128, 512), bf) for nm in ("Ca", "Za")}
    b128 = dn("b.bias128", (128, 512), var=0.1)
    raw = dn("b.raw", (B, 128, 512), bf)
    rawh = dn("b.rawh", (B, 128, 512), bf)
    q = dn("b.q", (B, 1, 64, 512), bf)
    qh = dn("b.qh", (B, 1, 64, 512), bf)
    w = synth.device_uniform("b.w", (B, 1, 64))
    sink = dn("b.sink", (64,))
    scores = torch.empty(B, 1, N4, dtype=bf, device="cuda")
    idx = torch.empty(B, 1, k, dtype=torch.int32, device="cuda")
    out, outh = torch.empty_like(q), torch.empty_like(qh)
    ws_t = _ws(torch, csa, csa.OP_TOPK, B, 1, N4, k)
    ws_a = _ws(torch, csa, csa.OP_SPARSE_ATTN, B, 1, N4, k)
    ws_h = _ws(torch, csa, csa.OP_HCA_ATTN, B, 1, N128, 0)
    ws_c = _ws(torch, csa, csa.OP_COMPRESS, B, 128, 512, 128)
    wk = Work("csa_hca_decode", "csa_hca_decode: CSA layer (C4A, indexer, top-512, sparse MQA) + HCA layer (C128A, "
              "dense MQA with sink), decode, batch 32 at 65,536 context", B, copies,
              dict(batch=B, context=ctx, c4a_entries=N4, c128a_entries=N128, topk=k, index_keys=keys, rope_dims=rope,
                   attention="batch_invariant" if batch_invariant else "split_kv", cache_copies_rotated=copies),
              "lightning_index")

    def key_job(r):
        j = dict(_c4_job(c4k, b4k, pos4, kb[r] if pairs is None else pairs[r][0], N4 - 1,
                         None if pairs is None else pairs[r][1]), rope_dims=rope)
        return j

    wk.add("compress_c4a_kv_keys", lambda r: csa.csa_compress_batch([
        dict(_c4_job(c4, b4, pos4, kv[r], N4 - 1), rope_dims=rope), key_job(r)]),
        _c4_decode_bytes(B, 512) + _c4_decode_bytes(B, 128, None if pairs is None else kbytes), 0, "hbm")
    if pairs is None:
        wk.add("lightning_index", lambda r: csa.lightning_index(qi, w, kb[r], q_pos0=t, scores=scores),
               B * N4 * 256 + B * 64 * 256 + B * 64 * 4 + B * N4 * 2, B * N4 * 64 * 128 * 2, "hbm")
    else:
        wk.add("lightning_index", lambda r: csa.lightning_index(qq[0], w, pairs[r][0], q_pos0=t, qk_dtype=qk,
                                                                q_scale=qq[1], k_scale=pairs[r][1], scores=scores,
                                                                N=N4),
               B * N4 * kbytes + B * 64 * kbytes + B * 64 * 4 + B * N4 * 2, B * N4 * 64 * 128 * 2, "hbm")
    wk.add("topk_select", lambda r: csa.topk_select(scores, k, q_pos0=t, idx=idx, workspace=ws_t),
           B * N4 * 2 + B * k * 4, 0, "hbm")
    wk.add("sparse_mqa_attn", lambda r: csa.sparse_mqa_attn(q, kv[r], idx, raw, q_pos0=t, raw_pos0=raw0, out=out,
                                                            workspace=ws_a, batch_invariant=batch_invariant,
                                                            rope_dims=rope),
           B * ((k + 128) * 1024 + k * 4 + 2 * 64 * 512 * 2), B * (k + 128) * 64 * 512 * 4, "hbm")
    wk.add("compress_c128a_kv", lambda r: csa.csa_compress(128, c128["Ca"], c128["Za"], b128, pos0=ctx - 128,
                                                           out=kvh[r], cache_entry0=N128 - 1, workspace=ws_c,
                                                           rope_dims=rope),
           B * 128 * 512 * 4 + B * 1024 + 128 * 512 * 4, 0, "hbm")
    wk.add("hca_attn", lambda r: csa.hca_attn(qh, kvh[r], rawh, q_pos0=t, raw_pos0=raw0, sink=sink, out=outh,
                                              workspace=ws_h, batch_invariant=batch_invariant, rope_dims=rope),
           B * ((N128 + 128) * 1024 + 2 * 64 * 512 * 2), B * (N128 + 128) * 64 * 512 * 4, "hbm")
    return wk


def c128a_1m(torch, csa, synth, copies=1):
    bf = torch.bfloat16
    dn = synth.device_normal
    ntok = 1048576
    c = {nm: dn(f"c.{nm}", (1, ntok, 512), bf) for nm in ("Ca", "Za")}
    b128 = dn("c.b", (128, 512), var=0.1)
    out = torch.empty(1, ntok // 128, 512, dtype=bf, device="cuda")
    wk = Work("c128a_1m", "c128a_1m: C128A compress of all 1,048,576 tokens (8,192 entries)", 0, copies,
              dict(tokens=ntok, c128a_entries=ntok // 128), "compress_c128a_kv", unit="raw-tokens/s", units=ntok)
    wk.add("compress_c128a_kv", lambda r: csa.csa_compress(128, c["Ca"], c["Za"], b128, pos0=0, out=out),
           ntok * 512 * 4 + ntok // 128 * 1024 + 128 * 512 * 4, 0, "hbm")
    return wk


def _reindex(torch, csa, synth, decode, copies=1):
    bf = torch.bfloat16
    dn = synth.device_normal
    B, T, N, q0 = (32, 1, 16384, 65535) if decode else (1, 4096, 33792, 131072)
    P, k = 2048, 512
    raw0 = q0 - 127
    keys = dn("r.keys", (B, N, 128), bf)
    # the Full layer (not timed): its own query over every key, top-P
    qf = dn("r.qf", (B, T, 64, 128), bf, var=1.0 / 128)
    wf = synth.device_uniform("r.wf", (B, T, 64))
    sf = csa.lightning_index(qf, wf, keys, q_pos0=q0, score_dtype=bf)
    pool = csa.topk_select(sf, P, q_pos0=q0)
    del sf, qf, wf
    qi = dn("r.qi", (B, T, 64, 128), bf, var=1.0 / 128)
    w = synth.device_uniform("r.w", (B, T, 64))
    kv = dn("r.kv", (B, N, 512), bf)
    q = dn("r.q", (B, T, 64, 512), bf)
    raw = dn("r.raw", (B, T + 127, 512), bf)
    scores = torch.empty(B, T, P, dtype=bf, device="cuda")
    idx = torch.empty(B, T, k, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    ws_a = _ws(torch, csa, csa.OP_SPARSE_ATTN, B, T, N, k)
    nq = B * T
    name = "csa_reindex_decode" if decode else "csa_reindex_prefill"
    wk = Work(name, f"{name}: a Reindex layer of the hierarchical sparse indexer (pool of {P} from a Full layer "
                    f"computed before timing): pool scoring, top-{k} inside the pool, sparse MQA", nq, copies,
              dict(batch=B, chunk=T, context=q0 + 1 if decode else q0 + T, c4a_entries=N, pool=P, topk=k),
              "lightning_index_pool")
    wk.add("lightning_index_pool", lambda r: csa.lightning_index_pool(qi, w, keys, pool, scores=scores),
           nq * (P * 256 + P * 4 + 64 * 128 * 2 + 64 * 4 + P * 2), nq * P * 64 * 128 * 2, "hbm" if decode else "bf16")
    wk.add("topk_select_pool", lambda r: csa.topk_select_pool(scores, pool, k, N=N, idx=idx),
           nq * (P * 2 + P * 4 + k * 4), 0, "hbm")
    wk.add("sparse_mqa_attn", lambda r: csa.sparse_mqa_attn(q, kv, idx, raw, q_pos0=q0, raw_pos0=raw0, out=out,
                                                            workspace=ws_a),
           nq * ((k + 128) * 1024 + k * 4 + 2 * 64 * 512 * 2), nq * (k + 128) * 64 * 512 * 4,
           "hbm" if decode else "bf16")
    return wk


def csa_reindex_decode(torch, csa, synth, copies=1):
    return _reindex(torch, csa, synth, True, copies)


def csa_reindex_prefill(torch, csa, synth, copies=1):
    return _reindex(torch, csa, synth, False, copies)


def csa_paged_decode(torch, csa, synth, copies=1):
    """Decode over the heterogeneous cache: 32 sequences at ragged positions, their
    C4A and C128A entries in shuffled 128-raw-token blocks of two pools under block
    tables, the window in 256-row rings."""
    bf = torch.bfloat16
    dn = synth.device_normal
    B, k, ring = 32, 512, 256
    g = np.random.default_rng(11)
    seq = [int(x) for x in g.integers(49152, 81920, size=B)]
    nblk = [(p + 1) // 128 + 1 for p in seq]
    max_blocks = max(nblk)
    n_pool = sum(nblk)
    perm = g.permutation(n_pool)
    table_np = np.full((B, max_blocks), -1, dtype=np.int32)
    o = 0
    for b in range(B):
        table_np[b, :nblk[b]] = perm[o:o + nblk[b]]
        o += nblk[b]
    table = torch.from_numpy(table_np).cuda()
    pool4 = dn("g.pool4", (n_pool, 32, 512), bf)
    pool128 = dn("g.pool128", (n_pool, 512), bf)
    win = dn("g.win", (B, ring, 512), bf)
    q = dn("g.q", (B, 64, 512), bf)
    qh = dn("g.qh", (B, 64, 512), bf)
    sink = dn("g.sink", (64,))
    sp = torch.tensor(seq, dtype=torch.int64, device="cuda")
    maxp = max(seq)
    out, outh = torch.empty_like(q), torch.empty_like(qh)
    ws_a = _ws(torch, csa, csa.OP_SPARSE_ATTN, B, 1, 1, 0)
    ws_h = _ws(torch, csa, csa.OP_HCA_ATTN, B, 1, 1, 0)
    vh = sum((p + 1) // 128 for p in seq)
    vis4 = sum((p + 1) // 4 for p in seq)
    kpool = dn("g.keys", (n_pool, 32, 128), bf)
    qi = dn("g.qi", (B, 64, 128), bf, var=1.0 / 128)
    wi = synth.device_uniform("g.wi", (B, 64))
    Nmax = 32 * max_blocks
    scores = torch.empty(B, Nmax, dtype=bf, device="cuda")
    idx = torch.empty(B, k, dtype=torch.int32, device="cuda")
    ws_t = _ws(torch, csa, csa.OP_TOPK, B, 1, Nmax, k)
    p0 = torch.tensor([p - p % 4 for p in seq], dtype=torch.int64, device="cuda")
    rb = {nm: dn(f"g.rb.{nm}", (B, 4, 512), bf) for nm in ("Ca", "Za", "pCb", "pZb")}
    rbk = {nm: dn(f"g.rbk.{nm}", (B, 4, 128), bf) for nm in ("Ca", "Za", "pCb", "pZb")}
    b4, b4k = dn("g.b4", (8, 512), var=0.1), dn("g.b4k", (8, 128), var=0.1)
    wk = Work("csa_paged_decode", "csa_paged_decode: CSA + HCA decode over the paged cache, 32 sequences at positions "
              "49,152..81,919: paged compressor writes, paged indexer, per-sequence Top-k, paged sparse MQA and HCA",
              B, copies, dict(batch=B, positions="49152..81919 (seeded)", topk=k, ring=ring, blocks=n_pool),
              "lightning_index_paged")
    # the latent and the indexer key in one launch
    wk.add("compress_paged_kv_keys", lambda r: csa.csa_compress_paged_batch([
        dict(ratio=4, Ca=rb["Ca"], Za=rb["Za"], bias=b4, pool=pool4, block_table=table, pos0=p0,
             prev_Cb=rb["pCb"], prev_Zb=rb["pZb"]),
        dict(ratio=4, Ca=rbk["Ca"], Za=rbk["Za"], bias=b4k, pool=kpool, block_table=table, pos0=p0,
             prev_Cb=rbk["pCb"], prev_Zb=rbk["pZb"])]),
           _c4_decode_bytes(B, 512) + _c4_decode_bytes(B, 128), 0, "hbm")
    wk.add("lightning_index_paged", lambda r: csa.lightning_index_paged(qi, wi, kpool, table, sp, scores=scores),
           vis4 * 256 + B * 64 * 128 * 2 + B * 64 * 4 + B * Nmax * 2, vis4 * 64 * 128 * 2, "hbm")
    wk.add("topk_select_paged", lambda r: csa.topk_select_paged(scores, k, sp, idx=idx, workspace=ws_t),
           B * Nmax * 2 + B * k * 4, 0, "hbm")
    wk.add("sparse_mqa_attn_paged", lambda r: csa.sparse_mqa_attn_paged(q, pool4, table, idx, win, sp, max_pos=maxp,
                                                                        out=out, workspace=ws_a),
           B * ((k + 128) * 1024 + k * 4 + 2 * 64 * 512 * 2), B * (k + 128) * 64 * 512 * 4, "hbm")
    wk.add("hca_attn_paged", lambda r: csa.hca_attn_paged(qh, pool128, table, win, sp, sink=sink, max_pos=maxp,
                                                          out=outh, workspace=ws_h),
           (vh + B * 128) * 1024 + B * 2 * 64 * 512 * 2, (vh + B * 128) * 64 * 512 * 4, "hbm")
    return wk


def csa_1m_decode_separate(torch, csa, synth, copies=4):
    """The 1M-context Pro decode with the compressor in a launch of its own (A/B
    against the headline's single launch)."""
    return csa_1m_decode(torch, csa, synth, copies=copies, fuse=False)


def csa_paged_1m_decode(torch, csa, synth, copies=2):
    """The 1M-context Pro decode over the heterogeneous cache: 8 sequences at ragged
    positions near 1,048,576, their C4A latents (bf16) and MXFP4 keys in shuffled
    32-entry blocks of two pools under block tables, the window in 256-row rings;
    paged compressor writes (latent, and the key quantized on write to MXFP4), the
    paged MXFP4 indexer, per-sequence top-1024, paged sparse MQA.  Key pools and
    their block tables are rotated over `copies` seeded copies (more than the
    Infinity Cache in all)."""
    bf = torch.bfloat16
    dn = synth.device_normal
    B, k, ring = 8, 1024, 256
    g = np.random.default_rng(13)
    seq = [int(x) for x in g.integers(1040384, 1048576, size=B)]
    nblk = [(p + 1) // 128 + 1 for p in seq]
    max_blocks = max(nblk)
    n_pool = sum(nblk)
    tables, kpools, kscales = [], [], []
    for r in range(copies):
        perm = g.permutation(n_pool)
        t_np = np.full((B, max_blocks), -1, dtype=np.int32)
        o = 0
        for b in range(B):
            t_np[b, :nblk[b]] = perm[o:o + nblk[b]]
            o += nblk[b]
        tables.append(torch.from_numpy(t_np).cuda())
        x = dn(f"pm.keys.{r}", (n_pool, 32, 128))
        a, sc = synth.device_quant_mxfp4(x)
        del x
        kpools.append(a)
        kscales.append(sc)
    pool4 = dn("pm.pool4", (n_pool, 32, 512), bf)
    win = dn("pm.win", (B, ring, 512), bf)
    q = dn("pm.q", (B, 64, 512), bf)
    sp = torch.tensor(seq, dtype=torch.int64, device="cuda")
    maxp = max(seq)
    out = torch.empty_like(q)
    ws_a = _ws(torch, csa, csa.OP_SPARSE_ATTN, B, 1, 1, 0)
    vis4 = sum((p + 1) // 4 for p in seq)
    qp, qs = synth.device_quant_mxfp4(dn("pm.qi", (B, 64, 128)))
    wi = synth.device_uniform("pm.wi", (B, 64))
    Nmax = 32 * max_blocks
    scores = torch.empty(B, Nmax, dtype=bf, device="cuda")
    idx = torch.empty(B, k, dtype=torch.int32, device="cuda")
    ws_t = _ws(torch, csa, csa.OP_TOPK, B, 1, Nmax, k)
    p0 = torch.tensor([p - p % 4 for p in seq], dtype=torch.int64, device="cuda")
    rb = {nm: dn(f"pm.rb.{nm}", (B, 4, 512), bf) for nm in ("Ca", "Za", "pCb", "pZb")}
    rbk = {nm: dn(f"pm.rbk.{nm}", (B, 4, 128), bf) for nm in ("Ca", "Za", "pCb", "pZb")}
    b4, b4k = dn("pm.b4", (8, 512), var=0.1), dn("pm.b4k", (8, 128), var=0.1)
    wk = Work("csa_paged_1m_decode", "csa_paged_1m_decode: the 1M-context Pro decode over the paged cache, 8 sequences "
              "at positions 1,040,384..1,048,575: paged compressor writes (latent bf16, key MXFP4), paged MXFP4 "
              "indexer, per-sequence top-1024, paged sparse MQA", B, copies,
              dict(batch=B, positions="1040384..1048575 (seeded)", topk=k, ring=ring, blocks=n_pool,
                   index_qk="mxfp4", key_pool_copies_rotated=copies),
              "lightning_index_paged")
    # the bf16 latent and the MXFP4 indexer key in one launch
    wk.add("compress_paged_kv_keys", lambda r: csa.csa_compress_paged_batch([
        dict(ratio=4, Ca=rb["Ca"], Za=rb["Za"], bias=b4, pool=pool4, block_table=tables[r], pos0=p0,
             prev_Cb=rb["pCb"], prev_Zb=rb["pZb"]),
        dict(ratio=4, Ca=rbk["Ca"], Za=rbk["Za"], bias=b4k, pool=kpools[r], block_table=tables[r], pos0=p0,
             prev_Cb=rbk["pCb"], prev_Zb=rbk["pZb"], scale_pool=kscales[r])]),
           _c4_decode_bytes(B, 512) + _c4_decode_bytes(B, 128, 64 + 4), 0, "hbm")
    wk.add("lightning_index_paged", lambda r: csa.lightning_index_paged(qp, wi, kpools[r], tables[r], sp,
                                                                        qk_dtype=csa.MXFP4, q_scale=qs,
                                                                        k_scale=kscales[r], scores=scores),
           vis4 * 68 + B * 64 * 68 + B * 64 * 4 + B * Nmax * 2, vis4 * 64 * 128 * 2, "hbm")
    wk.add("topk_select_paged", lambda r: csa.topk_select_paged(scores, k, sp, idx=idx, workspace=ws_t),
           B * Nmax * 2 + B * k * 4, 0, "hbm")
    wk.add("sparse_mqa_attn_paged", lambda r: csa.sparse_mqa_attn_paged(q, pool4, tables[r], idx, win, sp,
                                                                        max_pos=maxp, out=out, workspace=ws_a),
           B * ((k + 128) * 1024 + k * 4 + 2 * 64 * 512 * 2), B * (k + 128) * 64 * 512 * 4, "hbm")
    return wk


def hbm_copy(torch, csa, synth, copies=1):
    """A 1 GiB device copy: the calibration point of the HBM byte counters."""
    n = 1 << 28
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    wk = Work("hbm_copy", "hbm_copy: a 1 GiB device-to-device copy", 0, copies,
              dict(bytes_read=n * 4, bytes_written=n * 4), "copy_1GiB", unit="GB/s", units=2 * n * 4 / 1e9)
    wk.add("copy_1GiB", lambda r: y.copy_(x), 2 * n * 4, 0, "hbm")
    return wk


def hbm_read(torch, csa, synth, copies=4):
    """A plain streaming read (libcsa_probe.so) of as many bytes as the 1M decode's
    MXFP4 keys and scales, over rotating buffers: what a kernel that only reads
    HBM attains on this machine, beside the 8 TB/s peak."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(os.path.dirname(os.path.abspath(csa.__file__)), "libcsa_probe.so"))
    lib.csa_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_void_p]
    nbytes = 8 * 262144 * (64 + 4)
    grid = 1024
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(r + 1) for r in range(copies)]
    out = torch.empty(grid * 256, dtype=torch.int32, device="cuda")

    def run(r):
        st = torch.cuda.current_stream().cuda_stream
        assert lib.csa_probe_stream_read(bufs[r].data_ptr(), nbytes, out.data_ptr(), grid, ctypes.c_void_p(st)) == 0

    wk = Work("hbm_read", f"hbm_read: a streaming read of {nbytes:,} bytes (the 1M decode's MXFP4 keys and scales), "
              f"{copies} rotating buffers", 0, copies, dict(bytes_read=nbytes, grid=grid), "stream_read",
              unit="GB/s", units=nbytes / 1e9)
    wk.add("stream_read", run, nbytes, 0, "hbm")
    return wk


EXTRAS = {"csa_hca_decode": csa_hca_decode, "c128a_1m": c128a_1m, "csa_reindex_decode": csa_reindex_decode,
          "csa_reindex_prefill": csa_reindex_prefill, "csa_paged_decode": csa_paged_decode,
          "csa_paged_1m_decode": csa_paged_1m_decode, "csa_1m_decode_separate": csa_1m_decode_separate,
          "hca_decode_separate": hca_decode_separate, "csa_decode_separate": csa_decode_separate,
          "hbm_copy": hbm_copy,
          "hbm_read": hbm_read}
