"""Per-workload benchmark lines (``bench.py --workload NAME``).

Each workload is one pass of its stages over synthetic inputs resident in
HBM, captured in a HIP graph and replayed; every stage is also timed alone
(graph of repeated launches) to give its average kernel time and roofline.

  csa_prefill    1 sequence, 131,072 tokens of context + a 4,096-token chunk:
                 C4A compress of the chunk (512-d KV and 128-d keys in one launch),
                 fp8 indexer over 4,096 x 33,792, top-512, sparse MQA
  hca_decode     16 sequences at 1,048,576 context: C128A compress of the
                 last block, dense MQA with sink over 8,192 entries + window
  hca_prefill    the last 2,048 tokens of a 1,048,576 context: C128A compress
                 of the chunk, dense MQA with sink
  csa_1m_decode  8 sequences at 1,048,576 context: C4A compress (the KV latent, and
                 the key quantized on write into the MXFP4 cache),
                 MXFP4 indexer over 262,144 keys, top-1024, sparse MQA
  c128a_1m       C128A compress of all 1,048,576 tokens (8,192 entries)
  csa_reindex_decode / csa_reindex_prefill
                 a Reindex layer of the hierarchical sparse indexer: the pool
                 (2,048 entries per query) comes from a Full layer computed once
                 before timing (bf16 indexer + top-2,048); timed: pool scoring,
                 top-512 inside the pool, sparse MQA.  Decode: 32 sequences at
                 65,536 context (16,384 entries); prefill: the 4,096-token chunk
                 after 131,072 tokens (33,792 entries)
  csa_paged_decode
                 decode over the heterogeneous cache: 32 sequences at ragged
                 positions (49,152 .. 81,919; mean about 65,536), their C4A and
                 C128A entries in shuffled 128-raw-token blocks of two pools
                 under block tables, the window in 256-row rings: the paged
                 compressor write of every sequence's block (latent and key),
                 the paged indexer over bf16 keys, Top-k per sequence, sparse
                 MQA over the top-512 and HCA with sink, one query per sequence
  hbm_copy       a 1 GiB copy, the calibration point of the HBM byte counters
"""
from __future__ import annotations

import numpy as np

HBM = 8000.0
PEAK = {"bf16": 2500.0, "fp8": 5000.0, "mxfp4": 10100.0}


def _gtime(torch, st, fn, reps):
    with torch.cuda.stream(st):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            for _ in range(reps):
                fn()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        g.replay()
        e1.record(st)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps   # ms


def _quant_fp8_dev(torch, x):
    """Per-row E4M3 encoding on the device (input preparation, same rule as
    synth.quant_fp8_rows: scale = amax / 448, round to nearest even)."""
    amax = x.abs().amax(dim=-1).clamp_min(1e-30)
    scale = (amax / 448.0).float()
    codes = (x / scale[..., None]).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.contiguous()


def _rand_mxfp4_dev(torch, name, shape_rows, synth):
    """Random MXFP4 bytes: E2M1 nibbles drawn uniformly, E8M0 scales near 2^-2
    (the scale N(0,1) data gets).  Used only for throughput."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(synth.torch_seed(name))
    packed = torch.randint(0, 256, (*shape_rows, 64), generator=gen, device="cuda", dtype=torch.uint8)
    scales = torch.randint(125, 128, (*shape_rows, 4), generator=gen, device="cuda", dtype=torch.uint8)
    return packed, scales


def _etime(torch, st, fn, reps):
    """Eager launches between two events (the counter runs: kernels launched
    inside a graph are not seen by the profiler's counter collection)."""
    with torch.cuda.stream(st):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps   # ms


def run(args, torch, csa, synth):
    bf = torch.bfloat16
    dn = synth.device_normal
    st = torch.cuda.Stream()
    wl = args.workload
    stages = []          # (name, fn, alg_bytes, alg_flops, bound)
    queries = 0
    info = {}
    if wl == "csa_prefill":
        T, N, k, q0 = 4096, 33792, 512, 131072
        raw0 = q0 - 127
        c = {nm: dn(f"p.{nm}", (1, T, 512), bf) for nm in ("Ca", "Za", "Cb", "Zb")}
        ck = {nm: dn(f"p.k{nm}", (1, T, 128), bf) for nm in ("Ca", "Za", "Cb", "Zb")}
        h = {nm: dn(f"p.h{nm}", (1, 4, 512), bf) for nm in ("Cb", "Zb")}
        hk = {nm: dn(f"p.hk{nm}", (1, 4, 128), bf) for nm in ("Cb", "Zb")}
        b4, b4k = dn("p.b4", (8, 512), var=0.1), dn("p.b4k", (8, 128), var=0.1)
        kv = dn("p.kv", (1, N, 512), bf)
        keys_bf = torch.empty(1, N, 128, dtype=bf, device="cuda")
        qc, qs = _quant_fp8_dev(torch, dn("p.qi", (1, T, 64, 128)))
        kc, ks = _quant_fp8_dev(torch, dn("p.ki", (1, N, 128)))
        w = synth.device_uniform("p.w", (1, T, 64))
        q = dn("p.q", (1, T, 64, 512), bf)
        raw = dn("p.raw", (1, q0 + T - raw0, 512), bf)
        scores = torch.empty(1, T, N, dtype=bf, device="cuda")
        idx = torch.empty(1, T, k, dtype=torch.int32, device="cuda")
        out = torch.empty_like(q)
        n_vis = sum(min((q0 + t + 1) // 4, N) for t in range(T))
        stages = [
            ("compress_c4a_kv_keys", lambda: csa.csa_compress_batch([
                dict(ratio=4, Ca=c["Ca"], Za=c["Za"], bias=b4, Cb=c["Cb"], Zb=c["Zb"], prev_Cb=h["Cb"], prev_Zb=h["Zb"],
                     pos0=q0, out=kv, cache_entry0=q0 // 4),
                dict(ratio=4, Ca=ck["Ca"], Za=ck["Za"], bias=b4k, Cb=ck["Cb"], Zb=ck["Zb"], prev_Cb=hk["Cb"],
                     prev_Zb=hk["Zb"], pos0=q0, out=keys_bf, cache_entry0=q0 // 4)]),
             T * 4 * (512 + 128) * 2 + T // 4 * (512 + 128) * 2, 0, "hbm"),
            ("lightning_index", lambda: csa.lightning_index(qc, w, kc, q_pos0=q0, qk_dtype=csa.FP8_E4M3, q_scale=qs,
                                                            k_scale=ks, scores=scores),
             T * 64 * 132 + N * 132 + T * N * 2, n_vis * 64 * 128 * 2, "fp8"),
            ("topk_select", lambda: csa.topk_select(scores, k, q_pos0=q0, idx=idx), T * N * 2 + T * k * 4, 0, "hbm"),
            ("sparse_mqa_attn", lambda: csa.sparse_mqa_attn(q, kv, idx, raw, q_pos0=q0, raw_pos0=raw0, out=out),
             T * (k * 4 + 2 * 64 * 512 * 2) + (N + raw.shape[1]) * 1024, T * (k + 128) * 64 * 512 * 4, "bf16"),
        ]
        queries = T
        info = dict(batch=1, context=q0, chunk=T, c4a_entries=N, topk=k, indexer="fp8_e4m3")
    elif wl in ("hca_decode", "hca_prefill"):
        dec = wl == "hca_decode"
        B, T = (16, 1) if dec else (1, 2048)
        N = 8192
        q0 = 1048575 if dec else 1046528
        raw0 = q0 - 127
        cpos = q0 + 1 - 128 if dec else q0
        ntok = 128 if dec else T
        c = {nm: dn(f"h.{nm}", (B, ntok, 512), bf) for nm in ("Ca", "Za")}
        b128 = dn("h.b", (128, 512), var=0.1)
        kv = dn("h.kv", (B, N, 512), bf)
        q = dn("h.q", (B, T, 64, 512), bf)
        raw = dn("h.raw", (B, q0 + T - raw0, 512), bf)
        sink = dn("h.sink", (64,))
        out = torch.empty_like(q)
        ws = torch.empty(max(16, csa.workspace_bytes(csa.OP_HCA_ATTN, B, T, N, 0)), dtype=torch.uint8, device="cuda")
        wsc = torch.empty(max(16, csa.workspace_bytes(csa.OP_COMPRESS, B, ntok, 512, 128)), dtype=torch.uint8,
                          device="cuda")
        rows = sum(min((q0 + t + 1) // 128, N) + 128 for t in range(T))
        stages = [
            ("compress_c128a_kv", lambda: csa.csa_compress(128, c["Ca"], c["Za"], b128, pos0=cpos, out=kv,
                                                           cache_entry0=cpos // 128, workspace=wsc),
             B * ntok * 512 * 4 + B * ntok // 128 * 1024, 0, "hbm"),
            ("hca_attn", lambda: csa.hca_attn(q, kv, raw, q_pos0=q0, raw_pos0=raw0, sink=sink, out=out, workspace=ws),
             (B * rows * 1024 if dec else (N + raw.shape[1]) * 1024) + B * T * 2 * 64 * 512 * 2,
             B * rows * 64 * 512 * 4, "hbm" if dec else "bf16"),
        ]
        queries = B * T
        info = dict(batch=B, context=q0 + 1 if dec else 1048576, chunk=T, c128a_entries=N)
    elif wl == "csa_1m_decode":
        B, N, k, q0 = 8, 262144, 1024, 1048575
        raw0 = q0 - 127
        c = {nm: dn(f"m.{nm}", (B, 4, 512), bf) for nm in ("Ca", "Za", "Cb", "Zb", "pCb", "pZb")}
        ck = {nm: dn(f"m.k{nm}", (B, 4, 128), bf) for nm in ("Ca", "Za", "Cb", "Zb", "pCb", "pZb")}
        b4, b4k = dn("m.b4", (8, 512), var=0.1), dn("m.b4k", (8, 128), var=0.1)
        kv = dn("m.kv", (B, N, 512), bf)
        kp, ksc = _rand_mxfp4_dev(torch, "m.keys", (B, N), synth)
        qp, qsc = _rand_mxfp4_dev(torch, "m.qi", (B, 1, 64), synth)
        w = synth.device_uniform("m.w", (B, 1, 64))
        q = dn("m.q", (B, 1, 64, 512), bf)
        raw = dn("m.raw", (B, 128, 512), bf)
        scores = torch.empty(B, 1, N, dtype=bf, device="cuda")
        idx = torch.empty(B, 1, k, dtype=torch.int32, device="cuda")
        out = torch.empty_like(q)
        ws_t = torch.empty(max(16, csa.workspace_bytes(csa.OP_TOPK, B, 1, N, k)), dtype=torch.uint8, device="cuda")
        ws_a = torch.empty(max(16, csa.workspace_bytes(csa.OP_SPARSE_ATTN, B, 1, N, k)), dtype=torch.uint8,
                           device="cuda")
        stages = [
            ("compress_c4a_kv_keys", lambda: csa.csa_compress_batch([
                dict(ratio=4, Ca=c["Ca"], Za=c["Za"], bias=b4, Cb=c["Cb"], Zb=c["Zb"], prev_Cb=c["pCb"],
                     prev_Zb=c["pZb"], pos0=q0 - 3, out=kv, cache_entry0=N - 1),
                # the new key quantized on write into its MXFP4 cache slot
                dict(ratio=4, Ca=ck["Ca"], Za=ck["Za"], bias=b4k, Cb=ck["Cb"], Zb=ck["Zb"], prev_Cb=ck["pCb"],
                     prev_Zb=ck["pZb"], pos0=q0 - 3, out=kp, out_scale=ksc, cache_entry0=N - 1)]),
             B * 24 * (512 + 128) * 2 + B * (512 * 2 + 64 + 4) + 8 * (512 + 128) * 4, 0, "hbm"),
            ("lightning_index", lambda: csa.lightning_index(qp, w, kp, q_pos0=q0, qk_dtype=csa.MXFP4, q_scale=qsc,
                                                            k_scale=ksc, scores=scores, N=N),
             B * N * 68 + B * 64 * 68 + B * N * 2, B * N * 64 * 128 * 2, "hbm"),
            ("topk_select", lambda: csa.topk_select(scores, k, q_pos0=q0, idx=idx, workspace=ws_t),
             B * N * 2 + B * k * 4, 0, "hbm"),
            ("sparse_mqa_attn", lambda: csa.sparse_mqa_attn(q, kv, idx, raw, q_pos0=q0, raw_pos0=raw0, out=out,
                                                            workspace=ws_a),
             B * ((k + 128) * 1024 + k * 4 + 2 * 64 * 512 * 2), B * (k + 128) * 64 * 512 * 4, "hbm"),
        ]
        queries = B
        info = dict(batch=B, context=q0 + 1, c4a_entries=N, topk=k, indexer="mxfp4")
    elif wl == "c128a_1m":
        ntok = 1048576
        c = {nm: dn(f"c.{nm}", (1, ntok, 512), bf) for nm in ("Ca", "Za")}
        b128 = dn("c.b", (128, 512), var=0.1)
        out = torch.empty(1, ntok // 128, 512, dtype=bf, device="cuda")
        stages = [("compress_c128a_kv", lambda: csa.csa_compress(128, c["Ca"], c["Za"], b128, pos0=0, out=out),
                   ntok * 512 * 4 + ntok // 128 * 1024, 0, "hbm")]
        queries = 0
        info = dict(tokens=ntok, c128a_entries=ntok // 128)
    elif wl in ("csa_reindex_decode", "csa_reindex_prefill"):
        dec = wl == "csa_reindex_decode"
        B, T, N, q0 = (32, 1, 16384, 65535) if dec else (1, 4096, 33792, 131072)
        P, k = 2048, 512
        raw0 = q0 - 127
        keys = dn("r.keys", (B, N, 128), bf)
        # the Full layer (untimed): its own query over every key, top-P
        qf = dn("r.qf", (B, T, 64, 128), bf, var=1.0 / 128)
        wf = synth.device_uniform("r.wf", (B, T, 64))
        sf = csa.lightning_index(qf, wf, keys, q_pos0=q0, score_dtype=bf)
        pool = csa.topk_select(sf, P, q_pos0=q0)
        del sf, qf, wf
        # the Reindex layer
        qi = dn("r.qi", (B, T, 64, 128), bf, var=1.0 / 128)
        w = synth.device_uniform("r.w", (B, T, 64))
        kv = dn("r.kv", (B, N, 512), bf)
        q = dn("r.q", (B, T, 64, 512), bf)
        raw = dn("r.raw", (B, T + 127, 512), bf)
        scores = torch.empty(B, T, P, dtype=bf, device="cuda")
        idx = torch.empty(B, T, k, dtype=torch.int32, device="cuda")
        out = torch.empty_like(q)
        ws_a = torch.empty(max(16, csa.workspace_bytes(csa.OP_SPARSE_ATTN, B, T, N, k)), dtype=torch.uint8,
                           device="cuda")
        nq = B * T
        stages = [
            ("lightning_index_pool", lambda: csa.lightning_index_pool(qi, w, keys, pool, scores=scores),
             nq * (P * 256 + P * 4 + 64 * 128 * 2 + 64 * 4 + P * 2), nq * P * 64 * 128 * 2, "hbm" if dec else "bf16"),
            ("topk_select_pool", lambda: csa.topk_select_pool(scores, pool, k, N=N, idx=idx),
             nq * (P * 2 + 2 * k * 4), 0, "hbm"),
            ("sparse_mqa_attn", lambda: csa.sparse_mqa_attn(q, kv, idx, raw, q_pos0=q0, raw_pos0=raw0, out=out,
                                                            workspace=ws_a),
             nq * ((k + 128) * 1024 + k * 4 + 2 * 64 * 512 * 2), nq * (k + 128) * 64 * 512 * 4,
             "hbm" if dec else "bf16"),
        ]
        queries = nq
        info = dict(batch=B, chunk=T, context=q0 + 1 if dec else q0 + T, c4a_entries=N, pool=P, topk=k)
    elif wl == "csa_paged_decode":
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
        idx_np = np.stack([np.sort(g.choice((p + 1) // 4, size=k, replace=False)) for p in seq]).astype(np.int32)
        idx = torch.from_numpy(idx_np).cuda()
        sp = torch.tensor(seq, dtype=torch.int64, device="cuda")
        maxp = max(seq)
        out, outh = torch.empty_like(q), torch.empty_like(qh)
        ws_a = torch.empty(max(16, csa.workspace_bytes(csa.OP_SPARSE_ATTN, B, 1, 1, 0)), dtype=torch.uint8,
                           device="cuda")
        ws_h = torch.empty(max(16, csa.workspace_bytes(csa.OP_HCA_ATTN, B, 1, 1, 0)), dtype=torch.uint8,
                           device="cuda")
        vh = sum((p + 1) // 128 for p in seq)
        vis4 = sum((p + 1) // 4 for p in seq)
        kpool = dn("g.keys", (n_pool, 32, 128), bf)
        qi = dn("g.qi", (B, 64, 128), bf, var=1.0 / 128)
        wi = synth.device_uniform("g.wi", (B, 64))
        Nmax = 32 * max_blocks
        scores = torch.empty(B, Nmax, dtype=bf, device="cuda")
        idx2 = torch.empty(B, k, dtype=torch.int32, device="cuda")
        ws_t = torch.empty(max(16, csa.workspace_bytes(csa.OP_TOPK, B, 1, Nmax, k)), dtype=torch.uint8,
                           device="cuda")
        # the decode write: every sequence's current block (the most a step does)
        p0 = torch.tensor([p - p % 4 for p in seq], dtype=torch.int64, device="cuda")
        rb = {nm: dn(f"g.rb.{nm}", (B, 4, 512), bf) for nm in ("Ca", "Za", "pCb", "pZb")}
        rbk = {nm: dn(f"g.rbk.{nm}", (B, 4, 128), bf) for nm in ("Ca", "Za", "pCb", "pZb")}
        b4, b4k = dn("g.b4", (8, 512), var=0.1), dn("g.b4k", (8, 128), var=0.1)
        stages = [
            ("compress_paged_kv", lambda: csa.csa_compress_paged(4, rb["Ca"], rb["Za"], b4, pool4, table, p0,
                                                                 prev_Cb=rb["pCb"], prev_Zb=rb["pZb"]),
             B * 12 * 512 * 2 + B * 512 * 2 + 8 * 512 * 4, 0, "hbm"),
            ("compress_paged_keys", lambda: csa.csa_compress_paged(4, rbk["Ca"], rbk["Za"], b4k, kpool, table, p0,
                                                                   prev_Cb=rbk["pCb"], prev_Zb=rbk["pZb"]),
             B * 12 * 128 * 2 + B * 128 * 2 + 8 * 128 * 4, 0, "hbm"),
            ("lightning_index_paged", lambda: csa.lightning_index_paged(qi, wi, kpool, table, sp, scores=scores),
             vis4 * 256 + B * 64 * 128 * 2 + B * 64 * 4 + B * Nmax * 2, vis4 * 64 * 128 * 2, "hbm"),
            ("topk_select_paged", lambda: csa.topk_select_paged(scores, k, sp, idx=idx2, workspace=ws_t),
             B * Nmax * 2 + B * k * 4, 0, "hbm"),
            ("sparse_mqa_attn_paged", lambda: csa.sparse_mqa_attn_paged(q, pool4, table, idx, win, sp, max_pos=maxp,
                                                                        out=out, workspace=ws_a),
             B * ((k + 128) * 1024 + k * 4 + 2 * 64 * 512 * 2), B * (k + 128) * 64 * 512 * 4, "hbm"),
            ("hca_attn_paged", lambda: csa.hca_attn_paged(qh, pool128, table, win, sp, sink=sink, max_pos=maxp,
                                                          out=outh, workspace=ws_h),
             (vh + B * 128) * 1024 + B * 2 * 64 * 512 * 2, (vh + B * 128) * 64 * 512 * 4, "hbm"),
        ]
        queries = B
        info = dict(batch=B, positions="49152..81919 (seeded)", topk=k, ring=ring, blocks=n_pool)
    elif wl == "hbm_copy":
        # 1 GiB device-to-device copy: the reference point that turns the HBM
        # traffic counters (FETCH_SIZE, WRITE_SIZE) into bytes
        n = 1 << 28
        x = torch.ones(n, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        stages = [("copy_1GiB", lambda: y.copy_(x), 2 * n * 4, 0, "hbm")]
        queries = 0
        info = dict(bytes_read=n * 4, bytes_written=n * 4)
    else:
        raise SystemExit(f"unknown workload {wl}")

    # whole pass
    def whole():
        for s in stages:
            s[1]()

    timer = _etime if args.eager else _gtime
    ms = timer(torch, st, whole, max(2, min(args.steps, 20)))
    per = {}
    best = None
    for name, fn, nbytes, flops, bound in stages:
        t = timer(torch, st, fn, max(2, min(args.steps, 20)))
        gbs = nbytes / (t * 1e-3) / 1e9
        tfl = flops / (t * 1e-3) / 1e12 if flops else None
        if bound == "hbm":
            frac = gbs / HBM
            roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM, "unit": "GB/s"}
        else:
            frac = tfl / PEAK[bound]
            roof = {"bound": "mfma", "achieved": round(tfl, 1), "peak": PEAK[bound], "unit": "TFLOP/s",
                    "dtype": bound}
        roof["frac"] = round(frac, 4)
        per[name] = {"us": round(t * 1e3, 2), "GB/s": round(gbs, 1), "TFLOP/s": round(tfl, 2) if tfl else None,
                     "roofline": roof}
        if best is None or t > best[1]:
            best = (name, t, roof, nbytes)
    name, t, roof, nbytes = best
    roof = dict(roof, kernel=name, traffic=None, avg_launch_us=round(t * 1e3, 2), algorithmic_bytes_per_launch=nbytes)
    if wl == "hbm_copy":
        value, unit = nbytes / (ms * 1e-3) / 1e9, "GB/s"
    elif queries:
        value, unit = queries / (ms * 1e-3), "query-tokens/s"
    else:
        value, unit = 1048576 / (ms * 1e-3), "raw-tokens/s"
    return {
        "metric": "CSA/HCA query-tokens/s at 1 GPU; % peak HBM GB/s (decode), % MFMA (prefill)",
        "value": round(value, 1),
        "unit": unit,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "config": dict(workload=wl, **info, timing="eager" if args.eager else "hip_graph"),
        "roofline": roof, "stages": per,
    }
