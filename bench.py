#!/usr/bin/env python3
"""Benchmark of the compressed sparse attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload (one "step"): a decode step of one CSA layer and one HCA
layer for 32 sequences at 65,536 tokens of context (16,384 C4A entries,
512 C128A entries per sequence), all inputs synthetic and resident in HBM:

  CSA layer   csa_compress (C4A, 512-d KV, into cache entry 16,383)
              csa_compress (C4A, 128-d indexer keys, same slot)
              lightning_index (64 x 128 bf16 heads over 16,384 bf16 keys)
              topk_select (k = 512 over the bf16 scores)
              sparse_mqa_attn (64 x 512 heads over 512 entries + 128 window)
  HCA layer   csa_compress (C128A, 128 raw tokens into cache entry 511)
              hca_attn (64 x 512 heads over 512 entries + 128 window, sink)

Throughput is query tokens per second over the whole step.  Caches are
rotated over several copies (more than the 256 MB Infinity Cache in total)
so every step reads its keys and rows from HBM.  The step is captured in a
HIP graph per cache copy (launch overhead excluded; pass --eager to time
eager launches).  A second, eager pass brackets every stage with events on
the stream the kernels run on, to get each kernel's average duration; the
dominant kernel's roofline figure uses the algorithmic bytes of one launch.

The CPU baseline times the oracle (NumPy fp64, test infrastructure) on a
bounded sample of the same step's query tokens.

Other workloads (--workload): csa_prefill, hca_decode, hca_prefill,
csa_1m_decode, c128a_1m, csa_reindex_decode, csa_reindex_prefill,
csa_paged_decode -- each prints its own JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
FP4_PEAK_TFLOPS = 10100.0
METRIC = "CSA/HCA query-tokens/s at 1 GPU; % peak HBM GB/s (decode), % MFMA (prefill)"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="csa_hca_decode")
    p.add_argument("--rotate", type=int, default=4, help="cache copies cycled over the steps")
    p.add_argument("--eager", action="store_true",
                   help="time eager launches instead of HIP graphs (every workload; the counter runs need it)")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the CPU oracle sample")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--batch-invariant", action="store_true",
                   help="attention in batch-invariant mode (no row split; default workload only)")
    p.add_argument("--keys", choices=("bf16", "fp8", "fp4"), default="bf16",
                   help="index keys: bf16, or quantized on write (in the latent's compressor launch) to fp8 E4M3 "
                        "or MXFP4 and scored by the indexer of that format (default workload only)")
    p.add_argument("--fp8-keys", dest="keys", action="store_const", const="fp8", help="same as --keys fp8")
    p.add_argument("--rope", type=int, default=0,
                   help="partial RoPE dims fused into the compressors and the attention epilogues "
                        "(default workload only; 0 = none)")
    return p.parse_args()


# ---------------------------------------------------------------- workloads


class DecodeStep:
    """One CSA layer + one HCA layer decode step for B sequences at `ctx` context."""

    def __init__(self, csa, synth, torch, B=32, ctx=65536, k=512, rotate=4, batch_invariant=False, rope=0,
                 keys="bf16"):
        self.csa, self.torch = csa, torch
        self.bi = batch_invariant
        self.rope = rope
        self.kfmt = keys
        bf = torch.bfloat16
        dn = synth.device_normal
        self.B, self.ctx, self.k = B, ctx, k
        self.N4, self.N128 = ctx // 4, ctx // 128
        self.t = ctx - 1                    # the query token completes the last block
        self.raw0 = self.t - 127
        B, N4, N128 = self.B, self.N4, self.N128
        # per-copy caches (rotated)
        self.kv = [dn(f"b.kv.{r}", (B, N4, 512), bf) for r in range(rotate)]
        self.keys = [dn(f"b.keys.{r}", (B, N4, 128), bf) for r in range(rotate)]
        self.kvh = [dn(f"b.kvh.{r}", (B, N128, 512), bf) for r in range(rotate)]
        # per-step inputs: the last block's compressor projections, the window, queries
        self.c4 = {nm: dn(f"b.c4.{nm}", (B, 4, 512), bf) for nm in ("Ca", "Za", "Cb", "Zb", "pCb", "pZb")}
        self.c4k = {nm: dn(f"b.c4k.{nm}", (B, 4, 128), bf) for nm in ("Ca", "Za", "Cb", "Zb", "pCb", "pZb")}
        self.b4 = dn("b.bias4", (8, 512), var=0.1)
        self.b4k = dn("b.bias4k", (8, 128), var=0.1)
        self.c128 = {nm: dn(f"b.c128.{nm}", (B, 128, 512), bf) for nm in ("Ca", "Za")}
        self.b128 = dn("b.bias128", (128, 512), var=0.1)
        self.raw = dn("b.raw", (B, 128, 512), bf)
        self.rawh = dn("b.rawh", (B, 128, 512), bf)
        self.q = dn("b.q", (B, 1, 64, 512), bf)
        self.qh = dn("b.qh", (B, 1, 64, 512), bf)
        self.qi = dn("b.qi", (B, 1, 64, 128), bf, var=1.0 / 128)
        if keys == "fp8":
            # the key caches as fp8 codes + row scales (input preparation of the
            # resident cache; the step itself writes its new key quantized)
            self.keys, self.kscale = zip(*[_quant_fp8(torch, kk) for kk in self.keys])
            self.qi8, self.qscale = _quant_fp8(torch, self.qi)
        elif keys == "fp4":
            # MXFP4 codes (two per byte) + one E8M0 byte per 32 dims, same preparation
            self.keys, self.kscale = zip(*[_quant_mxfp4(torch, kk) for kk in self.keys])
            self.qi8, self.qscale = _quant_mxfp4(torch, self.qi)
        self.w = synth.device_uniform("b.w", (B, 1, 64))
        self.sink = dn("b.sink", (64,))
        # outputs and workspaces
        self.scores = torch.empty(B, 1, N4, dtype=bf, device="cuda")
        self.idx = torch.empty(B, 1, k, dtype=torch.int32, device="cuda")
        self.out = torch.empty(B, 1, 64, 512, dtype=bf, device="cuda")
        self.outh = torch.empty(B, 1, 64, 512, dtype=bf, device="cuda")
        self.ws_topk = self._ws(csa.OP_TOPK, N4, k)
        self.ws_attn = self._ws(csa.OP_SPARSE_ATTN, N4, k)
        self.ws_hca = self._ws(csa.OP_HCA_ATTN, N128, 0)
        n = csa.workspace_bytes(csa.OP_COMPRESS, B, 128, 512, 128)
        self.ws_c128 = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")

    def _ws(self, op, N, k):
        n = self.csa.workspace_bytes(op, self.B, 1, N, k)
        return self.torch.empty(max(n, 16), dtype=self.torch.uint8, device="cuda")

    def stages(self, r):
        csa, c4, c4k, c128 = self.csa, self.c4, self.c4k, self.c128
        pos4 = self.ctx - 4
        kv_job = dict(ratio=4, Ca=c4["Ca"], Za=c4["Za"], bias=self.b4, Cb=c4["Cb"], Zb=c4["Zb"], prev_Cb=c4["pCb"],
                      prev_Zb=c4["pZb"], pos0=pos4, out=self.kv[r], cache_entry0=self.N4 - 1, rope_dims=self.rope)
        key_job = dict(ratio=4, Ca=c4k["Ca"], Za=c4k["Za"], bias=self.b4k, Cb=c4k["Cb"], Zb=c4k["Zb"],
                       prev_Cb=c4k["pCb"], prev_Zb=c4k["pZb"], pos0=pos4, out=self.keys[r], cache_entry0=self.N4 - 1,
                       rope_dims=self.rope)
        if self.kfmt != "bf16":
            key_job["out_scale"] = self.kscale[r]
            qk = csa.FP8_E4M3 if self.kfmt == "fp8" else csa.MXFP4
            head = [
                # the 512-d latent in bf16 and the key quantized on write, one launch
                ("compress_c4a_kv_keys", lambda: csa.csa_compress_batch([kv_job, key_job])),
                ("lightning_index", lambda: csa.lightning_index(
                    self.qi8, self.w, self.keys[r], q_pos0=self.t, qk_dtype=qk, q_scale=self.qscale,
                    k_scale=self.kscale[r], scores=self.scores)),
            ]
        else:
            head = [
                # the block's 512-d latent and its 128-d indexer key, one launch
                ("compress_c4a_kv_keys", lambda: csa.csa_compress_batch([kv_job, key_job])),
                ("lightning_index", lambda: csa.lightning_index(
                    self.qi, self.w, self.keys[r], q_pos0=self.t, scores=self.scores)),
            ]
        return head + [
            ("topk_select", lambda: csa.topk_select(
                self.scores, self.k, q_pos0=self.t, idx=self.idx, workspace=self.ws_topk)),
            ("sparse_mqa_attn", lambda: csa.sparse_mqa_attn(
                self.q, self.kv[r], self.idx, self.raw, q_pos0=self.t, raw_pos0=self.raw0, out=self.out,
                workspace=self.ws_attn, batch_invariant=self.bi, rope_dims=self.rope)),
            ("compress_c128a_kv", lambda: csa.csa_compress(
                128, c128["Ca"], c128["Za"], self.b128, pos0=self.ctx - 128, out=self.kvh[r],
                cache_entry0=self.N128 - 1, workspace=self.ws_c128, rope_dims=self.rope)),
            ("hca_attn", lambda: csa.hca_attn(
                self.qh, self.kvh[r], self.rawh, q_pos0=self.t, raw_pos0=self.raw0, sink=self.sink,
                out=self.outh, workspace=self.ws_hca, batch_invariant=self.bi, rope_dims=self.rope)),
        ]

    queries_per_step = property(lambda self: self.B)

    def algorithmic(self):
        """Algorithmic bytes / flops of each stage for one launch (unique bytes only)."""
        B, N4, k = self.B, self.N4, self.k
        rows = k + 128
        if self.kfmt == "fp4":
            # a key row: 64 code bytes + 4 scale bytes; a query head the same
            head = {
                "compress_c4a_kv_keys": dict(bytes=B * 24 * (512 + 128) * 2 + B * (512 * 2 + 64 + 4)
                                             + 8 * (512 + 128) * 4, flops=0),
                "lightning_index": dict(bytes=B * N4 * 68 + B * 64 * 68 + B * 64 * 4 + B * N4 * 2,
                                        flops=B * N4 * 64 * 128 * 2),
            }
        elif self.kfmt == "fp8":
            head = {
                "compress_c4a_kv_keys": dict(bytes=B * 24 * (512 + 128) * 2 + B * (512 * 2 + 128 + 4)
                                             + 8 * (512 + 128) * 4, flops=0),
                "lightning_index": dict(bytes=B * N4 * 132 + B * 64 * 132 + B * 64 * 4 + B * N4 * 2,
                                        flops=B * N4 * 64 * 128 * 2),
            }
        else:
            head = {
                "compress_c4a_kv_keys": dict(bytes=B * (4 * 4 + 4 * 2) * (512 + 128) * 2 + B * (512 + 128) * 2
                                             + 8 * (512 + 128) * 4, flops=0),
                "lightning_index": dict(bytes=B * N4 * 128 * 2 + B * 64 * 128 * 2 + B * 64 * 4 + B * N4 * 2,
                                        flops=B * N4 * 64 * 128 * 2),
            }
        return {
            **head,
            "topk_select": dict(bytes=B * N4 * 2 + B * k * 4, flops=0),
            "sparse_mqa_attn": dict(bytes=B * (rows * 1024 + k * 4 + 2 * 64 * 512 * 2),
                                    flops=B * rows * 64 * 512 * 4),
            "compress_c128a_kv": dict(bytes=B * 2 * 128 * 512 * 2 + B * 512 * 2 + 128 * 512 * 4, flops=0),
            "hca_attn": dict(bytes=B * ((self.N128 + 128) * 1024 + 2 * 64 * 512 * 2),
                             flops=B * (self.N128 + 128) * 64 * 512 * 4),
        }


def _quant_fp8(torch, x):
    """Per-row E4M3 codes and fp32 scales (amax / 448) of a resident tensor, on
    the device (input preparation)."""
    amax = x.float().abs().amax(dim=-1).clamp_min(1e-30)
    scale = (amax / 448.0).contiguous()
    codes = (x.float() / scale[..., None]).to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    return codes, scale


def _quant_mxfp4(torch, x):
    """Per-32 MXFP4 codes of a resident tensor, on the device (input
    preparation): E8M0 exponent floor(log2 amax) - 2, elements rounded to the
    E2M1 grid, ties to the even code, even element in the low nibble."""
    xs = x.float().reshape(*x.shape[:-1], x.shape[-1] // 32, 32)
    amax = xs.abs().amax(dim=-1)
    e = torch.where(amax > 0, torch.floor(torch.log2(amax.clamp_min(1e-38))) - 2, torch.full_like(amax, -127))
    e = e.clamp(-127, 127)
    v = xs / torch.exp2(e)[..., None]
    a = v.abs()
    code = ((a > 0.25).int() + (a >= 0.75).int() + (a > 1.25).int() + (a >= 1.75).int() + (a > 2.5).int()
            + (a >= 3.5).int() + (a > 5).int())
    nib = code + 8 * ((v < 0) & (code > 0)).int()
    nib = nib.reshape(*x.shape[:-1], x.shape[-1])
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).to(torch.uint8).contiguous()
    return packed, (e + 127).to(torch.uint8).contiguous()


def cpu_oracle_decode(step, torch, budget_s):
    """Time the CPU oracle on a bounded sample of the decode step's query tokens.

    Each query token runs the whole path in the oracle: both compressors for
    the last block, the indexer over all 16,384 keys, Top-k over the stored
    bf16 scores, sparse attention, and the HCA compressor + dense attention
    with sink.  Host copies of the inputs are made before the clock starts."""
    from oracle import attention as oa, compressor as oc, indexer as oi, numerics as on, topk as ot

    def h(t):
        return t.float().cpu().numpy()

    r = 0
    samples = []
    for b in range(step.B):
        samples.append(dict(
            c4={k2: h(v[b]) for k2, v in step.c4.items()}, c4k={k2: h(v[b]) for k2, v in step.c4k.items()},
            c128={k2: h(v[b]) for k2, v in step.c128.items()},
            keys=h(step.keys[r][b]), kv=h(step.kv[r][b]), kvh=h(step.kvh[r][b]),
            raw=h(step.raw[b]), rawh=h(step.rawh[b]), q=h(step.q[b]), qh=h(step.qh[b]),
            qi=h(step.qi[b]), w=h(step.w[b])))
        if b >= 3:
            break
    b4, b4k, b128, sink = h(step.b4), h(step.b4k), h(step.b128), h(step.sink)
    t, N4 = step.t, step.N4
    done = 0
    t0 = time.perf_counter()
    while True:
        s = samples[done % len(samples)]
        c4, c4k = s["c4"], s["c4k"]
        ent, _ = oc.compress_sequence(c4["Ca"], c4["Za"], b4, 4, c4["Cb"], c4["Zb"], c4["pCb"], c4["pZb"],
                                      pos0=step.ctx - 4)
        key, _ = oc.compress_sequence(c4k["Ca"], c4k["Za"], b4k, 4, c4k["Cb"], c4k["Zb"], c4k["pCb"],
                                      c4k["pZb"], pos0=step.ctx - 4)
        keys = s["keys"].astype(np.float64)
        keys[N4 - 1] = key[0]
        sc = oi.index_scores(s["qi"][None], s["w"][None], keys[None], t, 4)
        idx = ot.topk_select(on.store_bf16(sc), step.k, t, 4)
        kv = s["kv"].astype(np.float64)
        kv[N4 - 1] = ent[0]
        sel = idx[0, 0]
        o, _ = oa.sparse_mqa(s["q"][None], kv[sel][None], np.arange(len(sel))[None, None], s["raw"][None],
                             step.raw0, t, 128)
        enth, _ = oc.compress_sequence(s["c128"]["Ca"], s["c128"]["Za"], b128, 128, pos0=step.ctx - 128)
        kvh = s["kvh"].astype(np.float64)
        kvh[step.N128 - 1] = enth[0]
        oh, _ = oa.hca_attention(s["qh"][None], kvh[None], s["rawh"][None], step.raw0, t, sink, ratio=128)
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    return {"value": done / el, "unit": "query-tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} query tokens of the same decode step (sequences 0..{len(samples) - 1} "
                      f"cycled), full path per token: both C4A compressors, indexer over {N4} keys, "
                      f"top-{step.k}, sparse MQA, C128A compressor and HCA attention; {el:.1f} s"}


def index_traffic():
    """HBM bytes per lightning_index launch from the committed counter runs
    (profiles/lightning_index_decode_traffic.md), or None once the kernel's
    sources differ from the ones the counters were taken on."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    try:
        text = open(os.path.join(here, "profiles", "lightning_index_decode_traffic.md")).read()
        rec = dict(line.split(" = ", 1) for line in text.splitlines() if " = " in line and "`" not in line)
        h = hashlib.sha256()
        for rel in ("csrc/indexer.hip", "csrc/device.h", "build.py"):
            with open(os.path.join(here, "long_context_sparse_compress_amd", rel), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != rec["source_sha256"].strip():
            return None
        return int(rec["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


# ---------------------------------------------------------------- timing


def time_graph(torch, step, steps, warmup, rotate, eager):
    stream = torch.cuda.Stream()
    graphs = []
    with torch.cuda.stream(stream):
        for r in range(rotate):           # eager warm run of each copy (also loads the kernels)
            for _, fn in step.stages(r):
                fn()
    torch.cuda.synchronize()
    if not eager:
        for r in range(rotate):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for _, fn in step.stages(r):
                    fn()
            graphs.append(g)
    torch.cuda.synchronize()

    def run(i):
        if eager:
            for _, fn in step.stages(i % rotate):
                fn()
        else:
            graphs[i % rotate].replay()

    with torch.cuda.stream(stream):
        for i in range(warmup):
            run(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(steps):
            run(i)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def time_stages(torch, step, steps, rotate):
    """Eager pass: events around every stage, on the stream the kernels are launched on."""
    stream = torch.cuda.Stream()
    names = [n for n, _ in step.stages(0)]
    acc = {n: 0.0 for n in names}
    with torch.cuda.stream(stream):
        for i in range(2):
            for _, fn in step.stages(i % rotate):
                fn()
        torch.cuda.synchronize()
        evs = []
        for i in range(steps):
            row = []
            for n, fn in step.stages(i % rotate):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn()
                b.record(stream)
                row.append((n, a, b))
            evs.append(row)
        torch.cuda.synchronize()
    for row in evs:
        for n, a, b in row:
            acc[n] += a.elapsed_time(b)
    return {n: acc[n] / steps for n in names}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import long_context_sparse_compress_amd as csa
    import synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    csa.library()
    if args.workload != "csa_hca_decode":
        import bench_workloads
        print(json.dumps(bench_workloads.run(args, torch, csa, synth)))
        return

    step = DecodeStep(csa, synth, torch, rotate=args.rotate, batch_invariant=args.batch_invariant,
                      rope=args.rope, keys=args.keys)
    ms, wall = time_graph(torch, step, args.steps, args.warmup, args.rotate, args.eager)
    per_stage = time_stages(torch, step, args.steps, args.rotate)
    alg = step.algorithmic()
    dom = "lightning_index"
    dom_ms = per_stage[dom]
    achieved = alg[dom]["bytes"] / (dom_ms * 1e-3) / 1e9
    stages = {}
    for n, t in per_stage.items():
        a = alg[n]
        stages[n] = {"us": round(t * 1e3, 2), "GB/s": round(a["bytes"] / (t * 1e-3) / 1e9, 1),
                     "TFLOP/s": round(a["flops"] / (t * 1e-3) / 1e12, 2) if a["flops"] else None}
    total_bytes = sum(a["bytes"] for a in alg.values())
    rec = {
        "metric": METRIC,
        "value": round(step.queries_per_step / (ms * 1e-3), 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "csa_hca_decode: CSA layer (C4A, indexer, top-512, sparse MQA) + HCA layer "
                               "(C128A, dense MQA with sink), decode",
                   "batch": step.B, "context": step.ctx, "c4a_entries": step.N4, "c128a_entries": step.N128,
                   "topk": step.k, "window": 128, "heads": 64, "head_dim": 512, "index_heads": 64,
                   "index_dim": 128, "cache_copies_rotated": args.rotate,
                   "timing": "eager" if args.eager else "hip_graph",
                   "attention": "batch_invariant" if args.batch_invariant else "split_kv",
                   "rope_dims": args.rope, "index_keys": {"bf16": "bf16", "fp8": "fp8_e4m3", "fp4": "mxfp4"}[args.keys]},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None if args.keys != "bf16" else index_traffic(),
                     "algorithmic_bytes_per_launch": alg[dom]["bytes"], "avg_launch_us": round(dom_ms * 1e3, 2)},
        "step_hbm_GBps": round(total_bytes / (ms * 1e-3) / 1e9, 1),
        "stages": stages,
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_cpu and args.keys == "bf16":
        rec["cpu_baseline"] = cpu_oracle_decode(step, torch, args.cpu_seconds)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
