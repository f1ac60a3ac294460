#!/usr/bin/env python3
"""Benchmark of the compressed sparse attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default: the five configurations of the method, one JSON line.  The headline
(`value`, `config`, `roofline`, `cpu_baseline`) is the largest single-GPU
configuration, the CSA decode at 1,048,576 tokens of context (Pro: batch 8,
262,144 C4A entries per sequence, MXFP4 indexer, top-1024); the line's
`configs` object carries the same record for the CSA decode at 65,536
context (batch 32), the CSA chunked prefill (4,096 queries after 131,072
tokens) and the HCA layer (decode, batch 16 at 1M context; a 2,048-token
prefill chunk).  A step is one pass of the workload's stages (see
bench_workloads.py) over synthetic inputs resident in HBM; decode caches are
rotated over several seeded copies, more than the 256 MB Infinity Cache in
total, so each step streams its keys and rows from HBM.

Timing: W untimed steps, then K steps between two HIP events on the stream
the kernels run on (one HIP graph holding a step on each cache copy in turn,
as a serving loop captures several layers in one graph, plus single-step
graphs for a remainder; --eager times eager launches), ms_per_step =
elapsed / K and value = query tokens / s.  A second,
eager pass brackets every stage with events on that stream: each stage's
average duration (which includes its launch's dispatch).  The dominant
kernel's launch duration is timed on its own: a HIP graph of its launches
back to back over the cache copies, replayed between two events on its
stream; from it the roofline fraction (algorithmic bytes or FLOPs of one
launch / duration, against 8 TB/s HBM or the MFMA peak of its dtype).
`traffic` is the HBM bytes per launch read
from the committed FETCH_SIZE / WRITE_SIZE counter record of that kernel
(profiles/), or null when the kernel's sources changed since.

The CPU baseline times the oracle (NumPy fp64, test infrastructure) on a
bounded sample of each configuration's step (about --cpu-seconds each).

--workload NAME prints the same record for one workload: a configuration
(csa_1m_decode, csa_decode, csa_prefill, hca_decode, hca_prefill) or another
workload (csa_hca_decode, c128a_1m, csa_reindex_decode, csa_reindex_prefill,
csa_paged_decode, csa_paged_1m_decode, csa_1m_decode_separate, hbm_copy,
hbm_read).
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
MFMA_PEAK = {"bf16": 2500.0, "fp8": 5000.0, "mxfp4": 10100.0}
METRIC = "CSA/HCA query-tokens/s at 1 GPU; % peak HBM GB/s (decode), % MFMA (prefill)"
HERE = os.path.dirname(os.path.abspath(__file__))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", default="all")
    p.add_argument("--rotate", type=int, default=4, help="cache copies cycled over the steps (decode workloads)")
    p.add_argument("--eager", action="store_true",
                   help="time eager launches instead of HIP graphs (the counter runs need it)")
    p.add_argument("--cpu-seconds", type=float, default=8.0, help="budget of each CPU oracle sample")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--batch-invariant", action="store_true", help="csa_hca_decode: batch-invariant attention")
    p.add_argument("--keys", choices=("bf16", "fp8", "fp4"), default="bf16",
                   help="csa_hca_decode: index keys bf16, or quantized on write to fp8 E4M3 or MXFP4")
    p.add_argument("--rope", type=int, default=0, help="csa_hca_decode: partial RoPE dims (0 = none)")
    return p.parse_args()


# ---------------------------------------------------------------- timing


def time_step(torch, wk, steps, warmup, eager):
    """Average step time over exactly `steps` steps, copy i % copies on step i.
    Graph timing: one HIP graph holds one step on each cache copy in turn (a
    serving loop likewise captures a step's layers in one graph, so the
    graph's own launch is paid once per several layers); `steps // copies`
    replays of it, then single-step graphs for the remainder."""
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        for r in range(wk.copies):                 # eager warm run of every copy (also loads the kernels)
            for s in wk.stages:
                s[1](r)
    torch.cuda.synchronize()
    graphs, multi = [], None
    if not eager:
        for r in range(wk.copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=st):
                for s in wk.stages:
                    s[1](r)
            graphs.append(g)
        if wk.copies > 1:
            multi = torch.cuda.CUDAGraph()
            with torch.cuda.graph(multi, stream=st):
                for r in range(wk.copies):
                    for s in wk.stages:
                        s[1](r)
        torch.cuda.synchronize()

    def run(n):
        """n steps, starting at copy 0."""
        if eager:
            for i in range(n):
                for s in wk.stages:
                    s[1](i % wk.copies)
            return
        i = 0
        if multi is not None:
            for _ in range(n // wk.copies):
                multi.replay()
            i = n - n % wk.copies
        for j in range(i, n):
            graphs[j % wk.copies].replay()

    with torch.cuda.stream(st):
        run(warmup)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(st)
        run(steps)
        e1.record(st)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    del graphs, multi
    return e0.elapsed_time(e1) / steps, wall


def time_stages(torch, wk, steps):
    """Eager pass: events around every stage on the stream its kernels run on;
    the median over the steps (ms), so that a one-off host-side stall does not
    stand for the stage."""
    st = torch.cuda.Stream()
    acc = {s[0]: [] for s in wk.stages}
    with torch.cuda.stream(st):
        for r in range(wk.copies):
            for s in wk.stages:
                s[1](r)
        torch.cuda.synchronize()
        evs = []
        for i in range(steps):
            for s in wk.stages:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(st)
                s[1](i % wk.copies)
                b.record(st)
                evs.append((s[0], a, b))
        torch.cuda.synchronize()
    for n, a, b in evs:
        acc[n].append(a.elapsed_time(b))
    return {n: sorted(v)[len(v) // 2] for n, v in acc.items()}


def time_kernel(torch, wk, stage, reps=10):
    """Average duration of one launch of `stage` alone: a HIP graph of 2 x copies
    back-to-back launches (cache copy i % copies each), replayed `reps` times
    between two events on its stream (ms per launch)."""
    fn = next(s for s in wk.stages if s[0] == stage)[1]
    st = torch.cuda.Stream()
    n = 2 * wk.copies
    with torch.cuda.stream(st):
        for i in range(n):
            fn(i % wk.copies)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        for i in range(n):
            fn(i % wk.copies)
    torch.cuda.synchronize()
    with torch.cuda.stream(st):
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            g.replay()
        e1.record(st)
        torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / (reps * n)


# ---------------------------------------------------------------- records


def counter_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` in `workload` from its committed counter
    record (profiles/traffic_<workload>_<kernel>.md), or None when absent or
    when the kernel's sources no longer hash to the recorded value."""
    path = os.path.join(HERE, "profiles", f"traffic_{workload}_{kernel}.md")
    try:
        text = open(path).read()
        rec = dict(line.split(" = ", 1) for line in text.splitlines() if " = " in line and "`" not in line)
        h = hashlib.sha256()
        for rel in rec["sources"].split(","):
            with open(os.path.join(HERE, "long_context_sparse_compress_amd", rel.strip()), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != rec["source_sha256"].strip():
            return None
        return int(rec["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def roofline(bound, nbytes, flops, ms):
    if bound == "hbm":
        a = nbytes / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4)}
    a = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "dtype": bound, "achieved": round(a, 1), "peak": MFMA_PEAK[bound],
            "unit": "TFLOP/s", "frac": round(a / MFMA_PEAK[bound], 4)}


def measure(torch, wk, args):
    ms, wall = time_step(torch, wk, args.steps, args.warmup, args.eager)
    per = time_stages(torch, wk, args.steps)
    stages = {}
    for name, _, nb, fl, bound in wk.stages:
        t = per[name]
        stages[name] = {"us": round(t * 1e3, 2), "GB/s": round(nb / (t * 1e-3) / 1e9, 1),
                        "TFLOP/s": round(fl / (t * 1e-3) / 1e12, 2) if fl else None,
                        "roofline": roofline(bound, nb, fl, t)}
    dom = next(s for s in wk.stages if s[0] == wk.dominant)
    # the dominant kernel's launch time: its launches back to back in a graph
    # (the stage table's eager events also hold each launch's dispatch)
    t_dom = time_kernel(torch, wk, dom[0]) if not args.eager else per[dom[0]]
    roof = dict(roofline(dom[4], dom[2], dom[3], t_dom), kernel=dom[0], traffic=counter_traffic(wk.key, dom[0]),
                avg_launch_us=round(t_dom * 1e3, 2), eager_event_us=stages[dom[0]]["us"])
    roof["algorithmic_bytes_per_launch" if dom[4] == "hbm" else "algorithmic_flops_per_launch"] = \
        dom[2] if dom[4] == "hbm" else dom[3]
    total = sum(s[2] for s in wk.stages)
    return {
        "value": round(wk.units / (ms * 1e-3), 1),
        "unit": wk.unit,
        "ms_per_step": round(ms, 5),
        "config": dict(workload=wk.label, **wk.info, timing="eager" if args.eager else "hip_graph"),
        "roofline": roof,
        "step_hbm_GBps": round(total / (ms * 1e-3) / 1e9, 1),
        "stages": stages,
        "wall_s_timed": round(wall, 3),
    }


def run_one(torch, csa, synth, bw, name, args):
    """Build, measure and (optionally) CPU-sample one workload; frees its inputs."""
    if name in bw.CONFIGS:
        build = bw.CONFIGS[name]
        wk = build(torch, csa, synth, copies=args.rotate) if name.endswith("decode") else build(torch, csa, synth)
    elif name == "csa_hca_decode":
        wk = bw.csa_hca_decode(torch, csa, synth, copies=args.rotate, keys=args.keys, rope=args.rope,
                               batch_invariant=args.batch_invariant)
    elif name in bw.EXTRAS:
        wk = bw.EXTRAS[name](torch, csa, synth)
    else:
        raise SystemExit(f"unknown workload {name}")
    rec = measure(torch, wk, args)
    print(f"# {name}: {rec['value']} {rec['unit']}, {rec['ms_per_step'] * 1e3:.1f} us/step", file=sys.stderr,
          flush=True)
    if not args.no_cpu and wk.cpu is not None:
        rec["cpu_baseline"] = wk.cpu(args.cpu_seconds)
        print(f"# {name}: cpu oracle {rec['cpu_baseline']['value']} {rec['cpu_baseline']['unit']}", file=sys.stderr,
              flush=True)
    del wk
    gc.collect()
    torch.cuda.empty_cache()
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import bench_workloads as bw
    import long_context_sparse_compress_amd as csa
    import synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    csa.library()
    names = bw.DEFAULT_ORDER if args.workload == "all" else [args.workload]
    recs = {n: run_one(torch, csa, synth, bw, n, args) for n in names}
    head = recs[names[0]]
    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
    }
    if "cpu_baseline" in head:
        line["cpu_baseline"] = head["cpu_baseline"]
    line["stages"] = head["stages"]
    line["step_hbm_GBps"] = head["step_hbm_GBps"]
    line["wall_s_timed"] = head["wall_s_timed"]
    if len(names) > 1:
        line["configs"] = {n: recs[n] for n in names[1:]}
    print(json.dumps(line))


if __name__ == "__main__":
    main()
