"""End-to-end chain on the tiny CSA prefill workload: the GPU path and the
oracle each run compressor -> indexer -> Top-k -> sparse MQA on their own
(the oracle never reads a GPU result), plus a C128A compressor and HCA
attention on the same raw tokens.  Used by tests/test_gpu_chain.py and by
__graft_entry__.smoke().

Workload ("Tiny CSA prefill"): 1 sequence of 256 raw tokens, fp32; Ca, Cb,
Za, Zb 256 x 512 ~ N(0,1), bias 8 x 512 ~ N(0, 0.1); the indexer keys come
from the same compressor on 256 x 128 inputs; q_I 256 x 64 x 128 ~ N(0,
1/128); w ~ U(0,1); k = 16; q 256 x 64 x 512 ~ N(0,1); raw window latents
256 x 512 ~ N(0,1); scale 1/sqrt(512); seed 0.

With ``rope`` (a number of dims R), partial RoPE runs through the chain on
both sides: the compressor rotates its entries (512-d and 128-d keys, anchor
offsets 1 for C4A and 5 for C128A), q, the indexer queries and the window
rows are rotated at their positions, and both attentions apply the inverse
RoPE to their outputs.

Top-k comparison: the selected sets must have the same size and be equal,
except that an entry whose oracle score lies within 1e-3 relative of the
row's k-th oracle score may be swapped for another such entry (ties within
fp32 rounding of the two summation orders).  Attention is compared on every
row: where the sets are equal against the oracle's own output; on a row
whose GPU set is one of those valid alternatives (checked first, against the
oracle's scores), against the oracle's attention over that set, with the
oracle's own compressed entries and window rows.
"""
from __future__ import annotations

import numpy as np
import torch

import long_context_sparse_compress_amd as csa
import synth
from oracle import attention as oa
from oracle import compressor as oc
from oracle import indexer as oi
from oracle import rope as orp
from oracle import topk as ot

N_TOK, K, WIN = 256, 16, 128
ANCHOR4, ANCHOR128 = 1, 5


def _d(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def inputs(seed=0):
    main = synth.compressor_inputs("tiny.main", 1, N_TOK, 512, 4, 0, seed=seed)
    keyc = synth.compressor_inputs("tiny.key", 1, N_TOK, 128, 4, 0, seed=seed)
    hca = synth.compressor_inputs("tiny.hca", 1, N_TOK, 512, 128, 0, seed=seed)
    return dict(
        main=main, keyc=keyc, hca=hca,
        qi=synth.normal("tiny.qi", (1, N_TOK, 64, 128), var=1.0 / 128, seed=seed),
        w=synth.uniform("tiny.w", (1, N_TOK, 64), seed=seed),
        q=synth.normal("tiny.q", (1, N_TOK, 64, 512), seed=seed),
        raw=synth.normal("tiny.raw", (1, N_TOK, 512), seed=seed),
        sink=synth.normal("tiny.sink", (64,), seed=seed),
    )


def run_gpu(x, rope=0):
    m, kc, hc = x["main"], x["keyc"], x["hca"]
    r4 = dict(rope_dims=rope, rope_anchor=ANCHOR4)
    kv = csa.csa_compress(4, _d(m["Ca"]), _d(m["Za"]), _d(m["bias"]), _d(m["Cb"]), _d(m["Zb"]), **r4)
    keys = csa.csa_compress(4, _d(kc["Ca"]), _d(kc["Za"]), _d(kc["bias"]), _d(kc["Cb"]), _d(kc["Zb"]), **r4)
    qi, q, raw = _d(x["qi"]), _d(x["q"]), _d(x["raw"])
    if rope:
        for t in (qi, q, raw):
            csa.rope(t, pos0=0, rope_dims=rope)
    scores = csa.lightning_index(qi, _d(x["w"]), keys, q_pos0=0, score_dtype=torch.float32)
    idx = csa.topk_select(scores, K, q_pos0=0)
    out = csa.sparse_mqa_attn(q, kv, idx, raw, q_pos0=0, raw_pos0=0, rope_dims=rope)
    kvh = csa.csa_compress(128, _d(hc["Ca"]), _d(hc["Za"]), _d(hc["bias"]), rope_dims=rope, rope_anchor=ANCHOR128)
    outh = csa.hca_attn(q, kvh, raw, q_pos0=0, raw_pos0=0, sink=_d(x["sink"]), rope_dims=rope)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in
            dict(kv=kv, keys=keys, scores=scores, idx=idx, out=out, kvh=kvh, outh=outh).items()}


def run_oracle(x, rows=None, rope=0):
    m, kc, hc = x["main"], x["keyc"], x["hca"]
    r4 = dict(rope_dims=rope, rope_anchor=ANCHOR4)
    kv = oc.compress(m["Ca"], m["Za"], m["bias"], 4, m["Cb"], m["Zb"], **r4)
    keys = oc.compress(kc["Ca"], kc["Za"], kc["bias"], 4, kc["Cb"], kc["Zb"], **r4)
    qi, q, raw = x["qi"], x["q"], x["raw"]
    if rope:
        qi, q, raw = (orp.rotate_rows(t, 0, rope) for t in (qi, q, raw))
    scores = oi.index_scores(qi, x["w"], keys, 0, 4)
    stored = scores.astype(np.float32).astype(np.float64)
    idx = ot.topk_select(stored, K, 0, 4)
    out, _ = oa.sparse_mqa(q, kv, idx, raw, 0, 0, WIN, rows=rows, rope_dims=rope)
    kvh = oc.compress(hc["Ca"], hc["Za"], hc["bias"], 128, rope_dims=rope, rope_anchor=ANCHOR128)
    outh, _ = oa.hca_attention(q, kvh, raw, 0, 0, x["sink"], ratio=128, rows=rows, rope_dims=rope)
    return dict(kv=kv, keys=keys, scores=scores, idx=idx, out=out, kvh=kvh, outh=outh)


def compare(g, o, rows=None, x=None, rope=0):
    """Returns a dict of diagnostics; raises AssertionError on a mismatch.
    ``x`` (the inputs) lets the rows whose selections differ inside the tie
    band be compared too (see the module docstring)."""
    rows = list(range(N_TOK)) if rows is None else list(rows)
    rep = {}
    rep["kv"] = float(np.max(np.abs(g["kv"] - o["kv"])))
    rep["keys"] = float(np.max(np.abs(g["keys"] - o["keys"])))
    rep["kvh"] = float(np.max(np.abs(g["kvh"] - o["kvh"])))
    assert rep["kv"] < 1e-4 and rep["keys"] < 1e-4 and rep["kvh"] < 1e-4, rep
    sc_o, sc_g = o["scores"][0], g["scores"][0]
    fin = np.isfinite(sc_o)
    assert np.array_equal(fin, np.isfinite(sc_g))
    rel = np.abs(sc_g[fin] - sc_o[fin]) / np.maximum(np.abs(sc_o[fin]), 1e-30)
    rep["scores_max_rel"] = float(rel.max()) if rel.size else 0.0
    assert np.all(np.abs(sc_g[fin] - sc_o[fin]) <= 1e-3 * np.abs(sc_o[fin]) + 1e-6), rep
    same_rows, tie_rows = [], []
    for t in range(N_TOK):
        gl = [int(s) for s in g["idx"][0, t] if s >= 0]
        ol = [int(s) for s in o["idx"][0, t] if s >= 0]
        gs, os_ = set(gl), set(ol)
        assert len(gl) == len(gs) == len(os_) == len(ol), f"row {t}: selection sizes differ"
        if gs == os_:
            same_rows.append(t)
            continue
        v = (t + 1) // 4
        kth = np.sort(sc_o[t, :v])[::-1][K - 1]
        band = np.abs(sc_o[t, :v] - kth) <= 1e-3 * abs(kth)
        for s in gs ^ os_:
            assert band[s], f"row {t}: entry {s} differs outside the tie band"
        tie_rows.append(t)
    rep["topk_rows_equal"] = len(same_rows)
    chk = [t for t in rows if t in set(same_rows)]
    oi_rows = {t: i for i, t in enumerate(rows)}
    errs = [np.max(np.abs(g["out"][0, t] - o["out"][0, oi_rows[t]])) for t in chk]
    tie_chk = [t for t in rows if t in set(tie_rows)]
    if tie_chk and x is not None:
        q = orp.rotate_rows(x["q"], 0, rope) if rope else x["q"]
        raw = orp.rotate_rows(x["raw"], 0, rope) if rope else x["raw"]
        alt = o["idx"].copy()
        for t in tie_chk:
            alt[0, t] = g["idx"][0, t]
        ot_out, _ = oa.sparse_mqa(q, o["kv"], alt, raw, 0, 0, WIN, rows=tie_chk, rope_dims=rope)
        errs += [np.max(np.abs(g["out"][0, t] - ot_out[0, i])) for i, t in enumerate(tie_chk)]
        rep["tie_rows_checked"] = len(tie_chk)
    rep["attn_max_abs"] = float(max(errs)) if errs else 0.0
    assert rep["attn_max_abs"] < 1e-4, rep
    errh = [np.max(np.abs(g["outh"][0, t] - o["outh"][0, oi_rows[t]])) for t in rows]
    rep["hca_max_abs"] = float(max(errh))
    assert rep["hca_max_abs"] < 1e-4, rep
    return rep
