"""GPU parity of lightning_index (stage 2) against the oracle, through the C ABI.

Pages: "DeepSeek Technical Reports" (DSA, the indexer equation); "DeepSeek V4
结构速览" (Lightning Indexer).  Tolerance: the workloads state 1e-3 relative on
fp32 accumulation (checked on fp32-stored scores); BF16-stored scores must be
within one bf16 ulp of the oracle's fp64 score rounded to bf16.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_compress_amd as csa
import synth
from oracle import indexer as oi
from oracle import numerics as on
from helpers import dev, host, index_close

pytestmark = pytest.mark.gpu


def _bf16_ulp(v):
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def _bf16_close(got, ref64):
    ref = on.store_bf16(ref64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin)
    assert np.all(got[~fin] == -np.inf)
    d = np.abs(got[fin] - ref[fin])
    assert np.all(d <= _bf16_ulp(ref[fin]) * 1.0001), f"max diff {d.max()}"


def _inputs(prefix, B, T, N, qk, q_var=1.0 / 128):
    q = synth.normal(prefix + ".q", (B, T, 64, 128), var=q_var)
    w = synth.uniform(prefix + ".w", (B, T, 64))
    k = synth.normal(prefix + ".k", (B, N, 128))
    if qk == "f32":
        return dict(q=dev(q), w=dev(w), k=dev(k), qk=csa.F32), (q, w, k)
    if qk == "bf16":
        qb, kb = synth.round_bf16(q), synth.round_bf16(k)
        return dict(q=dev(qb, torch.bfloat16), w=dev(w), k=dev(kb, torch.bfloat16), qk=csa.BF16), (qb, w, kb)
    if qk == "fp8":
        qc, qs = synth.quant_fp8_rows(q)
        kc, ks = synth.quant_fp8_rows(k)
        d = dict(q=dev(qc, torch.uint8), w=dev(w), k=dev(kc, torch.uint8), qk=csa.FP8_E4M3,
                 q_scale=dev(qs), k_scale=dev(ks))
        return d, (on.dequant_fp8_rows(qc, qs), w, on.dequant_fp8_rows(kc, ks))
    if qk == "mxfp4":
        qp, qs = synth.quant_mxfp4(q)
        kp, ks = synth.quant_mxfp4(k)
        d = dict(q=dev(qp, torch.uint8), w=dev(w), k=dev(kp, torch.uint8), qk=csa.MXFP4,
                 q_scale=dev(qs, torch.uint8), k_scale=dev(ks, torch.uint8))
        return d, (on.dequant_mxfp4(qp, qs), w, on.dequant_mxfp4(kp, ks))
    raise ValueError(qk)


def _gpu(d, q_pos0, ratio=4, score_dtype=torch.float32, N=None):
    s = csa.lightning_index(d["q"], d["w"], d["k"], q_pos0=q_pos0, ratio=ratio, qk_dtype=d["qk"],
                            q_scale=d.get("q_scale"), k_scale=d.get("k_scale"),
                            score_dtype=score_dtype, N=N)
    torch.cuda.synchronize()
    return host(s)


def test_tiny_prefill_fp32():
    """256 query tokens x 64 C4A entries, fp32 (keys here drawn directly)."""
    d, (q, w, k) = _inputs("tiny", 1, 256, 64, "f32")
    got = _gpu(d, 0)
    index_close(got, oi.index_scores(q, w, k, 0, 4))


@pytest.mark.parametrize("score", ["f32", "bf16"])
def test_csa_decode_bf16_full(score):
    """Batch 32 at 65,536 context: 16,384 bf16 keys per sequence, one query each."""
    d, (q, w, k) = _inputs("dec", 32, 1, 16384, "bf16")
    got = _gpu(d, 65535, score_dtype=torch.float32 if score == "f32" else torch.bfloat16)
    ref = oi.index_scores(q, w, k, 65535, 4)
    if score == "f32":
        index_close(got, ref)
    else:
        _bf16_close(got, ref)


def test_chunked_prefill_fp8_sampled_rows():
    """4,096 queries x 33,792 fp8 keys (per-row scales), bf16 scores; the oracle
    checks a sample of rows that includes the first, the last and the rows around
    entry boundaries."""
    T, N, q_pos0 = 4096, 33792, 131072
    d, (q, w, k) = _inputs("pf", 1, T, N, "fp8", q_var=1.0)
    got = _gpu(d, q_pos0, score_dtype=torch.bfloat16)
    rows = [0, 1, 2, 3, 4, 5, 1023, 2046, 2047, 2048, 4092, 4093, 4094, 4095]
    ref = oi.index_scores(q, w, k, q_pos0, 4, rows=rows)
    _bf16_close(got[:, rows], ref)
    # fp32 scores on the same rows against the 1e-3 rule
    got32 = _gpu(d, q_pos0, score_dtype=torch.float32)
    index_close(got32[:, rows], ref)


def test_decode_mxfp4():
    """MXFP4 q and keys (E2M1 + E8M0 per 32), bf16 and fp32 scores."""
    d, (q, w, k) = _inputs("mx", 3, 1, 20000, "mxfp4", q_var=1.0)
    ref = oi.index_scores(q, w, k, 4 * 20000 - 1, 4)
    index_close(_gpu(d, 4 * 20000 - 1), ref)
    _bf16_close(_gpu(d, 4 * 20000 - 1, score_dtype=torch.bfloat16), ref)


@pytest.mark.parametrize("qk,B,T,N,q_pos0,ratio", [
    ("bf16", 2, 5, 1000, 3996, 4),    # ragged T (not a multiple of 4) and N
    ("bf16", 1, 9, 17, 0, 4),         # rows with nothing visible, N barely larger than one tile
    ("fp8", 2, 7, 77, 280, 4),        # partly masked tiles
    ("fp8", 1, 1, 1, 3, 4),           # one entry
    ("mxfp4", 2, 6, 33, 125, 4),      # prefill-shaped MXFP4
    ("bf16", 1, 3, 40, 128 * 40 - 3, 128),   # ratio 128 visibility
    ("f32", 2, 3, 70, 270, 4),
])
def test_edge_shapes(qk, B, T, N, q_pos0, ratio):
    d, (q, w, k) = _inputs(f"edge{qk}{N}", B, T, N, qk)
    ref = oi.index_scores(q, w, k, q_pos0, ratio)
    index_close(_gpu(d, q_pos0, ratio=ratio), ref)


def test_scores_nonnegative_and_deterministic():
    d, _ = _inputs("nn", 4, 1, 5000, "bf16")
    a = _gpu(d, 4 * 5000 - 1, score_dtype=torch.bfloat16)
    b = _gpu(d, 4 * 5000 - 1, score_dtype=torch.bfloat16)
    assert np.all(a >= 0)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("T,q0", [(1, 399), (3, 399), (16, 0), (5, 12000)])
def test_key_runs_with_nothing_visible_still_write_every_score(T, q0):
    """Key runs wholly past every query's causal bound but inside N: the
    waves that own them score no tile and end early, and every one of their
    entries must still read -inf (the output starts as NaN).  T = 1 takes
    the decode kernel, T >= 3 the pipelined prefill kernel."""
    B, N = 2, 5000
    q = synth.round_bf16(synth.normal(f"ix.idle.{T}.q", (B, T, 64, 128), var=1.0 / 128))
    w = synth.uniform(f"ix.idle.{T}.w", (B, T, 64))
    k = synth.round_bf16(synth.normal(f"ix.idle.{T}.k", (B, N, 128)))
    ref = oi.index_scores(q, w, k, q0, 4)
    for sd in (torch.float32, torch.bfloat16):
        s = torch.full((B, T, N), float("nan"), dtype=sd, device="cuda")
        csa.lightning_index(dev(q, torch.bfloat16), dev(w), dev(k, torch.bfloat16), q_pos0=q0, ratio=4, scores=s)
        torch.cuda.synchronize()
        got = host(s)
        assert not np.isnan(got).any()
        if sd == torch.float32:
            index_close(got, ref)
        else:
            fin = np.isfinite(ref)
            assert np.array_equal(np.isfinite(got), fin) and np.all(got[~fin] == -np.inf)
            assert np.all(np.abs(got[fin] - ref[fin]) <= np.abs(ref[fin]) * 2.0 ** -8 + 1e-6)
