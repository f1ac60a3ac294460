"""GPU parity of quantize-on-write (csa_compress_ex with fp8 E4M3 output)
against the oracle, through the C ABI.

Pages: "DeepSeek V4 结构速览" (C4A Compressor; Lightning Indexer -- the
indexer keys are kept in low precision).  The oracle compresses in fp64 and
quantizes its own result (oracle.numerics.quant_fp8_rows_f32); the GPU
compresses in fp32 and quantizes its result.  Bounds: each entry's scale
within 1e-4 relative of the oracle's amax / 448; every decoded element within
half an E4M3 step (at its magnitude) of the oracle's value, plus the fp32
compressor tolerance; and the codes equal to the oracle's except where the
oracle's value lies within that tolerance of a rounding midpoint.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_compress_amd as csa
import synth
from oracle import compressor as oc
from oracle import numerics as on
from helpers import dev, host

pytestmark = pytest.mark.gpu
BF = torch.bfloat16
PRE_TOL = 1e-4        # fp32 compressor error on O(1) outputs (the compressor's own bound)


def _step(v):
    """E4M3 spacing at |v| (subnormal spacing below 2^-6)."""
    a = np.maximum(np.abs(v), 2.0 ** -6)
    return np.exp2(np.floor(np.log2(a)) - 3)


def _check(codes, scale, ref):
    """codes [.., c] uint8, scale [..] (GPU); ref [.., c] fp64 (oracle entries)."""
    amax = np.abs(ref).max(axis=-1)
    assert np.all(np.abs(scale - amax / 448.0) <= 1e-4 * amax / 448.0 + 1e-30)
    dec = on.decode_e4m3(codes) * scale[..., None]
    v = ref / scale[..., None]
    bound = (0.5 * _step(v) * (1 + 1e-6)) * scale[..., None] + PRE_TOL
    assert np.all(np.abs(dec - ref) <= bound), np.max(np.abs(dec - ref) - bound)
    oc_codes, _ = on.quant_fp8_rows_f32(ref)
    diff = codes != oc_codes
    if diff.any():
        # a differing code is only allowed next to a rounding midpoint
        lo = on.decode_e4m3(np.minimum(codes, oc_codes) & 0x7F)
        hi = on.decode_e4m3(np.maximum(codes, oc_codes) & 0x7F)
        mid = 0.5 * (lo + hi)
        near = np.abs(np.abs(v) - mid) <= PRE_TOL / scale[..., None] * 2 + 1e-6 * np.abs(v)
        assert np.all(near[diff]), "a code differs away from a rounding midpoint"
        assert diff.mean() < 1e-3


@pytest.mark.parametrize("B,n_tok,pos0,dtype,R", [
    (2, 4096, 131072, "bf16", 0),     # the chunked-prefill index keys
    (1, 256, 0, "f32", 0),            # tiny prefill, fp32 inputs
    (3, 37, 8, "bf16", 64),           # ragged chunk, with RoPE on the last 64 dims
])
def test_fp8_keys(B, n_tok, pos0, dtype, R):
    c = 128
    inp = synth.compressor_inputs(f"q8.{n_tok}.{pos0}", B, n_tok, c, 4, pos0, dtype=dtype)
    tdt = torch.float32 if dtype == "f32" else BF
    d = {k: dev(v, tdt if k != "bias" else torch.float32) for k, v in inp.items()}
    codes, scale = csa.csa_compress(4, d["Ca"], d["Za"], d["bias"], d["Cb"], d["Zb"], d.get("prev_Cb"),
                                    d.get("prev_Zb"), pos0=pos0, out_dtype=torch.uint8, rope_dims=R)
    torch.cuda.synchronize()
    ref = oc.compress(inp["Ca"], inp["Za"], inp["bias"], 4, inp["Cb"], inp["Zb"], inp.get("prev_Cb"),
                      inp.get("prev_Zb"), pos0=pos0, rope_dims=R)
    assert codes.dtype == torch.uint8 and codes.shape == (B, n_tok // 4, c)
    _check(host(codes), host(scale), ref)


def test_fp8_wide_rows_fp32_many_workgroups():
    """fp32 inputs with c = 1024 and 1,024 entries: one 256-thread row group per
    workgroup (the launch shape whose RMSNorm and amax reductions use only the
    small reduction area of the workgroup's LDS)."""
    B, n_tok, c = 1, 4096, 1024
    inp = synth.compressor_inputs("q8.wide", B, n_tok, c, 4, 0)
    d = {k: dev(v) for k, v in inp.items()}
    codes, scale = csa.csa_compress(4, d["Ca"], d["Za"], d["bias"], d["Cb"], d["Zb"], out_dtype=torch.uint8)
    torch.cuda.synchronize()
    ref = oc.compress(inp["Ca"], inp["Za"], inp["bias"], 4, inp["Cb"], inp["Zb"])
    assert codes.shape == (B, n_tok // 4, c)
    _check(host(codes), host(scale), ref)


def test_fp8_key_into_cache_slot_at_decode():
    """A decode step writes entry 16,383 of every sequence's fp8 key cache and
    its scale in place; nothing else in the caches changes."""
    B, N, c = 8, 64, 128
    inp = synth.compressor_inputs("q8.slot", B, 4, c, 4, 65532, dtype="bf16")
    d = {k: dev(v, BF if k != "bias" else torch.float32) for k, v in inp.items()}
    cache = torch.full((B, N, c), 0x11, dtype=torch.uint8, device="cuda")
    scales = torch.full((B, N), 7.0, dtype=torch.float32, device="cuda")
    csa.csa_compress(4, d["Ca"], d["Za"], d["bias"], d["Cb"], d["Zb"], d["prev_Cb"], d["prev_Zb"], pos0=65532,
                     out=cache, cache_entry0=N - 1, out_scale=scales)
    torch.cuda.synchronize()
    ref = oc.compress(inp["Ca"], inp["Za"], inp["bias"], 4, inp["Cb"], inp["Zb"], inp["prev_Cb"], inp["prev_Zb"],
                      pos0=65532)
    hc, hs = host(cache), host(scales)
    _check(hc[:, N - 1], hs[:, N - 1], ref[:, 0])
    assert np.all(hc[:, :N - 1] == 0x11) and np.all(hs[:, :N - 1] == 7.0)


def test_fp8_batch_of_key_streams():
    """Two fp8 key compressions of the same tokens in one csa_compress_batch launch."""
    jobs, refs = [], []
    for name in ("a", "b"):
        inp = synth.compressor_inputs(f"q8.batch.{name}", 4, 64, 128, 4, 128, dtype="bf16")
        d = {k: dev(v, BF if k != "bias" else torch.float32) for k, v in inp.items()}
        jobs.append(dict(ratio=4, Ca=d["Ca"], Za=d["Za"], bias=d["bias"], Cb=d["Cb"], Zb=d["Zb"],
                         prev_Cb=d["prev_Cb"], prev_Zb=d["prev_Zb"], pos0=128, out_dtype=torch.uint8))
        refs.append(oc.compress(inp["Ca"], inp["Za"], inp["bias"], 4, inp["Cb"], inp["Zb"], inp["prev_Cb"],
                                inp["prev_Zb"], pos0=128))
    outs = csa.csa_compress_batch(jobs)
    torch.cuda.synchronize()
    for (codes, scale), ref in zip(outs, refs):
        _check(host(codes), host(scale), ref)


def test_fp8_keys_feed_the_fp8_indexer():
    """Keys written by quantize-on-write are what lightning_index reads as fp8:
    the indexer's scores over them equal its scores over the same codes and
    scales handed over by the host (a byte-for-byte hand-over)."""
    B, n_tok, c, pos0 = 1, 512, 128, 0
    inp = synth.compressor_inputs("q8.idx", B, n_tok, c, 4, pos0, dtype="bf16")
    d = {k: dev(v, BF if k != "bias" else torch.float32) for k, v in inp.items()}
    codes, scale = csa.csa_compress(4, d["Ca"], d["Za"], d["bias"], d["Cb"], d["Zb"], pos0=pos0,
                                    out_dtype=torch.uint8)
    qc, qs = synth.quant_fp8_rows(synth.normal("q8.idx.q", (B, 16, 64, 128)))
    w = dev(synth.uniform("q8.idx.w", (B, 16, 64)))
    s1 = csa.lightning_index(dev(qc, torch.uint8), w, codes, q_pos0=n_tok - 16, qk_dtype=csa.FP8_E4M3,
                             q_scale=dev(qs), k_scale=scale, score_dtype=torch.float32)
    s2 = csa.lightning_index(dev(qc, torch.uint8), w, dev(host(codes), torch.uint8), q_pos0=n_tok - 16,
                             qk_dtype=csa.FP8_E4M3, q_scale=dev(qs), k_scale=dev(host(scale)),
                             score_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)


def test_mixed_batch_bf16_latent_and_fp8_key():
    """The CSA layer's decode write in one launch: the 512-d latent in bf16 and
    the 128-d indexer key quantized on write, into their cache slots."""
    B, N = 16, 64
    jobs, refs = [], []
    kv = torch.zeros(B, N, 512, dtype=BF, device="cuda")
    keys = torch.zeros(B, N, 128, dtype=torch.uint8, device="cuda")
    kscale = torch.zeros(B, N, dtype=torch.float32, device="cuda")
    for c, out in ((512, kv), (128, keys)):
        inp = synth.compressor_inputs(f"q8.mixed.{c}", B, 4, c, 4, 65532, dtype="bf16")
        d = {k: dev(v, BF if k != "bias" else torch.float32) for k, v in inp.items()}
        job = dict(ratio=4, Ca=d["Ca"], Za=d["Za"], bias=d["bias"], Cb=d["Cb"], Zb=d["Zb"], prev_Cb=d["prev_Cb"],
                   prev_Zb=d["prev_Zb"], pos0=65532, out=out, cache_entry0=N - 1, rope_dims=64)
        if c == 128:
            job["out_scale"] = kscale
        jobs.append(job)
        refs.append(oc.compress(inp["Ca"], inp["Za"], inp["bias"], 4, inp["Cb"], inp["Zb"], inp["prev_Cb"],
                                inp["prev_Zb"], pos0=65532, rope_dims=64))
    csa.csa_compress_batch(jobs)
    torch.cuda.synchronize()
    assert np.max(np.abs(host(kv)[:, N - 1] - refs[0][:, 0])) < 2e-2
    assert np.all(host(kv)[:, :N - 1] == 0)
    _check(host(keys)[:, N - 1], host(kscale)[:, N - 1], refs[1][:, 0])


# ---------------------------------------------------------------- MXFP4 (the pages' FP4 indexer keys)

def _check_fp4(packed, scales, ref):
    """packed [.., c/2], scales [.., c/32] (GPU); ref [.., c] fp64 (oracle)."""
    c = ref.shape[-1]
    dec = on.dequant_mxfp4(packed, scales)
    s = np.repeat(on.decode_e8m0(scales), 32, axis=-1)
    o_p, o_s = on.quant_mxfp4_rows_f32(ref)
    # the shared exponent may differ only when a block's amax lies next to a power of two
    blocks = np.abs(ref.reshape(*ref.shape[:-1], c // 32, 32)).max(axis=-1)
    near_pow2 = np.abs(np.log2(np.maximum(blocks, 1e-30)) - np.round(np.log2(np.maximum(blocks, 1e-30)))) < 1e-4
    assert np.all((scales == o_s) | near_pow2)
    v = ref / s
    a = np.abs(v)
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    err = np.abs(dec - ref)
    assert np.all((err <= (0.5 * step * (1 + 1e-6)) * s + PRE_TOL) | (a > 6)), np.max(err - 0.5 * step * s)
    # elements agree with the oracle's codes except next to a rounding midpoint
    same_scale = np.repeat(scales == o_s, 32, axis=-1)
    dec_o = on.dequant_mxfp4(o_p, o_s)
    diff = (dec != dec_o) & same_scale
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    near_mid = np.min(np.abs(a[..., None] - mids), axis=-1) <= PRE_TOL / s * 2 + 1e-6 * a
    assert np.all(near_mid[diff])


@pytest.mark.parametrize("B,n_tok,pos0,dtype,R", [
    (2, 4096, 131072, "bf16", 0),
    (1, 256, 0, "f32", 0),
    (3, 37, 8, "bf16", 64),
])
def test_mxfp4_keys(B, n_tok, pos0, dtype, R):
    c = 128
    inp = synth.compressor_inputs(f"q4.{n_tok}.{pos0}", B, n_tok, c, 4, pos0, dtype=dtype)
    tdt = torch.float32 if dtype == "f32" else BF
    d = {k: dev(v, tdt if k != "bias" else torch.float32) for k, v in inp.items()}
    packed, scales = csa.csa_compress(4, d["Ca"], d["Za"], d["bias"], d["Cb"], d["Zb"], d.get("prev_Cb"),
                                      d.get("prev_Zb"), pos0=pos0, out_dtype=csa.MXFP4, rope_dims=R)
    torch.cuda.synchronize()
    assert packed.shape == (B, n_tok // 4, c // 2) and scales.shape == (B, n_tok // 4, c // 32)
    ref = oc.compress(inp["Ca"], inp["Za"], inp["bias"], 4, inp["Cb"], inp["Zb"], inp.get("prev_Cb"),
                      inp.get("prev_Zb"), pos0=pos0, rope_dims=R)
    _check_fp4(host(packed), host(scales), ref)


def test_mxfp4_keys_feed_the_mxfp4_indexer_and_mix_in_a_batch():
    """A bf16 latent and MXFP4 keys in one batch launch, into cache slots; the
    keys are what lightning_index reads as CSA_MXFP4 (byte-for-byte hand-over)."""
    B, N = 4, 64
    kv = torch.zeros(B, N, 512, dtype=BF, device="cuda")
    keys = torch.zeros(B, N, 64, dtype=torch.uint8, device="cuda")
    ks = torch.zeros(B, N, 4, dtype=torch.uint8, device="cuda")
    jobs, refs = [], []
    for c, out in ((512, kv), (128, keys)):
        inp = synth.compressor_inputs(f"q4.mix.{c}", B, 4 * N, c, 4, 0, dtype="bf16")
        d = {k: dev(v, BF if k != "bias" else torch.float32) for k, v in inp.items()}
        job = dict(ratio=4, Ca=d["Ca"], Za=d["Za"], bias=d["bias"], Cb=d["Cb"], Zb=d["Zb"], pos0=0, out=out,
                   cache_entry0=0)
        if c == 128:
            job["out_scale"] = ks
        jobs.append(job)
        refs.append(oc.compress(inp["Ca"], inp["Za"], inp["bias"], 4, inp["Cb"], inp["Zb"], pos0=0))
    csa.csa_compress_batch(jobs)
    torch.cuda.synchronize()
    assert np.max(np.abs(host(kv) - refs[0])) < 2e-2
    _check_fp4(host(keys), host(ks), refs[1])
    qp, qs = synth.quant_mxfp4(synth.normal("q4.mix.q", (B, 8, 64, 128)))
    w = dev(synth.uniform("q4.mix.w", (B, 8, 64)))
    args = dict(q_pos0=4 * N - 8, qk_dtype=csa.MXFP4, q_scale=dev(qs, torch.uint8), score_dtype=torch.float32)
    s1 = csa.lightning_index(dev(qp, torch.uint8), w, keys, k_scale=ks, **args)
    s2 = csa.lightning_index(dev(qp, torch.uint8), w, dev(host(keys), torch.uint8),
                             k_scale=dev(host(ks), torch.uint8), **args)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
