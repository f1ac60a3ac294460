"""GPU parity of csa_compress (stage 1) against the oracle, through the C ABI.

Page: "DeepSeek V4 结构速览", C4A Compressor; "DeepSeek-V4技术报告解读，全适配国产
算力", 2.1.  Tolerances: fp32 output 1e-4 max-abs; bf16 output 2e-2 max-abs
(the outputs are RMS-normalised, |x| ~ 1, so this is a few bf16 ulps).
"""
import numpy as np
import pytest
import torch

import long_context_sparse_compress_amd as csa
import synth
from oracle import compressor as oc
from helpers import COMP_BF16_MAX_ABS, COMP_F32_MAX_ABS, dev, host, max_abs

pytestmark = pytest.mark.gpu


def _run(ratio, B, n_tok, c, pos0, dtype, out_dtype=None, prefix="cmp", gamma=False, eps=1e-6, workspace=None):
    inp = synth.compressor_inputs(prefix, B, n_tok, c, ratio, pos0, dtype=dtype)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    odt = tdt if out_dtype is None else out_dtype
    g = synth.normal(prefix + ".gamma", (c,)) if gamma else None
    d = {k: dev(v, tdt if k != "bias" else torch.float32) for k, v in inp.items()}
    out = csa.csa_compress(ratio, d["Ca"], d["Za"], d["bias"], d.get("Cb"), d.get("Zb"),
                           d.get("prev_Cb"), d.get("prev_Zb"), pos0=pos0,
                           gamma=None if g is None else dev(g), eps=eps, out_dtype=odt, workspace=workspace)
    torch.cuda.synchronize()
    ref = oc.compress(inp["Ca"], inp["Za"], inp["bias"], ratio, inp.get("Cb"), inp.get("Zb"),
                      inp.get("prev_Cb"), inp.get("prev_Zb"), pos0=pos0, gamma=g, eps=eps)
    return host(out), ref, out


@pytest.mark.parametrize("c", [512, 128])
def test_tiny_prefill_fp32(c):
    """The tiny CSA prefill: 256 raw tokens, fp32, main (512) and key (128) compressors."""
    got, ref, _ = _run(4, 1, 256, c, 0, "f32", prefix=f"tiny{c}")
    assert got.shape == (1, 64, c)
    assert max_abs(got, ref) < COMP_F32_MAX_ABS


@pytest.mark.parametrize("c", [512, 128])
def test_chunk_with_halo_bf16(c):
    """The chunked-prefill compressor: 4096 tokens after 131,072 of context, bf16, halo."""
    got, ref, _ = _run(4, 1, 4096, c, 131072, "bf16", prefix=f"chunk{c}")
    assert got.shape == (1, 1024, c)
    assert max_abs(got, ref) < COMP_BF16_MAX_ABS


def test_c128a_prefill_chunk_bf16():
    got, ref, _ = _run(128, 2, 2048, 512, 1046528, "bf16", prefix="hcachunk")
    assert got.shape == (2, 16, 512)
    assert max_abs(got, ref) < COMP_BF16_MAX_ABS


def test_c128a_decode_block_fp32_out():
    got, ref, _ = _run(128, 16, 128, 512, 1048448, "bf16", out_dtype=torch.float32, prefix="hcadec")
    assert max_abs(got, ref) < 1e-5 * 50


@pytest.mark.parametrize("ratio,B,n_tok,c,pos0", [
    (4, 3, 30, 64, 0),         # ragged tail, smallest channel count
    (4, 2, 4, 512, 65532),     # decode: one block plus halo
    (4, 5, 37, 192, 8),        # ragged, c not a power of two
    (128, 1, 300, 1024, 0),    # widest channel count, ragged
    (4, 1, 3, 512, 0),         # no complete block: nothing written
])
def test_edge_shapes_fp32(ratio, B, n_tok, c, pos0):
    got, ref, _ = _run(ratio, B, n_tok, c, pos0, "f32", prefix=f"edge{ratio}_{n_tok}_{c}", gamma=True)
    assert got.shape == ref.shape
    if got.size:
        assert max_abs(got, ref) < COMP_F32_MAX_ABS


def test_decode_writes_into_cache_slot():
    """out_batch_stride lets a decode step write entry 16383 of each sequence in place."""
    B, N, c = 4, 64, 512
    d = {k: dev(v, torch.bfloat16 if k != "bias" else torch.float32) for k, v in
         synth.compressor_inputs("slot", B, 4, c, 4, 252, dtype="bf16").items()}
    cache = torch.full((B, N, c), 7.0, dtype=torch.bfloat16, device="cuda")
    # the slot view is not contiguous across sequences: pass the slot's address and the stride
    slot = cache.view(-1)[(N - 1) * c:]
    st = csa.library().csa_compress(4, B, 4, c, 252, d["Ca"].data_ptr(), d["Za"].data_ptr(),
                                    d["Cb"].data_ptr(), d["Zb"].data_ptr(), d["prev_Cb"].data_ptr(),
                                    d["prev_Zb"].data_ptr(), d["bias"].data_ptr(), None, 1e-6,
                                    csa.BF16, csa.BF16, slot.data_ptr(), N * c, None, 0,
                                    torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    inpb = synth.compressor_inputs("slot", B, 4, c, 4, 252, dtype="bf16")
    ref = oc.compress(inpb["Ca"], inpb["Za"], inpb["bias"], 4, inpb["Cb"], inpb["Zb"],
                      inpb["prev_Cb"], inpb["prev_Zb"], pos0=252)
    got = host(cache)
    assert max_abs(got[:, N - 1], ref[:, 0]) < COMP_BF16_MAX_ABS
    assert np.all(got[:, :N - 1] == 7.0)


@pytest.mark.parametrize("B,n_tok,c,dtype", [
    (32, 128, 512, "bf16"),    # the decode step: 32 entries, 8 row ranges of 16
    (100, 128, 128, "f32"),    # 100 entries: 2 ranges of 64
    (3, 384, 1024, "bf16"),    # 9 entries, widest channels: 16 ranges of 8
])
def test_c128a_row_split_matches_single_pass(B, n_tok, c, dtype):
    """Few C128A entries: the row-split path (partial states merged by a second
    kernel) and the one-workgroup-per-entry path both match the oracle."""
    assert csa.workspace_bytes(csa.OP_COMPRESS, B, n_tok, c, 128) > 0
    pos0 = 1048576 - n_tok
    split, ref, _ = _run(128, B, n_tok, c, pos0, dtype, prefix=f"split{B}", gamma=True)
    single, ref2, _ = _run(128, B, n_tok, c, pos0, dtype, prefix=f"split{B}", gamma=True,
                           workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    assert np.array_equal(ref, ref2)
    for got in (split, single):
        if dtype == "f32":
            assert max_abs(got, ref) < COMP_F32_MAX_ABS
        else:
            # gamma scales outputs past |x| ~ 1: allow one bf16 ulp of each value
            # (2^-7 |x| bounds it) -- the fp32 result can sit on the other side
            # of a rounding boundary from the oracle's
            assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 2.0 ** -12)


@pytest.mark.parametrize("ratio,B,n_tok,pos0", [(4, 32, 4, 65532), (4, 3, 37, 8), (128, 4, 256, 0)])
def test_batch_matches_single_calls(ratio, B, n_tok, pos0):
    """csa_compress_batch: a 512-d and a 128-d compression of the same tokens in
    one launch match the two csa_compress results and the oracle (the batched
    kernel may contract multiply-adds differently, so equal up to rounding)."""
    jobs, singles, refs = [], [], []
    for c in (512, 128):
        inp = synth.compressor_inputs(f"batch{ratio}_{c}", B, n_tok, c, ratio, pos0, dtype="bf16")
        d = {k: dev(v, torch.bfloat16 if k != "bias" else torch.float32) for k, v in inp.items()}
        args = dict(ratio=ratio, Ca=d["Ca"], Za=d["Za"], bias=d["bias"], Cb=d.get("Cb"), Zb=d.get("Zb"),
                    prev_Cb=d.get("prev_Cb"), prev_Zb=d.get("prev_Zb"), pos0=pos0)
        jobs.append(args)
        singles.append(csa.csa_compress(args["ratio"], args["Ca"], args["Za"], args["bias"], args["Cb"], args["Zb"],
                                        args["prev_Cb"], args["prev_Zb"], pos0=pos0,
                                        workspace=torch.empty(0, dtype=torch.uint8, device="cuda")))
        refs.append(oc.compress(inp["Ca"], inp["Za"], inp["bias"], ratio, inp.get("Cb"), inp.get("Zb"),
                                inp.get("prev_Cb"), inp.get("prev_Zb"), pos0=pos0))
    outs = csa.csa_compress_batch(jobs)
    torch.cuda.synchronize()
    for got, one, ref in zip(outs, singles, refs):
        assert max_abs(host(got), host(one)) < COMP_BF16_MAX_ABS
        assert max_abs(host(got), ref) < COMP_BF16_MAX_ABS


def test_deterministic():
    _, _, a = _run(128, 2, 1024, 512, 0, "bf16", prefix="det")
    _, _, b = _run(128, 2, 1024, 512, 0, "bf16", prefix="det")
    assert torch.equal(a, b)


def test_row_split_workspace_reused_across_calls_and_shapes():
    """One workspace serves a run of row-split C128A calls of different shapes
    (the partial states of one call never leak into the next)."""
    ws = torch.empty(max(csa.workspace_bytes(csa.OP_COMPRESS, B, 128 * nb, 512, 128)
                         for B, nb in [(32, 1), (3, 3), (1, 1), (100, 1)]), dtype=torch.uint8, device="cuda")
    for rep, (B, nb, c) in enumerate([(32, 1, 512), (3, 3, 512), (32, 1, 512), (1, 1, 128), (100, 1, 512),
                                      (3, 3, 512)]):
        n_tok = 128 * nb
        got, ref, _ = _run(128, B, n_tok, c, 1048576 - n_tok, "f32", prefix=f"reuse{rep % 3}", workspace=ws)
        assert max_abs(got, ref) < COMP_F32_MAX_ABS, (rep, B, nb, c)
