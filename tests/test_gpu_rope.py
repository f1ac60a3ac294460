"""GPU parity of partial RoPE against the oracle, through the C ABI: csa_rope
on query and window rows, the compressor's RoPE at the entry anchor
(csa_compress_ex, every compressor path), and the attention epilogues'
inverse RoPE (sparse_mqa_attn_ex / hca_attn_ex: one-workgroup, split +
combine, batch-invariant and fp32 paths).

Pages: "DeepSeek Technical Reports" (DeepSeek-V4, Hybrid Attention, CSA:
position handled by partial RoPE) and "DeepSeek V4 结构速览" (RMSNorm +
RoPE in the compressor; inverse RoPE on the last 64 output dims).
Tolerances: fp32 rows 2e-6 max-abs (|x| ~ 1; the angles are fp64, the
rotation fp32); bf16 rows one bf16 ulp of the result (2^-8 |ref|, plus a
floor for values near zero); compressor and attention outputs as in their
own tests.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_compress_amd as csa
import synth
from oracle import attention as oa
from oracle import compressor as oc
from oracle import rope as orp
from helpers import (ATTN_BF16_MAX_ABS, ATTN_F32_MAX_ABS, ATTN_NORMWISE, COMP_BF16_MAX_ABS,
                     COMP_F32_MAX_ABS, dev, host, max_abs, normwise_rel)

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _bf16_close(got, ref):
    return np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 2.0 ** -14)


@pytest.mark.parametrize("shape,pos0,R,inverse", [
    ((2, 5, 64, 512), 0, 64, False),            # q rows, positions 0..4
    ((32, 1, 64, 512), 65535, 64, False),       # decode queries
    ((1, 300, 64, 512), 1048000, 64, True),     # long context, inverse, ragged T
    ((4, 128, 512), 1047000, 64, False),        # window rows [B, n_raw, 512]
    ((3, 7, 2, 128), 99, 128, False),           # the whole row rotated
    ((2, 3, 5, 1024), 12345, 1024, True),       # the widest rotated part
])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rope_rows(shape, pos0, R, inverse, dtype):
    x = synth.normal(f"rope.rows.{len(shape)}.{shape[-1]}.{pos0}", shape)
    tdt = torch.float32 if dtype == "f32" else BF
    xd = dev(x, tdt)
    xin = host(xd)                               # the bytes the kernel reads
    before = xd.clone()
    csa.rope(xd, pos0=pos0, rope_dims=R, inverse=inverse)
    torch.cuda.synchronize()
    got = host(xd)
    xr = xin if len(shape) == 4 else xin[:, :, None, :]
    ref = orp.rotate_rows(xr, pos0, R, inverse=inverse)
    ref = ref if len(shape) == 4 else ref[:, :, 0, :]
    D = shape[-1]
    assert torch.equal(xd[..., :D - R], before[..., :D - R])    # the unrotated part is untouched
    if dtype == "f32":
        assert max_abs(got, ref) < 2e-6
    else:
        assert _bf16_close(got, ref)


def test_rope_then_inverse_is_identity_fp32():
    x = dev(synth.normal("rope.id", (2, 9, 64, 512)))
    y = x.clone()
    csa.rope(y, pos0=1048570, rope_dims=64)
    csa.rope(y, pos0=1048570, rope_dims=64, inverse=True)
    torch.cuda.synchronize()
    assert max_abs(host(y), host(x)) < 1e-6


def _cmp(ratio, B, n_tok, c, pos0, dtype, R, anchor, out_dtype=None, workspace=None, prefix="rc"):
    inp = synth.compressor_inputs(prefix, B, n_tok, c, ratio, pos0, dtype=dtype)
    tdt = torch.float32 if dtype == "f32" else BF
    d = {k: dev(v, tdt if k != "bias" else torch.float32) for k, v in inp.items()}
    out = csa.csa_compress(ratio, d["Ca"], d["Za"], d["bias"], d.get("Cb"), d.get("Zb"), d.get("prev_Cb"),
                           d.get("prev_Zb"), pos0=pos0, out_dtype=out_dtype, workspace=workspace,
                           rope_dims=R, rope_anchor=anchor)
    torch.cuda.synchronize()
    ref = oc.compress(inp["Ca"], inp["Za"], inp["bias"], ratio, inp.get("Cb"), inp.get("Zb"),
                      inp.get("prev_Cb"), inp.get("prev_Zb"), pos0=pos0, rope_dims=R, rope_anchor=anchor)
    return host(out), ref


@pytest.mark.parametrize("ratio,B,n_tok,c,pos0,dtype,R,anchor", [
    (4, 1, 256, 512, 0, "f32", 64, 0),          # tiny prefill, main latent
    (4, 1, 256, 128, 0, "f32", 64, 3),          # indexer keys, last anchor offset
    (4, 2, 4096, 512, 131072, "bf16", 64, 0),   # chunk with halo
    (4, 32, 4, 512, 65532, "bf16", 64, 1),      # decode block
    (4, 3, 37, 192, 8, "f32", 192, 2),          # ragged; the whole entry rotated
    (128, 2, 2048, 512, 1046528, "bf16", 64, 127),   # C128A chunk at 1M context
])
def test_compress_rope(ratio, B, n_tok, c, pos0, dtype, R, anchor):
    got, ref = _cmp(ratio, B, n_tok, c, pos0, dtype, R, anchor, prefix=f"rc{ratio}.{c}.{pos0}")
    assert got.shape == ref.shape
    assert max_abs(got, ref) < (COMP_F32_MAX_ABS if dtype == "f32" else COMP_BF16_MAX_ABS)


@pytest.mark.parametrize("B,dtype", [(32, "bf16"), (3, "f32")])
def test_compress_rope_row_split_path(B, dtype):
    """Few C128A entries: the row-split path rotates in its merge kernel, the
    single-pass path in its epilogue; both match the oracle."""
    n_tok = 128 * (3 if B == 3 else 1)
    pos0 = 1048576 - n_tok
    assert csa.workspace_bytes(csa.OP_COMPRESS, B, n_tok, 512, 128) > 0
    split, ref = _cmp(128, B, n_tok, 512, pos0, dtype, 64, 64, prefix=f"rsplit{B}")
    single, _ = _cmp(128, B, n_tok, 512, pos0, dtype, 64, 64, prefix=f"rsplit{B}",
                     workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    tol = COMP_F32_MAX_ABS if dtype == "f32" else COMP_BF16_MAX_ABS
    assert max_abs(split, ref) < tol and max_abs(single, ref) < tol


def test_compress_batch_rope():
    """csa_compress_batch carries each job's RoPE arguments."""
    jobs, refs = [], []
    for c, R, anc in ((512, 64, 0), (128, 64, 2)):
        inp = synth.compressor_inputs(f"rbatch{c}", 8, 4, c, 4, 65532, dtype="bf16")
        d = {k: dev(v, BF if k != "bias" else torch.float32) for k, v in inp.items()}
        jobs.append(dict(ratio=4, Ca=d["Ca"], Za=d["Za"], bias=d["bias"], Cb=d["Cb"], Zb=d["Zb"],
                         prev_Cb=d["prev_Cb"], prev_Zb=d["prev_Zb"], pos0=65532, rope_dims=R, rope_anchor=anc))
        refs.append(oc.compress(inp["Ca"], inp["Za"], inp["bias"], 4, inp["Cb"], inp["Zb"], inp["prev_Cb"],
                                inp["prev_Zb"], pos0=65532, rope_dims=R, rope_anchor=anc))
    outs = csa.csa_compress_batch(jobs)
    torch.cuda.synchronize()
    for got, ref in zip(outs, refs):
        assert max_abs(host(got), ref) < COMP_BF16_MAX_ABS


def _assert_bf16(got, ref):
    assert max_abs(got, ref) < ATTN_BF16_MAX_ABS
    assert normwise_rel(got, ref) < ATTN_NORMWISE


def _visible(q_pos0, T, N):
    return [min((q_pos0 + t + 1) // 4, N) for t in range(T)]


def _sparse(name, B, T, N, k, q0, dtype=BF):
    rp0 = max(0, q0 - 127)
    q = synth.device_normal(name + ".q", (B, T, 64, 512), dtype)
    kv = synth.device_normal(name + ".kv", (B, N, 512), dtype)
    raw = synth.device_normal(name + ".raw", (B, q0 + T - rp0, 512), dtype)
    idx = synth.random_topk_indices(name + ".idx", B, T, k, _visible(q0, T, N))
    return q, kv, raw, idx, rp0


def _sparse_ref(q, kv, idx, raw, rp0, q0, b, t, R):
    sel = idx[b, t]
    valid = sel[sel >= 0]
    rows = host(kv[b, torch.as_tensor(valid, device=kv.device, dtype=torch.long)])
    pos = q0 + t
    w0 = max(0, pos - 127)
    rw = host(raw[b, w0 - rp0:pos - rp0 + 1])
    o, _ = oa.sparse_mqa(host(q[b, t])[None, None], rows[None], np.arange(len(valid))[None, None], rw[None],
                         w0, pos, 128, rope_dims=R)
    return o[0, 0]


@pytest.mark.parametrize("name,B,T,N,k,q0,bi", [
    ("ra.dec", 32, 1, 16384, 512, 65535, False),    # split decode: inverse RoPE in the combine
    ("ra.bi", 4, 1, 4096, 512, 16383, True),        # batch-invariant, one head block per workgroup
    ("ra.pf", 1, 512, 33792, 512, 131072, False),   # prefill: one workgroup per query
])
def test_sparse_attn_inverse_rope(name, B, T, N, k, q0, bi):
    q, kv, raw, idx, rp0 = _sparse(name, B, T, N, k, q0)
    out = csa.sparse_mqa_attn(q, kv, dev(idx, torch.int32), raw, q_pos0=q0, raw_pos0=rp0, rope_dims=64,
                              batch_invariant=bi)
    plain = csa.sparse_mqa_attn(q, kv, dev(idx, torch.int32), raw, q_pos0=q0, raw_pos0=rp0, batch_invariant=bi)
    torch.cuda.synchronize()
    got = host(out)
    # the first 448 dims are the plain output's, bit for bit
    assert torch.equal(out[..., :448], plain[..., :448])
    for b, t in ([(0, 0), (B - 1, 0), (B // 2, 0)] if T == 1 else [(0, 0), (0, 255), (0, T - 1)]):
        _assert_bf16(got[b, t], _sparse_ref(q, kv, idx, raw, rp0, q0, b, t, 64))


@pytest.mark.parametrize("B,T,q0,bi", [(16, 1, 1048575, False), (2, 1, 1048575, True), (1, 256, 1046528, False)])
def test_hca_attn_inverse_rope(B, T, q0, bi):
    N = (q0 + T) // 128
    rp0 = q0 - 127
    name = f"rh.{B}.{T}"
    q = synth.device_normal(name + ".q", (B, T, 64, 512), BF)
    kv = synth.device_normal(name + ".kv", (B, N, 512), BF)
    raw = synth.device_normal(name + ".raw", (B, q0 + T - rp0, 512), BF)
    sink = synth.device_normal(name + ".sink", (64,))
    out = csa.hca_attn(q, kv, raw, q_pos0=q0, raw_pos0=rp0, sink=sink, rope_dims=64, batch_invariant=bi)
    torch.cuda.synchronize()
    got = host(out)
    for b, t in [(0, 0), (B - 1, T - 1)]:
        pos = q0 + t
        V = (pos + 1) // 128
        rw = host(raw[b, pos - 127 - rp0:pos - rp0 + 1])
        o, _ = oa.dense_attention(host(q[b, t])[None, None], host(kv[b, :V])[None], rw[None], pos - 127, pos, 128,
                                  128, sink=host(sink), rope_dims=64)
        _assert_bf16(got[b, t], o[0, 0])


def test_fp32_attn_inverse_rope():
    """fp32 I/O: the plain fp32 kernel rotates its thread-local pairs."""
    q, kv, raw, idx, rp0 = _sparse("ra.f32", 1, 40, 64, 16, 200, torch.float32)
    out = csa.sparse_mqa_attn(q, kv, dev(idx, torch.int32), raw, q_pos0=200, raw_pos0=rp0, rope_dims=64,
                              rope_base=500.0)
    torch.cuda.synchronize()
    ref, _ = oa.sparse_mqa(host(q), host(kv), idx, host(raw), rp0, 200, 128, rope_dims=64, rope_base=500.0)
    assert max_abs(host(out), ref) < ATTN_F32_MAX_ABS
