"""GPU tests of hca_attn_compressed: an HCA decode step's C128A write and
the dense attention in one call.

Pages: "DeepSeek V4 结构速览" (HCA（c128a 路线）: an entry pools 128 raw
tokens; dense MQA over every visible entry plus the window, with a sink);
"DeepSeek-V4技术报告解读，全适配国产算力" 2.1 (the compression formula).

In the single launch the workgroup whose tiles hold the new entry pools it
(one pass over 128 rows, eight row groups) before it reads them.  Checked: the
written entry against the oracle compressor (and against the separate
csa_compress call within the same tolerance -- its row groups are summed in
another order), every other cache entry untouched, the attention output equal
bit for bit to hca_attn over the cache as written, and against the oracle's
attention.  The fallback route (a plan the fused kernel does not take) gives
exactly csa_compress + hca_attn.  A kernel trace shows which launches ran.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_compress_amd as csa
import synth
from oracle import attention as oa
from oracle import compressor as oc
from helpers import ATTN_BF16_MAX_ABS, ATTN_NORMWISE, COMP_BF16_MAX_ABS, host, max_abs, normwise_rel

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _case(tag, B, N, q0, e_new=None, rope=0, gamma=False):
    dn = synth.device_normal
    cpos = q0 + 1 - 128
    e_new = cpos // 128 if e_new is None else e_new
    d = dict(B=B, N=N, q0=q0, raw0=q0 - 127, cpos=cpos, e_new=e_new, rope=rope,
             kv=dn(f"{tag}.kv", (B, N, 512), BF), q=dn(f"{tag}.q", (B, 1, 64, 512), BF),
             raw=dn(f"{tag}.raw", (B, 128, 512), BF), sink=dn(f"{tag}.sink", (64,)),
             Ca=dn(f"{tag}.Ca", (B, 128, 512), BF), Za=dn(f"{tag}.Za", (B, 128, 512), BF),
             bias=dn(f"{tag}.b", (128, 512), var=0.1),
             gamma=(synth.device_uniform(f"{tag}.g", (512,)) + 0.5) if gamma else None)
    return d


def _job(d, kv):
    j = dict(ratio=128, Ca=d["Ca"], Za=d["Za"], bias=d["bias"], pos0=d["cpos"], out=kv, cache_entry0=d["e_new"])
    if d["gamma"] is not None:
        j["gamma"] = d["gamma"]
    if d["rope"]:
        j["rope_dims"] = d["rope"]
    return j


def _fused(d, kv):
    return csa.hca_attn_compressed(d["q"], kv, d["raw"], _job(d, kv), e_new=d["e_new"], q_pos0=d["q0"],
                                   raw_pos0=d["raw0"], sink=d["sink"])


def _separate(d, kv):
    csa.csa_compress(128, d["Ca"], d["Za"], d["bias"], pos0=d["cpos"], out=kv, cache_entry0=d["e_new"],
                     gamma=d["gamma"], rope_dims=d["rope"], workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    return csa.hca_attn(d["q"], kv, d["raw"], q_pos0=d["q0"], raw_pos0=d["raw0"], sink=d["sink"])


def _kernels(fn):
    from torch.profiler import ProfilerActivity, profile
    try:
        with profile(activities=[ProfilerActivity.CUDA]) as prof:
            fn()
            torch.cuda.synchronize()
    except Exception:
        return None
    names = [e.name for e in prof.events() if e.device_type.name == "CUDA"]
    return names or None


def _check(d, fused_launch=True, oracle_seqs=(0,)):
    kv0 = d["kv"]
    kv1, kv2 = kv0.clone(), kv0.clone()
    o1 = _fused(d, kv1)
    o2 = _separate(d, kv2)
    torch.cuda.synchronize()
    e = d["e_new"]
    # every other entry untouched
    mask = torch.ones(d["N"], dtype=torch.bool, device="cuda")
    mask[e] = False
    assert torch.equal(kv1[:, mask], kv0[:, mask])
    # the entry: the oracle's, and the separate call's, within the compressor tolerance
    ref = oc.compress(host(d["Ca"]), host(d["Za"]), host(d["bias"]), 128, pos0=d["cpos"],
                      gamma=None if d["gamma"] is None else host(d["gamma"]), rope_dims=d["rope"])
    got = host(kv1[:, e:e + 1])
    assert max_abs(got, ref) <= COMP_BF16_MAX_ABS, max_abs(got, ref)
    assert max_abs(got, host(kv2[:, e:e + 1])) <= COMP_BF16_MAX_ABS
    # the attention: hca_attn over the cache as written, bit for bit
    o3 = csa.hca_attn(d["q"], kv1, d["raw"], q_pos0=d["q0"], raw_pos0=d["raw0"], sink=d["sink"])
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))
    if not fused_launch:
        assert torch.equal(kv1, kv2) and torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    # and the oracle's attention on the written cache
    for b in oracle_seqs:
        r, _ = oa.hca_attention(host(d["q"][b:b + 1]), host(kv1[b:b + 1]), host(d["raw"][b:b + 1]), d["raw0"],
                             d["q0"], host(d["sink"]))
        g = host(o1[b:b + 1])
        assert max_abs(g, r) <= ATTN_BF16_MAX_ABS and normwise_rel(g, r) <= ATTN_NORMWISE
    names = _kernels(lambda: _fused(d, kv0.clone()))
    if names is not None:
        ours = [n for n in names if "attn" in n or "compress" in n]
        fused = [n for n in ours if "attn_bf16_kernel<2, 4, false, true>" in n]
        if fused_launch:
            assert len(fused) == 1 and not any("compress_" in n for n in ours), ours
        else:
            assert not fused and any("compress_kernel" in n for n in ours), ours


def test_fused_hca_decode_1m():
    """The HCA decode at 1,048,576 context, batch 16, 8,192 entries: the new
    entry is the last one, in the short last split."""
    d = _case("fh.1m", 16, 8192, 1048575)
    _check(d, oracle_seqs=(0, 15))


def test_fused_hca_rope_gamma():
    """Partial RoPE and RMSNorm gains on the written entry; 4,096 entries."""
    d = _case("fh.rope", 16, 4096, 4096 * 128 - 1, rope=64, gamma=True)
    _check(d, oracle_seqs=(2,))


def test_fused_hca_entry_not_last():
    """The written entry lies inside a middle split (a cache whose newest
    entry is not the list's last visible one)."""
    d = _case("fh.mid", 16, 4096, 4096 * 128 - 1, e_new=1500)
    _check(d, oracle_seqs=(1,))


def test_fallback_short_context():
    """A plan the fused kernel does not take (splits of 4 tiles): the
    compressor's launch, then the attention's -- exactly the two calls."""
    d = _case("fh.short", 4, 128, 100 * 128 - 1)
    _check(d, fused_launch=False, oracle_seqs=(3,))


def test_fallback_many_short_splits():
    """Batch 4 at 4,096 entries: the plan splits each query into 5-tile runs,
    which the fused kernel does not take -- the two calls, exactly."""
    d = _case("fh.b4", 4, 4096, 4096 * 128 - 1, rope=64)
    _check(d, fused_launch=False, oracle_seqs=(0,))


def test_fused_hca_graph_replays():
    """Captured in a HIP graph: every replay rewrites the entry and gives the
    eager call's bytes."""
    d = _case("fh.graph", 16, 4096, 4096 * 128 - 1)
    ref_kv = d["kv"].clone()
    ref_o = _fused(d, ref_kv)
    torch.cuda.synchronize()
    kv = d["kv"].clone()
    st = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        o = _fused(d, kv)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=st):
            o = _fused(d, kv)
    torch.cuda.synchronize()
    e = d["e_new"]
    for rep in range(3):
        kv[:, e].zero_()
        o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(kv, ref_kv), f"replay {rep}: cache"
        assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16)), f"replay {rep}: output"


def test_fused_hca_ragged_last_tile():
    """4,100 entries (the new entry alone in a partial tile of the short last
    split, followed by the window)."""
    d = _case("fh.rag", 16, 4100, 4100 * 128 - 1)
    _check(d, oracle_seqs=(5,))
