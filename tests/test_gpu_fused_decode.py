"""GPU tests of lightning_index_compressed: a decode step's compressor writes
and the lightning indexer in one call.

Pages: "DeepSeek V4 结构速览" (C4A Compressor: at decode the new entry pools
the current block with the previous one; Lightning Indexer: FP4 keys, BF16
scores), "DeepSeek Technical Reports" (DSA, the indexer equation).

The call must give exactly what csa_compress_batch followed by
lightning_index gives (both checked against the oracle by the compressor and
indexer tests): every byte of the caches the jobs write, and every score, bit
for bit -- in the single launch (MXFP4 keys, one query a sequence) and in
the two-launch fallback.  The new key's score is also checked against the
oracle on the decoded bytes.  A kernel trace shows which launches ran.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_compress_amd as csa
import synth
from oracle import indexer as oi
from oracle import numerics as on
from helpers import host, index_close

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _c4(tag, B, c):
    return {nm: synth.device_normal(f"{tag}.{nm}", (B, 4, c), BF) for nm in ("Ca", "Za", "Cb", "Zb", "pCb", "pZb")}


def _job(c4, bias, pos0, out, entry, out_scale=None, **kw):
    j = dict(ratio=4, Ca=c4["Ca"], Za=c4["Za"], bias=bias, Cb=c4["Cb"], Zb=c4["Zb"], prev_Cb=c4["pCb"],
             prev_Zb=c4["pZb"], pos0=pos0, out=out, cache_entry0=entry, **kw)
    if out_scale is not None:
        j["out_scale"] = out_scale
    return j


def _case(tag, B, N, e_new, q_pos0, keys="mxfp4", n_kv=16, kv_entry=5, rope=0, gamma=False, fp8_side=False,
          key_entry=None, key_only=False):
    """Inputs and two identical sets of caches (one per path)."""
    key_entry = e_new if key_entry is None else key_entry
    x = synth.device_normal(f"{tag}.keys", (B, N, 128))
    if keys == "mxfp4":
        k, ks = synth.device_quant_mxfp4(x)
        qx = synth.device_normal(f"{tag}.qi", (B, 1, 64, 128))
        q, qs = synth.device_quant_mxfp4(qx)
        qk = csa.MXFP4
    else:
        k, ks = x.to(BF), None
        q, qs = synth.device_normal(f"{tag}.qi", (B, 1, 64, 128), BF, var=1.0 / 128), None
        qk = csa.BF16
    w = synth.device_uniform(f"{tag}.w", (B, 1, 64))
    kv = synth.device_normal(f"{tag}.kv", (B, n_kv, 512), BF)
    c4, c4k = _c4(f"{tag}.c4", B, 512), _c4(f"{tag}.c4k", B, 128)
    b4 = synth.device_normal(f"{tag}.b4", (8, 512), var=0.1)
    b4k = synth.device_normal(f"{tag}.b4k", (8, 128), var=0.1)
    g512 = synth.device_uniform(f"{tag}.g", (512,)) + 0.5 if gamma else None
    g128 = synth.device_uniform(f"{tag}.gk", (128,)) + 0.5 if gamma else None
    f8 = torch.zeros(B, 8, 128, dtype=torch.uint8, device="cuda")
    f8s = torch.zeros(B, 8, dtype=torch.float32, device="cuda")
    pos4 = q_pos0 - 3

    def caches():
        return dict(kv=kv.clone(), k=k.clone(), ks=None if ks is None else ks.clone(), f8=f8.clone(),
                    f8s=f8s.clone())

    def jobs(cc):
        extra = dict(rope_dims=rope) if rope else {}
        j = [] if key_only else [_job(c4, b4, pos4, cc["kv"], kv_entry, gamma=g512, **extra)]
        if keys == "mxfp4":
            j.append(_job(c4k, b4k, pos4, cc["k"], key_entry, cc["ks"], gamma=g128, **extra))
        else:
            j.append(_job(c4k, b4k, pos4, cc["k"], key_entry, gamma=g128, **extra))
        if fp8_side:
            j.append(_job(c4k, b4k, pos4, cc["f8"], 3, cc["f8s"], gamma=g128, **extra))
        return j

    return dict(B=B, N=N, e_new=e_new, q_pos0=q_pos0, q=q, qs=qs, w=w, qk=qk, caches=caches, jobs=jobs)


def _separate(c, cc, score_dtype):
    csa.csa_compress_batch(c["jobs"](cc))
    return csa.lightning_index(c["q"], c["w"], cc["k"], q_pos0=c["q_pos0"], qk_dtype=c["qk"], q_scale=c["qs"],
                               k_scale=cc["ks"], score_dtype=score_dtype)


def _fused(c, cc, score_dtype):
    return csa.lightning_index_compressed(c["q"], c["w"], cc["k"], c["jobs"](cc), e_new=c["e_new"],
                                          q_pos0=c["q_pos0"], qk_dtype=c["qk"], q_scale=c["qs"], k_scale=cc["ks"],
                                          score_dtype=score_dtype)


def _kernels(fn):
    """Names of the kernels `fn` launches (None when the profiler records none)."""
    from torch.profiler import ProfilerActivity, profile
    try:
        with profile(activities=[ProfilerActivity.CUDA]) as prof:
            fn()
            torch.cuda.synchronize()
    except Exception:   # no device tracer: the launch count goes unchecked
        return None
    names = [e.name for e in prof.events() if e.device_type.name == "CUDA"]
    return names or None


def _same(a, b):
    if a is None:
        return b is None
    return torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                       b.view(torch.uint8) if b.dtype != torch.uint8 else b)


def _check(c, score_dtype=torch.bfloat16, fused_launch=True, kernel="index_mfma_jobs_kernel"):
    c1, c2 = c["caches"](), c["caches"]()
    s1 = _separate(c, c1, score_dtype)
    s2 = _fused(c, c2, score_dtype)
    torch.cuda.synchronize()
    for name in c1:
        assert _same(c1[name], c2[name]), f"{name} differs"
    assert torch.equal(s1.view(torch.int16 if s1.dtype == BF else torch.int32),
                       s2.view(torch.int16 if s2.dtype == BF else torch.int32))
    names = _kernels(lambda: _fused(c, c["caches"](), score_dtype))
    if names is not None:
        ours = [n for n in names if "compress" in n or "index" in n]
        fused = [n for n in ours if kernel in n]
        if fused_launch:
            assert len(fused) == 1 and not any("compress_batch_kernel" in n for n in ours), ours
        else:
            assert not fused and any("compress_batch_kernel" in n for n in ours), ours
    return c2, s2


def _bf16_close(got, ref64):
    """Within one bf16 ulp of the oracle's score rounded to bf16."""
    ref = on.store_bf16(ref64)
    a = np.maximum(np.abs(ref), 2.0 ** -126)
    assert np.all(np.abs(got - ref) <= np.exp2(np.floor(np.log2(a)) - 7) * 1.0001)


def _new_key_score(c, cc, s, b):
    """The new key's score (and its three neighbours') against the oracle on
    the decoded bytes: fp32 scores within 1e-3 relative, bf16 within one ulp."""
    e = c["e_new"]
    q = on.dequant_mxfp4(host(c["q"][b:b + 1]).astype(np.uint8), host(c["qs"][b:b + 1]).astype(np.uint8))
    lo = max(0, e - 3)
    kk = on.dequant_mxfp4(host(cc["k"][b:b + 1, lo:e + 1]).astype(np.uint8),
                          host(cc["ks"][b:b + 1, lo:e + 1]).astype(np.uint8))
    ref = oi.index_scores(q, host(c["w"][b:b + 1]), kk, 4 * (e + 1 - lo) - 1, 4)
    got = host(s[b:b + 1, :, lo:e + 1].float())
    if s.dtype == BF:
        _bf16_close(got, ref)
    else:
        index_close(got, ref)


def test_fused_pro_decode_1m():
    """The 1M-context Pro decode step: batch 8, 262,144 MXFP4 keys, the new
    entry last; bf16 latent and MXFP4 key written in the indexer's launch."""
    B, N = 8, 262144
    c = _case("fd.1m", B, N, N - 1, 4 * N - 1)
    cc, s = _check(c)
    for b in (0, B - 1):
        _new_key_score(c, cc, s, b)


def test_fused_entry_mid_run_rope_gamma_fp32_scores():
    """The written entry inside a middle key run (not the last), partial RoPE
    and RMSNorm gains on both jobs, fp32 scores, an fp8 job writing a third
    buffer in the same launch."""
    c = _case("fd.mid", 3, 5000, 1234, 4 * 5000 - 1, rope=64, gamma=True, fp8_side=True)
    cc, s = _check(c, torch.float32)
    _new_key_score(c, cc, s, 1)


def test_fused_single_key_run():
    """N small enough that one workgroup a sequence holds every key: every
    workgroup runs the jobs."""
    c = _case("fd.one", 4, 300, 299, 4 * 300 - 1)
    _check(c)


def test_fused_new_entry_partly_visible():
    """The query sees only part of the cache: entries past its visible range
    are -inf in both paths, the written entry the last visible one."""
    c = _case("fd.vis", 2, 4096, 2047, 4 * 2048 - 1)
    _check(c)


def test_fused_bf16_keys_ring():
    """bf16 keys: the jobs (latent and bf16 key) run by the ring indexer's
    workgroup of the new entry's key run, in one launch."""
    c = _case("fd.bf", 4, 3000, 2999, 4 * 3000 - 1, keys="bf16")
    _check(c, kernel="index_ring_kernel<1, 1, 32, 4, true, false, unsigned short, false, true>")


def test_fused_bf16_keys_ring_decode_size():
    """The CSA decode at 65,536 context: batch 32, 16,384 bf16 keys, the key
    job alone in the indexer's launch."""
    c = _case("fd.bf32", 32, 16384, 16383, 4 * 16384 - 1, keys="bf16", key_only=True)
    _check(c, kernel="index_ring_kernel<1, 1, 32, 4, true, false, unsigned short, false, true>")


def test_fallback_key_written_elsewhere():
    """A job writing the keys at another entry than e_new: two launches, the
    same results."""
    c = _case("fd.else", 2, 2048, 1000, 4 * 2048 - 1, key_entry=1500)
    _check(c, fused_launch=False)


def test_fused_in_graph_replays():
    """The fused call captured in a HIP graph (as the bench runs it): every
    replay, with eager work and synchronisations between replays, gives the
    eager call's bytes."""
    c = _case("fd.graph", 4, 4096, 4095, 4 * 4096 - 1)
    ref_c = c["caches"]()
    ref_s = _fused(c, ref_c, torch.bfloat16)
    torch.cuda.synchronize()
    cc = c["caches"]()
    st = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        s = _fused(c, cc, torch.bfloat16)        # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=st):
            s = _fused(c, cc, torch.bfloat16)
    torch.cuda.synchronize()
    e = c["e_new"]
    for rep in range(3):
        cc["k"][:, e].zero_()                     # the replay must rewrite the new entry
        cc["ks"][:, e].zero_()
        cc["kv"][:, 5].zero_()
        s.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(s.view(torch.int16), ref_s.view(torch.int16)), f"replay {rep}: scores"
        assert torch.equal(cc["k"][:, e], ref_c["k"][:, e]) and torch.equal(cc["ks"][:, e], ref_c["ks"][:, e])
        assert torch.equal(cc["kv"][:, 5], ref_c["kv"][:, 5])


def test_no_jobs_is_the_indexer():
    """n_jobs = 0: exactly lightning_index (e_new is not looked at)."""
    c = _case("fd.none", 2, 1000, 999, 4 * 1000 - 1)
    cc = c["caches"]()
    a = csa.lightning_index(c["q"], c["w"], cc["k"], q_pos0=c["q_pos0"], qk_dtype=c["qk"], q_scale=c["qs"],
                            k_scale=cc["ks"])
    b = csa.lightning_index_compressed(c["q"], c["w"], cc["k"], [], e_new=-1, q_pos0=c["q_pos0"],
                                       qk_dtype=c["qk"], q_scale=c["qs"], k_scale=cc["ks"])
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_fallback_two_queries_a_sequence():
    """T = 2 (two queries a sequence): two launches, the same results as the
    separate calls."""
    B, N, q0 = 3, 2000, 4 * 2000 - 2
    x = synth.device_normal("fd.t2.keys", (B, N, 128))
    k, ks = synth.device_quant_mxfp4(x)
    q, qs = synth.device_quant_mxfp4(synth.device_normal("fd.t2.qi", (B, 2, 64, 128)))
    w = synth.device_uniform("fd.t2.w", (B, 2, 64))
    c4k = _c4("fd.t2.c4k", B, 128)
    b4k = synth.device_normal("fd.t2.b4k", (8, 128), var=0.1)
    k1, ks1, k2, ks2 = k.clone(), ks.clone(), k.clone(), ks.clone()
    csa.csa_compress_batch([_job(c4k, b4k, q0 - 2, k1, N - 1, ks1)])
    s1 = csa.lightning_index(q, w, k1, q_pos0=q0, qk_dtype=csa.MXFP4, q_scale=qs, k_scale=ks1)
    s2 = csa.lightning_index_compressed(q, w, k2, [_job(c4k, b4k, q0 - 2, k2, N - 1, ks2)], e_new=N - 1, q_pos0=q0,
                                        qk_dtype=csa.MXFP4, q_scale=qs, k_scale=ks2)
    torch.cuda.synchronize()
    assert torch.equal(k1, k2) and torch.equal(ks1, ks2)
    assert torch.equal(s1.view(torch.int16), s2.view(torch.int16))


def test_fused_new_entry_in_a_ragged_last_tile():
    """N = 5,000 (the last key run and its last tile partial): the written
    entry is the very last key."""
    c = _case("fd.rag", 3, 5000, 4999, 4 * 5000 - 1)
    cc, s = _check(c)
    _new_key_score(c, cc, s, 2)



def _topk_case(tag, B, N, k, q_pos0):
    scores = synth.device_normal(f"{tag}.s", (B, 1, N), BF)
    kv = synth.device_normal(f"{tag}.kv", (B, 8, 512), BF)
    c4 = _c4(f"{tag}.c4", B, 512)
    b4 = synth.device_normal(f"{tag}.b4", (8, 512), var=0.1)
    g = synth.device_uniform(f"{tag}.g", (512,)) + 0.5
    return scores, kv, (lambda out: [_job(c4, b4, q_pos0 - 3, out, 6, gamma=g, rope_dims=64)])


@pytest.mark.parametrize("B,N,k,fused_launch", [
    (32, 16384, 512, True),      # the CSA decode at 65,536 context: the latent in spare workgroups
    (3, 2000, 512, True),        # rows shorter than one chunk a thread
    (2, 262144, 1024, False),    # long rows (the two-launch sliced path): the two calls
])
def test_topk_compressed(B, N, k, fused_launch):
    """topk_select_compressed = csa_compress_batch + topk_select: the same ids
    and the same written entry, bit for bit."""
    q0 = 4 * N - 1
    scores, kv, jobs = _topk_case(f"fd.tk{B}.{N}", B, N, k, q0)
    kv1, kv2 = kv.clone(), kv.clone()
    csa.csa_compress_batch(jobs(kv1))
    i1 = csa.topk_select(scores, k, q_pos0=q0)
    i2 = csa.topk_select_compressed(scores, k, jobs(kv2), q_pos0=q0)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(kv1, kv2)
    names = _kernels(lambda: csa.topk_select_compressed(scores, k, jobs(kv.clone()), q_pos0=q0))
    if names is not None:
        ours = [n for n in names if "topk" in n or "compress" in n]
        if fused_launch:
            assert any("topk_reg_jobs_kernel" in n for n in ours) and not any("compress_batch" in n for n in ours), ours
        else:
            assert any("compress_batch" in n for n in ours), ours
