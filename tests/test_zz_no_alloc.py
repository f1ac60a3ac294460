"""sparse_mqa_attn_noalloc (no allocation; split partials in the library's
static scratch) against sparse_mqa_attn with a caller workspace, through the
C ABI: two calls in a row, the second smaller, each equal bit for bit to the
workspace entry point on the same inputs (the same kernels and split plan),
and both within the attention tolerance of the oracle on sampled rows."""
import numpy as np
import pytest
import torch

import long_context_sparse_compress_amd as csa
import synth
from oracle import attention as oa
from helpers import ATTN_BF16_MAX_ABS, ATTN_NORMWISE, dev, host, max_abs, normwise_rel

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _case(name, B, T, N, k, q0):
    rp0 = max(0, q0 - 127)
    q = synth.device_normal(name + ".q", (B, T, 64, 512), BF)
    kv = synth.device_normal(name + ".kv", (B, N, 512), BF)
    raw = synth.device_normal(name + ".raw", (B, q0 + T - rp0, 512), BF)
    vis = [min((q0 + t + 1) // 4, N) for t in range(T)]
    idx = synth.random_topk_indices(name + ".idx", B, T, k, vis)
    return q, kv, raw, idx, rp0


def _oracle_row(q, kv, raw, idx, rp0, q0, b, t):
    sel = idx[b, t][idx[b, t] >= 0]
    rows = host(kv[b, torch.as_tensor(sel, device="cuda", dtype=torch.long)])
    pos = q0 + t
    w0 = max(0, pos - 127)
    rw = host(raw[b, w0 - rp0:pos - rp0 + 1])
    o, l = oa.sparse_mqa(host(q[b, t])[None, None], rows[None], np.arange(len(sel))[None, None], rw[None], w0, pos)
    return o[0, 0], l[0, 0]


@pytest.mark.parametrize("shapes", [[(32, 1, 16384, 512, 65535), (3, 1, 2000, 256, 7999)]])
def test_noalloc_matches_workspace_entry_point(shapes):
    for i, (B, T, N, k, q0) in enumerate(shapes):
        q, kv, raw, idx, rp0 = _case(f"na.{i}", B, T, N, k, q0)
        di = dev(idx, torch.int32)
        out_ws, lse_ws = csa.sparse_mqa_attn(q, kv, di, raw, q_pos0=q0, raw_pos0=rp0, return_lse=True)
        out = torch.full_like(q, float("nan"))
        lse = torch.full((B, T, 64), float("nan"), dtype=torch.float32, device="cuda")
        csa.sparse_mqa_attn_noalloc(q, kv, di, raw, q_pos0=q0, raw_pos0=rp0, out=out, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(out, out_ws), f"call {i}: output differs from the workspace entry point"
        assert torch.equal(lse, lse_ws), f"call {i}: lse differs from the workspace entry point"
        g, gl = host(out), host(lse)
        for b in sorted({0, B - 1}):
            ref, rl = _oracle_row(q, kv, raw, idx, rp0, q0, b, 0)
            assert max_abs(g[b, 0], ref) < ATTN_BF16_MAX_ABS and normwise_rel(g[b, 0], ref) < ATTN_NORMWISE
            assert max_abs(gl[b, 0], rl) < 1e-3


def test_noalloc_prefill_shape_needs_no_scratch():
    """B*T >= 256: no split, the scratch is not used; same bits as the workspace entry point."""
    B, T, N, k, q0 = 1, 300, 4096, 512, 16383 - 299
    q, kv, raw, idx, rp0 = _case("na.pf", B, T, N, k, q0)
    di = dev(idx, torch.int32)
    ref = csa.sparse_mqa_attn(q, kv, di, raw, q_pos0=q0, raw_pos0=rp0)
    out = torch.empty_like(q)
    csa.sparse_mqa_attn_noalloc(q, kv, di, raw, q_pos0=q0, raw_pos0=rp0, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
