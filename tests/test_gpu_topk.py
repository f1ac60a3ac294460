"""GPU parity of topk_select (stage 3) against the oracle, through the C ABI.

Pages: "DeepSeek Technical Reports" (DSA, the Top-k attention equation);
"DeepSeek V4 结构速览" (核心设计; Lightning Indexer: top-512, causal range).
Stage-isolated: both sides rank the same stored score tensor, so the selected
sets must be identical (ties go to the lower index).  The GPU writes the set in
ascending index order followed by -1 padding.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_compress_amd as csa
import synth
from oracle import topk as ot
from helpers import dev

pytestmark = pytest.mark.gpu


def _scores(prefix, B, T, N, dtype, ties=None):
    x = synth.normal(prefix, (B, T, N))
    if ties:
        x = np.round(x * ties) / ties          # few distinct values: heavy ties
    if dtype == "bf16":
        x = synth.round_bf16(x)
        return x, dev(x, torch.bfloat16)
    return x, dev(x)


def _check(got, ref):
    got = got.cpu().numpy()
    B, T, k = got.shape
    for b in range(B):
        for t in range(T):
            g, r = got[b, t], ref[b, t]
            nv = int((r >= 0).sum())
            assert np.all(g[nv:] == -1), (b, t)
            assert np.all(np.diff(g[:nv]) > 0), (b, t)          # ascending
            assert np.array_equal(g[:nv], np.sort(r[:nv])), (b, t)


def _run(x_dev, k, q_pos0, ratio=4):
    idx = csa.topk_select(x_dev, k, q_pos0=q_pos0, ratio=ratio)
    torch.cuda.synchronize()
    return idx


def test_tiny_fp32():
    """256 rows x 64 entries, k = 16 (rows t < 63 see fewer than 16 entries)."""
    x, d = _scores("tk.tiny", 1, 256, 64, "f32")
    _check(_run(d, 16, 0), ot.topk_select(x, 16, 0, 4))


def test_csa_decode_bf16():
    """Batch 32, 16,384 bf16 scores per row, k = 512."""
    x, d = _scores("tk.dec", 32, 1, 16384, "bf16")
    _check(_run(d, 512, 65535), ot.topk_select(x, 512, 65535, 4))


def test_chunked_prefill_bf16_sampled():
    """4,096 rows over 32,768..33,792 candidates, k = 512 (LDS path); sampled rows."""
    T, N, q0 = 4096, 33792, 131072
    x, d = _scores("tk.pf", 1, T, N, "bf16")
    got = _run(d, 512, q0)
    rows = [0, 1, 2, 3, 511, 2047, 2048, 4093, 4094, 4095]
    ref = ot.topk_select(x, 512, q0, 4, rows=rows)
    _check(got[:, rows], ref)


def test_1m_decode_bf16_global_path():
    """Batch 8, 262,144 candidates per row, k = 1024: the multi-workgroup path."""
    x, d = _scores("tk.1m", 8, 1, 262144, "bf16")
    _check(_run(d, 1024, 1048575), ot.topk_select(x, 1024, 1048575, 4))


def test_long_rows_partly_visible():
    """Long bf16 rows whose visible range ends inside the row (and mid-chunk:
    150,001 candidates), k = 1024."""
    x, d = _scores("tk.longvis", 1, 4, 200000, "bf16")
    _check(_run(d, 1024, 599999), ot.topk_select(x, 1024, 599999, 4))


def test_fp32_global_path():
    x, d = _scores("tk.f32g", 2, 3, 20000, "f32", ties=64)
    _check(_run(d, 700, 79997), ot.topk_select(x, 700, 79997, 4))


@pytest.mark.parametrize("dtype,ties,N,k", [
    ("bf16", 4, 5000, 300),        # heavy ties at the threshold
    ("f32", 2, 3000, 1000),
    ("bf16", 1, 300000, 2048),     # global path, max k, heavy ties
])
def test_ties_go_to_lower_index(dtype, ties, N, k):
    x, d = _scores(f"tk.ties{N}", 2, 1, N, dtype, ties=ties)
    _check(_run(d, k, 4 * N - 1), ot.topk_select(x, k, 4 * N - 1, 4))


def test_all_equal_and_signed_zero():
    x = np.zeros((1, 2, 4096), dtype=np.float32)
    x[0, 1, ::2] = -0.0
    d = dev(x, torch.bfloat16)
    got = _run(d, 100, 4 * 4096 - 2)
    assert np.array_equal(got[0, 0].cpu().numpy(), np.arange(100))
    assert np.array_equal(got[0, 1].cpu().numpy(), np.arange(100))


def test_infinite_scores_are_ranked():
    """-inf inside the visible range ranks last but can still be selected."""
    x = np.full((1, 1, 64), -np.inf, dtype=np.float32)
    x[0, 0, 10] = 1.0
    got = _run(dev(x), 3, 255)
    assert list(got[0, 0].cpu().numpy()) == [0, 1, 10]


@pytest.mark.parametrize("q_pos0,T,N,k", [(0, 40, 10, 4), (0, 4, 1, 1), (13, 6, 6, 5)])
def test_fewer_visible_than_k(q_pos0, T, N, k):
    x, d = _scores(f"tk.few{T}", 2, T, N, "f32")
    _check(_run(d, k, q_pos0), ot.topk_select(x, k, q_pos0, 4))


def test_deterministic():
    _, d = _scores("tk.det", 4, 1, 100000, "bf16", ties=8)
    a = _run(d, 1024, 399999)
    b = _run(d, 1024, 399999)
    assert torch.equal(a, b)


@pytest.mark.parametrize("e,ties", [(4, None), (20, None), (40, 64), (100, None), (100, 4)])
def test_key_range_spreads(e, ties):
    """Scores sign * 2^U(-e, e) (rounded to bf16) span about 2 * 2e * 128 distinct
    keys: the range histogram runs with no shift (e = 4) and with a shift of
    1, 2 and 3 bits plus the pass over the chosen bin's low bits; ties from
    coarse exponents where `ties` is set."""
    ex = synth.uniform(f"tk.spread{e}", (8, 1, 16384), lo=-e, hi=e)
    if ties:
        ex = np.round(ex * ties / e) * e / ties
    x = synth.round_bf16(np.sign(synth.normal(f"tk.sign{e}", ex.shape)) * np.exp2(ex))
    got = _run(dev(x, torch.bfloat16), 512, 65535)
    _check(got, ot.topk_select(x, 512, 65535, 4))


@pytest.mark.parametrize("dtype,N,k,ties", [
    ("f32", 16384, 512, None),    # fp32 row in LDS: 64 KiB of keys + the histogram
    ("f32", 18432, 2048, 16),     # the longest fp32 row the LDS path takes, max k, ties
    ("bf16", 30001, 512, None),   # bf16 row with N % 8 != 0: the LDS path, not the register one
])
def test_lds_path_large_rows(dtype, N, k, ties):
    """Rows whose LDS copy needs more than 64 KiB of dynamic LDS."""
    x, d = _scores(f"tk.lds{N}", 3, 1, N, dtype, ties=ties)
    _check(_run(d, k, 4 * N - 1), ot.topk_select(x, k, 4 * N - 1, 4))


def test_long_rows_ragged_batch_slice_edges():
    """The long-row (sliced) path with each sequence at its own position: visible
    lengths 0, k - 1, k, k + 1, one and just past one 16,384-key slice, a ragged
    mid-row end and the whole row, with heavy ties; k = 1024."""
    N, k = 262144, 1024
    V = [0, k - 1, k, k + 1, 16384, 16385, 100003, N]
    x, d = _scores("tk.ragged", len(V), 1, N, "bf16", ties=8)
    x, d = x[:, 0], d[:, 0].contiguous()
    sp = torch.as_tensor([4 * v + 2 for v in V], dtype=torch.int64, device="cuda")   # (pos + 1) // 4 = v
    got = csa.topk_select_paged(d, k, sp)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    for b, v in enumerate(V):
        r = ot.select_row(x[b], v, k)
        nv = int((r >= 0).sum())
        assert np.all(got[b, nv:] == -1), b
        assert np.array_equal(got[b, :nv], np.sort(r[:nv])), b
