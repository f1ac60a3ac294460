"""GPU parity of decode attention over the heterogeneous KV cache
(sparse_mqa_attn_paged, hca_attn_paged) against the oracle, through the C ABI.

Page: "DeepSeek-V4技术报告解读，全适配国产算力" (3.2: the classical paged cache
in blocks of 128 raw tokens, the per-request state cache holding the sliding
window).  Every sequence sits at its own position; the physical blocks are
shuffled; the window ring wraps.  The oracle gathers each sequence's entries
and window rows back into contiguous arrays (oracle.cache) and runs the
attention oracles.  Tolerances as for the contiguous attention (bf16 2e-2
max-abs plus the normwise guard, lse 1e-3); paged and contiguous layouts of
the same data give identical bits.
"""
import zlib

import numpy as np
import pytest
import torch

import long_context_sparse_compress_amd as csa
import synth
from oracle import attention as oa
from oracle import cache as occ
from helpers import ATTN_BF16_MAX_ABS, ATTN_NORMWISE, dev, host, max_abs, normwise_rel

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _assert_bf16(got, ref):
    assert max_abs(got, ref) < ATTN_BF16_MAX_ABS
    assert normwise_rel(got, ref) < ATTN_NORMWISE


def _paged_cache(name, seq_pos, per_block, ring, spare=5):
    """Blocks for every sequence's visible entries, shuffled in one pool;
    unused table slots hold -1.  Returns (pool, table, ring_win, n_blocks)."""
    B = len(seq_pos)
    ratio = 128 // per_block
    nblk = [(p + 1) // 128 + 1 for p in seq_pos]          # blocks covering positions 0..p
    max_blocks = max(nblk) + 2
    n_pool = sum(nblk) + spare
    g = np.random.default_rng(zlib.crc32(name.encode()))
    perm = g.permutation(n_pool)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    o = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[o:o + nblk[b]]
        o += nblk[b]
    shape = (n_pool, per_block, 512) if per_block > 1 else (n_pool, 512)
    pool = synth.device_normal(name + ".pool", shape, BF)
    win = synth.device_normal(name + ".win", (B, ring, 512), BF)
    return pool, table, win, ratio


def _entries(pool, table_row, n, per_block):
    return occ.paged_entries(host(pool), table_row, n, per_block)


def _window(win_b, pos, window=128):
    w0 = max(0, pos - window + 1)
    return occ.ring_rows(host(win_b), range(w0, pos + 1)), w0


SEQ_POS = [4095, 9000, 65535, 70001, 131071, 333, 12345, 65536]


@pytest.mark.parametrize("bi", [False, True])
def test_paged_sparse_decode(bi):
    """8 sequences at different positions, top-512 lists, shuffled blocks, a
    256-row window ring; the split decode and the batch-invariant kernel."""
    B, k, ring = len(SEQ_POS), 512, 256
    pool, table, win, _ = _paged_cache("pg.sp", SEQ_POS, 32, ring)
    q = synth.device_normal("pg.sp.q", (B, 64, 512), BF)
    idx = np.concatenate([synth.random_topk_indices(f"pg.sp.idx{b}", 1, 1, k, [(p + 1) // 4])[0]
                          for b, p in enumerate(SEQ_POS)])
    sp = torch.tensor(SEQ_POS, dtype=torch.int64, device="cuda")
    out, lse = csa.sparse_mqa_attn_paged(q, pool, dev(table, torch.int32), dev(idx, torch.int32), win, sp,
                                         return_lse=True, batch_invariant=bi)
    torch.cuda.synchronize()
    got, gl = host(out), host(lse)
    for b, pos in enumerate(SEQ_POS):
        sel = idx[b][idx[b] >= 0]
        rows = _entries(pool, table[b], int(sel.max()) + 1, 32)[sel]
        rw, w0 = _window(win[b], pos)
        o, l = oa.sparse_mqa(host(q[b])[None, None], rows[None], np.arange(len(sel))[None, None], rw[None],
                             w0, pos, 128)
        _assert_bf16(got[b], o[0, 0])
        assert max_abs(gl[b], l[0, 0]) < 1e-3


def test_paged_hca_decode_with_sink():
    """6 sequences up to 1M context (up to 8,192 C128A entries each), one entry
    per block, shuffled blocks, a 128-row ring, sink."""
    seq = [1048575, 300000, 128, 127, 65535, 777777]
    B, ring = len(seq), 128
    pool, table, win, _ = _paged_cache("pg.h", seq, 1, ring)
    q = synth.device_normal("pg.h.q", (B, 64, 512), BF)
    sink = synth.device_normal("pg.h.sink", (64,))
    sp = torch.tensor(seq, dtype=torch.int64, device="cuda")
    out, lse = csa.hca_attn_paged(q, pool, dev(table, torch.int32), win, sp, sink=sink, return_lse=True)
    torch.cuda.synchronize()
    got, gl = host(out), host(lse)
    for b, pos in enumerate(seq):
        V = (pos + 1) // 128
        kv = _entries(pool, table[b], V, 1) if V else np.zeros((0, 512))
        rw, w0 = _window(win[b], pos)
        o, l = oa.dense_attention(host(q[b])[None, None], kv[None], rw[None], w0, pos, 128, 128,
                                  sink=host(sink))
        _assert_bf16(got[b], o[0, 0])
        assert max_abs(gl[b], l[0, 0]) < 1e-3


def test_absent_blocks_are_padding():
    """Top-k slots that point into a block the table marks absent contribute
    nothing (and are not read)."""
    seq = [9000, 9000]
    B, k, ring = 2, 64, 128
    pool, table, win, _ = _paged_cache("pg.abs", seq, 32, ring)
    table = table.copy()
    table[0, 3] = -1                 # entries 96..127 of sequence 0: absent
    table[1, 5] = 10 ** 6            # past the pool: absent
    q = synth.device_normal("pg.abs.q", (B, 64, 512), BF)
    idx = np.tile(np.arange(80, 80 + 2 * k, 2, dtype=np.int32), (B, 1))   # entries 80..206
    sp = torch.tensor(seq, dtype=torch.int64, device="cuda")
    out = csa.sparse_mqa_attn_paged(q, pool, dev(table, torch.int32), dev(idx, torch.int32), win, sp)
    torch.cuda.synchronize()
    got = host(out)
    for b, pos in enumerate(seq):
        blk = table[b][idx[b] // 32]
        keep = idx[b][(blk >= 0) & (blk < pool.shape[0])]
        t = table[b].copy()
        t[(t < 0) | (t >= pool.shape[0])] = 0
        rows = _entries(pool, t, int(idx[b].max()) + 1, 32)[keep]
        rw, w0 = _window(win[b], pos)
        o, _ = oa.sparse_mqa(host(q[b])[None, None], rows[None], np.arange(len(keep))[None, None], rw[None], w0,
                             pos, 128)
        _assert_bf16(got[b], o[0, 0])


def test_paged_equals_contiguous_bits():
    """The same entries and window laid out contiguously (sparse_mqa_attn_ex,
    hca_attn_ex) and paged, all sequences at one position: identical bits."""
    B, N, k, pos = 16, 4096, 512, 16383
    kv = synth.device_normal("pg.eq.kv", (B, N, 512), BF)
    raw = synth.device_normal("pg.eq.raw", (B, 128, 512), BF)
    q = synth.device_normal("pg.eq.q", (B, 1, 64, 512), BF)
    idx = dev(synth.random_topk_indices("pg.eq.idx", B, 1, k, [N]), torch.int32)
    # pages: blocks of sequence b are b*128 + j, the pool shuffled under a table
    nb = N // 32
    g = np.random.default_rng(5)
    perm = g.permutation(B * nb).astype(np.int32)
    table = perm.reshape(B, nb)
    pool = torch.empty(B * nb, 32, 512, dtype=BF, device="cuda")
    pool[torch.as_tensor(table.reshape(-1), device="cuda").long()] = kv.reshape(B * nb, 32, 512)
    ring = torch.empty(B, 128, 512, dtype=BF, device="cuda")
    r0 = pos - 127
    ring[:, torch.arange(r0, pos + 1, device="cuda") % 128] = raw
    sp = torch.full((B,), pos, dtype=torch.int64, device="cuda")
    for bi in (False, True):
        a = csa.sparse_mqa_attn(q, kv, idx, raw, q_pos0=pos, raw_pos0=r0, batch_invariant=bi)
        p = csa.sparse_mqa_attn_paged(q[:, 0], pool, dev(table, torch.int32), idx[:, 0], ring, sp,
                                      batch_invariant=bi)
        torch.cuda.synchronize()
        assert torch.equal(a[:, 0], p), bi
    # HCA: one entry per block
    Nh = (pos + 1) // 128
    kvh = synth.device_normal("pg.eq.kvh", (B, Nh, 512), BF)
    sink = synth.device_normal("pg.eq.sink", (64,))
    permh = g.permutation(B * Nh).astype(np.int32).reshape(B, Nh)
    poolh = torch.empty(B * Nh, 512, dtype=BF, device="cuda")
    poolh[torch.as_tensor(permh.reshape(-1), device="cuda").long()] = kvh.reshape(B * Nh, 512)
    a = csa.hca_attn(q, kvh, raw, q_pos0=pos, raw_pos0=r0, sink=sink)
    p = csa.hca_attn_paged(q[:, 0], poolh, dev(permh, torch.int32), ring, sp, sink=sink)
    torch.cuda.synchronize()
    assert torch.equal(a[:, 0], p)


# ---------------------------------------------------------------- indexer / Top-k over paged keys

from oracle import indexer as oi  # noqa: E402
from oracle import numerics as on  # noqa: E402
from oracle import topk as ot  # noqa: E402
from helpers import index_close  # noqa: E402

IDX_POS = [4095, 9000, 65535, 70001, 131071, 333, 12345, 2]


def _key_pool(name, seq_pos, fmt):
    """bf16 keys (or their E4M3 codes + row scales, or MXFP4 codes + E8M0
    scales) for every sequence's visible entries, shuffled 32-entry blocks, -1
    past each sequence."""
    B = len(seq_pos)
    nblk = [(p + 1) // 128 + 1 for p in seq_pos]
    max_blocks = max(nblk) + 1
    n_pool = sum(nblk) + 3
    g = np.random.default_rng(zlib.crc32(name.encode()))
    perm = g.permutation(n_pool)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    o = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[o:o + nblk[b]]
        o += nblk[b]
    keys = synth.round_bf16(synth.normal(name + ".k", (n_pool, 32, 128)))
    if fmt == "fp8":
        codes, scale = synth.quant_fp8_rows(keys)
        return dev(codes, torch.uint8), dev(scale), on.dequant_fp8_rows(codes, scale), table
    if fmt == "mxfp4":
        packed, sc = synth.quant_mxfp4(keys)
        return dev(packed, torch.uint8), dev(sc, torch.uint8), on.dequant_mxfp4(packed, sc), table
    return dev(keys, BF), None, keys, table


def _queries(name, B, fmt):
    q = synth.normal(name + ".q", (B, 64, 128), var=1.0 if fmt != "bf16" else 1.0 / 128)
    w = synth.uniform(name + ".w", (B, 64))
    if fmt == "fp8":
        qc, qs = synth.quant_fp8_rows(q)
        return dev(qc, torch.uint8), dev(qs), on.dequant_fp8_rows(qc, qs), w
    if fmt == "mxfp4":
        qp, qs = synth.quant_mxfp4(q)
        return dev(qp, torch.uint8), dev(qs, torch.uint8), on.dequant_mxfp4(qp, qs), w
    qb = synth.round_bf16(q)
    return dev(qb, BF), None, qb, w


def _oracle_scores(qv, w, keys_host, table, seq_pos):
    """Per sequence: the indexer oracle over the entries gathered from the pool."""
    out = []
    for b, pos in enumerate(seq_pos):
        vis = (pos + 1) // 4
        kb = occ.paged_entries(keys_host, table[b], vis, 32) if vis else np.zeros((0, 128))
        out.append(oi.index_scores(qv[b][None, None], w[b][None, None], kb[None], pos, 4)[0, 0])
    return out


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
def test_paged_indexer_and_topk(fmt):
    """Ragged positions (2 .. 131,071, one with no visible entry), shuffled
    blocks, bf16, fp8 and MXFP4 keys: scores against the oracle, -inf past each
    sequence.  Per-sequence Top-k, stage-isolated: the GPU selects over the
    oracle's scores (stored in fp32) and must return the oracle's selection."""
    B, K = len(IDX_POS), 512
    kp, ks, keys_host, table = _key_pool(f"pg.ix.{fmt}", IDX_POS, fmt)
    q, qs, qv, w = _queries(f"pg.ix.{fmt}", B, fmt)
    sp = torch.tensor(IDX_POS, dtype=torch.int64, device="cuda")
    s = csa.lightning_index_paged(q, dev(w), kp, dev(table, torch.int32), sp, q_scale=qs, k_scale=ks,
                                  score_dtype=torch.float32)
    torch.cuda.synchronize()
    hs = host(s)
    ref = _oracle_scores(qv, w, keys_host, table, IDX_POS)
    Nmax = hs.shape[1]
    ref_rows = np.full((B, Nmax), -np.inf, dtype=np.float32)
    for b, pos in enumerate(IDX_POS):
        vis = (pos + 1) // 4
        if vis:
            index_close(hs[b, :vis][None], ref[b][None])
            ref_rows[b, :vis] = ref[b].astype(np.float32)
        assert np.all(np.isneginf(hs[b, vis:]))
    idx = csa.topk_select_paged(dev(ref_rows), K, sp)
    torch.cuda.synchronize()
    hi = host(idx)
    for b, pos in enumerate(IDX_POS):
        vis = (pos + 1) // 4
        want = np.sort(ot.select_row(ref_rows[b].astype(np.float64), vis, K))
        want = np.concatenate([want[want >= 0], want[want < 0]])
        assert np.array_equal(hi[b], want), b


def test_paged_decode_chain_against_the_oracle_chain():
    """The whole CSA decode step on the paged cache -- indexer over paged bf16
    keys, Top-k per sequence, sparse MQA over paged latents and the window
    ring -- against the oracle's own chain on the gathered data.  Selections
    may differ only between entries whose oracle scores tie within 1e-3; the
    attention is compared where the selections agree."""
    B, K, ring = len(IDX_POS), 512, 256
    kp, _, keys_host, table = _key_pool("pg.chain", IDX_POS, "bf16")
    q_i, _, qv, w = _queries("pg.chain", B, "bf16")
    pool = synth.device_normal("pg.chain.kv", (kp.shape[0], 32, 512), BF)
    win = synth.device_normal("pg.chain.win", (B, ring, 512), BF)
    q = synth.device_normal("pg.chain.q", (B, 64, 512), BF)
    dt = dev(table, torch.int32)
    sp = torch.tensor(IDX_POS, dtype=torch.int64, device="cuda")
    s = csa.lightning_index_paged(q_i, dev(w), kp, dt, sp, score_dtype=torch.float32)
    idx = csa.topk_select_paged(s, K, sp)
    out = csa.sparse_mqa_attn_paged(q, pool, dt, idx, win, sp)
    torch.cuda.synchronize()
    hi, got = host(idx), host(out)
    ref_scores = _oracle_scores(qv, w, keys_host, table, IDX_POS)
    agree = 0
    for b, pos in enumerate(IDX_POS):
        vis = (pos + 1) // 4
        so = ref_scores[b]
        osel = ot.select_row(so, vis, K)
        oset, gset = set(int(e) for e in osel if e >= 0), set(int(e) for e in hi[b] if e >= 0)
        if oset != gset:
            kth = np.sort(so[:vis])[::-1][min(K, vis) - 1]
            for e in oset ^ gset:
                assert abs(so[e] - kth) <= 1e-3 * abs(kth), (b, e)
            continue
        agree += 1
        sel = np.array(sorted(oset), dtype=np.int64)
        rows = occ.paged_entries(host(pool), table[b], int(sel.max()) + 1, 32)[sel] if len(sel) else \
            np.zeros((0, 512))
        rw, w0 = _window(win[b], pos)
        o, _ = oa.sparse_mqa(host(q[b])[None, None], rows[None], np.arange(len(sel))[None, None], rw[None], w0,
                             pos, 128)
        _assert_bf16(got[b], o[0, 0])
    assert agree >= B - 1


# ---------------------------------------------------------------- the rolling-buffer write into pages

from oracle import compressor as oc  # noqa: E402


@pytest.mark.parametrize("ratio,c,out", [(4, 512, "bf16"), (4, 128, "fp8"), (4, 128, "fp4"), (128, 512, "bf16"),
                                         (4, 192, "f32")])
def test_compress_paged_decode_write(ratio, c, out):
    """Sequences at different positions pool their current block into their
    own page slot; sequences not at a block start (and one whose block is
    absent) write nothing; every other slot of the pool is left alone."""
    per = 32 if ratio == 4 else 1
    pos = [4 * 1000, 128 * 7, 0, 65532, 77, 4 * 4095] if ratio == 4 else [128 * 7, 0, 128 * 8191, 130, 128 * 300]
    B = len(pos)
    nblk = [p // 128 + 1 for p in pos]
    max_blocks = max(nblk) + 1
    n_pool = sum(nblk) + 2
    g = np.random.default_rng(zlib.crc32(f"cp{ratio}{c}{out}".encode()))
    perm = g.permutation(n_pool)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    o = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[o:o + nblk[b]]
        o += nblk[b]
    absent = 1
    e_abs = pos[absent] // ratio
    table[absent, e_abs // per] = -1             # this sequence's block is not mapped
    dtype = "f32" if out == "f32" else "bf16"
    tdt = torch.float32 if dtype == "f32" else BF
    inp = {}
    for b, p in enumerate(pos):
        p0 = p - p % ratio
        inp[b] = synth.compressor_inputs(f"cp.{ratio}.{c}.{b}", 1, ratio, c, ratio, p0 if p0 else 0, dtype=dtype)
    Ca = np.concatenate([inp[b]["Ca"] for b in range(B)])
    Za = np.concatenate([inp[b]["Za"] for b in range(B)])
    bias = inp[0]["bias"]
    if ratio == 4:
        pC = np.concatenate([inp[b].get("prev_Cb", np.zeros((1, 4, c), np.float32)) for b in range(B)])
        pZ = np.concatenate([inp[b].get("prev_Zb", np.zeros((1, 4, c), np.float32)) for b in range(B)])
    shape = (n_pool, per, c) if per > 1 else (n_pool, c)
    if out == "fp8":
        pool = torch.full(shape, 0x33, dtype=torch.uint8, device="cuda")
        spool = torch.full((n_pool, per), 5.0, dtype=torch.float32, device="cuda")
    elif out == "fp4":
        pool = torch.full((n_pool, per, c // 2), 0x33, dtype=torch.uint8, device="cuda")
        spool = torch.full((n_pool, per, c // 32), 9, dtype=torch.uint8, device="cuda")
    else:
        pool = torch.full(shape, 3.0, dtype=torch.float32 if out == "f32" else BF, device="cuda")
        spool = None
    before = pool.clone()
    csa.csa_compress_paged(ratio, dev(Ca, tdt), dev(Za, tdt), dev(bias), pool, dev(table, torch.int32),
                           torch.tensor(pos, dtype=torch.int64, device="cuda"),
                           prev_Cb=dev(pC, tdt) if ratio == 4 else None, prev_Zb=dev(pZ, tdt) if ratio == 4 else None,
                           scale_pool=spool, rope_dims=64, rope_anchor=ratio - 1)
    torch.cuda.synchronize()
    hp, hb = host(pool), host(before)
    written = np.zeros(hp.shape[:2] if per > 1 else hp.shape[:1], dtype=bool)
    for b, p in enumerate(pos):
        if p % ratio or b == absent:
            continue
        e = p // ratio
        blk = table[b, e // per]
        slot = (blk, e % per) if per > 1 else (blk,)
        written[slot] = True
        ib = inp[b]
        # one bias for the call (sequence 0's), as the kernel got it
        ref = oc.compress(ib["Ca"], ib["Za"], bias, ratio, ib["Cb"], ib["Zb"],
                          ib.get("prev_Cb") if p else None, ib.get("prev_Zb") if p else None, pos0=p,
                          rope_dims=64, rope_anchor=ratio - 1)[0, 0] if ratio == 4 else \
            oc.compress(ib["Ca"], ib["Za"], bias, 128, pos0=p, rope_dims=64, rope_anchor=127)[0, 0]
        got = hp[slot]
        if out == "fp8":
            dec = on.decode_e4m3(got) * host(spool)[slot]
            assert np.max(np.abs(dec - ref)) <= np.abs(ref).max() / 448 * 16 + 1e-4
        elif out == "fp4":
            dec = on.dequant_mxfp4(got[None], host(spool)[slot][None])[0]
            # within half the largest E2M1 step (2 at scale 2^E, E = floor(log2 amax) - 2) of each value
            assert np.max(np.abs(dec - ref)) <= np.abs(ref).max() / 4 + 1e-4
        elif out == "f32":
            assert np.max(np.abs(got - ref)) < 1e-4
        else:
            assert np.max(np.abs(got - ref)) < 2e-2
    assert written.sum() == sum(1 for b, p in enumerate(pos) if p % ratio == 0 and b != absent)
    assert np.array_equal(hp[~written], hb[~written])


@pytest.mark.parametrize("ratio,c,out,n_tok,rope", [(4, 512, "bf16", 256, 64), (4, 128, "fp8", 130, 64),
                                                    (4, 128, "fp4", 64, 64), (128, 512, "bf16", 300, 64),
                                                    (4, 192, "f32", 36, 64), (128, 256, "f32", 384, 64),
                                                    (4, 512, "bf16", 40, 0), (128, 512, "f32", 256, 0)])
def test_compress_paged_chunk_write(ratio, c, out, n_tok, rope):
    """Chunked prefill into pages: each sequence compresses its own chunk,
    starting at its own block start, entry by entry into its page slots.
    The chunks cross page boundaries; one sequence has an absent page in the
    middle of its chunk (those entries are skipped), one is not at a block
    start (writes nothing); every other slot is left alone.  Each entry is
    compared with the oracle's compression of that sequence's chunk."""
    per = 32 if ratio == 4 else 1
    n_ent = n_tok // ratio
    pos = [0, 4 * 1000, 128 * 37, 6] if ratio == 4 else [0, 128 * 7, 128 * 8000, 130]
    B = len(pos)
    last = [(p // ratio + max(n_ent, 1) - 1) // per for p in pos]
    max_blocks = max(last) + 2
    nblk = [lb + 1 for lb in last]
    n_pool = sum(nblk) + 3
    g = np.random.default_rng(zlib.crc32(f"cpc{ratio}{c}{out}{n_tok}".encode()))
    perm = g.permutation(n_pool)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    o = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[o:o + nblk[b]]
        o += nblk[b]
    absent = 1                                    # the page of this sequence's chunk-middle entry is not mapped
    e_mid = pos[absent] // ratio + n_ent // 2
    table[absent, e_mid // per] = -1
    dtype = "f32" if out == "f32" else "bf16"
    tdt = torch.float32 if dtype == "f32" else BF
    inp = [synth.compressor_inputs(f"cpc.{ratio}.{c}.{n_tok}.{b}", 1, n_tok, c, ratio, p - p % ratio, dtype=dtype)
           for b, p in enumerate(pos)]
    cat = {nm: np.concatenate([x[nm] for x in inp]) for nm in (["Ca", "Za", "Cb", "Zb"] if ratio == 4 else
                                                               ["Ca", "Za"])}
    bias = inp[0]["bias"]
    if ratio == 4:
        for nm in ("prev_Cb", "prev_Zb"):
            cat[nm] = np.concatenate([x.get(nm, np.zeros((1, 4, c), np.float32)) for x in inp])
    shape = (n_pool, per, c) if per > 1 else (n_pool, c)
    if out == "fp8":
        pool = torch.full(shape, 0x33, dtype=torch.uint8, device="cuda")
        spool = torch.full((n_pool, per), 5.0, dtype=torch.float32, device="cuda")
    elif out == "fp4":
        pool = torch.full((n_pool, per, c // 2), 0x33, dtype=torch.uint8, device="cuda")
        spool = torch.full((n_pool, per, c // 32), 9, dtype=torch.uint8, device="cuda")
    else:
        pool = torch.full(shape, 3.0, dtype=torch.float32 if out == "f32" else BF, device="cuda")
        spool = None
    before = pool.clone()
    d = {nm: dev(v, tdt) for nm, v in cat.items()}
    csa.csa_compress_paged_chunk(ratio, d["Ca"], d["Za"], dev(bias), pool, dev(table, torch.int32),
                                 torch.tensor(pos, dtype=torch.int64, device="cuda"), Cb=d.get("Cb"),
                                 Zb=d.get("Zb"), prev_Cb=d.get("prev_Cb"), prev_Zb=d.get("prev_Zb"),
                                 scale_pool=spool, rope_dims=rope, rope_anchor=ratio - 1 if rope else 0)
    torch.cuda.synchronize()
    hp, hb = host(pool), host(before)
    written = np.zeros(hp.shape[:2] if per > 1 else hp.shape[:1], dtype=bool)
    for b, p in enumerate(pos):
        if p % ratio:
            continue
        x = inp[b]
        ref = oc.compress(x["Ca"], x["Za"], bias, ratio, x.get("Cb"), x.get("Zb"), x.get("prev_Cb"),
                          x.get("prev_Zb"), pos0=p, rope_dims=rope, rope_anchor=ratio - 1 if rope else 0)[0]
        for i in range(n_ent):
            e = p // ratio + i
            blk = table[b, e // per]
            if blk < 0:
                continue
            slot = (blk, e % per) if per > 1 else (blk,)
            written[slot] = True
            got = hp[slot]
            if out == "fp8":
                dec = on.decode_e4m3(got) * host(spool)[slot]
                assert np.max(np.abs(dec - ref[i])) <= np.abs(ref[i]).max() / 448 * 16 + 1e-4, (b, i)
            elif out == "fp4":
                dec = on.dequant_mxfp4(got[None], host(spool)[slot][None])[0]
                assert np.max(np.abs(dec - ref[i])) <= np.abs(ref[i]).max() / 4 + 1e-4, (b, i)
            elif out == "f32":
                assert np.max(np.abs(got - ref[i])) < 1e-4, (b, i)
            else:
                assert np.max(np.abs(got - ref[i])) < 2e-2, (b, i)
    skipped = sum(1 for i in range(n_ent) if table[absent, (pos[absent] // ratio + i) // per] < 0)
    assert skipped >= 1
    assert written.sum() == 3 * n_ent - skipped
    assert np.array_equal(hp[~written], hb[~written])


@pytest.mark.parametrize("kind", ["latent_fp4_key", "latent_fp8_key", "c128a_pair"])
def test_compress_paged_batch_equals_separate_calls(kind):
    """csa_compress_paged_batch writes exactly what the separate calls write:
    the paged decode step's bf16 latent with its MXFP4 (or fp8) indexer key in
    one launch, each with RoPE, and two C128A streams; sequences at ragged
    positions, one not at a block start and one with an absent block."""
    ratio = 128 if kind == "c128a_pair" else 4
    per = 32 if ratio == 4 else 1
    pos = [4 * 1000, 128 * 7, 0, 65532, 77, 4 * 4095] if ratio == 4 else [128 * 7, 0, 128 * 8191, 130, 128 * 300]
    B = len(pos)
    nblk = [p // 128 + 1 for p in pos]
    max_blocks = max(nblk) + 1
    n_pool = sum(nblk) + 2
    g = np.random.default_rng(zlib.crc32(f"cpb{kind}".encode()))
    perm = g.permutation(n_pool)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    o = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[o:o + nblk[b]]
        o += nblk[b]
    table[1, (pos[1] // ratio) // per] = -1
    streams = ([(512, "bf16", 64), (128, "fp4" if kind == "latent_fp4_key" else "fp8", 64)] if ratio == 4
               else [(512, "bf16", 64), (256, "bf16", 0)])
    tbl = dev(table, torch.int32)
    sp = torch.tensor(pos, dtype=torch.int64, device="cuda")
    jobs, sep = [], []
    for si, (c, out, R) in enumerate(streams):
        inp = synth.compressor_inputs(f"cpb.{kind}.{si}", B, ratio, c, ratio, ratio)   # pos0 > 0: with halo
        args = dict(Ca=dev(inp["Ca"], BF), Za=dev(inp["Za"], BF), bias=dev(inp["bias"]))
        if ratio == 4:
            args.update(prev_Cb=dev(inp["prev_Cb"], BF), prev_Zb=dev(inp["prev_Zb"], BF))
        if out == "fp8":
            mk = lambda: (torch.full((n_pool, per, c), 0x33, dtype=torch.uint8, device="cuda"),
                          torch.full((n_pool, per), 5.0, dtype=torch.float32, device="cuda"))
        elif out == "fp4":
            mk = lambda: (torch.full((n_pool, per, c // 2), 0x33, dtype=torch.uint8, device="cuda"),
                          torch.full((n_pool, per, c // 32), 9, dtype=torch.uint8, device="cuda"))
        else:
            shape = (n_pool, per, c) if per > 1 else (n_pool, c)
            mk = lambda: (torch.full(shape, 3.0, dtype=BF, device="cuda"), None)
        pa, sa = mk()
        pb, sb = mk()
        csa.csa_compress_paged(ratio, args["Ca"], args["Za"], args["bias"], pa, tbl, sp, prev_Cb=args.get("prev_Cb"),
                               prev_Zb=args.get("prev_Zb"), scale_pool=sa, rope_dims=R, rope_anchor=ratio - 1)
        sep.append((pa, sa))
        jobs.append(dict(ratio=ratio, pool=pb, scale_pool=sb, block_table=tbl, pos0=sp, rope_dims=R,
                         rope_anchor=ratio - 1, **args))
    csa.csa_compress_paged_batch(jobs)
    torch.cuda.synchronize()
    for (pa, sa), j in zip(sep, jobs):
        assert torch.equal(pa, j["pool"])
        if sa is not None:
            assert torch.equal(sa, j["scale_pool"])
