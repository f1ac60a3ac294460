"""Python binding of libcsa.so, the gfx950 compressed sparse attention library.

Argument marshalling only: every function checks that its tensors are
contiguous device tensors, passes their pointers and torch's current HIP
stream to the C ABI (include/csa.h), and raises on a non-zero status.  All of
the computation runs in the library's HIP kernels.  PyTorch provides device
memory and streams, nothing else.

The library is loaded from this package's directory; if it is missing the
import of any entry point raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["csa_compress", "csa_compress_batch", "lightning_index", "lightning_index_compressed", "hca_attn_compressed", "topk_select_compressed", "topk_select", "sparse_mqa_attn", "hca_attn",
           "sparse_mqa_attn_noalloc",
           "rope", "lightning_index_pool", "topk_select_pool", "csa_compress_paged", "csa_compress_paged_chunk",
           "csa_compress_paged_batch",
           "lightning_index_paged",
           "topk_select_paged",
           "sparse_mqa_attn_paged", "hca_attn_paged",
           "workspace_bytes", "library", "F32", "BF16",
           "FP8_E4M3", "MXFP4", "CsaError"]

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcsa.so")

F32, BF16, FP8_E4M3, MXFP4 = 0, 1, 2, 3
OP_COMPRESS, OP_INDEX, OP_TOPK, OP_SPARSE_ATTN, OP_HCA_ATTN = 0, 1, 2, 3, 4
ATTN_BATCH_INVARIANT = 1   # CSA_ATTN_BATCH_INVARIANT
ROPE_BASE = 10000.0        # the rotary base used when none is given

_i64, _int, _f32, _vp, _sz = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

_SIGS = {
    "csa_compress": [_int, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32,
                     _int, _int, _vp, _i64, _vp, _sz, _vp],
    "csa_compress_ex": [_int, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32,
                        _int, _int, _vp, _i64, _vp, _int, _f32, _int, _vp, _sz, _vp],
    "csa_rope": [_i64, _i64, _i64, _i64, _i64, _int, _f32, _int, _int, _vp, _vp],
    "csa_compress_paged": [_int, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _int, _int, _vp, _vp, _i64,
                           _vp, _i64, _int, _f32, _int, _vp],
    "csa_compress_paged_chunk": [_int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _int,
                                 _int, _vp, _vp, _i64, _vp, _i64, _int, _f32, _int, _vp],
    "lightning_index_paged": [_i64, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _int, _vp, _int,
                              _vp],
    "topk_select_paged": [_i64, _i64, _vp, _int, _int, _vp, _int, _vp, _vp, _sz, _vp],
    "sparse_mqa_attn_paged": [_i64, _int, _int, _int, _vp, _vp, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _i64,
                              _int, _f32, _int, _vp, _vp, _int, _int, _f32, _vp, _sz, _vp],
    "hca_attn_paged": [_i64, _int, _int, _vp, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _int, _f32, _vp, _int,
                       _vp, _vp, _int, _int, _f32, _vp, _sz, _vp],
    "lightning_index_pool": [_i64, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp, _int, _vp, _vp, _int, _vp],
    "topk_select_pool": [_i64, _i64, _i64, _i64, _int, _vp, _int, _vp, _vp, _vp],
    "lightning_index": [_i64, _i64, _i64, _i64, _int, _int, _int, _vp, _vp, _vp, _vp, _vp, _int,
                        _vp, _int, _vp],
    "topk_select": [_i64, _i64, _i64, _i64, _int, _int, _vp, _int, _vp, _vp, _sz, _vp],
    "sparse_mqa_attn": [_i64, _i64, _i64, _int, _i64, _int, _int, _vp, _vp, _vp, _vp, _i64, _i64,
                        _int, _f32, _int, _vp, _vp, _vp, _sz, _vp],
    "hca_attn": [_i64, _i64, _i64, _int, _i64, _int, _int, _vp, _vp, _vp, _i64, _i64, _int, _f32,
                 _vp, _int, _vp, _vp, _vp, _sz, _vp],
    "sparse_mqa_attn_ex": [_i64, _i64, _i64, _int, _i64, _int, _int, _vp, _vp, _vp, _vp, _i64, _i64,
                           _int, _f32, _int, _vp, _vp, _int, _int, _f32, _vp, _sz, _vp],
    "sparse_mqa_attn_noalloc": [_i64, _i64, _i64, _int, _i64, _int, _int, _vp, _vp, _vp, _vp, _i64, _i64,
                                _int, _f32, _int, _vp, _vp, _vp],
    "hca_attn_ex": [_i64, _i64, _i64, _int, _i64, _int, _int, _vp, _vp, _vp, _i64, _i64, _int, _f32,
                    _vp, _int, _vp, _vp, _int, _int, _f32, _vp, _sz, _vp],
}

_lib = None


class CsaError(RuntimeError):
    pass


def library() -> ctypes.CDLL:
    """Load libcsa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise CsaError(f"{LIB_PATH} is missing: build it with "
                           "`python -m long_context_sparse_compress_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.csa_compress_batch.argtypes = [ctypes.POINTER(_CompressJob), _int, _vp]
        lib.csa_compress_batch.restype = ctypes.c_int
        lib.lightning_index_compressed.argtypes = [_i64, _i64, _i64, _i64, _int, _int, _int, _vp, _vp, _vp, _vp,
                                                   _vp, _int, _vp, _int, ctypes.POINTER(_CompressJob), _int, _i64,
                                                   _vp]
        lib.lightning_index_compressed.restype = ctypes.c_int
        lib.hca_attn_compressed.argtypes = (_SIGS["hca_attn_ex"][:-1] + [ctypes.POINTER(_CompressJob), _i64, _vp])
        lib.hca_attn_compressed.restype = ctypes.c_int
        lib.topk_select_compressed.argtypes = [_i64, _i64, _i64, _i64, _int, _int, _vp, _int, _vp, _vp, _sz,
                                               ctypes.POINTER(_CompressJob), _int, _vp]
        lib.topk_select_compressed.restype = ctypes.c_int
        lib.csa_compress_paged_batch.argtypes = [ctypes.POINTER(_CompressPagedJob), _int, _vp]
        lib.csa_compress_paged_batch.restype = ctypes.c_int
        lib.csa_workspace_bytes.argtypes = [_int, _i64, _i64, _i64, _int]
        lib.csa_workspace_bytes.restype = ctypes.c_size_t
        lib.csa_last_error.restype = ctypes.c_char_p
        lib.csa_version.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def _check(status: int, name: str) -> None:
    if status != 0:
        msg = library().csa_last_error().decode()
        raise CsaError(f"{name} failed with status {status}: {msg}")


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def workspace_bytes(op: int, B: int, T: int, N: int, k: int) -> int:
    return int(library().csa_workspace_bytes(op, B, T, N, k))


def _workspace(op, B, T, N, k, device, workspace):
    need = workspace_bytes(op, B, T, N, k)
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


class _CompressJob(ctypes.Structure):
    """csa_compress_job of csa.h."""
    _fields_ = [("ratio", _int), ("B", _i64), ("n_tok", _i64), ("c", _i64), ("pos0", _i64),
                ("Ca", _vp), ("Za", _vp), ("Cb", _vp), ("Zb", _vp), ("prev_Cb", _vp), ("prev_Zb", _vp),
                ("bias", _vp), ("gamma", _vp), ("eps", _f32), ("in_dtype", _int), ("out_dtype", _int),
                ("out", _vp), ("out_batch_stride", _i64), ("rope_dims", _int), ("rope_base", _f32),
                ("rope_anchor", _int), ("out_scale", _vp)]


class _CompressPagedJob(ctypes.Structure):
    """csa_compress_paged_job of csa.h."""
    _fields_ = [("ratio", _int), ("B", _i64), ("n_tok", _i64), ("c", _i64), ("pos0", _vp),
                ("Ca", _vp), ("Za", _vp), ("Cb", _vp), ("Zb", _vp), ("prev_Cb", _vp), ("prev_Zb", _vp),
                ("bias", _vp), ("gamma", _vp), ("eps", _f32), ("in_dtype", _int), ("out_dtype", _int),
                ("pool", _vp), ("scale_pool", _vp), ("n_pool", _i64), ("block_table", _vp), ("max_blocks", _i64),
                ("rope_dims", _int), ("rope_base", _f32), ("rope_anchor", _int)]


def _out_dt(t: torch.Tensor, c=None) -> int:
    """Compressor output type: uint8 tensors hold fp8 E4M3 codes, or packed MXFP4
    (two elements per byte) when their rows are c / 2 bytes (quantize-on-write)."""
    if t.dtype == torch.uint8:
        return MXFP4 if (c is not None and t.shape[-1] * 2 == c) else FP8_E4M3
    return _dt(t)


def _compress_scale(out, out_scale, cache_entry0, n_ent, c):
    """Quantized output: the scale tensor (fp8: [B, n_ent] fp32; MXFP4: [B, n_ent, c/32]
    uint8; or the cache's) and the address of the first entry's scales."""
    if out.dtype != torch.uint8:
        if out_scale is not None:
            raise ValueError("out_scale is only for quantized (uint8) output")
        return None, None
    B = out.shape[0]
    fp4 = _out_dt(out, c) == MXFP4
    per = c // 32 if fp4 else 1
    if out_scale is None:
        if cache_entry0 is not None:
            raise ValueError("writing quantized entries into a cache needs the cache's out_scale")
        out_scale = torch.empty((B, n_ent, per) if fp4 else (B, n_ent), dtype=torch.uint8 if fp4 else torch.float32,
                                device=out.device)
    if out_scale.dtype != (torch.uint8 if fp4 else torch.float32) or not out_scale.is_contiguous():
        raise ValueError("out_scale must be contiguous uint8 (MXFP4) or float32 (fp8)")
    return out_scale, out_scale.data_ptr() + (cache_entry0 or 0) * (per if fp4 else 4)


def _compress_out(Ca, ratio, out, out_dtype, cache_entry0):
    """Output tensor, address of entry 0 of sequence 0, and batch stride."""
    B, n_tok, c = Ca.shape
    n_ent = n_tok // ratio
    if out is None:
        if out_dtype == MXFP4:       # packed fp4: c / 2 bytes per entry
            out = torch.empty(B, n_ent, c // 2, dtype=torch.uint8, device=Ca.device)
        else:
            odt = Ca.dtype if out_dtype is None else out_dtype
            out = torch.empty(B, n_ent, c, dtype=odt, device=Ca.device)
    row = out.shape[-1] if out.dim() == 3 else c     # stored elements (bytes for MXFP4) per entry
    per_elem = c // row                              # channels per stored element: 2 for MXFP4
    if cache_entry0 is None:
        if out.numel() < B * n_ent * row:
            raise ValueError("out is too small")
        return out, _ptr(out), 0
    if out.dim() != 3 or out.shape[0] != B or out.shape[2] * per_elem != c:
        raise ValueError("cache must be [B, N_cache, c] (c / 2 bytes for MXFP4)")
    if cache_entry0 < 0 or cache_entry0 + n_ent > out.shape[1]:
        raise ValueError("cache slot out of range")
    return out, _ptr(out) + cache_entry0 * row * out.element_size(), out.shape[1] * c


def _compress_jobs(jobs):
    """ctypes array of csa_compress_job for csa_compress_batch's job dicts, and the outputs."""
    arr = (_CompressJob * len(jobs))()
    outs = []
    for j, d in zip(arr, jobs):
        Ca = d["Ca"]
        B, n_tok, c = Ca.shape
        out, optr, stride = _compress_out(Ca, d["ratio"], d.get("out"), d.get("out_dtype"), d.get("cache_entry0"))
        sc, sptr = _compress_scale(out, d.get("out_scale"), d.get("cache_entry0"), n_tok // d["ratio"], c)
        outs.append(out if sc is None else (out, sc))
        j.ratio, j.B, j.n_tok, j.c, j.pos0 = d["ratio"], B, n_tok, c, d.get("pos0", 0)
        j.Ca, j.Za, j.Cb, j.Zb = _ptr(Ca), _ptr(d["Za"]), _ptr(d.get("Cb")), _ptr(d.get("Zb"))
        j.prev_Cb, j.prev_Zb = _ptr(d.get("prev_Cb")), _ptr(d.get("prev_Zb"))
        j.bias, j.gamma, j.eps = _ptr(d["bias"]), _ptr(d.get("gamma")), d.get("eps", 1e-6)
        j.in_dtype, j.out_dtype, j.out, j.out_batch_stride = _dt(Ca), _out_dt(out, c), optr, stride
        j.out_scale = sptr
        j.rope_dims, j.rope_base, j.rope_anchor = (d.get("rope_dims", 0), d.get("rope_base", ROPE_BASE),
                                                   d.get("rope_anchor", 0))
    return arr, outs


def csa_compress_batch(jobs, stream=None):
    """Several stage-1 calls of one ratio and dtype pair in one launch.  Each job
    is a dict of csa_compress's arguments (ratio, Ca, Za, bias and optionally
    Cb, Zb, prev_Cb, prev_Zb, pos0, gamma, eps, out, out_dtype, cache_entry0,
    rope_dims, rope_base, rope_anchor); returns the list of outputs."""
    arr, outs = _compress_jobs(jobs)
    st = library().csa_compress_batch(arr, len(jobs), _stream(stream))
    _check(st, "csa_compress_batch")
    return outs


def csa_compress(ratio, Ca, Za, bias, Cb=None, Zb=None, prev_Cb=None, prev_Zb=None, *, pos0=0,
                 gamma=None, eps=1e-6, out=None, out_dtype=None, cache_entry0=None, workspace=None,
                 rope_dims=0, rope_base=ROPE_BASE, rope_anchor=0, out_scale=None, stream=None):
    """Stage 1.  Ca, Za (Cb, Zb): [B, n_tok, c]; returns out [B, n_tok//ratio, c].

    With ``cache_entry0`` set, ``out`` is a [B, N_cache, c] cache and the new
    entries are written in place at entries cache_entry0 .. cache_entry0 +
    n_tok//ratio - 1 of every sequence.  ``workspace`` defaults to a fresh
    buffer of the size that enables the row split; an empty tensor disables it.
    ``rope_dims`` > 0: partial RoPE on each entry's last rope_dims channels at
    position pos0 + ratio*i + rope_anchor (csa_compress_ex).  ``out_dtype=torch.uint8``
    (or a uint8 ``out``) quantizes on write to fp8 E4M3 codes with one fp32 scale
    per entry (into ``out_scale``, the cache's [B, N_cache] with ``cache_entry0``);
    ``out_dtype=MXFP4`` (or a uint8 ``out`` of c / 2 bytes per entry) to packed
    MXFP4 with E8M0 scales [.., c / 32]; then (codes, scales) is returned."""
    B, n_tok, c = Ca.shape
    in_dt = _dt(Ca)
    out, optr, stride = _compress_out(Ca, ratio, out, out_dtype, cache_entry0)
    sc, sptr = _compress_scale(out, out_scale, cache_entry0, n_tok // ratio, c)
    ws, wsb = _workspace(OP_COMPRESS, B, n_tok, c, ratio, Ca.device, workspace)
    st = library().csa_compress_ex(ratio, B, n_tok, c, pos0, _ptr(Ca), _ptr(Za), _ptr(Cb), _ptr(Zb),
                                   _ptr(prev_Cb), _ptr(prev_Zb), _ptr(bias), _ptr(gamma), eps, in_dt,
                                   _out_dt(out, c), optr, stride, sptr, rope_dims, rope_base, rope_anchor, _ptr(ws),
                                   wsb, _stream(stream))
    _check(st, "csa_compress")
    return out if sc is None else (out, sc)


def lightning_index(q, w, k, *, q_pos0, ratio=4, qk_dtype=None, q_scale=None, k_scale=None,
                    score_dtype=torch.bfloat16, scores=None, N=None, stream=None):
    """Stage 2.  q: [B, T, 64, 128] (or uint8 encodings), w: [B, T, 64], k: [B, N, ...]."""
    B, T = q.shape[:2]
    N = k.shape[1] if N is None else N
    if qk_dtype is None:
        qk_dtype = _dt(q)
    if scores is None:
        scores = torch.empty(B, T, N, dtype=score_dtype, device=q.device)
    st = library().lightning_index(B, T, N, q_pos0, ratio, 64, 128, _ptr(q), _ptr(q_scale), _ptr(w),
                                   _ptr(k), _ptr(k_scale), qk_dtype, _ptr(scores), _dt(scores),
                                   _stream(stream))
    _check(st, "lightning_index")
    return scores


def lightning_index_compressed(q, w, k, jobs, *, e_new, q_pos0, ratio=4, qk_dtype=None, q_scale=None,
                               k_scale=None, score_dtype=torch.bfloat16, scores=None, N=None, stream=None):
    """A decode step's compressor writes (csa_compress_batch's job dicts), then
    stage 2, in one call: the results of csa_compress_batch(jobs) followed by
    lightning_index(...).  ``e_new`` is the key entry the jobs write."""
    B, T = q.shape[:2]
    N = k.shape[1] if N is None else N
    if qk_dtype is None:
        qk_dtype = _dt(q)
    if scores is None:
        scores = torch.empty(B, T, N, dtype=score_dtype, device=q.device)
    arr, _ = _compress_jobs(jobs) if jobs else (None, [])
    st = library().lightning_index_compressed(B, T, N, q_pos0, ratio, 64, 128, _ptr(q), _ptr(q_scale), _ptr(w),
                                              _ptr(k), _ptr(k_scale), qk_dtype, _ptr(scores), _dt(scores), arr,
                                              len(jobs), e_new, _stream(stream))
    _check(st, "lightning_index_compressed")
    return scores


def topk_select(scores, k, *, q_pos0, ratio=4, idx=None, workspace=None, stream=None):
    """Stage 3.  scores: [B, T, N]; returns idx [B, T, k] int32 (ascending, then -1)."""
    B, T, N = scores.shape
    if idx is None:
        idx = torch.empty(B, T, k, dtype=torch.int32, device=scores.device)
    ws, wsb = _workspace(OP_TOPK, B, T, N, k, scores.device, workspace)
    st = library().topk_select(B, T, N, q_pos0, ratio, k, _ptr(scores), _dt(scores), _ptr(idx),
                               _ptr(ws), wsb, _stream(stream))
    _check(st, "topk_select")
    return idx


def topk_select_compressed(scores, k, jobs, *, q_pos0, ratio=4, idx=None, workspace=None, stream=None):
    """A decode step's compressor writes (csa_compress_batch's job dicts), then
    stage 3, in one call: the results of csa_compress_batch(jobs) followed by
    topk_select(...)."""
    B, T, N = scores.shape
    if idx is None:
        idx = torch.empty(B, T, k, dtype=torch.int32, device=scores.device)
    ws, wsb = _workspace(OP_TOPK, B, T, N, k, scores.device, workspace)
    arr, _ = _compress_jobs(jobs) if jobs else (None, [])
    st = library().topk_select_compressed(B, T, N, q_pos0, ratio, k, _ptr(scores), _dt(scores), _ptr(idx), _ptr(ws),
                                          wsb, arr, len(jobs), _stream(stream))
    _check(st, "topk_select_compressed")
    return idx


def lightning_index_pool(q, w, k, pool, *, qk_dtype=None, q_scale=None, k_scale=None, score_dtype=torch.bfloat16,
                         scores=None, stream=None):
    """Hierarchical indexer, Reindex layer: scores of each query's candidate pool.
    q: [B, T, 64, 128] bf16 (or uint8 E4M3 codes with q_scale [B, T, 64], or packed
    MXFP4 [B, T, 64, 64] with E8M0 q_scale [B, T, 64, 4]), w: [B, T, 64], k: [B, N, 128]
    in the same form (k_scale [B, N] or [B, N, 4]), pool: [B, T, P] int32 (-1 = empty);
    returns scores [B, T, P] (-inf at empty slots)."""
    B, T, P = pool.shape
    N = k.shape[1]
    if qk_dtype is None:
        qk_dtype = (MXFP4 if q.shape[-1] == 64 else FP8_E4M3) if q.dtype == torch.uint8 else _dt(q)
    if scores is None:
        scores = torch.empty(B, T, P, dtype=score_dtype, device=q.device)
    st = library().lightning_index_pool(B, T, N, P, 64, 128, _ptr(q), _ptr(q_scale), _ptr(w), _ptr(k),
                                        _ptr(k_scale), qk_dtype, _ptr(pool), _ptr(scores), _dt(scores),
                                        _stream(stream))
    _check(st, "lightning_index_pool")
    return scores


def topk_select_pool(scores, pool, k, *, N, idx=None, stream=None):
    """Top-k inside the pool: returns idx [B, T, k] int32 of entry ids (ascending
    when the pool is), -1 padded.  N: entries in the cache (slots >= N are empty)."""
    B, T, P = pool.shape
    if idx is None:
        idx = torch.empty(B, T, k, dtype=torch.int32, device=pool.device)
    st = library().topk_select_pool(B, T, N, P, k, _ptr(scores), _dt(scores), _ptr(pool), _ptr(idx),
                                    _stream(stream))
    _check(st, "topk_select_pool")
    return idx


def sparse_mqa_attn(q, kv_cmp, idx, kv_raw, *, q_pos0, raw_pos0, window=128, scale=None,
                    out=None, lse=None, return_lse=False, workspace=None, batch_invariant=False,
                    rope_dims=0, rope_base=ROPE_BASE, stream=None):
    """Stage 4.  q: [B, T, 64, 512], kv_cmp: [B, N, 512], idx: [B, T, k], kv_raw: [B, n_raw, 512].
    ``batch_invariant``: no row split, so each query's bits do not depend on the batch.
    ``rope_dims`` > 0: inverse partial RoPE on the output at each query's position."""
    B, T, H, d = q.shape
    N = kv_cmp.shape[1]
    k = idx.shape[2]
    n_raw = kv_raw.shape[1]
    scale = d ** -0.5 if scale is None else scale
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty(B, T, H, dtype=torch.float32, device=q.device)
    if batch_invariant:
        ws, wsb = None, 0
    else:
        ws, wsb = _workspace(OP_SPARSE_ATTN, B, T, N, k, q.device, workspace)
    st = library().sparse_mqa_attn_ex(B, T, N, k, q_pos0, H, d, _ptr(q), _ptr(kv_cmp), _ptr(idx),
                                      _ptr(kv_raw), raw_pos0, n_raw, window, scale, _dt(q), _ptr(out),
                                      _ptr(lse), ATTN_BATCH_INVARIANT if batch_invariant else 0, rope_dims,
                                      rope_base, _ptr(ws), wsb, _stream(stream))
    _check(st, "sparse_mqa_attn")
    return (out, lse) if return_lse else out


def sparse_mqa_attn_noalloc(q, kv_cmp, idx, kv_raw, *, q_pos0, raw_pos0, out, window=128, scale=None, lse=None,
                            stream=None):
    """Stage 4 without any allocation: the split partials live in the library's
    static scratch (calls on one GPU must not overlap).  ``out`` (and ``lse``,
    optional) are the caller's; nothing is allocated here."""
    B, T, H, d = q.shape
    N = kv_cmp.shape[1]
    k = idx.shape[2]
    n_raw = kv_raw.shape[1]
    scale = d ** -0.5 if scale is None else scale
    st = library().sparse_mqa_attn_noalloc(B, T, N, k, q_pos0, H, d, _ptr(q), _ptr(kv_cmp), _ptr(idx), _ptr(kv_raw),
                                           raw_pos0, n_raw, window, scale, _dt(q), _ptr(out), _ptr(lse),
                                           _stream(stream))
    _check(st, "sparse_mqa_attn_noalloc")
    return out


def hca_attn(q, kv_cmp, kv_raw, *, q_pos0, raw_pos0, ratio=128, sink=None, window=128, scale=None,
             out=None, lse=None, return_lse=False, workspace=None, batch_invariant=False, rope_dims=0,
             rope_base=ROPE_BASE, stream=None):
    """Stage 5.  Dense MQA over all visible entries and the window, optional sink [64].
    ``batch_invariant``: no row split, so each query's bits do not depend on the batch.
    ``rope_dims`` > 0: inverse partial RoPE on the output at each query's position."""
    B, T, H, d = q.shape
    N = kv_cmp.shape[1]
    n_raw = kv_raw.shape[1]
    scale = d ** -0.5 if scale is None else scale
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty(B, T, H, dtype=torch.float32, device=q.device)
    if batch_invariant:
        ws, wsb = None, 0
    else:
        ws, wsb = _workspace(OP_HCA_ATTN, B, T, N, 0, q.device, workspace)
    st = library().hca_attn_ex(B, T, N, ratio, q_pos0, H, d, _ptr(q), _ptr(kv_cmp), _ptr(kv_raw),
                               raw_pos0, n_raw, window, scale, _ptr(sink), _dt(q), _ptr(out), _ptr(lse),
                               ATTN_BATCH_INVARIANT if batch_invariant else 0, rope_dims, rope_base, _ptr(ws),
                               wsb, _stream(stream))
    _check(st, "hca_attn")
    return (out, lse) if return_lse else out


def hca_attn_compressed(q, kv_cmp, kv_raw, job, *, e_new, q_pos0, raw_pos0, ratio=128, sink=None, window=128,
                        scale=None, out=None, lse=None, return_lse=False, workspace=None, rope_dims=0,
                        rope_base=ROPE_BASE, stream=None):
    """A decode step's C128A write (one csa_compress_batch job dict, ratio 128,
    writing entry ``e_new`` of ``kv_cmp``), then stage 5, in one call."""
    B, T, H, d = q.shape
    N = kv_cmp.shape[1]
    n_raw = kv_raw.shape[1]
    scale = d ** -0.5 if scale is None else scale
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty(B, T, H, dtype=torch.float32, device=q.device)
    ws, wsb = _workspace(OP_HCA_ATTN, B, T, N, 0, q.device, workspace)
    arr, _ = _compress_jobs([job])
    st = library().hca_attn_compressed(B, T, N, ratio, q_pos0, H, d, _ptr(q), _ptr(kv_cmp), _ptr(kv_raw),
                                       raw_pos0, n_raw, window, scale, _ptr(sink), _dt(q), _ptr(out), _ptr(lse), 0,
                                       rope_dims, rope_base, _ptr(ws), wsb, arr, e_new, _stream(stream))
    _check(st, "hca_attn_compressed")
    return (out, lse) if return_lse else out


def _paged_common(q, seq_pos, max_pos, out, lse, return_lse, workspace, batch_invariant, op):
    B = seq_pos.shape[0]
    if q.dim() == 4:
        if q.shape[1] != 1:
            raise ValueError("paged attention is a decode step: one query per sequence")
    elif q.dim() != 3:
        raise ValueError("q must be [B, 64, 512] or [B, 1, 64, 512]")
    if seq_pos.dtype != torch.int64:
        raise TypeError("seq_pos must be int64")
    if max_pos is None:
        max_pos = int(seq_pos.max().item()) if B else 0
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty(B, 64, dtype=torch.float32, device=q.device)
    if batch_invariant:
        ws, wsb = None, 0
    else:
        ws, wsb = _workspace(op, B, 1, 1, 0, q.device, workspace)
    return B, max_pos, out, lse, ws, wsb


def csa_compress_paged(ratio, Ca, Za, bias, pool, block_table, pos0, *, prev_Cb=None, prev_Zb=None, gamma=None,
                       eps=1e-6, scale_pool=None, rope_dims=0, rope_base=ROPE_BASE, rope_anchor=0, stream=None):
    """Decode write into the paged cache: sequence b pools its block starting at
    pos0[b] (int64 [B]) from the rolling buffer Ca, Za [B, ratio, c] (and, C4A, the
    previous block prev_Cb, prev_Zb [B, 4, c]) into its page slot of ``pool``
    ([n_pool, 32, c] C4A, [n_pool, c] C128A; uint8 for fp8 keys with ``scale_pool``)."""
    B, _, c = Ca.shape
    st = library().csa_compress_paged(ratio, B, c, _ptr(pos0), _ptr(Ca), _ptr(Za), _ptr(prev_Cb), _ptr(prev_Zb),
                                      _ptr(bias), _ptr(gamma), eps, _dt(Ca), _out_dt(pool, c), _ptr(pool),
                                      _ptr(scale_pool), pool.shape[0], _ptr(block_table), block_table.shape[1],
                                      rope_dims, rope_base, rope_anchor, _stream(stream))
    _check(st, "csa_compress_paged")
    return pool


def csa_compress_paged_chunk(ratio, Ca, Za, bias, pool, block_table, pos0, *, Cb=None, Zb=None, prev_Cb=None,
                             prev_Zb=None, gamma=None, eps=1e-6, scale_pool=None, rope_dims=0, rope_base=ROPE_BASE,
                             rope_anchor=0, stream=None):
    """Chunked-prefill write into the paged cache: sequence b compresses its chunk
    Ca, Za [B, n_tok, c] (C4A: with the chunk's Cb, Zb and the block before it,
    prev_Cb, prev_Zb [B, 4, c]) starting at block start pos0[b] (int64 [B]); entry
    pos0[b] / ratio + i lands in its page slot of ``pool`` as csa_compress_paged
    writes it."""
    B, n_tok, c = Ca.shape
    st = library().csa_compress_paged_chunk(ratio, B, n_tok, c, _ptr(pos0), _ptr(Ca), _ptr(Za), _ptr(Cb), _ptr(Zb),
                                            _ptr(prev_Cb), _ptr(prev_Zb), _ptr(bias), _ptr(gamma), eps, _dt(Ca),
                                            _out_dt(pool, c), _ptr(pool), _ptr(scale_pool), pool.shape[0],
                                            _ptr(block_table), block_table.shape[1], rope_dims, rope_base,
                                            rope_anchor, _stream(stream))
    _check(st, "csa_compress_paged_chunk")
    return pool


def csa_compress_paged_batch(jobs, stream=None):
    """Several csa_compress_paged_chunk calls in one launch.  Each job is a dict of
    that call's arguments (ratio, Ca, Za, bias, pool, block_table, pos0 and
    optionally Cb, Zb, prev_Cb, prev_Zb, gamma, eps, scale_pool, rope_dims,
    rope_base, rope_anchor); returns the pools."""
    arr = (_CompressPagedJob * len(jobs))()
    for j, d in zip(arr, jobs):
        Ca, pool, table = d["Ca"], d["pool"], d["block_table"]
        B, n_tok, c = Ca.shape
        j.ratio, j.B, j.n_tok, j.c, j.pos0 = d["ratio"], B, n_tok, c, _ptr(d["pos0"])
        j.Ca, j.Za, j.Cb, j.Zb = _ptr(Ca), _ptr(d["Za"]), _ptr(d.get("Cb")), _ptr(d.get("Zb"))
        j.prev_Cb, j.prev_Zb = _ptr(d.get("prev_Cb")), _ptr(d.get("prev_Zb"))
        j.bias, j.gamma, j.eps = _ptr(d["bias"]), _ptr(d.get("gamma")), d.get("eps", 1e-6)
        j.in_dtype, j.out_dtype = _dt(Ca), _out_dt(pool, c)
        j.pool, j.scale_pool, j.n_pool = _ptr(pool), _ptr(d.get("scale_pool")), pool.shape[0]
        j.block_table, j.max_blocks = _ptr(table), table.shape[1]
        j.rope_dims, j.rope_base, j.rope_anchor = (d.get("rope_dims", 0), d.get("rope_base", ROPE_BASE),
                                                   d.get("rope_anchor", 0))
    st = library().csa_compress_paged_batch(arr, len(jobs), _stream(stream))
    _check(st, "csa_compress_paged_batch")
    return [d["pool"] for d in jobs]


def lightning_index_paged(q, w, k_pool, block_table, seq_pos, *, qk_dtype=None, q_scale=None, k_scale=None,
                          score_dtype=torch.bfloat16, scores=None, stream=None):
    """Paged decode indexer: q [B, 64, 128] (bf16, or uint8 E4M3 codes with q_scale [B, 64],
    or packed MXFP4 [B, 64, 64] with E8M0 q_scale [B, 64, 4]), w [B, 64], k_pool [n_pool, 32, 128]
    (bf16, or uint8 codes with k_scale [n_pool, 32], or packed MXFP4 [n_pool, 32, 64] with
    k_scale [n_pool, 32, 4]), block_table [B, max_blocks] int32, seq_pos [B] int64; returns
    scores [B, 32 * max_blocks]."""
    B, max_blocks = block_table.shape
    if qk_dtype is None:
        if q.dtype == torch.uint8:
            qk_dtype = MXFP4 if q.shape[-1] == 64 else FP8_E4M3
        else:
            qk_dtype = _dt(q)
    if scores is None:
        scores = torch.empty(B, 32 * max_blocks, dtype=score_dtype, device=q.device)
    st = library().lightning_index_paged(B, max_blocks, 64, 128, _ptr(q), _ptr(q_scale), _ptr(w), _ptr(k_pool),
                                         _ptr(k_scale), k_pool.shape[0], _ptr(block_table), _ptr(seq_pos), qk_dtype,
                                         _ptr(scores), _dt(scores), _stream(stream))
    _check(st, "lightning_index_paged")
    return scores


def topk_select_paged(scores, k, seq_pos, *, ratio=4, idx=None, workspace=None, stream=None):
    """Top-k of each sequence's visible entries (row b: e < (seq_pos[b] + 1) // ratio);
    scores [B, N]; returns idx [B, k] int32."""
    B, N = scores.shape
    if idx is None:
        idx = torch.empty(B, k, dtype=torch.int32, device=scores.device)
    ws, wsb = _workspace(OP_TOPK, B, 1, N, k, scores.device, workspace)
    st = library().topk_select_paged(B, N, _ptr(seq_pos), ratio, k, _ptr(scores), _dt(scores), _ptr(idx), _ptr(ws),
                                     wsb, _stream(stream))
    _check(st, "topk_select_paged")
    return idx


def sparse_mqa_attn_paged(q, kv_pool, block_table, idx, win, seq_pos, *, max_pos=None, window=128, scale=None,
                          out=None, lse=None, return_lse=False, workspace=None, batch_invariant=False,
                          rope_dims=0, rope_base=ROPE_BASE, stream=None):
    """Paged decode, stage 4: one query per sequence at seq_pos[b] (int64 [B]).
    kv_pool [n_pool, 32, 512] (32 C4A entries per 128-raw-token block), block_table
    [B, max_blocks] int32, idx [B, k] entry ids, win [B, ring, 512] (position p at
    row p % ring, ring a power of two >= window)."""
    B, max_pos, out, lse, ws, wsb = _paged_common(q, seq_pos, max_pos, out, lse, return_lse, workspace,
                                                  batch_invariant, OP_SPARSE_ATTN)
    k = idx.shape[-1]
    d = q.shape[-1]
    scale = d ** -0.5 if scale is None else scale
    st = library().sparse_mqa_attn_paged(B, k, 64, d, _ptr(q), _ptr(kv_pool), kv_pool.shape[0], _ptr(block_table),
                                         block_table.shape[1], _ptr(idx), _ptr(win), win.shape[1], _ptr(seq_pos),
                                         max_pos, window, scale, _dt(q), _ptr(out), _ptr(lse),
                                         ATTN_BATCH_INVARIANT if batch_invariant else 0, rope_dims, rope_base,
                                         _ptr(ws), wsb, _stream(stream))
    _check(st, "sparse_mqa_attn_paged")
    return (out, lse) if return_lse else out


def hca_attn_paged(q, kv_pool, block_table, win, seq_pos, *, sink=None, max_pos=None, window=128, scale=None,
                   out=None, lse=None, return_lse=False, workspace=None, batch_invariant=False, rope_dims=0,
                   rope_base=ROPE_BASE, stream=None):
    """Paged decode, stage 5: dense MQA over the visible C128A entries of each
    sequence (kv_pool [n_pool, 512], one entry per block) and its window ring."""
    B, max_pos, out, lse, ws, wsb = _paged_common(q, seq_pos, max_pos, out, lse, return_lse, workspace,
                                                  batch_invariant, OP_HCA_ATTN)
    d = q.shape[-1]
    scale = d ** -0.5 if scale is None else scale
    st = library().hca_attn_paged(B, 64, d, _ptr(q), _ptr(kv_pool), kv_pool.shape[0], _ptr(block_table),
                                  block_table.shape[1], _ptr(win), win.shape[1], _ptr(seq_pos), max_pos, window,
                                  scale, _ptr(sink), _dt(q), _ptr(out), _ptr(lse),
                                  ATTN_BATCH_INVARIANT if batch_invariant else 0, rope_dims, rope_base, _ptr(ws),
                                  wsb, _stream(stream))
    _check(st, "hca_attn_paged")
    return (out, lse) if return_lse else out


def rope(x, *, pos0, rope_dims=64, rope_base=ROPE_BASE, inverse=False, stream=None):
    """Partial RoPE in place on x [B, T, H, D] or [B, T, D] (row t at pos0 + t); returns x."""
    if x.dim() == 3:
        B, T, D = x.shape
        H = 1
    else:
        B, T, H, D = x.shape
    st = library().csa_rope(B, T, H, D, pos0, rope_dims, rope_base, 1 if inverse else 0, _dt(x), _ptr(x),
                            _stream(stream))
    _check(st, "csa_rope")
    return x
