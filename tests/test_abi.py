"""The C-ABI library loads, exports every symbol include/csa.h declares, and
rejects bad arguments on the host before any HIP call (runs without a GPU)."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")

A = 0x10000          # a 16-byte-aligned fake device address; validation never dereferences it
MIS = 0x10008        # misaligned


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    import long_context_sparse_compress_amd as csa
    alt = os.environ.get("CSA_ABI_HOSTCHECK_LIB")
    if alt:
        # the sanitized host-only build of the same C-ABI layer (see
        # test_validation_under_sanitizers)
        csa.LIB_PATH = alt
    return csa.library()


def test_header_symbols_exported(lib):
    names = _declared()
    assert set(names) >= {"csa_compress", "lightning_index", "topk_select", "sparse_mqa_attn",
                          "hca_attn", "sparse_mqa_attn_ex", "hca_attn_ex", "csa_compress_ex", "csa_rope",
                          "lightning_index_pool", "topk_select_pool", "sparse_mqa_attn_paged", "hca_attn_paged",
                          "lightning_index_paged", "topk_select_paged", "csa_compress_paged",
                          "csa_compress_paged_chunk", "csa_compress_paged_batch", "csa_workspace_bytes",
                          "csa_last_error", "csa_version"}
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", os.path.join(ROOT, "long_context_sparse_compress_amd", "libcsa.so")],
                         capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", out, flags=re.M), n


def _err(lib):
    return lib.csa_last_error().decode()


def test_compress_validation(lib):
    f = lib.csa_compress
    ok = dict(ratio=4, B=2, n_tok=8, c=512, pos0=0, Ca=A, Za=A, Cb=A, Zb=A, pCb=None, pZb=None,
              bias=A, gamma=None, eps=1e-6, idt=1, odt=1, out=A, stride=0, ws=None, wsb=0, s=None)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["ratio"], a["B"], a["n_tok"], a["c"], a["pos0"], a["Ca"], a["Za"], a["Cb"], a["Zb"],
                 a["pCb"], a["pZb"], a["bias"], a["gamma"], a["eps"], a["idt"], a["odt"], a["out"],
                 a["stride"], a["ws"], a["wsb"], a["s"])

    assert call(ratio=8) == -1 and "ratio" in _err(lib)
    assert call(Ca=None) == -1 and "Ca is NULL" in _err(lib)
    assert call(Ca=MIS) == -1 and "aligned" in _err(lib)
    assert call(pos0=6) == -1 and "pos0" in _err(lib)
    assert call(pos0=8) == -1 and "prev_Cb is NULL" in _err(lib)
    assert call(pCb=A, pZb=A) == -1 and "must be NULL" in _err(lib)
    assert call(c=100) == -1 and "multiple of 64" in _err(lib)
    assert call(idt=2) == -2
    assert call(eps=0.0) == -1 and "eps" in _err(lib)
    assert call(ratio=128, n_tok=256) == -1 and "Cb must be NULL" in _err(lib)
    assert call(stride=100) == -1
    # the workspace is optional, but one that is declared must be a real, aligned buffer
    assert call(ws=None, wsb=4096) == -1 and "workspace is NULL" in _err(lib)
    assert call(ws=MIS, wsb=4096) == -1 and "aligned" in _err(lib)
    # nothing to do: succeeds without touching the GPU
    assert call(n_tok=3, Ca=None, Za=None, Cb=None, Zb=None, bias=None, out=None) == 0
    assert call(B=0, Ca=None, Za=None, Cb=None, Zb=None, bias=None, out=None) == 0


def test_compress_batch_layout_and_validation(lib, tmp_path):
    """csa_compress_job as the binding lays it out matches the C compiler's
    layout, and the batch entry point validates every job."""
    import ctypes
    import long_context_sparse_compress_amd as csa
    if shutil.which("g++"):
        src = tmp_path / "j.cpp"
        src.write_text('#include <cstddef>\n#include <cstdio>\n#include "csa.h"\n'
                       'int main(){printf("%zu %zu %zu %zu\\n", sizeof(csa_compress_job), '
                       'offsetof(csa_compress_job, eps), offsetof(csa_compress_job, out), '
                       'offsetof(csa_compress_job, out_batch_stride));}\n')
        exe = tmp_path / "j"
        r = subprocess.run(["g++", "-std=c++17", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        got = subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()
        J = csa._CompressJob
        assert [int(x) for x in got] == [ctypes.sizeof(J), J.eps.offset, J.out.offset, J.out_batch_stride.offset]
    lib.csa_compress_batch.argtypes = [ctypes.POINTER(csa._CompressJob), ctypes.c_int, ctypes.c_void_p]

    def job(**kw):
        d = dict(ratio=4, B=2, n_tok=8, c=512, pos0=0, Ca=A, Za=A, Cb=A, Zb=A, prev_Cb=None, prev_Zb=None,
                 bias=A, gamma=None, eps=1e-6, in_dtype=1, out_dtype=1, out=A, out_batch_stride=0)
        d.update(kw)
        return csa._CompressJob(**d)

    arr = (csa._CompressJob * 2)(job(), job(c=128, Ca=None))
    assert lib.csa_compress_batch(arr, 2, None) == -1 and "job 1: Ca is NULL" in _err(lib)
    arr = (csa._CompressJob * 2)(job(), job(ratio=128, n_tok=256, Cb=None, Zb=None))
    assert lib.csa_compress_batch(arr, 2, None) == -1 and "share ratio" in _err(lib)
    assert lib.csa_compress_batch(arr, 0, None) == -1 and "n_jobs" in _err(lib)
    assert lib.csa_compress_batch(None, 1, None) == -1
    # jobs with nothing to write: succeeds without touching the GPU
    arr = (csa._CompressJob * 2)(job(n_tok=3, Ca=None, Za=None, Cb=None, Zb=None, bias=None, out=None),
                                 job(B=0, Ca=None, Za=None, Cb=None, Zb=None, bias=None, out=None))
    assert lib.csa_compress_batch(arr, 2, None) == 0


def test_index_validation(lib):
    f = lib.lightning_index

    def call(B=1, T=4, N=64, q_pos0=252, ratio=4, H=64, d=128, q=A, qs=None, w=A, k=A, ks=None,
             qk=1, sc=A, sdt=1):
        return f(B, T, N, q_pos0, ratio, H, d, q, qs, w, k, ks, qk, sc, sdt, None)

    assert call(H=32) == -2 and "H_I=64" in _err(lib)
    assert call(N=10) == -1 and "visible" in _err(lib)
    assert call(qk=2) == -1 and "q_scale is NULL" in _err(lib)
    assert call(qk=1, qs=A) == -1 and "must be NULL" in _err(lib)
    assert call(qk=0, sdt=1) == -2
    assert call(ratio=5) == -1
    assert call(w=MIS) == -1 and "aligned" in _err(lib)
    assert call(qk=7) == -2


def test_index_compressed_validation(lib):
    """lightning_index_compressed: the indexer's checks, then the jobs' (as
    csa_compress_batch), then e_new (only with jobs).  Error cases only: a
    valid call would launch."""
    import ctypes
    import long_context_sparse_compress_amd as csa
    f = lib.lightning_index_compressed
    f.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int] * 3 + [ctypes.c_void_p] * 5 + [ctypes.c_int, ctypes.c_void_p,
                                                                                       ctypes.c_int,
                                                                                       ctypes.POINTER(csa._CompressJob),
                                                                                       ctypes.c_int, ctypes.c_int64,
                                                                                       ctypes.c_void_p]

    def job(**kw):
        d = dict(ratio=4, B=2, n_tok=4, c=512, pos0=4, Ca=A, Za=A, Cb=A, Zb=A, prev_Cb=A, prev_Zb=A,
                 bias=A, gamma=None, eps=1e-6, in_dtype=1, out_dtype=1, out=A, out_batch_stride=0)
        d.update(kw)
        return csa._CompressJob(**d)

    def call(jobs=None, n=None, e_new=63, B=2, N=64, q_pos0=255, H=64, qk=1, qs=None, ks=None):
        arr = (csa._CompressJob * max(1, len(jobs or [])))(*(jobs or []))
        n = len(jobs or []) if n is None else n
        return f(B, 1, N, q_pos0, 4, H, 128, A, qs, A, A, ks, qk, A, 1, arr, n, e_new, None)

    assert call(e_new=-5, H=32) == -2 and "H_I=64" in _err(lib)  # no jobs: e_new is not looked at
    assert call([job()], H=32) == -2 and "H_I=64" in _err(lib)   # the indexer is checked first
    assert call([job(), job(c=128, Ca=None)]) == -1 and "job 1: Ca is NULL" in _err(lib)
    assert call([job()], n=5) == -1 and "n_jobs" in _err(lib)
    assert call([job()], e_new=64) == -1 and "e_new" in _err(lib)
    assert call([job()], e_new=-1) == -1 and "e_new" in _err(lib)
    assert call([job(ratio=128, n_tok=128, Cb=None, Zb=None, prev_Cb=None, prev_Zb=None), job()]) == -1


def test_hca_compressed_validation(lib):
    """hca_attn_compressed: hca_attn_ex's checks, then the job's (ratio 128),
    then e_new.  Error cases only: a valid call would launch."""
    import ctypes
    import long_context_sparse_compress_amd as csa
    f = lib.hca_attn_compressed
    f.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t,
                  ctypes.POINTER(csa._CompressJob), ctypes.c_int64, ctypes.c_void_p]

    def job(**kw):
        d = dict(ratio=128, B=2, n_tok=128, c=512, pos0=1024 * 128 - 128, Ca=A, Za=A, Cb=None, Zb=None,
                 prev_Cb=None, prev_Zb=None, bias=A, gamma=None, eps=1e-6, in_dtype=1, out_dtype=1, out=A,
                 out_batch_stride=0)
        d.update(kw)
        return csa._CompressJob(**d)

    def call(j, e_new=1023, H=64, N=1024):
        arr = (csa._CompressJob * 1)(j)
        wsb = lib.csa_workspace_bytes(4, 2, 1, N, 0)
        return f(2, 1, N, 128, 1024 * 128 - 1, H, 512, A, A, A, 1024 * 128 - 128, 128, 128, 0.04, None, 1, A, None,
                 0, 0, 0.0, A, wsb, arr, e_new, None)

    assert call(job(), H=32) == -2                                   # the attention is checked first
    assert call(job(Ca=None)) == -1 and "job 0: Ca is NULL" in _err(lib)
    assert call(job(ratio=4, n_tok=4, Cb=A, Zb=A, prev_Cb=A, prev_Zb=A)) == -1 and "ratio 128" in _err(lib)
    assert call(job(), e_new=1024) == -1 and "e_new" in _err(lib)
    assert call(job(), e_new=-1) == -1 and "e_new" in _err(lib)


def test_topk_compressed_validation(lib):
    """topk_select_compressed: topk_select's checks, then the jobs'.  Error
    cases only: a valid call would launch."""
    import ctypes
    import long_context_sparse_compress_amd as csa
    f = lib.topk_select_compressed
    f.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(csa._CompressJob),
                                         ctypes.c_int, ctypes.c_void_p]

    def job(**kw):
        d = dict(ratio=4, B=2, n_tok=4, c=512, pos0=4, Ca=A, Za=A, Cb=A, Zb=A, prev_Cb=A, prev_Zb=A,
                 bias=A, gamma=None, eps=1e-6, in_dtype=1, out_dtype=1, out=A, out_batch_stride=0)
        d.update(kw)
        return csa._CompressJob(**d)

    def call(jobs, n=None, k=16):
        arr = (csa._CompressJob * len(jobs))(*jobs)
        return f(2, 1, 64, 255, 4, k, A, 1, A, None, 0, arr, len(jobs) if n is None else n, None)

    assert call([job()], k=0) == -1 and "k must be" in _err(lib)    # Top-k is checked first
    assert call([job(Za=None)]) == -1 and "job 0: Za is NULL" in _err(lib)
    assert call([job()], n=5) == -1 and "n_jobs" in _err(lib)


def test_topk_validation(lib):
    f = lib.topk_select
    assert f(1, 1, 64, 255, 4, 0, A, 1, A, None, 0, None) == -1 and "k must be" in _err(lib)
    assert f(1, 1, 64, 255, 4, 4096, A, 1, A, None, 0, None) == -1
    assert f(1, 1, 64, 255, 4, 16, A, 2, A, None, 0, None) == -2
    assert f(1, 1, 10, 255, 4, 16, A, 1, A, None, 0, None) == -1 and "visible" in _err(lib)
    # rows too long for LDS need a workspace
    assert f(1, 1, 262144, 1048575, 4, 1024, A, 1, A, None, 0, None) == -4
    need = lib.csa_workspace_bytes(2, 1, 1, 262144, 1024)
    assert need > 0
    assert f(1, 1, 262144, 1048575, 4, 1024, A, 1, A, A, need - 1, None) == -4


def test_attention_validation(lib):
    s = lib.sparse_mqa_attn
    h = lib.hca_attn
    ws = lib.csa_workspace_bytes(3, 2, 1, 64, 16)
    assert ws > 0

    def sp(H=64, d=512, window=128, raw_pos0=128, n_raw=128, io=1, wsp=A, wsb=ws, q=A):
        return s(2, 1, 64, 16, 255, H, d, q, A, A, A, raw_pos0, n_raw, window, 0.04, io, A, None,
                 wsp, wsb, None)

    assert sp(H=32) == -2
    assert sp(raw_pos0=129) == -1 and "first window position" in _err(lib)
    assert sp(n_raw=127) == -1 and "last query" in _err(lib)
    assert sp(window=0) == -1
    assert sp(io=2) == -2
    assert sp(wsp=None) == -4
    assert sp(wsb=ws - 1) == -4
    assert sp(q=None) == -1
    assert h(2, 1, 1, 128, 255, 64, 512, A, A, A, 128, 128, 128, 0.04, None, 1, A, None, A, ws, None) == -1
    assert h(2, 1, 2, 3, 255, 64, 512, A, A, A, 128, 128, 128, 0.04, None, 1, A, None, A, ws, None) == -1


def test_attention_flags_validation(lib):
    """The _ex entry points reject unknown flag bits before anything else, and
    the batch-invariant flag needs no workspace (the other checks still apply)."""
    se, he = lib.sparse_mqa_attn_ex, lib.hca_attn_ex
    ws = lib.csa_workspace_bytes(3, 2, 1, 64, 16)

    def sp(flags, wsp=None, wsb=0, H=64, n_raw=128, rd=0, rb=10000.0):
        return se(2, 1, 64, 16, 255, H, 512, A, A, A, A, 128, n_raw, 128, 0.04, 1, A, None, flags,
                  rd, rb, wsp, wsb, None)

    def hc(flags, wsp=None, wsb=0, n_raw=128, rd=0, rb=10000.0):
        return he(2, 1, 2, 128, 255, 64, 512, A, A, A, 128, n_raw, 128, 0.04, None, 1, A, None, flags,
                  rd, rb, wsp, wsb, None)

    for f in (2, 4, -1, 1 | 8):
        assert sp(f, A, ws) == -1 and "unknown attention flags" in _err(lib)
        assert hc(f, A, ws) == -1 and "unknown attention flags" in _err(lib)
    # without the flag the split decode wants its workspace
    assert sp(0) == -4 and "workspace" in _err(lib)
    assert hc(0) == -4 and "workspace" in _err(lib)
    # with it, the remaining argument checks still run
    assert sp(1, H=32) == -2
    assert sp(1, n_raw=127) == -1 and "last query" in _err(lib)
    assert hc(1, n_raw=127) == -1 and "last query" in _err(lib)
    # the output's inverse RoPE: a multiple of 8 up to 512, base > 1
    for rd in (4, 12, 520, -8):
        assert sp(1, rd=rd) == -1 and "rope_dims" in _err(lib), rd
        assert hc(1, rd=rd) == -1 and "rope_dims" in _err(lib), rd
    for rb in (1.0, 0.5, float("inf"), float("nan")):
        assert sp(1, rd=64, rb=rb) == -1 and "rope_base" in _err(lib), rb
    assert sp(1, rd=64, n_raw=127) == -1 and "last query" in _err(lib)


def test_rope_validation(lib):
    """csa_compress_ex's RoPE arguments and csa_rope's checks (host only)."""
    ce = lib.csa_compress_ex

    def cmp(rd=64, rb=10000.0, ra=0, ratio=4, c=512, odt=1, osc=None, stride=0):
        cb = A if ratio == 4 else None
        return ce(ratio, 2, 8, c, 0, A, A, cb, cb, None, None, A, None, 1e-6, 1, odt, A, stride, osc, rd, rb, ra,
                  None, 0, None)

    for rd in (4, 12, 520, -8):
        assert cmp(rd=rd) == -1 and "rope_dims" in _err(lib), rd
    assert cmp(rd=1024, c=512) == -1
    assert cmp(rb=1.0) == -1 and "rope_base" in _err(lib)
    assert cmp(ra=4) == -1 and "rope_anchor" in _err(lib)
    assert cmp(ra=-1) == -1 and "rope_anchor" in _err(lib)
    assert cmp(ra=127, ratio=128) == 0    # a valid anchor; 8 tokens complete no C128A block: no launch
    # quantize-on-write (fp8 output): C4A only, needs its scales, stride a multiple of c
    assert cmp(rd=0, odt=2) == -1 and "out_scale" in _err(lib)
    assert cmp(rd=0, odt=2, osc=A + 2) == -1 and "4-byte" in _err(lib)
    assert cmp(rd=0, odt=2, osc=A, stride=520) == -1 and "multiple of c" in _err(lib)
    assert cmp(rd=0, odt=2, osc=A, ratio=128, ra=0) == -2 and "ratio must be 4" in _err(lib)
    assert cmp(rd=0, odt=1, osc=A) == -1 and "out_scale must be NULL" in _err(lib)
    assert cmp(rd=0, odt=3) == -1 and "out_scale" in _err(lib)      # MXFP4 output needs its scale bytes
    assert cmp(rd=0, odt=4) == -2
    r = lib.csa_rope

    def rp(B=2, T=3, H=4, D=512, pos0=0, rd=64, rb=10000.0, inv=0, dt=1, x=A):
        return r(B, T, H, D, pos0, rd, rb, inv, dt, x, None)

    assert rp(rd=0) == -1 and "rope_dims" in _err(lib)
    assert rp(rd=2048, D=4096) == -1 and "rope_dims" in _err(lib)
    assert rp(rd=520) == -1
    assert rp(D=12) == -1 and "D must" in _err(lib)
    assert rp(inv=2) == -1 and "inverse" in _err(lib)
    assert rp(dt=2) == -2
    assert rp(x=None) == -1
    assert rp(pos0=-1) == -1 and "pos0" in _err(lib)
    assert rp(rb=0.9) == -1 and "rope_base" in _err(lib)
    assert rp(B=0, x=None) == 0           # nothing to do: no pointer needed, no launch


def test_workspace_query(lib):
    assert lib.csa_workspace_bytes(0, 8, 1, 64, 0) == 0
    assert lib.csa_workspace_bytes(3, 1, 4096, 33792, 512) == 0     # prefill: no split
    assert lib.csa_workspace_bytes(4, 16, 1, 8192, 0) > 0           # decode: split rows
    assert lib.csa_workspace_bytes(99, 1, 1, 1, 1) == 0
    # compressor (B, n_tok, c, ratio): C128A with few entries splits rows
    assert lib.csa_workspace_bytes(0, 32, 128, 512, 128) == 32 * 8 * 3 * 512 * 4   # 8 ranges of 16 rows
    assert lib.csa_workspace_bytes(0, 1, 128, 512, 128) == 16 * 3 * 512 * 4       # at most 16 ranges
    assert lib.csa_workspace_bytes(0, 2048, 128, 512, 128) == 0                   # enough entries
    assert lib.csa_workspace_bytes(0, 32, 128, 512, 4) == 0                       # C4A never splits


@pytest.mark.skipif(shutil.which("g++") is None, reason="no g++")
def test_validation_compiles_without_hip(tmp_path):
    """validate.h is plain C++: it builds with g++ and no HIP headers."""
    src = tmp_path / "v.cpp"
    src.write_text('#include "validate.h"\nint main(){auto c=csa::check_topk(1,1,8,0,4,0,nullptr,1,nullptr,nullptr,0);'
                   'return c.code==CSA_ERR_INVALID_ARG?0:1;}\n')
    exe = tmp_path / "v"
    r = subprocess.run(["g++", "-std=c++17", "-I", os.path.join(ROOT, "long_context_sparse_compress_amd", "csrc"),
                        str(src), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert subprocess.run([str(exe)]).returncode == 0


def test_pool_validation(lib):
    """lightning_index_pool / topk_select_pool argument checks (host only)."""
    ip, tp = lib.lightning_index_pool, lib.topk_select_pool

    def idx_pool(B=2, T=1, N=64, P=128, H=64, d=128, dt=1, sd=1, q=A, w=A, k=A, pool=A, sc=A, qs=None, ks=None):
        return ip(B, T, N, P, H, d, q, qs, w, k, ks, dt, pool, sc, sd, None)

    assert idx_pool(H=32) == -2 and "H_I=64" in _err(lib)
    assert idx_pool(dt=0) == -2 and "bf16, fp8 E4M3 or MXFP4" in _err(lib)
    assert idx_pool(dt=5) == -2
    assert idx_pool(dt=2) == -1 and "q_scale" in _err(lib)          # fp8 needs both scale arrays
    assert idx_pool(dt=3, qs=A) == -1 and "k_scale" in _err(lib)     # MXFP4 too
    assert idx_pool(qs=A) == -1 and "must be NULL" in _err(lib)      # bf16 takes none
    assert idx_pool(sd=2) == -2
    assert idx_pool(P=65537) == -1 and "P must" in _err(lib)
    assert idx_pool(P=-1) == -1
    assert idx_pool(pool=None) == -1 and "pool" in _err(lib)
    assert idx_pool(k=MIS) == -1
    assert idx_pool(N=0, k=None, B=0) == 0          # nothing to do
    assert idx_pool(P=0, q=None, w=None, k=None, pool=None, sc=None) == 0

    def top_pool(B=2, T=1, N=64, P=128, k=16, sd=1, sc=A, pool=A, idx=A):
        return tp(B, T, N, P, k, sc, sd, pool, idx, None)

    assert top_pool(P=16385) == -1 and "P must" in _err(lib)
    assert top_pool(k=0) == -1 and "k must" in _err(lib)
    assert top_pool(k=2049) == -1
    assert top_pool(sd=3) == -2
    assert top_pool(pool=None) == -1 and "pool" in _err(lib)
    assert top_pool(idx=None) == -1
    assert top_pool(B=0, sc=None, pool=None, idx=None) == 0


def test_paged_validation(lib):
    """sparse_mqa_attn_paged / hca_attn_paged argument checks (host only)."""
    sp, hp = lib.sparse_mqa_attn_paged, lib.hca_attn_paged
    ws = lib.csa_workspace_bytes(3, 4, 1, 1, 0)

    def s_(B=4, k=16, H=64, nb=8, ring=256, win=128, maxpos=1000, flags=0, wsp=A, wsb=ws, tbl=A, sp_=A, idx=A):
        return sp(B, k, H, 512, A, A, 100, tbl, nb, idx, A, ring, sp_, maxpos, win, 0.04, 1, A, None, flags, 0,
                  10000.0, wsp, wsb, None)

    def h_(B=4, ring=256, sink=None, wsp=A, wsb=ws):
        return hp(B, 64, 512, A, A, 100, A, 8, A, ring, A, 1000, 128, 0.04, sink, 1, A, None, 0, 0, 10000.0,
                  wsp, wsb, None)

    assert s_(H=32) == -2
    assert s_(ring=100) == -1 and "fewer than the window" in _err(lib)
    assert s_(ring=192) == -1 and "power of two" in _err(lib)
    assert s_(nb=0) == -1 and "max_blocks" in _err(lib)
    assert s_(maxpos=-1) == -1
    assert s_(tbl=None) == -1 and "block_table" in _err(lib)
    assert s_(sp_=None) == -1 and "seq_pos" in _err(lib)
    assert s_(idx=None) == -1 and "idx" in _err(lib)
    assert s_(k=2049) == -1
    assert s_(wsp=None) == -4
    assert s_(flags=2) == -1 and "unknown attention flags" in _err(lib)
    assert h_(ring=64) == -1
    assert h_(wsp=None) == -4
    assert h_(sink=MIS) == -1
    assert s_(B=0, wsp=None, tbl=None, sp_=None, idx=None) == 0


def test_paged_index_topk_validation(lib):
    ip, tp = lib.lightning_index_paged, lib.topk_select_paged

    def ix(B=4, mb=8, H=64, dt=1, qs=None, ks=None, npool=10, tbl=A, sp_=A, sd=1):
        return ip(B, mb, H, 128, A, qs, A, A, ks, npool, tbl, sp_, dt, A, sd, None)

    assert ix(H=32) == -2
    assert ix(dt=0) == -2 and "bf16, fp8 E4M3 or MXFP4" in _err(lib)
    assert ix(dt=3) == -1 and "q_scale" in _err(lib)        # MXFP4 keys need both scale arrays
    assert ix(dt=3, qs=A) == -1 and "k_scale" in _err(lib)
    assert ix(dt=2) == -1 and "q_scale" in _err(lib)
    assert ix(dt=1, qs=A) == -1 and "must be NULL" in _err(lib)
    assert ix(npool=0) == -1 and "no block" in _err(lib)
    assert ix(mb=0) == -1
    assert ix(tbl=None) == -1 and "block_table" in _err(lib)
    assert ix(sp_=None) == -1 and "seq_pos" in _err(lib)
    assert ix(B=0, tbl=None, sp_=None, npool=0) == 0

    def tk(B=4, N=1024, k=16, sp_=A, ratio=4, ws=None, wsb=0):
        return tp(B, N, sp_, ratio, k, A, 1, A, ws, wsb, None)

    assert tk(ratio=3) == -1
    assert tk(k=0) == -1
    assert tk(sp_=None) == -1 and "seq_pos" in _err(lib)
    assert tk(N=262144) == -4            # long rows need a workspace
    assert tk(B=0, sp_=None) == 0


def test_compress_paged_validation(lib):
    cp = lib.csa_compress_paged

    def c_(ratio=4, B=4, c=512, od=1, sc=None, pc=A, npool=10, mb=8, tbl=A, p0=A, ra=0):
        return cp(ratio, B, c, p0, A, A, pc, pc, A, None, 1e-6, 1, od, A, sc, npool, tbl, mb, 0, 10000.0, ra, None)

    assert c_(ratio=8) == -1
    assert c_(c=100) == -1
    assert c_(od=2) == -1 and "scale_pool" in _err(lib)
    assert c_(od=2, sc=A, ratio=128, pc=None) == -2
    assert c_(od=1, sc=A) == -1 and "scale_pool must be NULL" in _err(lib)
    assert c_(pc=None) == -1 and "prev_Cb" in _err(lib)
    assert c_(ratio=128) == -1 and "must be NULL" in _err(lib)
    assert c_(mb=0) == -1
    assert c_(tbl=None) == -1 and "block_table" in _err(lib)
    assert c_(p0=None) == -1 and "pos0" in _err(lib)
    assert c_(ra=4) == -1 and "rope_anchor" in _err(lib)
    assert c_(npool=0) == 0 and c_(B=0, p0=None, tbl=None) == 0      # nothing to write


def test_compress_paged_chunk_validation(lib):
    cp = lib.csa_compress_paged_chunk

    def c_(ratio=4, B=4, n=64, c=512, cb=A, pc=A, od=1, sc=None, npool=10, mb=8, tbl=A, p0=A):
        return cp(ratio, B, n, c, p0, A, A, cb, cb, pc, pc, A, None, 1e-6, 1, od, A, sc, npool, tbl, mb, 0, 10000.0, 0,
                  None)

    # the pointers are fake: every call below must fail validation or have nothing to write
    assert c_(n=-1) == -1 and "n_tok" in _err(lib)
    assert c_(n=4 * ((1 << 22) + 1)) == -1 and "2^22" in _err(lib)
    assert c_(cb=None) == -1 and "Cb" in _err(lib)          # more than one entry: the chunk's own previous blocks
    assert c_(pc=None) == -1 and "prev_Cb" in _err(lib)
    # C128A takes no Cb / prev_Cb: with them absent, the call gets as far as the scale_pool check
    assert c_(ratio=128, cb=None, pc=None, n=256, sc=A) == -1 and "scale_pool must be NULL" in _err(lib)
    assert c_(ratio=128, cb=A, pc=None, n=256) == -1 and "Cb" in _err(lib)
    assert c_(od=2) == -1 and "scale_pool" in _err(lib)
    assert c_(n=3) == 0 and c_(n=3, p0=None, tbl=None, cb=None, pc=None) == 0   # fewer tokens than one block
    assert c_(B=0, p0=None, tbl=None, cb=None, pc=None) == 0
    # one entry reads prev_Cb only: without Cb the call gets as far as the scale_pool check
    assert c_(n=4, cb=None, od=2) == -1 and "scale_pool is NULL" in _err(lib)


def test_compress_paged_batch_layout_and_validation(lib, tmp_path):
    """csa_compress_paged_job as the binding lays it out matches the C
    compiler's layout, and the batch entry point validates every job."""
    import long_context_sparse_compress_amd as csa
    J = csa._CompressPagedJob
    if shutil.which("g++"):
        src = tmp_path / "pj.cpp"
        src.write_text('#include <cstddef>\n#include <cstdio>\n#include "csa.h"\n'
                       'int main(){printf("%zu %zu %zu %zu %zu\\n", sizeof(csa_compress_paged_job), '
                       'offsetof(csa_compress_paged_job, eps), offsetof(csa_compress_paged_job, pool), '
                       'offsetof(csa_compress_paged_job, max_blocks), offsetof(csa_compress_paged_job, rope_anchor));}\n')
        exe = tmp_path / "pj"
        r = subprocess.run(["g++", "-std=c++17", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        got = subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()
        assert [int(x) for x in got] == [ctypes.sizeof(J), J.eps.offset, J.pool.offset, J.max_blocks.offset,
                                         J.rope_anchor.offset]
    lib.csa_compress_paged_batch.argtypes = [ctypes.POINTER(J), ctypes.c_int, ctypes.c_void_p]

    def job(ratio=4, od=1, n=4, cb=None, pc=A, sc=None, c=512):
        j = J()
        j.ratio, j.B, j.n_tok, j.c, j.pos0 = ratio, 4, n, c, A
        j.Ca, j.Za, j.Cb, j.Zb, j.prev_Cb, j.prev_Zb = A, A, cb, cb, pc, pc
        j.bias, j.gamma, j.eps, j.in_dtype, j.out_dtype = A, None, 1e-6, 1, od
        j.pool, j.scale_pool, j.n_pool, j.block_table, j.max_blocks = A, sc, 10, A, 8
        j.rope_dims, j.rope_base, j.rope_anchor = 0, 10000.0, 0
        return j

    def call(*jobs, n=None):
        arr = (J * max(1, len(jobs)))(*jobs)
        return lib.csa_compress_paged_batch(arr, len(jobs) if n is None else n, None)

    # the pointers are fake: every call below must fail validation
    assert lib.csa_compress_paged_batch(None, 1, None) == -1 and "NULL" in _err(lib)
    assert call(job(), n=0) == -1 and "n_jobs" in _err(lib)
    assert call(job(), n=5) == -1 and "n_jobs" in _err(lib)
    assert call(job(), job(od=2)) == -1 and "job 1" in _err(lib) and "scale_pool" in _err(lib)
    assert call(job(), job(ratio=128, pc=None)) == -1 and "share ratio" in _err(lib)
    assert call(job(od=1), job(od=0, c=128)) == -1 and "share ratio" in _err(lib)   # two float output types
    assert call(job(n=-1)) == -1 and "job 0" in _err(lib)


@pytest.mark.skipif(shutil.which("g++") is None or os.environ.get("CSA_ABI_HOSTCHECK_LIB") is not None,
                    reason="no g++, or already inside the sanitized run")
def test_validation_under_sanitizers(tmp_path):
    """The C-ABI's host side -- capi.cpp and validate.h, with the kernel
    launchers replaced by host stubs (abi_host_stub.cpp) -- built with g++ under
    AddressSanitizer and UndefinedBehaviorSanitizer (any report aborts), then
    every argument-validation test of this file run against it in a child
    process."""
    so = tmp_path / "libcsa_hostcheck.so"
    csrc = os.path.join(ROOT, "long_context_sparse_compress_amd", "csrc")
    cmd = ["g++", "-std=c++17", "-shared", "-fPIC", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", csrc, "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined",
           "-o", str(so), os.path.join(csrc, "capi.cpp"), os.path.join(ROOT, "tests", "abi_host_stub.cpp")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ, CSA_ABI_HOSTCHECK_LIB=str(so), LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run(["python", "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py"), "-k", "validation or workspace_query"],
                       capture_output=True, text=True, env=env, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "passed" in r.stdout and "failed" not in r.stdout


def test_noalloc_validation(lib):
    """sparse_mqa_attn_noalloc: sparse_mqa_attn's argument checks, plus the
    static scratch's bound (host only: rejected calls make no HIP call)."""
    f = lib.sparse_mqa_attn_noalloc

    def call(B=32, T=1, N=16384, k=512, q0=65535, H=64, q=A, kv=A, idx=A, raw=A, rp0=65408, nraw=128, out=A,
             lse=None):
        return f(B, T, N, k, q0, H, 512, q, kv, idx, raw, rp0, nraw, 128, 0.0442, 1, out, lse, None)

    assert call(H=32) == -2
    assert call(idx=None) == -1 and "idx" in _err(lib)
    assert call(out=MIS) == -1
    assert call(k=2049) == -1
    assert call(nraw=64) == -1
    # B*T = 200: the split plan needs 2 x 200 partials of 66,048 bytes > 24 MiB
    assert call(B=200) == -4 and "static scratch" in _err(lib) and "26419200" in _err(lib)
    assert call(B=255) == -4
    assert call(B=0, q=None, kv=None, idx=None, raw=None, out=None) == 0      # nothing to do, no HIP call
