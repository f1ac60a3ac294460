"""CPU oracle for DeepSeek-V4 compressed sparse attention (CSA / HCA).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import or call anything in this package.
The product path (the HIP library and its Python binding) never does, and
shares no code with it.

Every function is a plain, slow, direct transcription of what the pages
define, evaluated in float64 with NumPy.  A library primitive (matmul, exp,
sort) is used as a step; there is no blocking, fusion, streaming or
reordering beyond what the definitions state.  Quantized inputs (fp8 E4M3
with a row scale, MXFP4) are decoded exactly from their bytes first.

Pages and the parts each module follows:

* ``compressor`` -- "DeepSeek V4 结构速览" (核心设计; C4A Compressor) and
  "DeepSeek-V4技术报告解读，全适配国产算力" (2.1, the compression formula).
* ``indexer`` -- "DeepSeek Technical Reports" (DSA, the lightning-indexer
  equation) and "DeepSeek V4 结构速览" (Lightning Indexer).
* ``topk`` -- "DeepSeek Technical Reports" (DSA, the Top-k attention
  equation) and "DeepSeek V4 结构速览" (核心设计; Lightning Indexer).
* ``attention`` -- "DeepSeek V4 结构速览" (CSA（c4a 路线）; HCA（c128a 路线）)
  and "DeepSeek-V4 技术解读：百万 Token 上下文的新里程碑" (2.1, shared-KV MQA).
* ``kv_accounting`` -- "DeepSeek V4 结构速览" (KV cache 账).
* ``cache`` -- "DeepSeek-V4技术报告解读，全适配国产算力" (3.2, the heterogeneous
  KV cache: paged classical cache, per-request state cache).
* ``rope`` -- "DeepSeek Technical Reports" (DeepSeek-V4, Hybrid Attention,
  CSA: the Partial Rotary Positional Embedding section is named there) and
  "DeepSeek V4 结构速览" (the CSA operator graph; RoPE anchors of the compressor; inverse RoPE on the output).
* ``numerics`` -- decoding of the quantized inputs and bf16 score storage.

Parity status: every function is pinned by the CPU tests against closed forms,
library routines, brute force or values the pages print.  The conventions the
pages leave open (which block is "a", bias row order, the block-0 fill, the
RMSNorm eps, no indexer scale, the sink semantics) are readings that no page
value fixes; they are listed with each function.
"""
from . import attention, cache, compressor, indexer, kv_accounting, numerics, rope, topk  # noqa: F401
