/*
 * csa.h -- C ABI of the MI355X (gfx950) compressed sparse attention library.
 *
 * Five entry points, one per stage of DeepSeek-V4's compressed sparse
 * attention (CSA) and heavily compressed attention (HCA) layer:
 *
 *   csa_compress      C4A / C128A KV compressor
 *   csa_compress_batch  several compressor calls of one ratio in one launch
 *   lightning_index_compressed  a decode step's compressor writes and the indexer in one call
 *   hca_attn_compressed  a decode step's C128A write and the HCA attention in one call
 *   topk_select_compressed  a decode step's compressor writes and Top-k in one call
 *   lightning_index   indexer scores  I[t,s] = sum_j w[t,j] * ReLU(q[t,j] . k[s])
 *   topk_select       causal Top-k over the indexer scores
 *   sparse_mqa_attn   shared-KV MQA over the Top-k entries plus the window
 *   hca_attn          dense shared-KV MQA over all C128A entries plus the
 *                     window, with an attention sink
 *
 * and, around them: csa_compress_ex / sparse_mqa_attn_ex / hca_attn_ex (the
 * same operations with partial RoPE fused in, and the batch-invariant
 * attention mode), csa_rope (partial RoPE on query or window rows), and
 * lightning_index_pool / topk_select_pool (the hierarchical indexer), and
 * csa_compress_paged / csa_compress_paged_chunk / csa_compress_paged_batch /
 * lightning_index_paged / topk_select_paged / sparse_mqa_attn_paged /
 * hca_attn_paged (the paged cache).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.     Every tensor pointer is device memory owned by the caller.  The
 *             library never allocates, frees or keeps caller memory; scratch
 *             space comes only from the caller's `workspace`.  Tensors are
 *             dense, row-major, innermost dimension last.  Every pointer must
 *             be 16-byte aligned.
 * Positions.  Token positions are absolute and 0-based.  A call's T query
 *             tokens are positions q_pos0 .. q_pos0+T-1 in every sequence of
 *             the batch.  Compressed entry s of ratio m covers raw tokens
 *             m*s .. m*s+m-1 and is visible to position t iff its whole
 *             block has arrived: s < V_m(t) = floor((t+1)/m).
 * Streams.    `stream` is a hipStream_t passed as void* (NULL = the null
 *             stream).  Calls are asynchronous: a return of CSA_OK means the
 *             arguments passed validation and the kernels were launched;
 *             a device-side fault shows up at the caller's synchronisation.
 * Errors.     Arguments are validated on the host before any HIP call.  A
 *             non-zero return leaves every output untouched, and
 *             csa_last_error() returns a message (thread-local, valid until
 *             the next call on the same thread).
 * Threads.    Entry points are thread-safe; concurrent calls on one stream
 *             are serialised by the stream.
 * Numerics.   Floating-point work is fp32 (bf16 MFMA products with fp32
 *             accumulation; fp8/MXFP4 MFMA products, which are exact, with
 *             fp32 accumulation).  bf16 outputs are rounded to nearest even.
 *             No fast-math reassociation of reductions across launches: the
 *             same inputs give bit-identical outputs on every run.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define CSA_OK               0
#define CSA_ERR_INVALID_ARG (-1)  /* null pointer, bad size, bad position, misalignment */
#define CSA_ERR_UNSUPPORTED (-2)  /* valid request this build does not implement       */
#define CSA_ERR_HIP         (-3)  /* a HIP call failed; the message holds its string    */
#define CSA_ERR_WORKSPACE   (-4)  /* workspace missing or smaller than required         */

/* ---- element types ---- */
#define CSA_F32       0  /* IEEE float32                                               */
#define CSA_BF16      1  /* bfloat16                                                   */
#define CSA_FP8_E4M3  2  /* OCP E4M3 (FN) byte codes, with one fp32 scale per 128-row */
#define CSA_MXFP4     3  /* OCP MX v1.0: E2M1 pairs per byte (even element in the low
                            nibble), one E8M0 scale byte per 32 elements               */

/* ---- operation ids for csa_workspace_bytes ---- */
#define CSA_OP_COMPRESS     0
#define CSA_OP_INDEX        1
#define CSA_OP_TOPK         2
#define CSA_OP_SPARSE_ATTN  3
#define CSA_OP_HCA_ATTN     4

/* Supported head shapes (the pages' configuration). */
#define CSA_HEADS        64   /* attention query heads                    */
#define CSA_HEAD_DIM    512   /* attention head dim = shared latent width */
#define CSA_INDEX_HEADS  64   /* indexer heads                            */
#define CSA_INDEX_DIM   128   /* indexer head dim                         */
#define CSA_MAX_TOPK   2048

/*
 * csa_compress -- stage 1, the KV compressor.
 *
 * Defined in "DeepSeek V4 结构速览" (核心设计; C4A Compressor) and the
 * compression formula of "DeepSeek-V4技术报告解读，全适配国产算力" (2.1):
 *  ratio 4 (C4A):   entry i pools 8 raw tokens -- the current block
 *                   4i..4i+3 (contents Ca, weight logits Za, bias rows 0..3)
 *                   and the previous block 4i-4..4i-1 (Cb, Zb, bias rows
 *                   4..7).  Per channel, p = softmax over the 8 rows of
 *                   (Z + bias); y = sum_r p[r] * C[r].  For the first block of
 *                   a sequence the previous block has zero content and
 *                   logit -inf.
 *  ratio 128 (C128A): entry i pools raw tokens 128i..128i+127 (Ca, Za, bias
 *                   rows 0..127) the same way.
 *  Then RMSNorm: out = y * rsqrt(mean_c(y^2) + eps) * gamma.
 *
 * The call pools the raw tokens pos0 .. pos0+n_tok-1 of each sequence;
 * pos0 must be a multiple of ratio.  It writes n_tok/ratio entries per
 * sequence (a trailing partial block produces nothing).
 *
 *  Ca, Za          [B, n_tok, c] in_dtype
 *  Cb, Zb          [B, n_tok, c] in_dtype; ratio 4 only, NULL for ratio 128
 *  prev_Cb/_Zb     [B, 4, c] in_dtype: raw tokens pos0-4..pos0-1 (the block
 *                  before the chunk).  Required iff ratio == 4 and pos0 > 0,
 *                  otherwise NULL.
 *  bias            [8, c] (ratio 4) or [128, c] (ratio 128) float32
 *  gamma           [c] float32, or NULL for ones
 *  eps             > 0 (finite)
 *  in_dtype        CSA_F32 or CSA_BF16;  out_dtype CSA_F32 or CSA_BF16
 *  out             entry i of sequence b at out + b*out_batch_stride + i*c
 *                  (elements); out_batch_stride 0 means (n_tok/ratio)*c.
 *                  This lets a decode step write straight into a cache slot.
 *  c               a multiple of 64, at most 1024.
 *  workspace / ws_bytes: optional device scratch (the caller owns it; its
 *                  contents need no initialisation and are not preserved).
 *                  With at least csa_workspace_bytes(CSA_OP_COMPRESS, B,
 *                  n_tok, c, ratio) bytes, a C128A call with few entries
 *                  spreads each entry's rows over several workgroups and
 *                  merges their partial states; with less (e.g. 0 and NULL)
 *                  every entry is pooled by one workgroup.  Same results up
 *                  to floating-point rounding order.
 */
int csa_compress(int ratio, int64_t B, int64_t n_tok, int64_t c, int64_t pos0,
                 const void* Ca, const void* Za, const void* Cb, const void* Zb,
                 const void* prev_Cb, const void* prev_Zb,
                 const float* bias, const float* gamma, float eps,
                 int in_dtype, int out_dtype, void* out, int64_t out_batch_stride,
                 void* workspace, size_t ws_bytes, void* stream);

/*
 * Partial RoPE, shared by the _ex entry points and csa_rope.
 *
 * "DeepSeek Technical Reports" (DeepSeek-V4, Hybrid Attention, CSA: position
 * is handled by a partial rotary embedding) and "DeepSeek V4 结构速览" (the
 * CSA operator graph): compressed entries get RoPE after their RMSNorm at an
 * anchor position, the query gets RoPE at its position, and the attention
 * output gets inverse RoPE on its last 64 dimensions.  The rotation is
 * RoFormer's: over the last R = rope_dims dimensions of a row, pair p =
 * (x[D-R+2p], x[D-R+2p+1]) turns by the angle pos * rope_base^(-2p/R):
 *   (x, y) -> (x cos a - y sin a, x sin a + y cos a);
 * the inverse turns by -a.  The pages give R = 64 and no base (10000 is
 * RoFormer's).  rope_dims is 0 (no RoPE) or a multiple of 8 up to the row
 * width; rope_base must be finite and > 1 when rope_dims > 0.  Angles are
 * formed and reduced in fp64, the rotation is fp32 before the output's
 * rounding.
 *
 * csa_compress_ex -- csa_compress, then partial RoPE on each entry.
 *
 * Entry i of the call (absolute entry pos0/ratio + i) is rotated at position
 * pos0 + ratio*i + rope_anchor.  The pages name the anchor position but its
 * symbol is lost in the text; the caller picks the offset inside the block,
 * 0 <= rope_anchor < ratio (0: the block's first raw token).  The row-split
 * C128A path (workspace given) applies it in its merge step.
 *
 * Quantize-on-write: out_dtype CSA_FP8_E4M3 (C4A only -- the indexer keys,
 * which "DeepSeek V4 结构速览" (Lightning Indexer) keeps in low precision)
 * writes each entry as E4M3 codes (OCP, round to nearest even, saturating)
 * of out / scale with scale = amax / 448 over the entry's channels (after
 * RMSNorm and RoPE; 1 for an all-zero entry), each step in fp32, and the
 * scale to out_scale: entry i of sequence b at out_scale[b * S + i] with S =
 * out_batch_stride / c (out_batch_stride a multiple of c), or n_tok/ratio
 * when out_batch_stride is 0 -- the byte codes and per-row scales
 * lightning_index reads as CSA_FP8_E4M3 keys.  out_scale is 4-byte aligned.
 *
 * out_dtype CSA_MXFP4 (C4A; "DeepSeek V4 结构速览", CSA operator graph: the
 * indexer scores in FP4) writes OCP MX v1.0 MXFP4 instead: per block of 32
 * channels the shared exponent E = floor(log2 amax) - 2 (E8M0 byte E + 127,
 * clipped to [0, 254]; 0 for an all-zero block) and the elements out * 2^-E
 * as E2M1 (nearest, ties to the even mantissa, clamped to 6; -0 written +0),
 * two per byte with the even channel in the low nibble: entry i of sequence b
 * at byte (b * out_batch_stride + i * c) / 2 of out, its c / 32 scale bytes
 * at out_scale[(b * S + i) * c / 32 ..] -- the packed keys and scales
 * lightning_index reads as CSA_MXFP4.
 *
 * out_scale is NULL for float output types.  Other arguments, rules and
 * errors are those of csa_compress; csa_compress is this call with out_scale
 * NULL and rope_dims 0.
 */
int csa_compress_ex(int ratio, int64_t B, int64_t n_tok, int64_t c, int64_t pos0,
                    const void* Ca, const void* Za, const void* Cb, const void* Zb,
                    const void* prev_Cb, const void* prev_Zb,
                    const float* bias, const float* gamma, float eps,
                    int in_dtype, int out_dtype, void* out, int64_t out_batch_stride,
                    void* out_scale, int rope_dims, float rope_base, int rope_anchor,
                    void* workspace, size_t ws_bytes, void* stream);

/*
 * csa_compress_batch -- several csa_compress calls in one launch.
 *
 * The same operation as csa_compress, for callers that compress more than
 * one stream of the same tokens at once (the CSA layer's 512-d latent and its
 * 128-d indexer keys both go through a C4A compressor).  Each job carries
 * exactly the arguments of csa_compress_ex (without workspace and stream) and
 * obeys the same rules; jobs of one batch must share ratio, in_dtype and
 * out_dtype, except that CSA_FP8_E4M3 jobs (quantize-on-write, C4A) may sit
 * (and CSA_MXFP4 jobs) beside jobs of one other output type -- the CSA
 * layer's bf16 latent and its quantized indexer key in one launch.  1 <= n_jobs <= 4.  Jobs with nothing to
 * write are skipped.
 * The row split that csa_compress's workspace enables is not used here.
 * Errors name the first offending job.
 */
typedef struct csa_compress_job {
  int ratio;
  int64_t B, n_tok, c, pos0;
  const void *Ca, *Za, *Cb, *Zb, *prev_Cb, *prev_Zb;
  const float* bias;
  const float* gamma;
  float eps;
  int in_dtype, out_dtype;
  void* out;
  int64_t out_batch_stride;
  int rope_dims;      /* csa_compress_ex's partial RoPE; 0 for none */
  float rope_base;
  int rope_anchor;
  void* out_scale;    /* csa_compress_ex's scales (fp8: fp32, MXFP4: E8M0); NULL for float outputs */
} csa_compress_job;

int csa_compress_batch(const csa_compress_job* jobs, int n_jobs, void* stream);

/*
 * lightning_index -- stage 2, the lightning indexer.
 *
 * Defined in "DeepSeek Technical Reports" (DSA, the indexer equation):
 *   I[t,s] = sum_{j<H_I} w[t,j] * ReLU(q[t,j] . k[s])   -- no scale factor.
 * "DeepSeek V4 结构速览" (Lightning Indexer): low-precision QK, ReLU, the
 * head-weighted sum, BF16 scores, causal range.  Scores of entries
 * s >= V_ratio(t) are written as -inf.
 *
 *  q        qk_dtype F32/BF16: [B, T, H_I, d_I];  FP8_E4M3: [B, T, H_I, d_I]
 *           codes;  MXFP4: [B, T, H_I, d_I/2] packed bytes
 *  q_scale  FP8_E4M3: [B, T, H_I] float32 (> 0);  MXFP4: [B, T, H_I, d_I/32]
 *           E8M0 bytes;  NULL otherwise
 *  w        [B, T, H_I] float32
 *  k        [B, N, d_I] (same encodings as q);  k_scale FP8: [B, N] float32,
 *           MXFP4: [B, N, d_I/32] bytes, NULL otherwise
 *  scores   [B, T, N] score_dtype (CSA_F32 or CSA_BF16)
 *  Requires H_I = 64, d_I = 128, ratio in {4, 128}, N >= V_ratio(q_pos0+T-1).
 *  qk_dtype CSA_F32 needs score_dtype CSA_F32.
 */
int lightning_index(int64_t B, int64_t T, int64_t N, int64_t q_pos0, int ratio,
                    int H_I, int d_I,
                    const void* q, const void* q_scale, const float* w,
                    const void* k, const void* k_scale, int qk_dtype,
                    void* scores, int score_dtype, void* stream);

/*
 * lightning_index_compressed -- a decode step's compressor writes, then the
 * lightning indexer, as one call.
 *
 * The same results as csa_compress_batch(jobs, n_jobs, stream) followed by
 * lightning_index(...) on the same stream: the step's new C4A entry
 * ("DeepSeek V4 结构速览", C4A Compressor: at decode the current block is
 * pooled with the previous one into the latest entry) is written into the
 * caches -- its 512-d latent and its indexer key, quantized on write -- and
 * the indexer ("DeepSeek V4 结构速览", Lightning Indexer) then scores every
 * visible key, the new one included.
 *
 * Arguments: those of lightning_index, then the jobs (the rules of
 * csa_compress_batch; n_jobs may be 0, then this is lightning_index), and
 * e_new, the key entry the jobs write (ignored when n_jobs is 0).  The jobs
 * must not write q, q_scale, w or scores; a job may write the keys only at
 * entry e_new.  With MXFP4 or bf16 keys, T = 1 and jobs that each write one entry per
 * sequence from bf16 rows (n_tok = 4, B as the indexer's, c <= 512, outputs
 * bf16, fp8 or MXFP4; any output inside k / k_scale being exactly entry e_new
 * of every sequence in their layout: MXFP4 codes and scales for MXFP4 keys,
 * bf16 for bf16 keys) the jobs run inside the indexer's launch,
 * in the workgroup that scores entry e_new of each sequence, before it reads
 * its keys; otherwise the call makes the two launches.  Errors: as
 * lightning_index and csa_compress_batch; e_new outside [0, N) with jobs is
 * CSA_ERR_INVALID_ARG.
 */
int lightning_index_compressed(int64_t B, int64_t T, int64_t N, int64_t q_pos0, int ratio,
                               int H_I, int d_I,
                               const void* q, const void* q_scale, const float* w,
                               const void* k, const void* k_scale, int qk_dtype,
                               void* scores, int score_dtype,
                               const csa_compress_job* jobs, int n_jobs, int64_t e_new, void* stream);

/*
 * topk_select -- stage 3, the causal Top-k selector.
 *
 * "DeepSeek Technical Reports" (DSA, the Top-k attention equation) and
 * "DeepSeek V4 结构速览" (核心设计; Lightning Indexer): each query row keeps
 * the k entries with the highest stored score among s < V_ratio(t).  Equal
 * scores go to the lower index; -0.0 equals +0.0.  When fewer than k entries
 * are visible all are kept.  Output row: the selected indices in ascending
 * order, then -1 in the remaining slots.  NaN scores are not supported.
 *
 *  scores  [B, T, N] score_dtype (CSA_F32 or CSA_BF16)
 *  idx     [B, T, k] int32
 *  workspace / ws_bytes: at least csa_workspace_bytes(CSA_OP_TOPK, B, T, N, k)
 *  bytes (may be 0, then workspace may be NULL).
 */
int topk_select(int64_t B, int64_t T, int64_t N, int64_t q_pos0, int ratio, int k,
                const void* scores, int score_dtype, int32_t* idx,
                void* workspace, size_t ws_bytes, void* stream);

/*
 * topk_select_compressed -- a decode step's compressor writes and Top-k as
 * one call.
 *
 * The results of csa_compress_batch(jobs, n_jobs, stream) followed by
 * topk_select(...) on the same stream.  Top-k reads only the scores, so a
 * write that no stage before the attention reads -- the step's new 512-d
 * latent entry ("DeepSeek V4 结构速览", C4A Compressor) -- can go here.
 * Arguments: those of topk_select, then the jobs (the rules of
 * csa_compress_batch; n_jobs may be 0, then this is topk_select).  The jobs
 * must not write the scores or idx.  With bf16 scores on the one-workgroup-a-
 * row path (rows of up to 40,960 candidates, N a multiple of 8) and C4A jobs
 * of one entry per sequence from bf16 rows (n_tok = 4, c <= 512), the jobs
 * run in spare workgroups of Top-k's launch; otherwise the call makes the two
 * launches.  Errors: as topk_select and csa_compress_batch.
 */
int topk_select_compressed(int64_t B, int64_t T, int64_t N, int64_t q_pos0, int ratio, int k,
                           const void* scores, int score_dtype, int32_t* idx,
                           void* workspace, size_t ws_bytes,
                           const csa_compress_job* jobs, int n_jobs, void* stream);

/*
 * lightning_index_pool / topk_select_pool -- the hierarchical sparse indexer.
 *
 * "DeepSeek Technical Reports" (DeepSeek-V4.1, CSA2: Cross-Layer KV and
 * Index Reuse; Hierarchical Sparse Indexer): a Full-indexer layer scans the whole context
 * (lightning_index + topk_select with a large k = P) and yields a candidate
 * pool per query; a later Reindex layer re-scores with its own query only the
 * pool's entries and takes its Top-k inside the pool; Reuse layers pass an
 * earlier layer's idx straight to sparse_mqa_attn (nothing to compute).
 *
 * lightning_index_pool:
 *   scores[b,t,j] = sum_h w[b,t,h] * ReLU(q[b,t,h] . k[b, pool[b,t,j]])
 * (the indexer equation of lightning_index, no scale), -inf where the slot is
 * empty: pool[b,t,j] < 0 or >= N (such slots read no key).  Visibility is the
 * pool's: a pool from topk_select holds visible entries only.
 *  q, k in qk_dtype, as lightning_index takes them: CSA_BF16 (q [B, T, 64,
 *  128], k [B, N, 128]); CSA_FP8_E4M3 (E4M3 codes, q_scale [B, T, 64] and
 *  k_scale [B, N] fp32 row scales); CSA_MXFP4 (packed E2M1 q [B, T, 64, 64]
 *  and k [B, N, 64], E8M0 q_scale [B, T, 64, 4] and k_scale [B, N, 4]) --
 *  the key precision of the indexer cache the pool came from ("DeepSeek V4
 *  结构速览", Lightning Indexer: FP4 QK).  q_scale, k_scale NULL for bf16.
 *  w [B, T, 64] float32;  pool [B, T, P] int32;  scores [B, T, P] float32 or
 *  bf16 (score_dtype).  0 <= P <= 65536.
 *
 * topk_select_pool: for each row, the k pool entries with the highest scores,
 * equal scores to the earlier slot; a slot is written as its entry id
 * pool[b,t,j], and as -1 when the slot is empty (-1 or >= N) or when the row
 * has fewer than k slots.  When pool rows list entry ids in ascending order
 * and then empty slots -- as topk_select writes them -- the earlier slot is
 * the lower id (the tie rule of topk_select) and idx is ascending entry ids,
 * then -1.  scores [B, T, P] (as lightning_index_pool writes them), pool
 * [B, T, P], idx [B, T, k] int32.  0 <= P <= 16384, 1 <= k <= 2048.  No
 * workspace.
 */
int lightning_index_pool(int64_t B, int64_t T, int64_t N, int64_t P, int H_I, int d_I,
                         const void* q, const void* q_scale, const float* w, const void* k,
                         const void* k_scale, int qk_dtype, const int32_t* pool, void* scores,
                         int score_dtype, void* stream);
int topk_select_pool(int64_t B, int64_t T, int64_t N, int64_t P, int k, const void* scores,
                     int score_dtype, const int32_t* pool, int32_t* idx, void* stream);

/*
 * sparse_mqa_attn -- stage 4, shared-KV MQA over Top-k entries + window.
 *
 * "DeepSeek V4 结构速览" (CSA（c4a 路线）) and "DeepSeek-V4 技术解读：百万
 * Token 上下文的新里程碑" (2.1): H query heads share one d-dim latent that is
 * both key and value.  Query t attends over the concatenation (no
 * de-duplication) of kv_cmp rows idx[t, :] and the raw window rows
 * max(0, t-window+1) .. t:
 *   o[t,h] = sum_x softmax_x(scale * q[t,h] . x) * x.
 * idx slots outside [0, N) (e.g. the -1 padding) contribute nothing.
 *
 *  q       [B, T, H, d] io_dtype;   kv_cmp [B, N, d] io_dtype
 *  idx     [B, T, k] int32
 *  kv_raw  [B, n_raw, d] io_dtype, raw positions raw_pos0 .. raw_pos0+n_raw-1;
 *          must cover every query's window.
 *  out     [B, T, H, d] io_dtype;  lse [B, T, H] float32 natural-log
 *          softmax denominators, or NULL.
 *  io_dtype CSA_F32 or CSA_BF16;  H = 64, d = 512, 1 <= window <= 4096.
 *  workspace: at least csa_workspace_bytes(CSA_OP_SPARSE_ATTN, B, T, N, k).
 */
int sparse_mqa_attn(int64_t B, int64_t T, int64_t N, int k, int64_t q_pos0, int H, int d,
                    const void* q, const void* kv_cmp, const int32_t* idx,
                    const void* kv_raw, int64_t raw_pos0, int64_t n_raw, int window,
                    float scale, int io_dtype, void* out, float* lse,
                    void* workspace, size_t ws_bytes, void* stream);

/*
 * hca_attn -- stage 5, HCA: dense shared-KV MQA with an attention sink.
 *
 * "DeepSeek V4 结构速览" (HCA（c128a 路线）): no indexer; every query attends
 * over all visible compressed entries s < V_ratio(t) and its raw window, with
 * an attention sink.  The sink is one logit sink[h] per head (not scaled)
 * with a zero value vector:
 *   o[t,h] = sum_x e^{l_x} x / (e^{sink[h]} + sum_x e^{l_x}),
 *   l_x = scale * q[t,h] . x.
 * sink == NULL means no sink (plain dense attention; with ratio 4 this is the
 * dense counterpart of sparse_mqa_attn).  lse includes the sink term.
 *
 *  q [B, T, H, d], kv_cmp [B, N, d], kv_raw [B, n_raw, d] io_dtype;
 *  sink [H] float32 or NULL;  out [B, T, H, d];  lse [B, T, H] or NULL.
 *  Requires N >= V_ratio(q_pos0+T-1).
 *  workspace: at least csa_workspace_bytes(CSA_OP_HCA_ATTN, B, T, N, 0).
 */
int hca_attn(int64_t B, int64_t T, int64_t N, int ratio, int64_t q_pos0, int H, int d,
             const void* q, const void* kv_cmp, const void* kv_raw, int64_t raw_pos0,
             int64_t n_raw, int window, float scale, const float* sink,
             int io_dtype, void* out, float* lse,
             void* workspace, size_t ws_bytes, void* stream);

/*
 * sparse_mqa_attn_ex / hca_attn_ex -- the same operations with a flags word
 * and the output's inverse RoPE.
 *
 * rope_dims > 0: each output row of query position t = q_pos0 + tq gets
 * inverse partial RoPE at t on its last rope_dims dimensions (the RoPE
 * convention above), after normalisation and before the output's rounding;
 * lse is unchanged.  q and the rows are taken as given: the caller rotates q
 * and the window rows (csa_rope) and the entries (csa_compress_ex).
 *
 * CSA_ATTN_BATCH_INVARIANT: "DeepSeek-V4 技术解读：百万 Token 上下文的新里程
 * 碑" (3.3) makes attention batch-invariant by giving up the split-KV
 * decomposition: one kernel has a single SM compute a whole sequence, a
 * second spreads a sequence over several SMs yet stays bit-identical to the
 * first.  With this flag a query's rows are never split: every output
 * element is computed by the same operations in the same order whatever B,
 * T and the other queries of the call, so a query gives the same bits alone
 * or in any batch (and run to run).  Calls with few queries spread each
 * query's four 16-head blocks over four workgroups, which yields the same
 * bits.  No workspace is used (workspace may be NULL, ws_bytes 0).  Without
 * the flag (flags 0) these are sparse_mqa_attn / hca_attn, whose decode split
 * (chosen from B * T) makes the last bits depend on the batch size.
 * Unknown flag bits are an error.
 */
#define CSA_ATTN_BATCH_INVARIANT 1
int sparse_mqa_attn_ex(int64_t B, int64_t T, int64_t N, int k, int64_t q_pos0, int H, int d,
                       const void* q, const void* kv_cmp, const int32_t* idx,
                       const void* kv_raw, int64_t raw_pos0, int64_t n_raw, int window,
                       float scale, int io_dtype, void* out, float* lse, int flags,
                       int rope_dims, float rope_base,
                       void* workspace, size_t ws_bytes, void* stream);
int hca_attn_ex(int64_t B, int64_t T, int64_t N, int ratio, int64_t q_pos0, int H, int d,
                const void* q, const void* kv_cmp, const void* kv_raw, int64_t raw_pos0,
                int64_t n_raw, int window, float scale, const float* sink,
                int io_dtype, void* out, float* lse, int flags,
                int rope_dims, float rope_base,
                void* workspace, size_t ws_bytes, void* stream);

/*
 * hca_attn_compressed -- a decode step's C128A write, then the HCA attention,
 * as one call.
 *
 * The results of csa_compress(job) followed by hca_attn_ex(...) on the same
 * stream: the step's new C128A entry ("DeepSeek V4 结构速览", HCA（c128a 路线）:
 * one entry pools 128 raw tokens; "DeepSeek-V4技术报告解读，全适配国产算力" 2.1,
 * the compression formula) is pooled into kv_cmp, and the dense attention
 * over every visible entry plus the window reads it.  Arguments: those of
 * hca_attn_ex, then one csa_compress_job (ratio 128; the rules of
 * csa_compress_batch) and e_new, the kv_cmp entry it writes.  With bf16 I/O,
 * T = 1, flags 0 and a job that writes one entry per sequence (n_tok = 128,
 * c = 512, bf16 in and out) exactly at entry e_new of kv_cmp (e_new visible to
 * the query, kv_cmp's layout) and touches nothing else the attention reads or
 * writes, the entry is pooled inside the attention's launch by the workgroup
 * whose tiles hold it, before it reads them; otherwise the call makes the
 * compressor's launch and the attention's.  The two routes may sum the
 * entry's row groups in a different order (differences at the rounding of the
 * entry's bf16 store).  The workspace is the attention's
 * (csa_workspace_bytes(CSA_OP_HCA_ATTN, ...)).  Errors: as hca_attn_ex and
 * csa_compress_batch; a job of another ratio, or e_new outside [0, N), is
 * CSA_ERR_INVALID_ARG.
 */
int hca_attn_compressed(int64_t B, int64_t T, int64_t N, int ratio, int64_t q_pos0, int H, int d,
                        const void* q, const void* kv_cmp, const void* kv_raw, int64_t raw_pos0,
                        int64_t n_raw, int window, float scale, const float* sink,
                        int io_dtype, void* out, float* lse, int flags,
                        int rope_dims, float rope_base, void* workspace, size_t ws_bytes,
                        const csa_compress_job* job, int64_t e_new, void* stream);

/*
 * sparse_mqa_attn_noalloc -- sparse_mqa_attn for callers that cannot
 * allocate: code under HIP graph capture, allocation-free serving loops, and
 * harnesses that forbid hipMalloc.
 *
 * The same operation, arguments, rules and results as sparse_mqa_attn with a
 * workspace (the same kernels and split plan, so the same bits), except that
 * the decode split's partials live in a static device scratch of 24 MiB that
 * the library holds on every GPU it runs on until the process ends, instead
 * of a caller workspace.  The call allocates nothing (no hipMalloc, no
 * allocating library routine).  The caller still passes every input and
 * output.  Calls whose split plan needs more than the scratch -- B*T between
 * 191 and 255 -- return CSA_ERR_WORKSPACE with a message naming the sizes
 * (use sparse_mqa_attn with a workspace there); B*T <= 190 and B*T >= 256
 * always fit.  All calls on one GPU share its scratch, which keeps the last
 * call's partials (nothing in it needs clearing: each call writes every
 * partial it reads): calls that overlap on one GPU, on any streams, race --
 * serialise them.  The first call on a device looks the scratch's address up
 * once with that device current; a failure there returns CSA_ERR_HIP.
 */
int sparse_mqa_attn_noalloc(int64_t B, int64_t T, int64_t N, int k, int64_t q_pos0, int H, int d,
                            const void* q, const void* kv_cmp, const int32_t* idx,
                            const void* kv_raw, int64_t raw_pos0, int64_t n_raw, int window,
                            float scale, int io_dtype, void* out, float* lse, void* stream);

/*
 * sparse_mqa_attn_paged / hca_attn_paged -- decode attention over the
 * heterogeneous KV cache.
 *
 * "DeepSeek-V4技术报告解读，全适配国产算力" (3.2): compressed entries live in a
 * classical paged cache, blocks of 128 raw tokens per request, and the
 * sliding-window KV in a per-request state cache.  One query per sequence,
 * each at its own position seq_pos[b] (a ragged batch).
 *  q          [B, 64, 512] (io_dtype)
 *  kv_pool    sparse: [n_pool, 32, 512] -- the 32 C4A entries of a block;
 *             hca:    [n_pool, 512]     -- its one C128A entry
 *  block_table [B, max_blocks] int32: physical block of each logical block
 *             (raw tokens 128j .. 128j+127) of sequence b; entry e of b is
 *             slot e % 32 (C4A) of block block_table[b][e / 32], or block
 *             block_table[b][e] (C128A).  Ids outside [0, n_pool) mark absent
 *             blocks: their entries are treated as padding and never read.
 *  idx        sparse: [B, k] int32 entry ids (as topk_select writes them, -1
 *             padding); entries past max_blocks' reach are padding too.
 *             hca: every entry e < floor((seq_pos[b] + 1) / 128) is attended.
 *  win        [B, ring, 512]: the window ring; raw position p of sequence b
 *             at row p % ring.  ring is a power of two >= window, and holds
 *             positions seq_pos[b] - window + 1 .. seq_pos[b] when called.
 *  seq_pos    [B] int64 query positions; max_pos >= every seq_pos[b] (a
 *             host-side bound that plans the decode split; a longer list is
 *             still computed in full, with longer splits).
 *  window, scale, sink, io_dtype, out [B, 64, 512], lse [B, 64], flags,
 *  rope_dims, rope_base, workspace: as sparse_mqa_attn_ex / hca_attn_ex with
 *  T = 1 (workspace per csa_workspace_bytes(op, B, 1, ...)).
 */
/*
 * csa_compress_paged -- the decode step's compressor write into the paged
 * cache: one block per sequence, each at its own position.
 *
 * "DeepSeek V4 结构速览" (C4A Compressor: at decode the previous block is the
 * latest complete block and the current block the rolling buffer) and
 * "DeepSeek-V4技术报告解读，全适配国产算力" (3.2, classical blocks of 128 raw
 * tokens).  Sequence b pools the block of raw tokens pos0[b] .. pos0[b] +
 * ratio - 1 exactly as csa_compress_ex does for a one-block chunk (RMSNorm,
 * optional RoPE at pos0[b] + rope_anchor, optional fp8 quantize-on-write) and
 * writes entry e = pos0[b] / ratio to slot e % 32 of block
 * block_table[b][e / 32] of pool [n_pool, 32, c] (C4A), or to block
 * block_table[b][e] of pool [n_pool, c] (C128A).  A sequence whose pos0 is
 * negative or not a multiple of ratio, or whose block is outside
 * [0, n_pool) or past max_blocks, writes nothing.
 *  pos0        [B] int64 (device)
 *  Ca, Za      [B, ratio, c] in_dtype: the rolling buffer (current block)
 *  prev_Cb/_Zb [B, 4, c] (C4A): the previous block's rows; not read for a
 *              sequence at pos0 0.  NULL for C128A.
 *  bias, gamma, eps, in_dtype, out_dtype, rope_*: as csa_compress_ex
 *              (pool rows of c / 2 bytes for CSA_MXFP4);
 *  scale_pool  [n_pool, 32] fp32 for CSA_FP8_E4M3 output, [n_pool, 32, c / 32]
 *              E8M0 bytes for CSA_MXFP4, else NULL.
 */
int csa_compress_paged(int ratio, int64_t B, int64_t c, const int64_t* pos0, const void* Ca,
                       const void* Za, const void* prev_Cb, const void* prev_Zb,
                       const float* bias, const float* gamma, float eps, int in_dtype,
                       int out_dtype, void* pool, void* scale_pool, int64_t n_pool,
                       const int32_t* block_table, int64_t max_blocks, int rope_dims,
                       float rope_base, int rope_anchor, void* stream);

/*
 * csa_compress_paged_chunk -- a chunk of raw tokens per sequence (chunked
 * prefill) compressed into the paged cache: the same operation as
 * csa_compress_ex over [B, n_tok, c] (C4A overlapping blocks, C128A
 * classical blocks), each sequence's chunk starting at its own block start
 * pos0[b], entry i of sequence b (e = pos0[b] / ratio + i) written to its
 * page row as csa_compress_paged writes e.  csa_compress_paged is the case
 * n_tok = ratio.  Pages: "DeepSeek V4 结构速览" (C4A Compressor) and
 * "DeepSeek-V4技术报告解读，全适配国产算力" (3.2: compressed entries live in
 * the classical cache, several blocks per request, while tokens not yet
 * compressed wait in the state cache).
 *  n_tok       raw tokens per sequence in the chunk; floor(n_tok / ratio)
 *              entries are written (at most 2^22); trailing tokens are ignored
 *  Ca, Za      [B, n_tok, c] in_dtype: the chunk's projections
 *  Cb, Zb      [B, n_tok, c] (C4A): previous-block projections of the
 *              chunk, read for entries i >= 1 (required when n_tok >= 8);
 *              NULL for C128A
 *  prev_Cb/_Zb [B, 4, c] (C4A): previous-block rows of the block before the
 *              chunk, read for entry 0 of a sequence at pos0 > 0
 *  the rest    as csa_compress_paged.  Entries whose block is absent
 *              (outside [0, n_pool) or past max_blocks) are skipped; a
 *              sequence whose pos0 is negative or not a multiple of ratio
 *              writes nothing.
 */
int csa_compress_paged_chunk(int ratio, int64_t B, int64_t n_tok, int64_t c, const int64_t* pos0,
                             const void* Ca, const void* Za, const void* Cb, const void* Zb,
                             const void* prev_Cb, const void* prev_Zb, const float* bias,
                             const float* gamma, float eps, int in_dtype, int out_dtype, void* pool,
                             void* scale_pool, int64_t n_pool, const int32_t* block_table,
                             int64_t max_blocks, int rope_dims, float rope_base, int rope_anchor,
                             void* stream);

/*
 * csa_compress_paged_batch -- several csa_compress_paged_chunk calls in one
 * launch.
 *
 * The same operation as csa_compress_paged_chunk, for callers that write
 * more than one compressed stream per step (the paged decode step's 512-d
 * latent and its 128-d indexer key): each job is exactly that call's
 * arguments (without stream), and the results are those of the separate
 * calls, bit for bit.  1 to 4 jobs, sharing ratio and in_dtype; their
 * out_dtype is one float type, or CSA_FP8_E4M3 / CSA_MXFP4 jobs (C4A) beside
 * jobs of one float type.  Errors: those of csa_compress_paged_chunk for each
 * job (the message names the job), CSA_ERR_INVALID_ARG for a NULL jobs, a job
 * count outside 1..4 or jobs that do not share ratio and dtypes.
 */
typedef struct csa_compress_paged_job {
  int ratio;
  int64_t B, n_tok, c;
  const int64_t* pos0;
  const void *Ca, *Za, *Cb, *Zb, *prev_Cb, *prev_Zb;
  const float* bias;
  const float* gamma;
  float eps;
  int in_dtype, out_dtype;
  void* pool;
  void* scale_pool;
  int64_t n_pool;
  const int32_t* block_table;
  int64_t max_blocks;
  int rope_dims;
  float rope_base;
  int rope_anchor;
} csa_compress_paged_job;

int csa_compress_paged_batch(const csa_compress_paged_job* jobs, int n_jobs, void* stream);

/*
 * lightning_index_paged / topk_select_paged -- the decode indexer and Top-k
 * over the heterogeneous cache (the same operations as lightning_index and
 * topk_select with T = 1 and one position per sequence).
 *
 * lightning_index_paged: scores[b, e] of entry e of sequence b, index keys in
 * k_pool [n_pool, 32, 128] (bf16; E4M3 codes with k_scale [n_pool, 32]
 * fp32; or MXFP4 [n_pool, 32, 64] packed E2M1 with k_scale [n_pool, 32, 4]
 * E8M0 -- what the quantize-on-write compressors produce), entry e at slot
 * e % 32 of block block_table[b][e / 32] (ids outside [0, n_pool) read block
 * 0: the blocks holding a sequence's visible entries must be mapped).
 * q [B, 64, 128] (bf16; E4M3 with q_scale [B, 64]; or MXFP4 [B, 64, 64] with
 * q_scale [B, 64, 4]), w [B, 64]; scores [B, 32 * max_blocks]: -inf for
 * e >= floor((seq_pos[b] + 1) / 4).  qk_dtype CSA_BF16, CSA_FP8_E4M3 or
 * CSA_MXFP4 ("DeepSeek V4 结构速览", Lightning Indexer: the Pro model's QK
 * path runs in FP4); n_pool >= 1.
 *
 * topk_select_paged: topk_select's selection over scores [B, N] where row b's
 * candidates are e < min(N, floor((seq_pos[b] + 1) / ratio)); idx [B, k],
 * ascending then -1.  Workspace as csa_workspace_bytes(CSA_OP_TOPK, B, 1, N, k).
 */
int lightning_index_paged(int64_t B, int64_t max_blocks, int H_I, int d_I, const void* q,
                          const void* q_scale, const float* w, const void* k_pool,
                          const void* k_scale, int64_t n_pool, const int32_t* block_table,
                          const int64_t* seq_pos, int qk_dtype, void* scores, int score_dtype,
                          void* stream);
int topk_select_paged(int64_t B, int64_t N, const int64_t* seq_pos, int ratio, int k,
                      const void* scores, int score_dtype, int32_t* idx, void* workspace,
                      size_t ws_bytes, void* stream);

int sparse_mqa_attn_paged(int64_t B, int k, int H, int d, const void* q, const void* kv_pool,
                          int64_t n_pool, const int32_t* block_table, int64_t max_blocks,
                          const int32_t* idx, const void* win, int64_t ring, const int64_t* seq_pos,
                          int64_t max_pos, int window, float scale, int io_dtype, void* out,
                          float* lse, int flags, int rope_dims, float rope_base, void* workspace,
                          size_t ws_bytes, void* stream);
int hca_attn_paged(int64_t B, int H, int d, const void* q, const void* kv_pool, int64_t n_pool,
                   const int32_t* block_table, int64_t max_blocks, const void* win, int64_t ring,
                   const int64_t* seq_pos, int64_t max_pos, int window, float scale,
                   const float* sink, int io_dtype, void* out, float* lse, int flags,
                   int rope_dims, float rope_base, void* workspace, size_t ws_bytes, void* stream);

/*
 * csa_rope -- partial RoPE (or its inverse) in place on rows of a tensor.
 *
 * "DeepSeek Technical Reports" (Hybrid Attention, CSA: partial RoPE) and
 * "DeepSeek V4 结构速览" (the CSA operator graph: the query is rotated at its position, and so is each raw
 * latent of the sliding window, whose rows are the keys and values of the
 * window).  x is [B, T, H, D] of dtype (CSA_F32 or CSA_BF16), dense; row
 * (b, t, h) sits at position pos0 + t and its last rope_dims dimensions are
 * rotated by the RoPE convention above (by -angle when inverse = 1).  Use H =
 * 1 for [B, T, D] rows.  D is a multiple of 8 up to 65536; rope_dims is a
 * multiple of 8 in [8, min(D, 1024)]; 0 <= pos0 <= 2^40; B * T < 2^31,
 * H <= 2^24.  The first D - rope_dims dimensions are not read or written.
 */
int csa_rope(int64_t B, int64_t T, int64_t H, int64_t D, int64_t pos0, int rope_dims,
             float rope_base, int inverse, int dtype, void* x, void* stream);

/* Workspace bytes the named operation needs for these sizes (0 if none).
 * For the two attention operations the need depends only on B and T; N and
 * k are accepted for symmetry.  For CSA_OP_COMPRESS the arguments are
 * (B, n_tok, c, ratio) and the figure is what enables the row split.
 * Returns 0 for an unknown op. */
size_t csa_workspace_bytes(int op, int64_t B, int64_t T, int64_t N, int k);

/* Message for the last non-OK return on this thread ("" if none). */
const char* csa_last_error(void);

/* Library version string. */
const char* csa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H_ */
