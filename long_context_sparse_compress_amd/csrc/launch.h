// Internal launcher interface between the C ABI (capi.cpp) and the kernels.
// Arguments arrive here already validated by validate.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/csa.h"

namespace csa {

struct CompressArgs {
  int ratio;
  int64_t B, n_tok, c, pos0;
  const void *Ca, *Za, *Cb, *Zb, *prev_Cb, *prev_Zb;
  const float* bias;
  const float* gamma;
  float eps;
  int in_dtype, out_dtype;
  void* out;
  int64_t out_batch_stride;
  void* ws;          // optional row-split workspace
  size_t ws_bytes;
  int rope_dims;     // partial RoPE on the last rope_dims channels (0: none)
  float rope_base;
  int rope_anchor;   // entry i's position: pos0 + ratio * i + rope_anchor
  void* out_scale;   // fp8: fp32 scale of entry i of sequence b at [b * (stride / c) + i]; fp4: E8M0 bytes, c / 32 per entry
};

// The decode write of one block per sequence into the paged cache.
struct CompressPagedArgs {
  int ratio;
  int64_t B, c;
  const int64_t* pos0;          // [B] chunk start of each sequence (a block start)
  int64_t n_tok;                // raw tokens per sequence in the chunk (ratio at decode)
  const void *Ca, *Za;          // [B, n_tok, c]: the chunk (at decode the rolling buffer)
  const void *Cb, *Zb;          // [B, n_tok, c]: previous-block projections of the chunk (C4A, entries >= 1)
  const void *prev_Cb, *prev_Zb;  // [B, 4, c]: the block before the chunk (C4A)
  const float* bias;
  const float* gamma;
  float eps;
  int in_dtype, out_dtype;
  void* pool;                   // [n_pool, 32, c] (C4A) or [n_pool, c] (C128A)
  void* scale_pool;             // fp8: [n_pool, 32] fp32; fp4: [n_pool, 32, c / 32] E8M0
  int64_t n_pool;
  const int32_t* block_table;   // [B, max_blocks]
  int64_t max_blocks;
  int rope_dims;
  float rope_base;
  int rope_anchor;
};

struct IndexArgs {
  int64_t B, T, N, q_pos0;
  int ratio;
  const void* q;
  const void* q_scale;
  const float* w;
  const void* k;
  const void* k_scale;
  int qk_dtype;
  void* scores;
  int score_dtype;
  // paged decode keys (NULL otherwise): k is a pool of 32-entry blocks
  const int32_t* block_table = nullptr;
  int64_t max_blocks = 0, n_pool = 0;
  const int64_t* seq_pos = nullptr;
};

struct TopkArgs {
  int64_t B, T, N, q_pos0;
  int ratio, k;
  const void* scores;
  int score_dtype;
  int32_t* idx;
  void* ws;
  const int32_t* pool;   // pool mode: a selected slot j is written as pool[row][j] (-1 if outside 0..n_ent-1)
  int64_t n_ent;
  const int64_t* seq_pos = nullptr;   // ragged decode: row b's position (T = 1)
};

struct IndexPoolArgs {
  int64_t B, T, N, P;
  const void* q;         // [B, T, 64, 128] in qk_dtype
  const void* q_scale;   // fp8: [B, T, 64] fp32; MXFP4: [B, T, 64, 4] E8M0; else NULL
  const float* w;        // [B, T, 64]
  const void* k;         // [B, N, 128] in qk_dtype
  const void* k_scale;   // fp8: [B, N] fp32; MXFP4: [B, N, 4] E8M0; else NULL
  int qk_dtype;
  const int32_t* pool;   // [B, T, P]
  void* scores;          // [B, T, P]
  int score_dtype;
};

struct AttnArgs {
  int64_t B, T, N;
  int k;              // top-k slots per query (sparse); 0 for dense
  int ratio;          // dense: compressed entries visible are s < (t+1)/ratio
  int64_t q_pos0;
  const void* q;
  const void* kv_cmp;
  const int32_t* idx; // NULL for dense
  const void* kv_raw;
  int64_t raw_pos0, n_raw;
  int window;
  float scale;
  const float* sink;  // dense only, may be NULL
  int io_dtype;
  void* out;
  float* lse;
  void* ws;
  int flags;          // CSA_ATTN_* bits
  int rope_dims;      // inverse RoPE on the output's last rope_dims dims (0: none)
  float rope_base;
  // paged decode (all zero / NULL otherwise): see Params in attention.hip
  const int32_t* block_table = nullptr;
  int64_t max_blocks = 0, n_pool = 0;
  int page_shift = 0;
  int64_t ring = 0;
  const int64_t* seq_pos = nullptr;
  int64_t max_pos = 0;
};

struct RopeArgs {
  int64_t B, T, H, D, pos0;
  int dims;
  float base;
  int inverse;
  int dtype;
  void* x;
};

hipError_t launch_compress(const CompressArgs& a, hipStream_t s);
// up to 4 jobs of one ratio and dtype pair, one launch
hipError_t launch_compress_batch(const CompressArgs* jobs, int n, hipStream_t s);
hipError_t launch_compress_paged(const CompressPagedArgs* jobs, int n, hipStream_t s);   // 1..4 jobs
hipError_t launch_index(const IndexArgs& a, hipStream_t s);
// The compressor jobs (1..4), then the indexer: in one launch where the
// indexer's decode kernel can run them (MXFP4 or bf16 keys, one query a
// sequence, one-entry bf16 jobs whose writes into the keys are entry e_new), else as a
// compressor launch followed by the indexer's.  Same results either way.
hipError_t launch_index_jobs(const IndexArgs& a, const CompressArgs* jobs, int n, int64_t e_new, hipStream_t s);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
// The compressor jobs (1..4, one entry a sequence), then Top-k: in one launch
// where the register kernel applies (the jobs in spare workgroups), else as a
// compressor launch followed by Top-k's.  Same results either way.
hipError_t launch_topk_jobs(const TopkArgs& a, const CompressArgs* jobs, int n, hipStream_t s);
hipError_t launch_index_pool(const IndexPoolArgs& a, hipStream_t s);
hipError_t launch_attn(const AttnArgs& a, hipStream_t s);
// A dense decode's C128A write (one entry a sequence, at entry e_new of
// kv_cmp), then the attention: one launch where the attention's decode plan
// allows, else the compressor's launch and the attention's.  The entry's
// pooling may sum its row groups in another order on the two routes.
hipError_t launch_attn_jobs(const AttnArgs& a, const CompressArgs& job, int64_t e_new, hipStream_t s);
// Device address, on the current device, of the attention kernels' static
// scratch (kAttnStaticScratchBytes bytes); looked up once per device.
hipError_t attn_static_scratch(void** ptr);
hipError_t launch_rope(const RopeArgs& a, hipStream_t s);

}  // namespace csa
