// The extern "C" entry points declared in include/csa.h: validate on the
// host (validate.h), then hand the arguments to the kernel launchers.
#include <hip/hip_runtime.h>

#include <string>

#include "../../include/csa.h"
#include "launch.h"
#include "validate.h"

namespace {

thread_local std::string g_last_error;

int finish(const csa::Check& c) {
  g_last_error = c.msg;
  return c.code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) {
    g_last_error.clear();
    return CSA_OK;
  }
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return CSA_ERR_HIP;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int csa_compress_ex(int ratio, int64_t B, int64_t n_tok, int64_t c, int64_t pos0, const void* Ca,
                    const void* Za, const void* Cb, const void* Zb, const void* prev_Cb,
                    const void* prev_Zb, const float* bias, const float* gamma, float eps, int in_dtype,
                    int out_dtype, void* out, int64_t out_batch_stride, void* out_scale, int rope_dims,
                    float rope_base, int rope_anchor, void* workspace, size_t ws_bytes, void* stream) {
  csa::Check ck = csa::check_compress(ratio, B, n_tok, c, pos0, Ca, Za, Cb, Zb, prev_Cb, prev_Zb, bias,
                                      gamma, eps, in_dtype, out_dtype, out, out_batch_stride, workspace, ws_bytes,
                                      rope_dims, rope_base, rope_anchor, out_scale);
  if (!ck.ok()) return finish(ck);
  csa::CompressArgs a{ratio, B, n_tok, c, pos0, Ca, Za, Cb, Zb, prev_Cb, prev_Zb,
                      bias, gamma, eps, in_dtype, out_dtype, out, out_batch_stride, workspace, ws_bytes,
                      rope_dims, rope_base, rope_anchor, out_scale};
  return hip_status(csa::launch_compress(a, as_stream(stream)), "csa_compress launch");
}

int csa_compress(int ratio, int64_t B, int64_t n_tok, int64_t c, int64_t pos0, const void* Ca,
                 const void* Za, const void* Cb, const void* Zb, const void* prev_Cb,
                 const void* prev_Zb, const float* bias, const float* gamma, float eps, int in_dtype,
                 int out_dtype, void* out, int64_t out_batch_stride, void* workspace, size_t ws_bytes,
                 void* stream) {
  return csa_compress_ex(ratio, B, n_tok, c, pos0, Ca, Za, Cb, Zb, prev_Cb, prev_Zb, bias, gamma, eps, in_dtype,
                         out_dtype, out, out_batch_stride, nullptr, 0, 0.f, 0, workspace, ws_bytes, stream);
}

namespace {

// The rules of csa_compress_batch for 1..4 jobs; the jobs' launch arguments
// go to `a`.
csa::Check check_jobs(const csa_compress_job* jobs, int n_jobs, csa::CompressArgs* a) {
  csa::Check ck;
  if (!jobs) ck.fail(CSA_ERR_INVALID_ARG, "jobs is NULL");
  else if (n_jobs < 1 || n_jobs > 4) ck.fail(CSA_ERR_INVALID_ARG, "n_jobs must be 1..4, got " + csa::i2s(n_jobs));
  if (!ck.ok()) return ck;
  for (int q = 0; q < n_jobs; ++q) {
    const csa_compress_job& j = jobs[q];
    csa::Check cj = csa::check_compress(j.ratio, j.B, j.n_tok, j.c, j.pos0, j.Ca, j.Za, j.Cb, j.Zb, j.prev_Cb,
                                        j.prev_Zb, j.bias, j.gamma, j.eps, j.in_dtype, j.out_dtype, j.out,
                                        j.out_batch_stride, nullptr, 0, j.rope_dims, j.rope_base, j.rope_anchor,
                                        j.out_scale);
    // quantized jobs (quantize-on-write, C4A) may sit beside jobs of one float output type
    auto quant = [](int dt) { return dt == CSA_FP8_E4M3 || dt == CSA_MXFP4; };
    bool same_out = true;
    for (int p = 0; p < q; ++p)
      if (jobs[p].out_dtype != j.out_dtype && !quant(jobs[p].out_dtype) && !quant(j.out_dtype)) same_out = false;
    if (cj.ok() && (j.ratio != jobs[0].ratio || j.in_dtype != jobs[0].in_dtype || !same_out))
      cj.fail(CSA_ERR_INVALID_ARG, "jobs of one batch must share ratio, in_dtype and out_dtype (fp8 jobs may join "
                                   "jobs of one other output type)");
    if (!cj.ok()) {
      cj.msg = "job " + csa::i2s(q) + ": " + cj.msg;
      return cj;
    }
    a[q] = csa::CompressArgs{j.ratio, j.B, j.n_tok, j.c, j.pos0, j.Ca, j.Za, j.Cb, j.Zb, j.prev_Cb, j.prev_Zb,
                             j.bias, j.gamma, j.eps, j.in_dtype, j.out_dtype, j.out, j.out_batch_stride, nullptr, 0,
                             j.rope_dims, j.rope_base, j.rope_anchor, j.out_scale};
  }
  return ck;
}

}  // namespace

int csa_compress_batch(const csa_compress_job* jobs, int n_jobs, void* stream) {
  csa::CompressArgs a[4];
  const csa::Check ck = check_jobs(jobs, n_jobs, a);
  if (!ck.ok()) return finish(ck);
  return hip_status(csa::launch_compress_batch(a, n_jobs, as_stream(stream)), "csa_compress_batch launch");
}

int lightning_index_compressed(int64_t B, int64_t T, int64_t N, int64_t q_pos0, int ratio, int H_I, int d_I,
                               const void* q, const void* q_scale, const float* w, const void* k,
                               const void* k_scale, int qk_dtype, void* scores, int score_dtype,
                               const csa_compress_job* jobs, int n_jobs, int64_t e_new, void* stream) {
  csa::Check ck = csa::check_index(B, T, N, q_pos0, ratio, H_I, d_I, q, q_scale, w, k, k_scale, qk_dtype,
                                   scores, score_dtype);
  if (!ck.ok()) return finish(ck);
  csa::CompressArgs a[4];
  if (n_jobs != 0) {
    ck = check_jobs(jobs, n_jobs, a);
    if (!ck.ok()) return finish(ck);
  }
  if (n_jobs != 0 && (e_new < 0 || e_new >= N)) {
    ck.fail(CSA_ERR_INVALID_ARG, "e_new must lie in [0, N), got " + csa::i2s(e_new));
    return finish(ck);
  }
  csa::IndexArgs ia{B, T, N, q_pos0, ratio, q, q_scale, w, k, k_scale, qk_dtype, scores, score_dtype};
  return hip_status(csa::launch_index_jobs(ia, a, n_jobs, e_new, as_stream(stream)),
                    "lightning_index_compressed launch");
}

int lightning_index(int64_t B, int64_t T, int64_t N, int64_t q_pos0, int ratio, int H_I, int d_I,
                    const void* q, const void* q_scale, const float* w, const void* k,
                    const void* k_scale, int qk_dtype, void* scores, int score_dtype, void* stream) {
  csa::Check ck = csa::check_index(B, T, N, q_pos0, ratio, H_I, d_I, q, q_scale, w, k, k_scale, qk_dtype,
                                   scores, score_dtype);
  if (!ck.ok()) return finish(ck);
  csa::IndexArgs a{B, T, N, q_pos0, ratio, q, q_scale, w, k, k_scale, qk_dtype, scores, score_dtype};
  return hip_status(csa::launch_index(a, as_stream(stream)), "lightning_index launch");
}

int topk_select(int64_t B, int64_t T, int64_t N, int64_t q_pos0, int ratio, int k, const void* scores,
                int score_dtype, int32_t* idx, void* workspace, size_t ws_bytes, void* stream) {
  csa::Check ck = csa::check_topk(B, T, N, q_pos0, ratio, k, scores, score_dtype, idx, workspace, ws_bytes);
  if (!ck.ok()) return finish(ck);
  csa::TopkArgs a{B, T, N, q_pos0, ratio, k, scores, score_dtype, idx, workspace, nullptr, 0};
  return hip_status(csa::launch_topk(a, as_stream(stream)), "topk_select launch");
}

int topk_select_compressed(int64_t B, int64_t T, int64_t N, int64_t q_pos0, int ratio, int k, const void* scores,
                           int score_dtype, int32_t* idx, void* workspace, size_t ws_bytes,
                           const csa_compress_job* jobs, int n_jobs, void* stream) {
  csa::Check ck = csa::check_topk(B, T, N, q_pos0, ratio, k, scores, score_dtype, idx, workspace, ws_bytes);
  if (!ck.ok()) return finish(ck);
  csa::CompressArgs a[4];
  if (n_jobs != 0) {
    ck = check_jobs(jobs, n_jobs, a);
    if (!ck.ok()) return finish(ck);
  }
  csa::TopkArgs ta{B, T, N, q_pos0, ratio, k, scores, score_dtype, idx, workspace, nullptr, 0};
  return hip_status(csa::launch_topk_jobs(ta, a, n_jobs, as_stream(stream)), "topk_select_compressed launch");
}

int lightning_index_pool(int64_t B, int64_t T, int64_t N, int64_t P, int H_I, int d_I, const void* q,
                         const void* q_scale, const float* w, const void* k, const void* k_scale, int qk_dtype,
                         const int32_t* pool, void* scores, int score_dtype, void* stream) {
  csa::Check ck = csa::check_index_pool(B, T, N, P, H_I, d_I, q, q_scale, w, k, k_scale, qk_dtype, pool, scores,
                                        score_dtype);
  if (!ck.ok()) return finish(ck);
  csa::IndexPoolArgs a{B, T, N, P, q, q_scale, w, k, k_scale, qk_dtype, pool, scores, score_dtype};
  return hip_status(csa::launch_index_pool(a, as_stream(stream)), "lightning_index_pool launch");
}

int topk_select_pool(int64_t B, int64_t T, int64_t N, int64_t P, int k, const void* scores, int score_dtype,
                     const int32_t* pool, int32_t* idx, void* stream) {
  csa::Check ck = csa::check_topk_pool(B, T, N, P, k, scores, score_dtype, pool, idx);
  if (!ck.ok()) return finish(ck);
  // every slot of a row is a candidate (ratio 1, positions past the row):
  // the register / LDS selection over P slots, each selected slot written as
  // its pool entry
  csa::TopkArgs a{B, T, P, P, 1, k, scores, score_dtype, idx, nullptr, pool, N};
  return hip_status(csa::launch_topk(a, as_stream(stream)), "topk_select_pool launch");
}

int sparse_mqa_attn_ex(int64_t B, int64_t T, int64_t N, int k, int64_t q_pos0, int H, int d, const void* q,
                       const void* kv_cmp, const int32_t* idx, const void* kv_raw, int64_t raw_pos0,
                       int64_t n_raw, int window, float scale, int io_dtype, void* out, float* lse, int flags,
                       int rope_dims, float rope_base, void* workspace, size_t ws_bytes, void* stream) {
  csa::Check ck = csa::check_sparse(B, T, N, k, q_pos0, H, d, q, kv_cmp, idx, kv_raw, raw_pos0, n_raw,
                                    window, scale, io_dtype, out, lse, workspace, ws_bytes, flags, rope_dims,
                                    rope_base);
  if (!ck.ok()) return finish(ck);
  csa::AttnArgs a{B, T, N, k, 4, q_pos0, q, kv_cmp, idx, kv_raw, raw_pos0, n_raw, window, scale,
                  nullptr, io_dtype, out, lse, workspace, flags, rope_dims, rope_base};
  return hip_status(csa::launch_attn(a, as_stream(stream)), "sparse_mqa_attn launch");
}

int sparse_mqa_attn(int64_t B, int64_t T, int64_t N, int k, int64_t q_pos0, int H, int d, const void* q,
                    const void* kv_cmp, const int32_t* idx, const void* kv_raw, int64_t raw_pos0,
                    int64_t n_raw, int window, float scale, int io_dtype, void* out, float* lse,
                    void* workspace, size_t ws_bytes, void* stream) {
  return sparse_mqa_attn_ex(B, T, N, k, q_pos0, H, d, q, kv_cmp, idx, kv_raw, raw_pos0, n_raw, window, scale,
                            io_dtype, out, lse, 0, 0, 0.f, workspace, ws_bytes, stream);
}

int sparse_mqa_attn_noalloc(int64_t B, int64_t T, int64_t N, int k, int64_t q_pos0, int H, int d, const void* q,
                            const void* kv_cmp, const int32_t* idx, const void* kv_raw, int64_t raw_pos0,
                            int64_t n_raw, int window, float scale, int io_dtype, void* out, float* lse,
                            void* stream) {
  csa::Check ck = csa::check_sparse_noalloc(B, T, N, k, q_pos0, H, d, q, kv_cmp, idx, kv_raw, raw_pos0, n_raw,
                                            window, scale, io_dtype, out, lse);
  if (!ck.ok()) return finish(ck);
  if (B == 0 || T == 0) return finish(ck);
  void* ws = nullptr;
  const hipError_t e = csa::attn_static_scratch(&ws);
  if (e != hipSuccess) return hip_status(e, "sparse_mqa_attn_noalloc scratch lookup");
  csa::AttnArgs a{B, T, N, k, 4, q_pos0, q, kv_cmp, idx, kv_raw, raw_pos0, n_raw, window, scale,
                  nullptr, io_dtype, out, lse, ws, 0, 0, 0.f};
  return hip_status(csa::launch_attn(a, as_stream(stream)), "sparse_mqa_attn_noalloc launch");
}

int hca_attn_ex(int64_t B, int64_t T, int64_t N, int ratio, int64_t q_pos0, int H, int d, const void* q,
                const void* kv_cmp, const void* kv_raw, int64_t raw_pos0, int64_t n_raw, int window,
                float scale, const float* sink, int io_dtype, void* out, float* lse, int flags, int rope_dims,
                float rope_base, void* workspace, size_t ws_bytes, void* stream) {
  csa::Check ck = csa::check_hca(B, T, N, ratio, q_pos0, H, d, q, kv_cmp, kv_raw, raw_pos0, n_raw, window,
                                 scale, sink, io_dtype, out, lse, workspace, ws_bytes, flags, rope_dims, rope_base);
  if (!ck.ok()) return finish(ck);
  csa::AttnArgs a{B, T, N, 0, ratio, q_pos0, q, kv_cmp, nullptr, kv_raw, raw_pos0, n_raw, window, scale,
                  sink, io_dtype, out, lse, workspace, flags, rope_dims, rope_base};
  return hip_status(csa::launch_attn(a, as_stream(stream)), "hca_attn launch");
}

int hca_attn_compressed(int64_t B, int64_t T, int64_t N, int ratio, int64_t q_pos0, int H, int d, const void* q,
                        const void* kv_cmp, const void* kv_raw, int64_t raw_pos0, int64_t n_raw, int window,
                        float scale, const float* sink, int io_dtype, void* out, float* lse, int flags, int rope_dims,
                        float rope_base, void* workspace, size_t ws_bytes, const csa_compress_job* job, int64_t e_new,
                        void* stream) {
  csa::Check ck = csa::check_hca(B, T, N, ratio, q_pos0, H, d, q, kv_cmp, kv_raw, raw_pos0, n_raw, window,
                                 scale, sink, io_dtype, out, lse, workspace, ws_bytes, flags, rope_dims, rope_base);
  if (!ck.ok()) return finish(ck);
  csa::CompressArgs j[4];
  ck = check_jobs(job, 1, j);
  if (!ck.ok()) return finish(ck);
  if (job->ratio != 128) {
    ck.fail(CSA_ERR_INVALID_ARG, "the job must be a C128A compression (ratio 128), got ratio " + csa::i2s(job->ratio));
    return finish(ck);
  }
  if (e_new < 0 || e_new >= N) {
    ck.fail(CSA_ERR_INVALID_ARG, "e_new must lie in [0, N), got " + csa::i2s(e_new));
    return finish(ck);
  }
  csa::AttnArgs a{B, T, N, 0, ratio, q_pos0, q, kv_cmp, nullptr, kv_raw, raw_pos0, n_raw, window, scale,
                  sink, io_dtype, out, lse, workspace, flags, rope_dims, rope_base};
  return hip_status(csa::launch_attn_jobs(a, j[0], e_new, as_stream(stream)), "hca_attn_compressed launch");
}

int hca_attn(int64_t B, int64_t T, int64_t N, int ratio, int64_t q_pos0, int H, int d, const void* q,
             const void* kv_cmp, const void* kv_raw, int64_t raw_pos0, int64_t n_raw, int window,
             float scale, const float* sink, int io_dtype, void* out, float* lse, void* workspace,
             size_t ws_bytes, void* stream) {
  return hca_attn_ex(B, T, N, ratio, q_pos0, H, d, q, kv_cmp, kv_raw, raw_pos0, n_raw, window, scale, sink,
                     io_dtype, out, lse, 0, 0, 0.f, workspace, ws_bytes, stream);
}

int csa_compress_paged_chunk(int ratio, int64_t B, int64_t n_tok, int64_t c, const int64_t* pos0, const void* Ca,
                             const void* Za, const void* Cb, const void* Zb, const void* prev_Cb, const void* prev_Zb,
                             const float* bias, const float* gamma, float eps, int in_dtype, int out_dtype, void* pool,
                             void* scale_pool, int64_t n_pool, const int32_t* block_table, int64_t max_blocks,
                             int rope_dims, float rope_base, int rope_anchor, void* stream) {
  csa::Check ck = csa::check_compress_paged(ratio, B, n_tok, c, pos0, Ca, Za, Cb, Zb, prev_Cb, prev_Zb, bias, gamma,
                                            eps, in_dtype, out_dtype, pool, scale_pool, n_pool, block_table,
                                            max_blocks, rope_dims, rope_base, rope_anchor);
  if (!ck.ok()) return finish(ck);
  if (n_pool == 0 || B == 0 || n_tok < ratio) return finish(ck);   // nothing to write
  csa::CompressPagedArgs a{ratio, B, c, pos0, n_tok, Ca, Za, Cb, Zb, prev_Cb, prev_Zb, bias, gamma, eps, in_dtype,
                           out_dtype, pool, scale_pool, n_pool, block_table, max_blocks, rope_dims, rope_base,
                           rope_anchor};
  return hip_status(csa::launch_compress_paged(&a, 1, as_stream(stream)), "csa_compress_paged launch");
}

int csa_compress_paged_batch(const csa_compress_paged_job* jobs, int n_jobs, void* stream) {
  csa::Check ck;
  if (!jobs) ck.fail(CSA_ERR_INVALID_ARG, "jobs is NULL");
  else if (n_jobs < 1 || n_jobs > 4) ck.fail(CSA_ERR_INVALID_ARG, "n_jobs must be 1..4, got " + csa::i2s(n_jobs));
  if (!ck.ok()) return finish(ck);
  csa::CompressPagedArgs a[4];
  auto quant = [](int dt) { return dt == CSA_FP8_E4M3 || dt == CSA_MXFP4; };
  for (int q = 0; q < n_jobs; ++q) {
    const csa_compress_paged_job& j = jobs[q];
    csa::Check cj = csa::check_compress_paged(j.ratio, j.B, j.n_tok, j.c, j.pos0, j.Ca, j.Za, j.Cb, j.Zb, j.prev_Cb,
                                              j.prev_Zb, j.bias, j.gamma, j.eps, j.in_dtype, j.out_dtype, j.pool,
                                              j.scale_pool, j.n_pool, j.block_table, j.max_blocks, j.rope_dims,
                                              j.rope_base, j.rope_anchor);
    bool same_out = true;
    for (int p = 0; p < q; ++p)
      if (jobs[p].out_dtype != j.out_dtype && !quant(jobs[p].out_dtype) && !quant(j.out_dtype)) same_out = false;
    if (cj.ok() && (j.ratio != jobs[0].ratio || j.in_dtype != jobs[0].in_dtype || !same_out))
      cj.fail(CSA_ERR_INVALID_ARG, "jobs of one batch must share ratio, in_dtype and out_dtype (fp8 / MXFP4 jobs "
                                   "may join jobs of one other output type)");
    if (!cj.ok()) {
      cj.msg = "job " + csa::i2s(q) + ": " + cj.msg;
      return finish(cj);
    }
    a[q] = csa::CompressPagedArgs{j.ratio, j.B, j.c, j.pos0, j.n_tok, j.Ca, j.Za, j.Cb, j.Zb, j.prev_Cb, j.prev_Zb,
                                  j.bias, j.gamma, j.eps, j.in_dtype, j.out_dtype, j.pool, j.scale_pool, j.n_pool,
                                  j.block_table, j.max_blocks, j.rope_dims, j.rope_base, j.rope_anchor};
  }
  return hip_status(csa::launch_compress_paged(a, n_jobs, as_stream(stream)), "csa_compress_paged_batch launch");
}

int csa_compress_paged(int ratio, int64_t B, int64_t c, const int64_t* pos0, const void* Ca, const void* Za,
                       const void* prev_Cb, const void* prev_Zb, const float* bias, const float* gamma, float eps,
                       int in_dtype, int out_dtype, void* pool, void* scale_pool, int64_t n_pool,
                       const int32_t* block_table, int64_t max_blocks, int rope_dims, float rope_base, int rope_anchor,
                       void* stream) {
  // one block per sequence: a chunk of ratio raw tokens whose previous block is prev_Cb / prev_Zb
  return csa_compress_paged_chunk(ratio, B, ratio, c, pos0, Ca, Za, nullptr, nullptr, prev_Cb, prev_Zb, bias, gamma,
                                  eps, in_dtype, out_dtype, pool, scale_pool, n_pool, block_table, max_blocks,
                                  rope_dims, rope_base, rope_anchor, stream);
}

int lightning_index_paged(int64_t B, int64_t max_blocks, int H_I, int d_I, const void* q, const void* q_scale,
                          const float* w, const void* k_pool, const void* k_scale, int64_t n_pool,
                          const int32_t* block_table, const int64_t* seq_pos, int qk_dtype, void* scores,
                          int score_dtype, void* stream) {
  csa::Check ck = csa::check_index_paged(B, max_blocks, H_I, d_I, q, q_scale, w, k_pool, k_scale, n_pool, block_table,
                                         seq_pos, qk_dtype, scores, score_dtype);
  if (!ck.ok()) return finish(ck);
  csa::IndexArgs a{B, 1, max_blocks * 32, 0, 4, q, q_scale, w, k_pool, k_scale, qk_dtype, scores, score_dtype,
                   block_table, max_blocks, n_pool, seq_pos};
  return hip_status(csa::launch_index(a, as_stream(stream)), "lightning_index_paged launch");
}

int topk_select_paged(int64_t B, int64_t N, const int64_t* seq_pos, int ratio, int k, const void* scores,
                      int score_dtype, int32_t* idx, void* workspace, size_t ws_bytes, void* stream) {
  csa::Check ck = csa::check_topk_paged(B, N, seq_pos, ratio, k, scores, score_dtype, idx, workspace, ws_bytes);
  if (!ck.ok()) return finish(ck);
  csa::TopkArgs a{B, 1, N, 0, ratio, k, scores, score_dtype, idx, workspace, nullptr, 0, seq_pos};
  return hip_status(csa::launch_topk(a, as_stream(stream)), "topk_select_paged launch");
}

int sparse_mqa_attn_paged(int64_t B, int k, int H, int d, const void* q, const void* kv_pool, int64_t n_pool,
                          const int32_t* block_table, int64_t max_blocks, const int32_t* idx, const void* win,
                          int64_t ring, const int64_t* seq_pos, int64_t max_pos, int window, float scale,
                          int io_dtype, void* out, float* lse, int flags, int rope_dims, float rope_base,
                          void* workspace, size_t ws_bytes, void* stream) {
  csa::Check ck = csa::check_paged(true, B, k, H, d, q, kv_pool, n_pool, block_table, max_blocks, idx, win, ring,
                                   seq_pos, max_pos, window, scale, nullptr, io_dtype, out, lse, flags, rope_dims,
                                   rope_base, workspace, ws_bytes);
  if (!ck.ok()) return finish(ck);
  // 32 C4A entries per block of 128 raw tokens
  csa::AttnArgs a{B, 1, max_blocks << 5, k, 4, 0, q, kv_pool, idx, win, 0, ring, window, scale,
                  nullptr, io_dtype, out, lse, workspace, flags, rope_dims, rope_base,
                  block_table, max_blocks, n_pool, 5, ring, seq_pos, max_pos};
  return hip_status(csa::launch_attn(a, as_stream(stream)), "sparse_mqa_attn_paged launch");
}

int hca_attn_paged(int64_t B, int H, int d, const void* q, const void* kv_pool, int64_t n_pool,
                   const int32_t* block_table, int64_t max_blocks, const void* win, int64_t ring,
                   const int64_t* seq_pos, int64_t max_pos, int window, float scale, const float* sink, int io_dtype,
                   void* out, float* lse, int flags, int rope_dims, float rope_base, void* workspace,
                   size_t ws_bytes, void* stream) {
  csa::Check ck = csa::check_paged(false, B, 0, H, d, q, kv_pool, n_pool, block_table, max_blocks, nullptr, win,
                                   ring, seq_pos, max_pos, window, scale, sink, io_dtype, out, lse, flags,
                                   rope_dims, rope_base, workspace, ws_bytes);
  if (!ck.ok()) return finish(ck);
  // one C128A entry per block of 128 raw tokens
  csa::AttnArgs a{B, 1, max_blocks, 0, 128, 0, q, kv_pool, nullptr, win, 0, ring, window, scale,
                  sink, io_dtype, out, lse, workspace, flags, rope_dims, rope_base,
                  block_table, max_blocks, n_pool, 0, ring, seq_pos, max_pos};
  return hip_status(csa::launch_attn(a, as_stream(stream)), "hca_attn_paged launch");
}

int csa_rope(int64_t B, int64_t T, int64_t H, int64_t D, int64_t pos0, int rope_dims, float rope_base,
             int inverse, int dtype, void* x, void* stream) {
  csa::Check ck = csa::check_rope_rows(B, T, H, D, pos0, rope_dims, rope_base, inverse, dtype, x);
  if (!ck.ok()) return finish(ck);
  csa::RopeArgs a{B, T, H, D, pos0, rope_dims, rope_base, inverse, dtype, x};
  return hip_status(csa::launch_rope(a, as_stream(stream)), "csa_rope launch");
}

size_t csa_workspace_bytes(int op, int64_t B, int64_t T, int64_t N, int k) {
  return csa::workspace_bytes(op, B, T, N, k);
}

const char* csa_last_error(void) { return g_last_error.c_str(); }

const char* csa_version(void) { return "csa-gfx950 0.1"; }

}  // extern "C"
