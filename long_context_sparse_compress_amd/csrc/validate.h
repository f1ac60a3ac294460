// Host-side argument validation for every entry point of csa.h.
//
// Plain C++ with no HIP dependency, so the same checks compile with g++ and
// run on a machine without a GPU.  Each check returns CSA_OK or an error code
// and fills `msg`.  The rules are the ones csa.h documents for each call.
#pragma once

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/csa.h"

namespace csa {

constexpr int kAttnTile = 32;        // rows per attention tile
constexpr int kMaxWindow = 4096;
constexpr int kMaxSplits = 32;

inline int64_t visible(int64_t t, int64_t ratio) { return (t + 1) / ratio; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Check {
  int code = CSA_OK;
  std::string msg;
  bool fail(int c, const std::string& m) {
    if (code == CSA_OK) { code = c; msg = m; }
    return false;
  }
  bool ptr(const void* p, const char* name, bool required = true) {
    if (!p) return required ? fail(CSA_ERR_INVALID_ARG, std::string(name) + " is NULL") : true;
    if (!aligned16(p)) return fail(CSA_ERR_INVALID_ARG, std::string(name) + " is not 16-byte aligned");
    return true;
  }
  bool must_be_null(const void* p, const char* name, const char* why) {
    if (p) return fail(CSA_ERR_INVALID_ARG, std::string(name) + " must be NULL " + why);
    return true;
  }
  bool ok() const { return code == CSA_OK; }
};

inline std::string i2s(int64_t v) { return std::to_string(v); }

// Partial RoPE parameters: 0 dims (none), or a multiple of 8 up to the row
// width with a finite base > 1.
inline bool check_rope(Check& k, int dims, float base, int64_t width) {
  if (dims < 0 || dims % 8 != 0 || dims > width) {
    k.fail(CSA_ERR_INVALID_ARG, "rope_dims must be 0 or a multiple of 8 up to " + std::to_string(width) + ", got " +
                                    std::to_string(dims));
    return false;
  }
  if (dims > 0 && !(base > 1.0f && std::isfinite(base))) {
    k.fail(CSA_ERR_INVALID_ARG, "rope_base must be finite and > 1");
    return false;
  }
  return true;
}

inline void check_attn_flags(Check& k, int flags) {
  if (flags & ~CSA_ATTN_BATCH_INVARIANT) k.fail(CSA_ERR_INVALID_ARG, "unknown attention flags " + std::to_string(flags));
}

// Split plan of the attention kernels: how many workgroups share one query's
// rows.  The workspace bound depends only on B*T; the split count used at run
// time never exceeds it.
inline int attn_max_splits(int64_t B, int64_t T) {
  const int64_t q = B * T;
  if (q <= 0 || q >= 256) return 1;
  // about one workgroup per CU: more splits shorten the kernel but every split
  // adds a 128 KB partial that the combine must read back
  int64_t s = (256 + q - 1) / q;
  if (s > kMaxSplits) s = kMaxSplits;
  return static_cast<int>(s < 1 ? 1 : s);
}

inline int attn_splits(int64_t B, int64_t T, int64_t rows) {
  int64_t s = attn_max_splits(B, T);
  const int64_t by_rows = (rows + 4 * kAttnTile - 1) / (4 * kAttnTile);  // >= 4 tiles each
  if (s > by_rows) s = by_rows;
  return static_cast<int>(s < 1 ? 1 : s);
}

// Per split and query: 64 x 512 bf16 partial output + 64 running maxima + 64 sums (fp32).
inline size_t attn_split_bytes() { return size_t(CSA_HEADS) * CSA_HEAD_DIM * 2 + 2 * size_t(CSA_HEADS) * sizeof(float); }

inline size_t attn_workspace_bytes(int64_t B, int64_t T) {
  const int s = attn_max_splits(B, T);
  if (s <= 1) return 0;
  return size_t(B) * size_t(T) * size_t(s) * attn_split_bytes();
}

// Size of the static device scratch that sparse_mqa_attn_noalloc's split
// partials live in: 24 MiB, enough for the split plan of every call with
// B*T <= 190 (and B*T >= 256 needs none).
constexpr size_t kAttnStaticScratchBytes = size_t(24) << 20;

// Top-k keeps rows of up to this many candidates in LDS; longer rows use the
// multi-pass global path, which needs a per-row histogram workspace.
constexpr int64_t kTopkLdsMax16 = 36864;   // bf16 keys
constexpr int64_t kTopkLdsMax32 = 18432;   // fp32 keys
constexpr int kTopkSlices = 64;            // workgroups per row on the global path

inline bool topk_row_in_lds(int64_t N, int dtype) {
  return N <= (dtype == CSA_BF16 ? kTopkLdsMax16 : kTopkLdsMax32);
}

// Global path scratch per row: one 2048-bin histogram per digit pass (at most
// three) and a (greater, equal) count pair per slice.
inline size_t topk_row_ws_bytes() { return (3 * 2048 + 2 * kTopkSlices) * sizeof(uint32_t); }

// Long bf16 rows: one record per slice of 16384 keys -- two 1024-word coarse
// count tables and a list of at most k + 63 (key, count) words, the record
// rounded up to 16 bytes.
constexpr int64_t kTopkFineSlice = 16384;
constexpr int kTopkFineCoarse = 1024;
inline int64_t topk_fine_rec_words(int k) { return 2 * kTopkFineCoarse + (int64_t(k) + 64 + 3) / 4 * 4; }
inline size_t topk_fine_row_ws_bytes(int64_t N, int k) {
  return size_t((N + kTopkFineSlice - 1) / kTopkFineSlice) * size_t(topk_fine_rec_words(k)) * sizeof(uint32_t);
}

inline size_t topk_workspace_bytes(int64_t B, int64_t T, int64_t N, int k, int dtype) {
  if (topk_row_in_lds(N, dtype)) return 0;
  size_t per = topk_row_ws_bytes();
  if (dtype == CSA_BF16 && topk_fine_row_ws_bytes(N, k) > per) per = topk_fine_row_ws_bytes(N, k);
  return size_t(B) * size_t(T) * per;
}

// Compressor row split: a C128A call with few (entry, sequence) pairs spreads
// each entry's 128 rows over P workgroups (P a power of two up to 16, about
// 256 workgroups in all) and merges their partial states in a second kernel.
inline int compress_splits(int ratio, int64_t B, int64_t n_tok) {
  if (ratio != 128) return 1;
  const int64_t n_wg = B * (n_tok / ratio);
  if (n_wg <= 0 || n_wg >= 128) return 1;
  int P = 16;
  while (P > 2 && n_wg * P > 256) P /= 2;
  return P;
}

// (m, s, y) per channel per row range, fp32.
inline size_t compress_workspace_bytes(int ratio, int64_t B, int64_t n_tok, int64_t c) {
  const int P = compress_splits(ratio, B, n_tok);
  if (P <= 1) return 0;
  return size_t(B) * size_t(n_tok / ratio) * size_t(P) * 3 * size_t(c) * sizeof(float);
}

inline Check check_compress(int ratio, int64_t B, int64_t n_tok, int64_t c, int64_t pos0,
                            const void* Ca, const void* Za, const void* Cb, const void* Zb,
                            const void* prev_Cb, const void* prev_Zb, const float* bias,
                            const float* gamma, float eps, int in_dtype, int out_dtype,
                            const void* out, int64_t out_batch_stride, const void* ws, size_t ws_bytes,
                            int rope_dims = 0, float rope_base = 0.f, int rope_anchor = 0,
                            const void* out_scale = nullptr) {
  Check k;
  if (ratio != 4 && ratio != 128) { k.fail(CSA_ERR_INVALID_ARG, "ratio must be 4 or 128, got " + i2s(ratio)); return k; }
  if (B < 0 || n_tok < 0) { k.fail(CSA_ERR_INVALID_ARG, "B and n_tok must be >= 0"); return k; }
  if (c <= 0 || c % 64 != 0 || c > 1024) { k.fail(CSA_ERR_INVALID_ARG, "c must be a positive multiple of 64, at most 1024, got " + i2s(c)); return k; }
  if (!check_rope(k, rope_dims, rope_base, c)) return k;
  if (rope_anchor < 0 || rope_anchor >= ratio) { k.fail(CSA_ERR_INVALID_ARG, "rope_anchor must be in [0, ratio), got " + i2s(rope_anchor)); return k; }
  if (pos0 < 0 || pos0 % ratio != 0) { k.fail(CSA_ERR_INVALID_ARG, "pos0 must be >= 0 and a multiple of ratio, got " + i2s(pos0)); return k; }
  if (in_dtype != CSA_F32 && in_dtype != CSA_BF16) { k.fail(CSA_ERR_UNSUPPORTED, "in_dtype must be CSA_F32 or CSA_BF16"); return k; }
  if (out_dtype != CSA_F32 && out_dtype != CSA_BF16 && out_dtype != CSA_FP8_E4M3 && out_dtype != CSA_MXFP4) { k.fail(CSA_ERR_UNSUPPORTED, "out_dtype must be CSA_F32, CSA_BF16, CSA_FP8_E4M3 or CSA_MXFP4"); return k; }
  if (out_dtype == CSA_FP8_E4M3 || out_dtype == CSA_MXFP4) {
    if (ratio != 4) { k.fail(CSA_ERR_UNSUPPORTED, "quantized output (quantize-on-write) is for C4A keys: ratio must be 4"); return k; }
    if (out_batch_stride % c != 0) { k.fail(CSA_ERR_INVALID_ARG, "quantized output needs out_batch_stride to be a multiple of c"); return k; }
    if (!out_scale && B > 0 && n_tok / ratio > 0) { k.fail(CSA_ERR_INVALID_ARG, "out_scale is NULL"); return k; }
    if (out_dtype == CSA_FP8_E4M3 && (reinterpret_cast<uintptr_t>(out_scale) & 3u) != 0) { k.fail(CSA_ERR_INVALID_ARG, "out_scale is not 4-byte aligned"); return k; }
  } else if (out_scale) {
    k.fail(CSA_ERR_INVALID_ARG, "out_scale must be NULL unless the output is quantized (CSA_FP8_E4M3, CSA_MXFP4)");
    return k;
  }
  if (!(eps > 0.0f) || !std::isfinite(eps)) { k.fail(CSA_ERR_INVALID_ARG, "eps must be positive and finite"); return k; }
  const int64_t n_ent = n_tok / ratio;
  if (out_batch_stride != 0 && out_batch_stride < n_ent * c) { k.fail(CSA_ERR_INVALID_ARG, "out_batch_stride smaller than one sequence's output"); return k; }
  if (out_batch_stride % 8 != 0) { k.fail(CSA_ERR_INVALID_ARG, "out_batch_stride must be a multiple of 8 elements"); return k; }
  const bool empty = (B == 0 || n_ent == 0);
  k.ptr(Ca, "Ca", !empty) && k.ptr(Za, "Za", !empty) && k.ptr(bias, "bias", !empty) &&
      k.ptr(gamma, "gamma", false) && k.ptr(out, "out", !empty);
  if (!k.ok()) return k;
  if (ratio == 4) {
    k.ptr(Cb, "Cb", !empty) && k.ptr(Zb, "Zb", !empty);
    if (!k.ok()) return k;
    if (pos0 > 0) {
      k.ptr(prev_Cb, "prev_Cb", !empty) && k.ptr(prev_Zb, "prev_Zb", !empty);
    } else {
      k.must_be_null(prev_Cb, "prev_Cb", "when pos0 == 0") && k.must_be_null(prev_Zb, "prev_Zb", "when pos0 == 0");
    }
  } else {
    k.must_be_null(Cb, "Cb", "for ratio 128") && k.must_be_null(Zb, "Zb", "for ratio 128") &&
        k.must_be_null(prev_Cb, "prev_Cb", "for ratio 128") && k.must_be_null(prev_Zb, "prev_Zb", "for ratio 128");
  }
  if (!k.ok()) return k;
  if (ws_bytes > 0) k.ptr(ws, "workspace");   // optional: too small a workspace just means no split
  return k;
}

inline Check check_index(int64_t B, int64_t T, int64_t N, int64_t q_pos0, int ratio, int H_I, int d_I,
                         const void* q, const void* q_scale, const float* w, const void* kk,
                         const void* k_scale, int qk_dtype, const void* scores, int score_dtype) {
  Check k;
  if (B < 0 || T < 0 || N < 0) { k.fail(CSA_ERR_INVALID_ARG, "B, T and N must be >= 0"); return k; }
  if (q_pos0 < 0) { k.fail(CSA_ERR_INVALID_ARG, "q_pos0 must be >= 0"); return k; }
  if (ratio != 4 && ratio != 128) { k.fail(CSA_ERR_INVALID_ARG, "ratio must be 4 or 128, got " + i2s(ratio)); return k; }
  if (H_I != CSA_INDEX_HEADS || d_I != CSA_INDEX_DIM) { k.fail(CSA_ERR_UNSUPPORTED, "indexer shape must be H_I=64, d_I=128"); return k; }
  if (qk_dtype < CSA_F32 || qk_dtype > CSA_MXFP4) { k.fail(CSA_ERR_UNSUPPORTED, "unknown qk_dtype " + i2s(qk_dtype)); return k; }
  if (score_dtype != CSA_F32 && score_dtype != CSA_BF16) { k.fail(CSA_ERR_UNSUPPORTED, "score_dtype must be CSA_F32 or CSA_BF16"); return k; }
  if (qk_dtype == CSA_F32 && score_dtype != CSA_F32) { k.fail(CSA_ERR_UNSUPPORTED, "fp32 QK needs fp32 scores"); return k; }
  if (T > 0 && N < visible(q_pos0 + T - 1, ratio)) { k.fail(CSA_ERR_INVALID_ARG, "N = " + i2s(N) + " is smaller than the entries visible to the last query (" + i2s(visible(q_pos0 + T - 1, ratio)) + ")"); return k; }
  const bool empty = (B == 0 || T == 0 || N == 0);
  const bool scaled = (qk_dtype == CSA_FP8_E4M3 || qk_dtype == CSA_MXFP4);
  k.ptr(q, "q", !empty) && k.ptr(w, "w", !empty) && k.ptr(kk, "k", !empty) && k.ptr(scores, "scores", !empty);
  if (!k.ok()) return k;
  if (scaled) {
    k.ptr(q_scale, "q_scale", !empty) && k.ptr(k_scale, "k_scale", !empty);
  } else {
    k.must_be_null(q_scale, "q_scale", "for unscaled qk_dtype") && k.must_be_null(k_scale, "k_scale", "for unscaled qk_dtype");
  }
  return k;
}

inline Check check_topk(int64_t B, int64_t T, int64_t N, int64_t q_pos0, int ratio, int kk,
                        const void* scores, int score_dtype, const void* idx, const void* ws, size_t ws_bytes) {
  Check k;
  if (B < 0 || T < 0 || N < 0) { k.fail(CSA_ERR_INVALID_ARG, "B, T and N must be >= 0"); return k; }
  if (q_pos0 < 0) { k.fail(CSA_ERR_INVALID_ARG, "q_pos0 must be >= 0"); return k; }
  if (ratio != 4 && ratio != 128) { k.fail(CSA_ERR_INVALID_ARG, "ratio must be 4 or 128, got " + i2s(ratio)); return k; }
  if (kk < 1 || kk > CSA_MAX_TOPK) { k.fail(CSA_ERR_INVALID_ARG, "k must be in [1, 2048], got " + i2s(kk)); return k; }
  if (score_dtype != CSA_F32 && score_dtype != CSA_BF16) { k.fail(CSA_ERR_UNSUPPORTED, "score_dtype must be CSA_F32 or CSA_BF16"); return k; }
  if (T > 0 && N < visible(q_pos0 + T - 1, ratio)) { k.fail(CSA_ERR_INVALID_ARG, "N = " + i2s(N) + " is smaller than the entries visible to the last query (" + i2s(visible(q_pos0 + T - 1, ratio)) + ")"); return k; }
  const bool empty = (B == 0 || T == 0);
  k.ptr(scores, "scores", !empty && N > 0) && k.ptr(idx, "idx", !empty);
  if (!k.ok()) return k;
  const size_t need = topk_workspace_bytes(B, T, N, kk, score_dtype);
  if (need > 0) {
    if (!ws || ws_bytes < need) { k.fail(CSA_ERR_WORKSPACE, "topk_select needs " + i2s((int64_t)need) + " workspace bytes, got " + i2s((int64_t)ws_bytes)); return k; }
    k.ptr(ws, "workspace");
  }
  return k;
}

// Hierarchical indexer: pool scoring and Top-k inside the pool.
constexpr int64_t kMaxPool = 65536;       // pool slots a query may score
constexpr int64_t kMaxPoolTopk = 16384;   // pool slots Top-k selects from (one workgroup per row, no workspace)

inline Check check_index_pool(int64_t B, int64_t T, int64_t N, int64_t P, int H_I, int d_I, const void* q,
                              const void* q_scale, const float* w, const void* kk, const void* k_scale, int qk_dtype,
                              const int32_t* pool, const void* scores, int score_dtype) {
  Check k;
  if (B < 0 || T < 0 || N < 0 || P < 0) { k.fail(CSA_ERR_INVALID_ARG, "B, T, N and P must be >= 0"); return k; }
  if (P > kMaxPool) { k.fail(CSA_ERR_INVALID_ARG, "P must be at most 65536, got " + i2s(P)); return k; }
  if (H_I != CSA_INDEX_HEADS || d_I != CSA_INDEX_DIM) { k.fail(CSA_ERR_UNSUPPORTED, "indexer shape must be H_I=64, d_I=128"); return k; }
  if (qk_dtype != CSA_BF16 && qk_dtype != CSA_FP8_E4M3 && qk_dtype != CSA_MXFP4) { k.fail(CSA_ERR_UNSUPPORTED, "lightning_index_pool takes bf16, fp8 E4M3 or MXFP4 q and keys"); return k; }
  if (score_dtype != CSA_F32 && score_dtype != CSA_BF16) { k.fail(CSA_ERR_UNSUPPORTED, "score_dtype must be CSA_F32 or CSA_BF16"); return k; }
  if (B * T * ((P + 255) / 256) > 0x7fffffff) { k.fail(CSA_ERR_INVALID_ARG, "B * T * ceil(P / 256) must be below 2^31"); return k; }
  const bool empty = (B == 0 || T == 0 || P == 0);
  k.ptr(q, "q", !empty) && k.ptr(w, "w", !empty) && k.ptr(kk, "k", !empty && N > 0) && k.ptr(pool, "pool", !empty) &&
      k.ptr(scores, "scores", !empty);
  if (!k.ok()) return k;
  if (qk_dtype == CSA_BF16) {
    k.must_be_null(q_scale, "q_scale", "for bf16") && k.must_be_null(k_scale, "k_scale", "for bf16");
  } else {
    k.ptr(q_scale, "q_scale", !empty) && k.ptr(k_scale, "k_scale", !empty && N > 0);
  }
  return k;
}

inline Check check_topk_pool(int64_t B, int64_t T, int64_t N, int64_t P, int kk, const void* scores, int score_dtype,
                             const int32_t* pool, const void* idx) {
  Check k;
  if (B < 0 || T < 0 || N < 0 || P < 0) { k.fail(CSA_ERR_INVALID_ARG, "B, T, N and P must be >= 0"); return k; }
  if (P > kMaxPoolTopk) { k.fail(CSA_ERR_INVALID_ARG, "P must be at most 16384, got " + i2s(P)); return k; }
  if (kk < 1 || kk > CSA_MAX_TOPK) { k.fail(CSA_ERR_INVALID_ARG, "k must be in [1, 2048], got " + i2s(kk)); return k; }
  if (score_dtype != CSA_F32 && score_dtype != CSA_BF16) { k.fail(CSA_ERR_UNSUPPORTED, "score_dtype must be CSA_F32 or CSA_BF16"); return k; }
  if (B * T > 0x7fffffff) { k.fail(CSA_ERR_INVALID_ARG, "B * T must be below 2^31"); return k; }
  const bool empty = (B == 0 || T == 0);
  k.ptr(scores, "scores", !empty && P > 0) && k.ptr(pool, "pool", !empty && P > 0) && k.ptr(idx, "idx", !empty);
  return k;
}

inline bool check_attn_common(Check& k, int64_t B, int64_t T, int64_t q_pos0, int H, int d,
                               int64_t raw_pos0, int64_t n_raw, int window, float scale, int io_dtype) {
  if (B < 0 || T < 0) { k.fail(CSA_ERR_INVALID_ARG, "B and T must be >= 0"); return false; }
  if (q_pos0 < 0) { k.fail(CSA_ERR_INVALID_ARG, "q_pos0 must be >= 0"); return false; }
  if (H != CSA_HEADS || d != CSA_HEAD_DIM) { k.fail(CSA_ERR_UNSUPPORTED, "attention shape must be H=64, d=512"); return false; }
  if (window < 1 || window > kMaxWindow) { k.fail(CSA_ERR_INVALID_ARG, "window must be in [1, 4096], got " + i2s(window)); return false; }
  if (!std::isfinite(scale)) { k.fail(CSA_ERR_INVALID_ARG, "scale must be finite"); return false; }
  if (io_dtype != CSA_F32 && io_dtype != CSA_BF16) { k.fail(CSA_ERR_UNSUPPORTED, "io_dtype must be CSA_F32 or CSA_BF16"); return false; }
  if (T > 0) {
    const int64_t wstart = q_pos0 - window + 1 > 0 ? q_pos0 - window + 1 : 0;
    if (raw_pos0 < 0 || raw_pos0 > wstart) { k.fail(CSA_ERR_INVALID_ARG, "kv_raw starts at " + i2s(raw_pos0) + ", after the first window position " + i2s(wstart)); return false; }
    if (raw_pos0 + n_raw < q_pos0 + T) { k.fail(CSA_ERR_INVALID_ARG, "kv_raw ends before the last query position"); return false; }
  }
  return true;
}

inline Check check_sparse(int64_t B, int64_t T, int64_t N, int kk, int64_t q_pos0, int H, int d,
                          const void* q, const void* kv_cmp, const void* idx, const void* kv_raw,
                          int64_t raw_pos0, int64_t n_raw, int window, float scale, int io_dtype,
                          const void* out, const void* lse, const void* ws, size_t ws_bytes, int flags = 0,
                          int rope_dims = 0, float rope_base = 0.f) {
  Check k;
  check_attn_flags(k, flags);
  if (!k.ok()) return k;
  if (!check_attn_common(k, B, T, q_pos0, H, d, raw_pos0, n_raw, window, scale, io_dtype)) return k;
  if (!check_rope(k, rope_dims, rope_base, d)) return k;
  if (N < 0) { k.fail(CSA_ERR_INVALID_ARG, "N must be >= 0"); return k; }
  if (kk < 0 || kk > CSA_MAX_TOPK) { k.fail(CSA_ERR_INVALID_ARG, "k must be in [0, 2048], got " + i2s(kk)); return k; }
  const bool empty = (B == 0 || T == 0);
  k.ptr(q, "q", !empty) && k.ptr(kv_cmp, "kv_cmp", !empty && N > 0 && kk > 0) &&
      k.ptr(idx, "idx", !empty && kk > 0) && k.ptr(kv_raw, "kv_raw", !empty) && k.ptr(out, "out", !empty) &&
      k.ptr(lse, "lse", false);
  if (!k.ok()) return k;
  // the batch-invariant mode never splits rows, so it uses no workspace
  const size_t need = (flags & CSA_ATTN_BATCH_INVARIANT) ? 0 : attn_workspace_bytes(B, T);
  if (need > 0 && !empty) {
    if (!ws || ws_bytes < need) { k.fail(CSA_ERR_WORKSPACE, "sparse_mqa_attn needs " + i2s((int64_t)need) + " workspace bytes, got " + i2s((int64_t)ws_bytes)); return k; }
    k.ptr(ws, "workspace");
  }
  return k;
}

// sparse_mqa_attn_noalloc: the arguments of sparse_mqa_attn (flags 0, no
// RoPE), with the split partials in the library's static scratch instead of a
// caller workspace -- calls whose plan needs more than it are rejected.
inline Check check_sparse_noalloc(int64_t B, int64_t T, int64_t N, int kk, int64_t q_pos0, int H, int d,
                                  const void* q, const void* kv_cmp, const void* idx, const void* kv_raw,
                                  int64_t raw_pos0, int64_t n_raw, int window, float scale, int io_dtype,
                                  const void* out, const void* lse) {
  Check k = check_sparse(B, T, N, kk, q_pos0, H, d, q, kv_cmp, idx, kv_raw, raw_pos0, n_raw, window, scale,
                         io_dtype, out, lse, nullptr, 0, CSA_ATTN_BATCH_INVARIANT);
  if (!k.ok()) return k;
  const size_t need = (B == 0 || T == 0) ? 0 : attn_workspace_bytes(B, T);
  if (need > kAttnStaticScratchBytes)
    k.fail(CSA_ERR_WORKSPACE, "sparse_mqa_attn_noalloc: the split partials of B*T = " + i2s(B * T) +
                                  " queries need " + i2s((int64_t)need) + " bytes, more than its static scratch of " +
                                  i2s((int64_t)kAttnStaticScratchBytes) + " (call sparse_mqa_attn with a workspace)");
  return k;
}

inline Check check_hca(int64_t B, int64_t T, int64_t N, int ratio, int64_t q_pos0, int H, int d,
                       const void* q, const void* kv_cmp, const void* kv_raw, int64_t raw_pos0,
                       int64_t n_raw, int window, float scale, const void* sink, int io_dtype,
                       const void* out, const void* lse, const void* ws, size_t ws_bytes, int flags = 0,
                       int rope_dims = 0, float rope_base = 0.f) {
  Check k;
  check_attn_flags(k, flags);
  if (!k.ok()) return k;
  if (ratio != 4 && ratio != 128) { k.fail(CSA_ERR_INVALID_ARG, "ratio must be 4 or 128, got " + i2s(ratio)); return k; }
  if (!check_attn_common(k, B, T, q_pos0, H, d, raw_pos0, n_raw, window, scale, io_dtype)) return k;
  if (!check_rope(k, rope_dims, rope_base, d)) return k;
  if (N < 0) { k.fail(CSA_ERR_INVALID_ARG, "N must be >= 0"); return k; }
  if (T > 0 && N < visible(q_pos0 + T - 1, ratio)) { k.fail(CSA_ERR_INVALID_ARG, "N = " + i2s(N) + " is smaller than the entries visible to the last query"); return k; }
  const bool empty = (B == 0 || T == 0);
  k.ptr(q, "q", !empty) && k.ptr(kv_cmp, "kv_cmp", !empty && N > 0) && k.ptr(kv_raw, "kv_raw", !empty) &&
      k.ptr(out, "out", !empty) && k.ptr(lse, "lse", false) && k.ptr(sink, "sink", false);
  if (!k.ok()) return k;
  // the batch-invariant mode never splits rows, so it uses no workspace
  const size_t need = (flags & CSA_ATTN_BATCH_INVARIANT) ? 0 : attn_workspace_bytes(B, T);
  if (need > 0 && !empty) {
    if (!ws || ws_bytes < need) { k.fail(CSA_ERR_WORKSPACE, "hca_attn needs " + i2s((int64_t)need) + " workspace bytes, got " + i2s((int64_t)ws_bytes)); return k; }
    k.ptr(ws, "workspace");
  }
  return k;
}

inline Check check_rope_rows(int64_t B, int64_t T, int64_t H, int64_t D, int64_t pos0, int dims, float base,
                             int inverse, int dtype, const void* x) {
  Check k;
  if (B < 0 || T < 0 || H < 0) { k.fail(CSA_ERR_INVALID_ARG, "B, T and H must be >= 0"); return k; }
  if (D <= 0 || D % 8 != 0 || D > 65536) { k.fail(CSA_ERR_INVALID_ARG, "D must be a positive multiple of 8, at most 65536, got " + i2s(D)); return k; }
  if (dims == 0 || dims > 1024) { k.fail(CSA_ERR_INVALID_ARG, "rope_dims must be in [8, 1024], got " + i2s(dims)); return k; }
  if (!check_rope(k, dims, base, D)) return k;
  if (B * T > 0x7fffffff) { k.fail(CSA_ERR_INVALID_ARG, "B * T must be below 2^31"); return k; }
  if (H > (int64_t{1} << 24)) { k.fail(CSA_ERR_INVALID_ARG, "H must be at most 2^24"); return k; }
  if (pos0 < 0 || pos0 > (int64_t{1} << 40)) { k.fail(CSA_ERR_INVALID_ARG, "pos0 must be in [0, 2^40]"); return k; }
  if (inverse != 0 && inverse != 1) { k.fail(CSA_ERR_INVALID_ARG, "inverse must be 0 or 1"); return k; }
  if (dtype != CSA_F32 && dtype != CSA_BF16) { k.fail(CSA_ERR_UNSUPPORTED, "dtype must be CSA_F32 or CSA_BF16"); return k; }
  k.ptr(x, "x", B > 0 && T > 0 && H > 0);
  return k;
}

inline Check check_compress_paged(int ratio, int64_t B, int64_t n_tok, int64_t c, const int64_t* pos0, const void* Ca,
                                  const void* Za, const void* Cb, const void* Zb,
                                  const void* pCb, const void* pZb, const float* bias, const float* gamma, float eps,
                                  int in_dtype, int out_dtype, const void* pool, const void* scale_pool,
                                  int64_t n_pool, const int32_t* table, int64_t max_blocks, int rope_dims,
                                  float rope_base, int rope_anchor) {
  Check k;
  if (ratio != 4 && ratio != 128) { k.fail(CSA_ERR_INVALID_ARG, "ratio must be 4 or 128, got " + i2s(ratio)); return k; }
  if (B < 0) { k.fail(CSA_ERR_INVALID_ARG, "B must be >= 0"); return k; }
  if (c <= 0 || c % 64 != 0 || c > 1024) { k.fail(CSA_ERR_INVALID_ARG, "c must be a positive multiple of 64, at most 1024, got " + i2s(c)); return k; }
  if (!check_rope(k, rope_dims, rope_base, c)) return k;
  if (rope_anchor < 0 || rope_anchor >= ratio) { k.fail(CSA_ERR_INVALID_ARG, "rope_anchor must be in [0, ratio), got " + i2s(rope_anchor)); return k; }
  if (in_dtype != CSA_F32 && in_dtype != CSA_BF16) { k.fail(CSA_ERR_UNSUPPORTED, "in_dtype must be CSA_F32 or CSA_BF16"); return k; }
  if (out_dtype != CSA_F32 && out_dtype != CSA_BF16 && out_dtype != CSA_FP8_E4M3 && out_dtype != CSA_MXFP4) { k.fail(CSA_ERR_UNSUPPORTED, "out_dtype must be CSA_F32, CSA_BF16, CSA_FP8_E4M3 or CSA_MXFP4"); return k; }
  const bool quant = out_dtype == CSA_FP8_E4M3 || out_dtype == CSA_MXFP4;
  if (quant && ratio != 4) { k.fail(CSA_ERR_UNSUPPORTED, "quantized output (quantize-on-write) is for C4A keys: ratio must be 4"); return k; }
  if (!(eps > 0.0f) || !std::isfinite(eps)) { k.fail(CSA_ERR_INVALID_ARG, "eps must be positive and finite"); return k; }
  if (n_pool < 0) { k.fail(CSA_ERR_INVALID_ARG, "n_pool must be >= 0"); return k; }
  if (max_blocks < 1 || max_blocks > (int64_t{1} << 26)) { k.fail(CSA_ERR_INVALID_ARG, "max_blocks must be in [1, 2^26]"); return k; }
  if (B > 0x7fffffff) { k.fail(CSA_ERR_INVALID_ARG, "B must be below 2^31"); return k; }
  // one workgroup of at most 1024 threads per entry: entries * threads stay below 2^32
  if (n_tok < 0 || n_tok / ratio > (int64_t{1} << 22)) { k.fail(CSA_ERR_INVALID_ARG, "n_tok must be >= 0 with at most 2^22 entries per sequence, got " + i2s(n_tok)); return k; }
  const bool empty = B == 0 || n_tok < ratio;   // nothing to write
  k.ptr(pos0, "pos0", !empty) && k.ptr(Ca, "Ca", !empty) && k.ptr(Za, "Za", !empty) && k.ptr(bias, "bias", !empty) &&
      k.ptr(gamma, "gamma", false) && k.ptr(pool, "pool", !empty && n_pool > 0) && k.ptr(table, "block_table", !empty);
  if (!k.ok()) return k;
  if (ratio == 4) {
    // entries after the chunk's first take their previous block from the chunk itself
    k.ptr(pCb, "prev_Cb", !empty) && k.ptr(pZb, "prev_Zb", !empty) && k.ptr(Cb, "Cb", !empty && n_tok >= 8) &&
        k.ptr(Zb, "Zb", !empty && n_tok >= 8);
  } else {
    k.must_be_null(pCb, "prev_Cb", "for ratio 128") && k.must_be_null(pZb, "prev_Zb", "for ratio 128") &&
        k.must_be_null(Cb, "Cb", "for ratio 128") && k.must_be_null(Zb, "Zb", "for ratio 128");
  }
  if (!k.ok()) return k;
  if (quant) {
    if (!scale_pool && !empty && n_pool > 0) { k.fail(CSA_ERR_INVALID_ARG, "scale_pool is NULL"); return k; }
    if (out_dtype == CSA_FP8_E4M3 && (reinterpret_cast<uintptr_t>(scale_pool) & 3u) != 0) { k.fail(CSA_ERR_INVALID_ARG, "scale_pool is not 4-byte aligned"); return k; }
  } else if (scale_pool) {
    k.fail(CSA_ERR_INVALID_ARG, "scale_pool must be NULL unless the output is quantized (CSA_FP8_E4M3, CSA_MXFP4)");
    return k;
  }
  return k;
}

// Paged decode indexer / Top-k (heterogeneous cache): one query per sequence
// at seq_pos[b], index keys in a pool of 32-entry blocks under a block table.
inline Check check_index_paged(int64_t B, int64_t max_blocks, int H_I, int d_I, const void* q, const void* q_scale,
                               const float* w, const void* kpool, const void* kscale, int64_t n_pool,
                               const int32_t* table, const int64_t* seq_pos, int qk_dtype, const void* scores,
                               int score_dtype) {
  Check k;
  if (B < 0) { k.fail(CSA_ERR_INVALID_ARG, "B must be >= 0"); return k; }
  if (max_blocks < 1 || max_blocks > (int64_t{1} << 26)) { k.fail(CSA_ERR_INVALID_ARG, "max_blocks must be in [1, 2^26]"); return k; }
  if (H_I != CSA_INDEX_HEADS || d_I != CSA_INDEX_DIM) { k.fail(CSA_ERR_UNSUPPORTED, "indexer shape must be H_I=64, d_I=128"); return k; }
  if (qk_dtype != CSA_BF16 && qk_dtype != CSA_FP8_E4M3 && qk_dtype != CSA_MXFP4) { k.fail(CSA_ERR_UNSUPPORTED, "paged keys are bf16, fp8 E4M3 or MXFP4"); return k; }
  if (score_dtype != CSA_F32 && score_dtype != CSA_BF16) { k.fail(CSA_ERR_UNSUPPORTED, "score_dtype must be CSA_F32 or CSA_BF16"); return k; }
  if (B > 0 && n_pool < 1) { k.fail(CSA_ERR_INVALID_ARG, "the key pool holds no block"); return k; }
  if (B * max_blocks * 32 > (int64_t{1} << 40)) { k.fail(CSA_ERR_INVALID_ARG, "B * max_blocks too large"); return k; }
  const bool empty = B == 0;
  const bool quant = qk_dtype == CSA_FP8_E4M3 || qk_dtype == CSA_MXFP4;
  k.ptr(q, "q", !empty) && k.ptr(w, "w", !empty) && k.ptr(kpool, "k_pool", !empty) &&
      k.ptr(table, "block_table", !empty) && k.ptr(seq_pos, "seq_pos", !empty) && k.ptr(scores, "scores", !empty);
  if (!k.ok()) return k;
  if (quant) {
    k.ptr(q_scale, "q_scale", !empty) && k.ptr(kscale, "k_scale", !empty);
  } else {
    k.must_be_null(q_scale, "q_scale", "for bf16") && k.must_be_null(kscale, "k_scale", "for bf16");
  }
  return k;
}

inline Check check_topk_paged(int64_t B, int64_t N, const int64_t* seq_pos, int ratio, int kk, const void* scores,
                              int score_dtype, const void* idx, const void* ws, size_t ws_bytes) {
  Check k;
  if (B < 0 || N < 0) { k.fail(CSA_ERR_INVALID_ARG, "B and N must be >= 0"); return k; }
  if (ratio != 4 && ratio != 128) { k.fail(CSA_ERR_INVALID_ARG, "ratio must be 4 or 128, got " + i2s(ratio)); return k; }
  if (kk < 1 || kk > CSA_MAX_TOPK) { k.fail(CSA_ERR_INVALID_ARG, "k must be in [1, 2048], got " + i2s(kk)); return k; }
  if (score_dtype != CSA_F32 && score_dtype != CSA_BF16) { k.fail(CSA_ERR_UNSUPPORTED, "score_dtype must be CSA_F32 or CSA_BF16"); return k; }
  const bool empty = B == 0;
  k.ptr(scores, "scores", !empty && N > 0) && k.ptr(idx, "idx", !empty) && k.ptr(seq_pos, "seq_pos", !empty);
  if (!k.ok()) return k;
  const size_t need = topk_workspace_bytes(B, 1, N, kk, score_dtype);
  if (need > 0) {
    if (!ws || ws_bytes < need) { k.fail(CSA_ERR_WORKSPACE, "topk_select_paged needs " + i2s((int64_t)need) + " workspace bytes, got " + i2s((int64_t)ws_bytes)); return k; }
    k.ptr(ws, "workspace");
  }
  return k;
}

// Paged decode attention (heterogeneous cache): one query per sequence at
// seq_pos[b], compressed entries through a block table, the window from a ring.
inline Check check_paged(bool sparse, int64_t B, int kk, int H, int d, const void* q, const void* kv_pool,
                         int64_t n_pool, const int32_t* block_table, int64_t max_blocks, const int32_t* idx,
                         const void* win, int64_t ring, const int64_t* seq_pos, int64_t max_pos, int window,
                         float scale, const float* sink, int io_dtype, const void* out, const float* lse, int flags,
                         int rope_dims, float rope_base, const void* ws, size_t ws_bytes) {
  Check k;
  check_attn_flags(k, flags);
  if (!k.ok()) return k;
  if (!check_attn_common(k, B, 0, 0, H, d, 0, 0, window, scale, io_dtype)) return k;
  if (!check_rope(k, rope_dims, rope_base, d)) return k;
  if (sparse && (kk < 0 || kk > CSA_MAX_TOPK)) { k.fail(CSA_ERR_INVALID_ARG, "k must be in [0, 2048], got " + i2s(kk)); return k; }
  if (n_pool < 0) { k.fail(CSA_ERR_INVALID_ARG, "n_pool must be >= 0"); return k; }
  if (max_blocks < 1 || max_blocks > (int64_t{1} << 26)) { k.fail(CSA_ERR_INVALID_ARG, "max_blocks must be in [1, 2^26]"); return k; }
  if (ring < window) { k.fail(CSA_ERR_INVALID_ARG, "the window ring holds " + i2s(ring) + " rows, fewer than the window " + i2s(window)); return k; }
  if (ring & (ring - 1)) { k.fail(CSA_ERR_INVALID_ARG, "the window ring size must be a power of two, got " + i2s(ring)); return k; }
  if (max_pos < 0) { k.fail(CSA_ERR_INVALID_ARG, "max_pos must be >= 0"); return k; }
  const bool empty = (B == 0);
  k.ptr(q, "q", !empty) && k.ptr(kv_pool, "kv_pool", !empty && n_pool > 0) &&
      k.ptr(block_table, "block_table", !empty) && k.ptr(idx, "idx", sparse && !empty && kk > 0) &&
      k.ptr(win, "win", !empty) && k.ptr(seq_pos, "seq_pos", !empty) && k.ptr(out, "out", !empty) &&
      k.ptr(lse, "lse", false) && k.ptr(sink, "sink", false);
  if (!k.ok()) return k;
  if (sparse && sink) { k.fail(CSA_ERR_INVALID_ARG, "sparse attention has no sink"); return k; }
  const size_t need = (flags & CSA_ATTN_BATCH_INVARIANT) ? 0 : attn_workspace_bytes(B, 1);
  if (need > 0 && !empty) {
    if (!ws || ws_bytes < need) { k.fail(CSA_ERR_WORKSPACE, "paged attention needs " + i2s((int64_t)need) + " workspace bytes, got " + i2s((int64_t)ws_bytes)); return k; }
    k.ptr(ws, "workspace");
  }
  return k;
}

inline size_t workspace_bytes(int op, int64_t B, int64_t T, int64_t N, int kk) {
  (void)kk;
  switch (op) {
    case CSA_OP_COMPRESS: return compress_workspace_bytes(kk, B, T, N);   // (B, n_tok, c, ratio)
    case CSA_OP_TOPK: return topk_workspace_bytes(B, T, N, kk, CSA_BF16) > topk_workspace_bytes(B, T, N, kk, CSA_F32)
                                 ? topk_workspace_bytes(B, T, N, kk, CSA_BF16) : topk_workspace_bytes(B, T, N, kk, CSA_F32);
    case CSA_OP_SPARSE_ATTN:
    case CSA_OP_HCA_ATTN: return attn_workspace_bytes(B, T);
    default: return 0;
  }
}

}  // namespace csa
