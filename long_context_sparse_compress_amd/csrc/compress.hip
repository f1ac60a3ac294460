// Stage 1: the C4A / C128A KV compressor on gfx950.
//
// "DeepSeek V4 结构速览" (核心设计; C4A Compressor) and the compression
// formula of "DeepSeek-V4技术报告解读，全适配国产算力" (2.1): each entry is a
// per-channel softmax-weighted sum of 8 raw tokens at stride 4 (C4A: the
// current block from Ca/Za, the previous block from Cb/Zb, a positional bias
// on the 8 logits) or 128 raw tokens at stride 128 (C128A), then RMSNorm and,
// when asked, partial RoPE at the entry's anchor position ("DeepSeek
// Technical Reports", Hybrid Attention, CSA; the CSA operator graph's
// RMSNorm + RoPE in "DeepSeek V4 结构速览").
//
// The work is pure streaming (C128A reads 257 rows' worth of bytes per
// entry), so the kernel is organised for HBM bandwidth:
//  * one workgroup per (sequence, entry); each thread owns VEC consecutive
//    channels and loads 16 bytes per row per tensor (fully coalesced rows);
//  * the window rows are split across G row groups that each keep an online
//    softmax state (running max, running sum, running weighted content) per
//    channel in registers, so every input byte is read exactly once;
//  * the G partial states are merged through LDS, then RMSNorm is a
//    block-wide reduction over channels.
#include <cmath>
#include <type_traits>

#include "compress_entry.h"
#include "device.h"
#include "launch.h"
#include "validate.h"

namespace csa {
namespace {

// C4A workgroups hold at most 512 threads (c / 4 channel threads x 2 row
// groups), C128A ones up to 1024; the bound sets the register budget.
template <int RATIO> constexpr int kCompressThreads = RATIO == 4 ? 512 : 1024;

template <typename TI, typename TO, int RATIO, bool SPLIT, int VEC = Vec<TI>::n, int UC = kChunkRows>
__global__ void __launch_bounds__(kCompressThreads<RATIO>)
compress_kernel(int64_t n_tok, int c, int64_t pos0,
                const TI* __restrict__ Ca, const TI* __restrict__ Za,
                const TI* __restrict__ Cb, const TI* __restrict__ Zb,
                const TI* __restrict__ pCb, const TI* __restrict__ pZb,
                const float* __restrict__ bias, const float* __restrict__ gamma, float eps,
                TO* __restrict__ out, int64_t out_stride, int G, float* __restrict__ part, int rope_R,
                double rope_l2b, int rope_anchor, void* __restrict__ out_scale, int64_t scale_stride) {
  compress_entry<TI, TO, RATIO, SPLIT, VEC, UC>(blockIdx.x, blockIdx.y, static_cast<int>(blockIdx.z),
                                       static_cast<int>(gridDim.z), n_tok, c, pos0, Ca, Za, Cb, Zb, pCb, pZb, bias,
                                       gamma, eps, out, out_stride, G, part, rope_R, rope_l2b, rope_anchor,
                                       out_scale, scale_stride);
}

// The rolling-buffer write of a decode step into the heterogeneous cache's
// pages ("DeepSeek V4 结构速览": at decode the previous block is the latest
// complete one, the current block the rolling buffer; "DeepSeek-V4技术报告解读"
// 3.2: compressed entries live in blocks of 128 raw tokens).  Workgroup b
// pools sequence b's block starting at pos0s[b] into entry pos0s[b] / RATIO,
// slot (e % 32 for C4A) of its physical block table[b][e / (32 or 1)].  A
// sequence whose position is not a block start, or whose block is absent,
// writes nothing (the whole workgroup returns before any barrier).
// One compression into pages (a call's arguments on the device).
struct PagedJobDev {
  const void *Ca, *Za, *Cb, *Zb, *pCb, *pZb;
  const float* bias;
  const float* gamma;
  void* pool;
  void* scale_pool;
  const int64_t* pos0s;
  const int32_t* table;
  int64_t n_tok, n_ent, B, n_pool, max_blocks;
  float eps;
  int c, G;
  int rope_R;
  double rope_l2b;
  int rope_anchor;
  int qfmt;   // MIXED batches: 1 fp8, 2 fp4, 0 the float type
};
constexpr int kMaxPagedJobs = 4;
struct PagedBatch {
  PagedJobDev j[kMaxPagedJobs];
};

template <typename TI, typename TO, int RATIO, int VEC, int UC>
__device__ __forceinline__ void paged_entry(const PagedJobDev& J) {
  constexpr int SH = RATIO == 4 ? 5 : 0;   // log2 entries per block
  const int64_t b = blockIdx.y;
  const int64_t i = blockIdx.x;            // entry of the chunk
  const int64_t p0 = J.pos0s[b];
  if (p0 < 0 || p0 % RATIO) return;
  const int64_t e = p0 / RATIO + i;
  if ((e >> SH) >= J.max_blocks) return;
  const int64_t blk = J.table[b * J.max_blocks + (e >> SH)];
  if (blk < 0 || blk >= J.n_pool) return;
  const int64_t row = (blk << SH) + (e & ((int64_t{1} << SH) - 1));
  const int c = J.c;
  // entry i of the chunk, written at `row` (no batch stride)
  constexpr bool kFp4 = std::is_same_v<TO, E2M1x2>;
  TO* dst = kFp4 ? reinterpret_cast<TO*>(static_cast<uint8_t*>(J.pool) + row * c / 2) : static_cast<TO*>(J.pool) + row * c;
  void* sdst = !J.scale_pool ? nullptr
               : kFp4        ? static_cast<void*>(static_cast<uint8_t*>(J.scale_pool) + row * (c / 32))
                             : static_cast<void*>(static_cast<float*>(J.scale_pool) + row);
  compress_entry<TI, TO, RATIO, false, VEC, UC>(i, b, 0, 1, J.n_tok, c, p0, static_cast<const TI*>(J.Ca),
                                       static_cast<const TI*>(J.Za), static_cast<const TI*>(J.Cb),
                                       static_cast<const TI*>(J.Zb), static_cast<const TI*>(J.pCb),
                                       static_cast<const TI*>(J.pZb), J.bias, J.gamma, J.eps, dst, 0, J.G, nullptr,
                                       J.rope_R, J.rope_l2b, J.rope_anchor, sdst, 0, 0);
}

// Up to four writes into pages in one launch (blockIdx.z picks the job; the
// paged decode step's bf16 latent and quantized indexer key together).
// MIXED: jobs writing fp8 or MXFP4 codes sit beside jobs of the float type TO.
template <typename TI, typename TO, int RATIO, bool MIXED = false, int VEC = Vec<TI>::n, int UC = kChunkRows>
__global__ void __launch_bounds__(kCompressThreads<RATIO>)
compress_paged_kernel(PagedBatch jb) {
  const PagedJobDev& J = jb.j[blockIdx.z];
  if (static_cast<int64_t>(blockIdx.x) >= J.n_ent || static_cast<int64_t>(blockIdx.y) >= J.B) return;
  if constexpr (MIXED) {
    if (J.qfmt == 1) return paged_entry<TI, uint8_t, RATIO, VEC, UC>(J);
    if (J.qfmt == 2) return paged_entry<TI, E2M1x2, RATIO, VEC, UC>(J);
  }
  paged_entry<TI, TO, RATIO, VEC, UC>(J);
}

// MIXED: some jobs write fp8 codes (quantize-on-write; their out_scale is
// set) and the others TO -- the CSA layer's bf16 latent and fp8 indexer keys
// in one launch.  The choice is per workgroup (one job each).
template <typename TI, typename TO, int RATIO, bool MIXED = false, int VEC = Vec<TI>::n, int UC = kChunkRows>
__global__ void __launch_bounds__(kCompressThreads<RATIO>)
compress_batch_kernel(CompressBatch jb) {
  const CompressJobDev& J = jb.j[blockIdx.z];
  if (static_cast<int64_t>(blockIdx.x) >= J.n_ent || static_cast<int64_t>(blockIdx.y) >= J.B) return;
  if (MIXED && J.qfmt == 1) {
    compress_entry<TI, uint8_t, RATIO, false, VEC, UC>(blockIdx.x, blockIdx.y, 0, 1, J.n_tok, J.c, J.pos0,
                                              static_cast<const TI*>(J.Ca), static_cast<const TI*>(J.Za),
                                              static_cast<const TI*>(J.Cb), static_cast<const TI*>(J.Zb),
                                              static_cast<const TI*>(J.pCb), static_cast<const TI*>(J.pZb), J.bias,
                                              J.gamma, J.eps, static_cast<uint8_t*>(J.out), J.out_stride, J.G,
                                              nullptr, J.rope_R, J.rope_l2b, J.rope_anchor, J.out_scale,
                                              J.scale_stride);
    return;
  }
  if (MIXED && J.qfmt == 2) {
    compress_entry<TI, E2M1x2, RATIO, false, VEC, UC>(blockIdx.x, blockIdx.y, 0, 1, J.n_tok, J.c, J.pos0,
                                             static_cast<const TI*>(J.Ca), static_cast<const TI*>(J.Za),
                                             static_cast<const TI*>(J.Cb), static_cast<const TI*>(J.Zb),
                                             static_cast<const TI*>(J.pCb), static_cast<const TI*>(J.pZb), J.bias,
                                             J.gamma, J.eps, static_cast<E2M1x2*>(J.out), J.out_stride, J.G,
                                             nullptr, J.rope_R, J.rope_l2b, J.rope_anchor, J.out_scale,
                                             J.scale_stride);
    return;
  }
  compress_entry<TI, TO, RATIO, false, VEC, UC>(blockIdx.x, blockIdx.y, 0, 1, J.n_tok, J.c, J.pos0,
                                       static_cast<const TI*>(J.Ca), static_cast<const TI*>(J.Za),
                                       static_cast<const TI*>(J.Cb), static_cast<const TI*>(J.Zb),
                                       static_cast<const TI*>(J.pCb), static_cast<const TI*>(J.pZb), J.bias, J.gamma,
                                       J.eps, static_cast<TO*>(J.out), J.out_stride, J.G, nullptr, J.rope_R,
                                       J.rope_l2b, J.rope_anchor, J.out_scale, J.scale_stride);
}

// Merge of the row-range states of one (entry, sequence), then RMSNorm.  One
// workgroup of c threads (one channel each) per (entry, sequence); all P
// states of a channel are loaded before any arithmetic, then combined in
// range order against their common maximum.
template <typename TO>
__global__ void __launch_bounds__(1024)
compress_merge_kernel(int64_t n_ent, int c, int P, const float* __restrict__ part,
                      const float* __restrict__ gamma, float eps, TO* __restrict__ out, int64_t out_stride,
                      int64_t pos0, int ratio, int rope_R, double rope_l2b, int rope_anchor) {
  constexpr int kMaxP = 16;
  __shared__ float red[16];
  const int ch = threadIdx.x;
  const int64_t i = blockIdx.x, b = blockIdx.y;
  const float* pp = part + (b * n_ent + i) * P * 3 * c + ch;
  float m[kMaxP], sv[kMaxP], yv[kMaxP];
#pragma unroll
  for (int p = 0; p < kMaxP; ++p) {
    const bool in = p < P;
    m[p] = in ? pp[static_cast<int64_t>(p) * 3 * c] : -INFINITY;
    sv[p] = in ? pp[static_cast<int64_t>(p) * 3 * c + c] : 0.f;
    yv[p] = in ? pp[static_cast<int64_t>(p) * 3 * c + 2 * c] : 0.f;
  }
  float M = -INFINITY;
#pragma unroll
  for (int p = 0; p < kMaxP; ++p) M = fmaxf(M, m[p]);
  float S = 0.f, Y = 0.f;
#pragma unroll
  for (int p = 0; p < kMaxP; ++p) {
    const float e = (m[p] == -INFINITY) ? 0.f : exp2_le0(m[p] - M);
    S = fmaf(sv[p], e, S);
    Y = fmaf(yv[p], e, Y);
  }
  const float y = Y / S;
  float ss = wave_sum(y * y);
  if ((ch & 63) == 0) red[ch / 64] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < (c + 63) / 64; ++w) tot += red[w];
  float o = y * rsqrtf(tot / static_cast<float>(c) + eps) * (gamma ? gamma[ch] : 1.f);
  if (__builtin_expect(rope_R > 0, 0)) {   // partial RoPE: the pair partner of channel ch is lane ch ^ 1
    const float other = __shfl_xor(o, 1, 64);
    if (ch >= c - rope_R) {
      float cs, sn;
      rope_cos_sin(pos0 + i * ratio + rope_anchor, (ch - (c - rope_R)) / 2, rope_R, rope_l2b, cs, sn);
      float x = (ch & 1) ? other : o, yv = (ch & 1) ? o : other;
      rope_pair(x, yv, cs, sn);
      o = (ch & 1) ? yv : x;
    }
  }
  TO* dst = out + b * out_stride + i * c + ch;
  if constexpr (sizeof(TO) == 4) *reinterpret_cast<float*>(dst) = o;
  else *reinterpret_cast<uint16_t*>(dst) = f32_to_bf16(o);
}

double rope_log2_base(const CompressArgs& a) { return a.rope_dims > 0 ? std::log2(static_cast<double>(a.rope_base)) : 0.0; }

// A C4A launch of fewer workgroups than this (a decode step) spreads each
// entry over c / 2 threads, each pooling all 8 rows of two channels.
constexpr int64_t kNarrowWgs = 256;
constexpr int kNarrowVec = 2;
// Each job takes the layout its own call would, so a batch computes every
// job exactly as the separate calls do (jobs of both kinds go out as two
// launches).
template <typename Args>
bool narrow_job(const Args& a) { return a.ratio == 4 && (a.n_tok / a.ratio) * a.B < kNarrowWgs; }

template <typename TI, typename TO, int RATIO, int VEC = Vec<TI>::n, int UC = kChunkRows>
hipError_t launch_vt(const CompressArgs& a, hipStream_t s) {
  constexpr int ROWS = (RATIO == 4) ? 8 : RATIO;
  const int CT = static_cast<int>(a.c / VEC);
  const int64_t n_ent = a.n_tok / RATIO;
  const int64_t n_wg = n_ent * a.B;
  const int64_t stride = a.out_batch_stride ? a.out_batch_stride : n_ent * a.c;
  const int P = compress_splits(RATIO, a.B, a.n_tok);
  const bool split = P > 1 && a.ws_bytes >= compress_workspace_bytes(RATIO, a.B, a.n_tok, a.c);
  // Row groups: enough that a thread holds at most one chunk of UC rows when
  // the workgroups are few (latency), at most 256 threads per workgroup when
  // they are many; never more groups than rows / UC.
  const int rows = split ? ROWS / P : ROWS;
  const int max_threads = (split ? n_wg * P : n_wg) >= 1024 ? 256 : 1024;
  int G = 1;
  while (G * 2 * CT <= max_threads && G * 2 * UC <= rows) G *= 2;
  const int threads = (CT * G + 63) / 64 * 64;   // whole waves: the wave reductions use every lane
  // + 64 floats: the RMSNorm sums (red[0..15]) and the fp8 amax (red_max = red + 32)
  const size_t smem = (G > 1 ? static_cast<size_t>(G / 2) * 3 * a.c : 0) * sizeof(float) + 64 * sizeof(float);
  const auto* Ca = static_cast<const TI*>(a.Ca);
  const auto* Za = static_cast<const TI*>(a.Za);
  const auto* Cb = static_cast<const TI*>(a.Cb);
  const auto* Zb = static_cast<const TI*>(a.Zb);
  const auto* pCb = static_cast<const TI*>(a.prev_Cb);
  const auto* pZb = static_cast<const TI*>(a.prev_Zb);
  if constexpr (RATIO == 128) {
    if (split) {
      float* part = static_cast<float*>(a.ws);
      const dim3 grid(static_cast<uint32_t>(n_ent), static_cast<uint32_t>(a.B), static_cast<uint32_t>(P));
      hipLaunchKernelGGL((compress_kernel<TI, TO, RATIO, true>), grid, dim3(threads), smem, s, a.n_tok,
                         static_cast<int>(a.c), a.pos0, Ca, Za, Cb, Zb, pCb, pZb, a.bias, a.gamma, a.eps,
                         static_cast<TO*>(a.out), stride, G, part, 0, 0.0, 0, nullptr, 0);
      hipLaunchKernelGGL((compress_merge_kernel<TO>), dim3(static_cast<uint32_t>(n_ent), static_cast<uint32_t>(a.B)),
                         dim3(static_cast<uint32_t>(a.c)), 0, s, n_ent, static_cast<int>(a.c), P, part, a.gamma,
                         a.eps, static_cast<TO*>(a.out), stride, a.pos0, RATIO, a.rope_dims, rope_log2_base(a),
                         a.rope_anchor);
      return hipGetLastError();
    }
  }
  const dim3 grid(static_cast<uint32_t>(n_ent), static_cast<uint32_t>(a.B), 1);
  hipLaunchKernelGGL((compress_kernel<TI, TO, RATIO, false, VEC, UC>), grid, dim3(threads), smem, s, a.n_tok,
                     static_cast<int>(a.c), a.pos0, Ca, Za, Cb, Zb, pCb, pZb, a.bias, a.gamma, a.eps,
                     static_cast<TO*>(a.out), stride, G, nullptr, a.rope_dims, rope_log2_base(a), a.rope_anchor,
                     a.out_scale, stride / a.c);
  return hipGetLastError();
}

template <typename TI, typename TO, int RATIO>
hipError_t launch_t(const CompressArgs& a, hipStream_t s) {
  if constexpr (RATIO == 4) {
    if (narrow_job(a)) return launch_vt<TI, TO, RATIO, kNarrowVec, 8>(a, s);
  }
  return launch_vt<TI, TO, RATIO>(a, s);
}

template <typename TI, typename TO, int RATIO, bool MIXED, int VEC, int UC>
hipError_t launch_batch_vt(const CompressArgs* jobs, int n, hipStream_t s) {
  constexpr int ROWS = (RATIO == 4) ? 8 : RATIO;
  CompressBatch jb{};
  int threads = 64;
  size_t smem = 0;
  int64_t gx = 1, gy = 1;
  for (int q = 0; q < n; ++q) {
    const CompressArgs& a = jobs[q];
    const int CT = static_cast<int>(a.c / VEC);
    const int64_t n_ent = a.n_tok / RATIO;
    const int max_threads = n_ent * a.B >= 1024 ? 256 : 1024;
    int G = 1;
    while (G * 2 * CT <= max_threads && G * 2 * UC <= ROWS) G *= 2;
    threads = CT * G > threads ? CT * G : threads;
    const size_t sm = (G > 1 ? static_cast<size_t>(G / 2) * 3 * a.c : 0) * sizeof(float);
    smem = sm > smem ? sm : smem;
    gx = n_ent > gx ? n_ent : gx;
    gy = a.B > gy ? a.B : gy;
    jb.j[q] = CompressJobDev{a.Ca, a.Za, a.Cb, a.Zb, a.prev_Cb, a.prev_Zb, a.bias, a.gamma, a.out, a.n_tok, a.pos0,
                             a.out_batch_stride ? a.out_batch_stride : n_ent * a.c, n_ent, a.B, a.eps,
                             static_cast<int>(a.c), G, a.rope_dims, rope_log2_base(a), a.rope_anchor, a.out_scale,
                             (a.out_batch_stride ? a.out_batch_stride : n_ent * a.c) / a.c,
                             a.out_dtype == CSA_FP8_E4M3 ? 1 : (a.out_dtype == CSA_MXFP4 ? 2 : 0)};
  }
  threads = (threads + 63) / 64 * 64;   // whole waves: the wave reductions use every lane
  hipLaunchKernelGGL((compress_batch_kernel<TI, TO, RATIO, MIXED, VEC, UC>),
                     dim3(static_cast<uint32_t>(gx), static_cast<uint32_t>(gy), static_cast<uint32_t>(n)),
                     dim3(static_cast<uint32_t>(threads)), smem + 64 * sizeof(float), s, jb);
  return hipGetLastError();
}

template <typename TI, typename TO, int RATIO, bool MIXED = false>
hipError_t launch_batch_t(const CompressArgs* jobs, int n, hipStream_t s) {
  CompressArgs nar[kMaxBatchJobs], wide[kMaxBatchJobs];
  int nn = 0, nw = 0;
  for (int q = 0; q < n; ++q) {
    if (narrow_job(jobs[q])) nar[nn++] = jobs[q];
    else wide[nw++] = jobs[q];
  }
  hipError_t e = hipSuccess;
  if constexpr (RATIO == 4) {
    if (nn) e = launch_batch_vt<TI, TO, RATIO, MIXED, kNarrowVec, 8>(nar, nn, s);
  }
  if (e == hipSuccess && nw) e = launch_batch_vt<TI, TO, RATIO, MIXED, Vec<TI>::n, kChunkRows>(wide, nw, s);
  return e;
}

template <typename TI, typename TO>
hipError_t launch_batch_r(const CompressArgs* jobs, int n, hipStream_t s) {
  return jobs[0].ratio == 4 ? launch_batch_t<TI, TO, 4>(jobs, n, s) : launch_batch_t<TI, TO, 128>(jobs, n, s);
}

template <typename TI, typename TO>
hipError_t launch_r(const CompressArgs& a, hipStream_t s) {
  return a.ratio == 4 ? launch_t<TI, TO, 4>(a, s) : launch_t<TI, TO, 128>(a, s);
}

}  // namespace

hipError_t launch_compress(const CompressArgs& a, hipStream_t s) {
  if (a.B == 0 || a.n_tok / a.ratio == 0) return hipSuccess;
  if (a.out_dtype == CSA_FP8_E4M3)   // C4A only (validated): the indexer keys
    return a.in_dtype == CSA_F32 ? launch_t<float, uint8_t, 4>(a, s) : launch_t<uint16_t, uint8_t, 4>(a, s);
  if (a.out_dtype == CSA_MXFP4)
    return a.in_dtype == CSA_F32 ? launch_t<float, E2M1x2, 4>(a, s) : launch_t<uint16_t, E2M1x2, 4>(a, s);
  if (a.in_dtype == CSA_F32)
    return a.out_dtype == CSA_F32 ? launch_r<float, float>(a, s) : launch_r<float, uint16_t>(a, s);
  return a.out_dtype == CSA_F32 ? launch_r<uint16_t, float>(a, s) : launch_r<uint16_t, uint16_t>(a, s);
}

namespace {

template <typename TI, typename TO, int RATIO, bool MIXED, int VEC, int UC>
hipError_t launch_paged_vt(const CompressPagedArgs* jobs, int n, hipStream_t s) {
  constexpr int ROWS = (RATIO == 4) ? 8 : RATIO;
  PagedBatch jb{};
  int threads = 64;
  size_t smem = 0;
  int64_t gx = 1, gy = 1;
  for (int q = 0; q < n; ++q) {
    const CompressPagedArgs& a = jobs[q];
    const int CT = static_cast<int>(a.c / VEC);
    const int64_t n_ent = a.n_tok / RATIO;
    const int max_threads = a.B * n_ent >= 1024 ? 256 : (RATIO == 4 ? 512 : 1024);
    int G = 1;
    while (G * 2 * CT <= max_threads && G * 2 * UC <= ROWS) G *= 2;
    threads = CT * G > threads ? CT * G : threads;
    const size_t sm = (G > 1 ? static_cast<size_t>(G / 2) * 3 * a.c : 0) * sizeof(float);
    smem = sm > smem ? sm : smem;
    gx = n_ent > gx ? n_ent : gx;
    gy = a.B > gy ? a.B : gy;
    const double l2b = a.rope_dims > 0 ? std::log2(static_cast<double>(a.rope_base)) : 0.0;
    jb.j[q] = PagedJobDev{a.Ca, a.Za, a.Cb, a.Zb, a.prev_Cb, a.prev_Zb, a.bias, a.gamma, a.pool, a.scale_pool, a.pos0,
                          a.block_table, a.n_tok, n_ent, a.B, a.n_pool, a.max_blocks, a.eps, static_cast<int>(a.c), G,
                          a.rope_dims, l2b, a.rope_anchor,
                          a.out_dtype == CSA_FP8_E4M3 ? 1 : (a.out_dtype == CSA_MXFP4 ? 2 : 0)};
  }
  // + 64 floats: the RMSNorm sums and the fp8 amax
  threads = (threads + 63) / 64 * 64;   // whole waves: the wave reductions use every lane
  hipLaunchKernelGGL((compress_paged_kernel<TI, TO, RATIO, MIXED, VEC, UC>),
                     dim3(static_cast<uint32_t>(gx), static_cast<uint32_t>(gy), static_cast<uint32_t>(n)),
                     dim3(static_cast<uint32_t>(threads)), smem + 64 * sizeof(float), s, jb);
  return hipGetLastError();
}

template <typename TI, typename TO, int RATIO, bool MIXED = false>
hipError_t launch_paged_t(const CompressPagedArgs* jobs, int n, hipStream_t s) {
  CompressPagedArgs nar[kMaxPagedJobs], wide[kMaxPagedJobs];
  int nn = 0, nw = 0;
  for (int q = 0; q < n; ++q) {
    if (narrow_job(jobs[q])) nar[nn++] = jobs[q];
    else wide[nw++] = jobs[q];
  }
  hipError_t e = hipSuccess;
  if constexpr (RATIO == 4) {
    if (nn) e = launch_paged_vt<TI, TO, RATIO, MIXED, kNarrowVec, 8>(nar, nn, s);
  }
  if (e == hipSuccess && nw) e = launch_paged_vt<TI, TO, RATIO, MIXED, Vec<TI>::n, kChunkRows>(wide, nw, s);
  return e;
}

// jobs share ratio and input type; quantized jobs (C4A fp8, MXFP4) may sit
// beside jobs of one float output type
template <typename TI>
hipError_t launch_paged_i(const CompressPagedArgs* jobs, int n, hipStream_t s) {
  auto quant = [](int dt) { return dt == CSA_FP8_E4M3 || dt == CSA_MXFP4; };
  int odt = -1, nq8 = 0, nq4 = 0;
  for (int q = 0; q < n; ++q) {
    if (!quant(jobs[q].out_dtype)) odt = jobs[q].out_dtype;
    nq8 += jobs[q].out_dtype == CSA_FP8_E4M3;
    nq4 += jobs[q].out_dtype == CSA_MXFP4;
  }
  if (odt < 0 && nq4 == 0) return launch_paged_t<TI, uint8_t, 4>(jobs, n, s);
  if (odt < 0 && nq8 == 0) return launch_paged_t<TI, E2M1x2, 4>(jobs, n, s);
  if (odt < 0) odt = CSA_BF16;   // fp8 and fp4 jobs only: any float type serves as the third path
  if (nq8 + nq4 > 0)
    return odt == CSA_F32 ? launch_paged_t<TI, float, 4, true>(jobs, n, s)
                          : launch_paged_t<TI, uint16_t, 4, true>(jobs, n, s);
  if (jobs[0].ratio == 4)
    return odt == CSA_F32 ? launch_paged_t<TI, float, 4>(jobs, n, s) : launch_paged_t<TI, uint16_t, 4>(jobs, n, s);
  return odt == CSA_F32 ? launch_paged_t<TI, float, 128>(jobs, n, s) : launch_paged_t<TI, uint16_t, 128>(jobs, n, s);
}

}  // namespace

hipError_t launch_compress_paged(const CompressPagedArgs* jobs, int n, hipStream_t s) {
  // jobs with nothing to write are dropped
  CompressPagedArgs live[kMaxPagedJobs];
  int m = 0;
  for (int q = 0; q < n && q < kMaxPagedJobs; ++q)
    if (jobs[q].B > 0 && jobs[q].n_pool > 0 && jobs[q].n_tok / jobs[q].ratio > 0) live[m++] = jobs[q];
  if (m == 0) return hipSuccess;
  return live[0].in_dtype == CSA_F32 ? launch_paged_i<float>(live, m, s) : launch_paged_i<uint16_t>(live, m, s);
}

hipError_t launch_compress_batch(const CompressArgs* jobs, int n, hipStream_t s) {
  // jobs with nothing to write are dropped; the rest share ratio and dtypes
  CompressArgs live[kMaxBatchJobs];
  int m = 0;
  for (int q = 0; q < n; ++q)
    if (jobs[q].B > 0 && jobs[q].n_tok / jobs[q].ratio > 0) live[m++] = jobs[q];
  if (m == 0) return hipSuccess;
  // quantized jobs (fp8, fp4) may sit beside jobs of one float type
  auto quant = [](int dt) { return dt == CSA_FP8_E4M3 || dt == CSA_MXFP4; };
  int odt = -1;
  int nq8 = 0, nq4 = 0;
  for (int q = 0; q < m; ++q) {
    if (!quant(live[q].out_dtype)) odt = live[q].out_dtype;
    nq8 += live[q].out_dtype == CSA_FP8_E4M3;
    nq4 += live[q].out_dtype == CSA_MXFP4;
  }
  const CompressArgs& a = live[0];
  if (odt < 0 && nq4 == 0)
    return a.in_dtype == CSA_F32 ? launch_batch_t<float, uint8_t, 4>(live, m, s)
                                 : launch_batch_t<uint16_t, uint8_t, 4>(live, m, s);
  if (odt < 0 && nq8 == 0)
    return a.in_dtype == CSA_F32 ? launch_batch_t<float, E2M1x2, 4>(live, m, s)
                                 : launch_batch_t<uint16_t, E2M1x2, 4>(live, m, s);
  if (odt < 0) odt = CSA_BF16;   // fp8 and fp4 jobs only: any float type serves as the third path
  if (nq8 + nq4 > 0) {   // C4A (validated): float outputs with quantized ones
    if (a.in_dtype == CSA_F32)
      return odt == CSA_F32 ? launch_batch_t<float, float, 4, true>(live, m, s)
                            : launch_batch_t<float, uint16_t, 4, true>(live, m, s);
    return odt == CSA_F32 ? launch_batch_t<uint16_t, float, 4, true>(live, m, s)
                          : launch_batch_t<uint16_t, uint16_t, 4, true>(live, m, s);
  }
  if (a.in_dtype == CSA_F32)
    return odt == CSA_F32 ? launch_batch_r<float, float>(live, m, s) : launch_batch_r<float, uint16_t>(live, m, s);
  return odt == CSA_F32 ? launch_batch_r<uint16_t, float>(live, m, s) : launch_batch_r<uint16_t, uint16_t>(live, m, s);
}

}  // namespace csa
