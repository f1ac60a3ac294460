// Stages 4 and 5: shared-KV MQA over Top-k entries + window (CSA) and dense
// MQA with an attention sink over all compressed entries + window (HCA).
//
// "DeepSeek V4 结构速览" (CSA（c4a 路线）; HCA（c128a 路线）) and "DeepSeek-V4 技术
// 解读：百万 Token 上下文的新里程碑" (2.1): 64 query heads of dim 512 attend over
// one shared 512-d latent that is both key and value.  CSA attends over the
// selected entries concatenated with the 128-token raw window; HCA attends
// over every visible C128A entry and the window, with one sink logit per head
// whose value is zero.
//
// Both stages are one kernel that walks a per-query "list" of rows: first the
// compressed slots (the Top-k indices, or entries 0..V(t)-1 for the dense
// form), then the window's raw rows.  A workgroup owns one query (all 64
// heads) and a contiguous run of 32-row tiles of that list; wave w owns heads
// 16w..16w+15.
//
// Per tile (bf16 path):
//  * every thread loads 8 rows x 16 bytes (one 1 KB row per wave-wide load)
//    for the next tile into registers while the current tile is computed;
//  * the tile goes to LDS twice: row-major (padded rows) for S^T = K Q^T, and
//    as 4 groups of 8 rows transposed to [d][8 rows] for P V -- an in-register
//    8x8 transpose of bf16 makes that layout without scattered LDS writes;
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 with the wave's 16 heads' q in
//    registers.  The C layout of S^T gives lane (head j, group g) the logits of
//    rows {4g..4g+3, 16+4g..16+4g+3}; the P V MFMA takes exactly those rows as
//    lane (j, g)'s K slice, so P goes from registers into the next MFMA with no
//    data movement, as long as the transposed V groups use the same rows;
//  * online softmax in the exp2 domain (logits pre-multiplied by log2 e);
//  * O (16 heads x 512 fp32 per wave) stays in registers.
// Decode has few queries, so a query's tiles are split over several
// workgroups whose partial (max, sum, O) go to the workspace; a combine
// kernel merges them in a fixed order (bit-reproducible results).
#include "device.h"
#include "launch.h"
#include "validate.h"

namespace csa {
namespace {

constexpr int kH = 64;
constexpr int kD = 512;
constexpr int kTile = kAttnTile;            // 32 rows
constexpr int kKsStride = kD * 2 + 16;      // bytes per row of the row-major tile (padded)
constexpr float kLn2 = 0.69314718055994531f;

struct Params {
  int64_t B, T, N;
  int k;
  int ratio;
  int64_t q_pos0;
  const void* q;
  const void* kv_cmp;
  const int32_t* idx;
  const void* kv_raw;
  int64_t raw_pos0, n_raw;
  int window;
  float scale_log2;     // scale * log2(e)
  const float* sink;
  void* out;
  float* lse;
  float* ws;
  int splits;
};

struct List {
  int64_t n_cmp;   // compressed slots at the head of the list
  int64_t wstart;  // first window position
  int64_t L;       // list length
};

__device__ __forceinline__ List make_list(const Params& P, int64_t t) {
  const int64_t pos = P.q_pos0 + t;
  List l;
  l.wstart = pos - P.window + 1 > 0 ? pos - P.window + 1 : 0;
  if (P.idx) {
    l.n_cmp = P.k;
  } else {
    const int64_t v = (pos + 1) / P.ratio;
    l.n_cmp = v < P.N ? v : P.N;
  }
  l.L = l.n_cmp + (pos - l.wstart + 1);
  return l;
}

// Address of list row `p` of query (b, t), or nullptr for padding / past the end.
// `sidx` (optional) is the query's Top-k row already staged in LDS.
template <typename E>
__device__ __forceinline__ const E* row_ptr(const Params& P, int64_t b, int64_t t, const List& l, int64_t p,
                                            const int32_t* sidx = nullptr) {
  if (p >= l.L) return nullptr;
  if (p < l.n_cmp) {
    int64_t e = p;
    if (P.idx) e = sidx ? sidx[p] : P.idx[(b * P.T + t) * P.k + p];
    if (e < 0 || e >= P.N) return nullptr;
    return static_cast<const E*>(P.kv_cmp) + (b * P.N + e) * kD;
  }
  const int64_t u = l.wstart + (p - l.n_cmp) - P.raw_pos0;
  return static_cast<const E*>(P.kv_raw) + (b * P.n_raw + u) * kD;
}

__device__ __forceinline__ void split_range(const Params& P, const List& l, int split, int64_t& t0,
                                            int64_t& t1) {
  const int64_t nt = (l.L + kTile - 1) / kTile;
  const int64_t per = (nt + P.splits - 1) / P.splits;
  t0 = split * per;
  t1 = t0 + per < nt ? t0 + per : nt;
  if (t0 > t1) t0 = t1;
}

// ------------------------------------------------------------ bf16 MFMA kernel
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kTileBytes = kTile * kKsStride;   // one row-major tile in LDS

// One 1 KB latent row straight from global memory into LDS (16 bytes per lane,
// lane l's bytes land at dst + 16 l): no registers, no staging.
__device__ __forceinline__ void row_to_lds(const uint16_t* src_row, uint8_t* dst_row, int lane) {
  __builtin_amdgcn_global_load_lds(static_cast<const void*>(src_row + lane * 8),
                                   (lds_void*)(dst_row), 16, 0, 0);
}

// B operand of the P V MFMA (rows x 16 columns, k-slice of lane group g) read
// transposed from the row-major tile: within a 16-lane group, lane k points at
// row base + k/4, columns 4(k%4)..4(k%4)+3 of the 16-column block; the
// transposing read hands lane j column j of rows base..base+3.
__device__ __forceinline__ bf16x8 v_operand(const uint8_t* tile, int n, int g, int k) {
  const uint8_t* p0 = tile + (4 * g + (k >> 2)) * kKsStride + (n * 16 + 4 * (k & 3)) * 2;
  const uint8_t* p1 = p0 + 16 * kKsStride;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p1));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

#ifndef ATTN_WAVES_PER_SIMD
#define ATTN_WAVES_PER_SIMD 2
#endif
__global__ void __launch_bounds__(256, ATTN_WAVES_PER_SIMD)
attn_bf16_kernel(Params P) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* tiles = smem;                                                    // [2][32][kKsStride]
  uint32_t* rvalid = reinterpret_cast<uint32_t*>(smem + 2 * kTileBytes);    // [2][32]
  int32_t* sidx = reinterpret_cast<int32_t*>(rvalid + 2 * kTile);           // [k] Top-k row of this query

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int x16 = (lane ^ 16) << 2, x32 = (lane ^ 32) << 2;   // ds_bpermute addresses
  int hsrc[4];                                                 // lanes holding heads 4g..4g+3
#pragma unroll
  for (int i = 0; i < 4; ++i) hsrc[i] = (4 * g + i) << 2;
  const int64_t gq = blockIdx.x / P.splits;
  const int split = static_cast<int>(blockIdx.x % P.splits);
  const int64_t b = gq / P.T, t = gq % P.T;
  const List l = make_list(P, t);
  int64_t tile0, tile1;
  split_range(P, l, split, tile0, tile1);

  // Stage the slice of this query's Top-k row that this workgroup's tiles use.
  if (P.idx) {
    const int64_t p0 = tile0 * kTile;
    const int64_t p1 = tile1 * kTile < l.n_cmp ? tile1 * kTile : l.n_cmp;
    const int32_t* src = P.idx + gq * P.k;
    for (int64_t p = p0 + tid; p < p1; p += 256) sidx[p] = src[p];
    __syncthreads();
  }

  // q fragments of head 16*wid + j, d in [g*128, g*128+128)
  uint4 qf[16];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(P.q) +
                                                     ((gq * kH) + 16 * wid + j) * kD + g * 128);
#pragma unroll
    for (int s = 0; s < 16; ++s) qf[s] = qp[s];
  }

  f32x4 o[32];
#pragma unroll
  for (int n = 0; n < 32; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // The query's own raw row is always in the list: padding rows load it (and are masked).
  const uint16_t* safe_row = static_cast<const uint16_t*>(P.kv_raw) +
                             (b * P.n_raw + (P.q_pos0 + t - P.raw_pos0)) * kD;
  // wave w brings rows 8w..8w+7 of a tile
  auto issue_tile = [&](int64_t tile, int buf) {
    uint8_t* dst = tiles + buf * kTileBytes;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = 8 * wid + e;
      const uint16_t* p = row_ptr<uint16_t>(P, b, t, l, tile * kTile + r, sidx);
      row_to_lds(p ? p : safe_row, dst + r * kKsStride, lane);
      if (lane == 0) rvalid[buf * kTile + r] = p != nullptr;
    }
  };

  if (tile0 < tile1) issue_tile(tile0, 0);
  for (int64_t tile = tile0; tile < tile1; ++tile) {
    const int cur = static_cast<int>((tile - tile0) & 1);
    __builtin_amdgcn_s_waitcnt(0);   // this wave's row loads into `cur` have landed
    __syncthreads();                 // ... and every wave's; nobody still reads `cur ^ 1`
    if (tile + 1 < tile1) issue_tile(tile + 1, cur ^ 1);
    const uint8_t* Ks = tiles + cur * kTileBytes;
    const uint32_t* rv = rvalid + cur * kTile;

    // S^T = K Q^T for rows 0..15 (s0) and 16..31 (s1); the operands of step
    // s+1 are read from LDS while step s's MFMAs run
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    const uint8_t* ka = Ks + j * kKsStride + g * 256;
    uint4 a0 = *reinterpret_cast<const uint4*>(ka);
    uint4 a1 = *reinterpret_cast<const uint4*>(ka + 16 * kKsStride);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      uint4 n0 = a0, n1 = a1;
      if (s + 1 < 16) {
        n0 = *reinterpret_cast<const uint4*>(ka + (s + 1) * 16);
        n1 = *reinterpret_cast<const uint4*>(ka + 16 * kKsStride + (s + 1) * 16);
      }
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0), as_bf16x8(qf[s]), s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1), as_bf16x8(qf[s]), s1, 0, 0, 0);
      a0 = n0;
      a1 = n1;
    }
    float lg[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lg[i] = rv[4 * g + i] ? s0[i] * P.scale_log2 : -INFINITY;
      lg[4 + i] = rv[16 + 4 * g + i] ? s1[i] * P.scale_log2 : -INFINITY;
    }
    float mt = lg[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, lg[i]);
    mt = fmaxf(mt, lane_read(x16, mt));
    mt = fmaxf(mt, lane_read(x32, mt));
    const float m_new = fmaxf(m_run, mt);
    const bool none = (m_new == -INFINITY);
    const float alpha = none ? 1.f : fast_exp2(m_run - m_new);
    float p[8], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = none ? 0.f : fast_exp2(lg[i] - m_new);
      psum += p[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {   // some head's running max moved: rescale O
      float a4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a4[i] = lane_read(hsrc[i], alpha);
#pragma unroll
      for (int n = 0; n < 32; ++n) {
        o[n][0] *= a4[0]; o[n][1] *= a4[1]; o[n][2] *= a4[2]; o[n][3] *= a4[3];
      }
    }
    const uint4 pa = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));
    const bf16x8 pav = as_bf16x8(pa);
    bf16x8 vb = v_operand(Ks, 0, g, j);
#pragma unroll
    for (int n = 0; n < 32; ++n) {
      const bf16x8 vn = (n + 1 < 32) ? v_operand(Ks, n + 1, g, j) : vb;
      o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pav, vb, o[n], 0, 0, 0);
      vb = vn;
    }
  }

  // per-head totals: lanes with (lane & 15) == h hold head 16*wid + h
  float l_tot = l_run;
  l_tot += lane_read(x16, l_tot);
  l_tot += lane_read(x32, l_tot);
  const int head_j = 16 * wid + j;

  if (P.splits == 1) {
    float M = m_run;
    float zl = -INFINITY;
    if (P.sink) {
      zl = P.sink[head_j] * kLog2e;
      M = fmaxf(M, zl);
    }
    const float em = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - M);
    const float denom = l_tot * em + (P.sink ? fast_exp2(zl - M) : 0.f);
    const float f = em / denom;
    if (P.lse && g == 0) P.lse[gq * kH + head_j] = kLn2 * (M + log2f(denom));
    float f4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) f4[i] = lane_read(hsrc[i], f);
    uint16_t* out = static_cast<uint16_t*>(P.out) + (gq * kH + 16 * wid + 4 * g) * kD;
#pragma unroll
    for (int n = 0; n < 32; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) out[i * kD + n * 16 + j] = f32_to_bf16(o[n][i] * f4[i]);
  } else {
    float* w = P.ws + (gq * P.splits + split) * (kH * (kD + 2));
    float* wo = w + (16 * wid + 4 * g) * kD;
#pragma unroll
    for (int n = 0; n < 32; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) wo[i * kD + n * 16 + j] = o[n][i];
    if (g == 0) {
      w[kH * kD + head_j] = m_run;
      w[kH * kD + kH + head_j] = l_tot;
    }
  }
}

// ------------------------------------------------------------ fp32 kernel
// Plain fp32 arithmetic for fp32 I/O (small problems).  One workgroup per
// (query, group of 8 heads); 32 lanes per head, 16 dims per lane; rows are
// staged in LDS 16 at a time.
__global__ void __launch_bounds__(256)
attn_f32_kernel(Params P) {
  __shared__ float xs[16][kD];
  __shared__ uint32_t xv[16];
  const int tid = threadIdx.x;
  const int64_t gq = blockIdx.x / 8;
  const int hg = static_cast<int>(blockIdx.x % 8);
  const int64_t b = gq / P.T, t = gq % P.T;
  const int head = hg * 8 + tid / 32;
  const int part = tid % 32;
  const List l = make_list(P, t);
  float qv[16], ov[16];
  const float* qp = static_cast<const float*>(P.q) + (gq * kH + head) * kD + part * 16;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    qv[i] = qp[i];
    ov[i] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  for (int64_t base = 0; base < l.L; base += 16) {
    __syncthreads();
    for (int i = tid; i < 16 * kD; i += 256) {
      const int r = i / kD, c = i % kD;
      const float* p = row_ptr<float>(P, b, t, l, base + r);
      xs[r][c] = p ? p[c] : 0.f;
      if (c == 0) xv[r] = p != nullptr;
    }
    __syncthreads();
    for (int r = 0; r < 16; ++r) {
      if (!xv[r]) continue;
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) dot = fmaf(qv[i], xs[r][part * 16 + i], dot);
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) dot += __shfl_xor(dot, o, 32);
      const float lg = dot * P.scale_log2;
      const float mn = fmaxf(m_run, lg);
      const float a = fast_exp2(m_run - mn);
      const float pr = fast_exp2(lg - mn);
      l_run = l_run * a + pr;
#pragma unroll
      for (int i = 0; i < 16; ++i) ov[i] = ov[i] * a + pr * xs[r][part * 16 + i];
      m_run = mn;
    }
  }
  float M = m_run, zl = -INFINITY;
  if (P.sink) {
    zl = P.sink[head] * kLog2e;
    M = fmaxf(M, zl);
  }
  const float em = fast_exp2(m_run - M);
  const float denom = l_run * em + (P.sink ? fast_exp2(zl - M) : 0.f);
  const float f = em / denom;
  float* out = static_cast<float*>(P.out) + (gq * kH + head) * kD + part * 16;
#pragma unroll
  for (int i = 0; i < 16; ++i) out[i] = ov[i] * f;
  if (P.lse && part == 0) P.lse[gq * kH + head] = kLn2 * (M + log2f(denom));
}

// ------------------------------------------------------------ split combine
// One workgroup per (query, head); 128 threads x 4 dims.  Partials are merged
// in split order.
__global__ void __launch_bounds__(128)
attn_combine_kernel(Params P) {
  const int64_t gq = blockIdx.x / kH;
  const int h = static_cast<int>(blockIdx.x % kH);
  const int S = P.splits;
  const float* base = P.ws + gq * S * (kH * (kD + 2));
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, base[s * (kH * (kD + 2)) + kH * kD + h]);
  float zl = -INFINITY;
  if (P.sink) {
    zl = P.sink[h] * kLog2e;
    M = fmaxf(M, zl);
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float denom = 0.f;
  const int d0 = threadIdx.x * 4;
  for (int s = 0; s < S; ++s) {
    const float* w = base + s * (kH * (kD + 2));
    const float ms = w[kH * kD + h];
    const float e = (ms == -INFINITY) ? 0.f : fast_exp2(ms - M);
    denom += w[kH * kD + kH + h] * e;
    const float4 v = *reinterpret_cast<const float4*>(w + h * kD + d0);
    acc.x += v.x * e; acc.y += v.y * e; acc.z += v.z * e; acc.w += v.w * e;
  }
  if (P.sink) denom += fast_exp2(zl - M);
  const float f = 1.f / denom;
  uint16_t* out = static_cast<uint16_t*>(P.out) + (gq * kH + h) * kD + d0;
  uint2 pk;
  pk.x = pack_bf16x2(acc.x * f, acc.y * f);
  pk.y = pack_bf16x2(acc.z * f, acc.w * f);
  *reinterpret_cast<uint2*>(out) = pk;
  if (P.lse && threadIdx.x == 0) P.lse[gq * kH + h] = kLn2 * (M + log2f(denom));
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  if (a.B == 0 || a.T == 0) return hipSuccess;
  Params P{};
  P.B = a.B; P.T = a.T; P.N = a.N; P.k = a.k; P.ratio = a.ratio; P.q_pos0 = a.q_pos0;
  P.q = a.q; P.kv_cmp = a.kv_cmp; P.idx = a.idx; P.kv_raw = a.kv_raw;
  P.raw_pos0 = a.raw_pos0; P.n_raw = a.n_raw; P.window = a.window;
  P.scale_log2 = a.scale * kLog2e; P.sink = a.sink; P.out = a.out; P.lse = a.lse;
  P.ws = static_cast<float*>(a.ws);
  const int64_t nq = a.B * a.T;
  if (a.io_dtype == CSA_F32) {
    P.splits = 1;
    hipLaunchKernelGGL(attn_f32_kernel, dim3(static_cast<uint32_t>(nq * 8)), dim3(256), 0, s, P);
    return hipGetLastError();
  }
  // longest list over the call's queries bounds the split count
  const int64_t last = a.q_pos0 + a.T - 1;
  const int64_t wlen = last - (last - a.window + 1 > 0 ? last - a.window + 1 : 0) + 1;
  int64_t ncmp = a.idx ? a.k : (last + 1) / a.ratio;
  if (!a.idx && ncmp > a.N) ncmp = a.N;
  P.splits = attn_splits(a.B, a.T, ncmp + wlen);
  const size_t smem = 2 * kTile * kKsStride + 2 * kTile * 4 + (a.idx ? a.k * 4 : 0);
  hipLaunchKernelGGL(attn_bf16_kernel, dim3(static_cast<uint32_t>(nq * P.splits)), dim3(256), smem, s, P);
  if (P.splits > 1)
    hipLaunchKernelGGL(attn_combine_kernel, dim3(static_cast<uint32_t>(nq * kH)), dim3(128), 0, s, P);
  return hipGetLastError();
}

}  // namespace csa
