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

#include "device.h"
#include "launch.h"
#include "validate.h"

namespace csa {
namespace {

template <typename T> struct Vec;
template <> struct Vec<float> { static constexpr int n = 4; };
template <> struct Vec<uint16_t> { static constexpr int n = 8; };

// VEC consecutive elements of T as raw bytes (16, 8 or 4), converted when used.
template <int BYTES> struct RawBytes;
template <> struct RawBytes<16> { using type = uint4; };
template <> struct RawBytes<8> { using type = uint2; };
template <> struct RawBytes<4> { using type = uint32_t; };
template <typename T, int VEC> using Raw = typename RawBytes<VEC * static_cast<int>(sizeof(T))>::type;

template <typename T, int VEC>
__device__ __forceinline__ void unpack_raw(const Raw<T, VEC>& r, float* f) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(&r);
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) f[v] = __uint_as_float(w[v]);
  } else {
#pragma unroll
    for (int v = 0; v < VEC / 2; ++v) {
      f[2 * v] = __uint_as_float(w[v] << 16);
      f[2 * v + 1] = __uint_as_float(w[v] & 0xffff0000u);
    }
  }
}

// VEC consecutive fp32 values (VEC = 2, 4 or 8).
template <int VEC>
__device__ __forceinline__ void load_f32(const float* p, float* f) {
  if constexpr (VEC % 4 == 0) {
#pragma unroll
    for (int v = 0; v < VEC; v += 4) {
      const float4 q = *reinterpret_cast<const float4*>(p + v);
      f[v] = q.x; f[v + 1] = q.y; f[v + 2] = q.z; f[v + 3] = q.w;
    }
  } else {
    const float2 q = *reinterpret_cast<const float2*>(p);
    f[0] = q.x; f[1] = q.y;
  }
}

template <typename T>
__device__ __forceinline__ void store_vec(T* p, const float* f);
template <>
__device__ __forceinline__ void store_vec<float>(float* p, const float* f) {
  *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
}
template <>
__device__ __forceinline__ void store_vec<uint16_t>(uint16_t* p, const float* f) {
  uint4 v;
  v.x = pack_bf16x2(f[0], f[1]);
  v.y = pack_bf16x2(f[2], f[3]);
  v.z = pack_bf16x2(f[4], f[5]);
  v.w = pack_bf16x2(f[6], f[7]);
  *reinterpret_cast<uint4*>(p) = v;
}
// A thread's VEC output channels (VEC = 2, 4 or 8) in one store.
template <typename TO, int VEC>
__device__ __forceinline__ void store_out(TO* p, const float* f) {
  if constexpr (sizeof(TO) == 4) {
    if constexpr (VEC % 4 == 0) {
#pragma unroll
      for (int i = 0; i < VEC; i += 4) store_vec<float>(reinterpret_cast<float*>(p) + i, f + i);
    } else {
      *reinterpret_cast<float2*>(p) = make_float2(f[0], f[1]);
    }
  } else {
    if constexpr (VEC == 8) {
      store_vec<uint16_t>(reinterpret_cast<uint16_t*>(p), f);
    } else if constexpr (VEC == 4) {
      uint2 v;
      v.x = pack_bf16x2(f[0], f[1]);
      v.y = pack_bf16x2(f[2], f[3]);
      *reinterpret_cast<uint2*>(p) = v;
    } else {
      *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(f[0], f[1]);
    }
  }
}

// Output type of MXFP4 quantize-on-write: two E2M1 elements per byte (the
// element pointer of an entry then counts bytes of c / 2).
struct E2M1x2 {
  uint8_t b;
};

constexpr int kChunkRows = 4;   // rows per thread whose loads are in flight together
constexpr int kMaxRopePairs = 512;   // c <= 1024

struct Online {
  float m, s, y;   // running max (log2 domain), sum of weights, weighted content
};

// exp2 of a non-positive argument: v_exp_f32 directly.  A result below the
// smallest normal flushes to zero instead of a denormal, an absolute change
// of < 2^-126 to weights whose largest is 1.
__device__ __forceinline__ float exp2_le0(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void online_merge(Online& st, const Online& o) {
  if (o.m == -INFINITY) return;
  if (st.m == -INFINITY) { st = o; return; }
  const float mn = fmaxf(st.m, o.m);
  const float a = exp2_le0(st.m - mn);
  const float b = exp2_le0(o.m - mn);
  st.s = st.s * a + o.s * b;
  st.y = st.y * a + o.y * b;
  st.m = mn;
}

// One workgroup per (entry i, sequence b) -- or, with SPLIT, per (entry,
// sequence, row range z) when there are too few entries to fill the chip.
// blockDim.x = CT * G with CT = c / VEC channel threads and G (a power of
// two) row groups; group g owns rows rlo + g, rlo + g + G, ... of the range.
// Every row slot of a chunk is loaded unconditionally (a missing row reads a
// harmless in-range address and is masked), so all loads of a chunk,
// including its bias rows, are in flight together.
// Entry i of sequence b (rows of range z of nz), by a workgroup of at least
// CT * G threads (threads past that only join the barriers).  VEC channels a
// thread (16-byte row loads by default) and chunks of UC rows.  Few
// workgroups (a decode step) take VEC = 2 and UC = 8 with one row group: each
// thread then pools all 8 rows of its two channels with no merge, and the
// work of an entry spreads over four times the threads.
template <typename TI, typename TO, int RATIO, bool SPLIT, int VEC = Vec<TI>::n, int UC = kChunkRows>
__device__ __forceinline__ void compress_entry(int64_t i, int64_t b, int z, int nz, int64_t n_tok, int c, int64_t pos0,
                                               const TI* __restrict__ Ca, const TI* __restrict__ Za,
                                               const TI* __restrict__ Cb, const TI* __restrict__ Zb,
                                               const TI* __restrict__ pCb, const TI* __restrict__ pZb,
                                               const float* __restrict__ bias, const float* __restrict__ gamma,
                                               float eps, TO* __restrict__ out, int64_t out_stride, int G,
                                               float* __restrict__ part, int rope_R, double rope_l2b,
                                               int rope_anchor, void* __restrict__ out_scale,
                                               int64_t scale_stride, int64_t out_i = -1) {
  const int64_t io = out_i >= 0 ? out_i : i;   // where the entry is written (a paged row: 0 from its row)
  constexpr int ROWS = (RATIO == 4) ? 8 : RATIO;
  static_assert(VEC % 2 == 0 && 32 % VEC == 0 && UC <= ROWS, "whole RoPE pairs, whole MXFP4 blocks");
  const int CT = c / VEC;
  const int tid = threadIdx.x;
  const int ct = tid % CT;
  const int g = tid / CT;
  const int ch0 = ct * VEC;
  const int rows_per = ROWS / nz;
  const int rlo = z * rows_per, rhi = g < G ? rlo + rows_per : rlo;   // idle threads own no rows

  float gm[VEC];   // RMSNorm gain, fetched while the rows load
  if (!SPLIT && g == 0) {
    if (gamma) {
      load_f32<VEC>(gamma + ch0, gm);
    } else {
#pragma unroll
      for (int v = 0; v < VEC; ++v) gm[v] = 1.f;
    }
  }

  Online st[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) st[v] = Online{-INFINITY, 0.f, 0.f};

  // Partial RoPE (cos, sin) of the entry's R/2 channel pairs at its anchor
  // position: one pair per thread, into LDS, before the rows stream in (kept
  // in registers through the loop they would push it past the register limit
  // of 1024-thread workgroups; formed after it by the few threads that own
  // them, their latency would add up).  Read after the RMSNorm barrier.
  __shared__ float2 rope_tab[kMaxRopePairs];
  if (!SPLIT && __builtin_expect(rope_R > 0, 0)) {
    for (int p = tid; p < rope_R / 2; p += blockDim.x) {
      float cs, sn;
      rope_cos_sin(pos0 + i * RATIO + rope_anchor, p, rope_R, rope_l2b, cs, sn);
      rope_tab[p] = make_float2(cs, sn);
    }
  }


  const int64_t seq = b * n_tok * c;
  for (int r0 = rlo + g; r0 < rhi; r0 += G * UC) {
    Raw<TI, VEC> zl[UC], xl[UC];    // raw row slices; converted when consumed
    float bl[UC][VEC];
    bool have[UC];
#pragma unroll
    for (int u = 0; u < UC; ++u) {
      const int r = r0 + u * G;
      const bool in = r < rhi;
      const int rr = in ? r : rlo;
      const TI* zp;
      const TI* xp;
      bool ok = true;
      if constexpr (RATIO == 128) {
        const int64_t tok = i * RATIO + rr;
        zp = Za + seq + tok * c + ch0;
        xp = Ca + seq + tok * c + ch0;
      } else {
        // rows 0..3: the current block; 4..7: the block before it, from
        // this chunk (i > 0), from prev_* (i == 0, pos0 > 0) or absent
        const bool cur = rr < 4;
        const int64_t tok = cur ? i * 4 + rr : i * 4 - 4 + (rr - 4);
        const bool here = cur || i > 0;
        const int64_t off = (b * 4 + (rr & 3)) * c + ch0;
        ok = here || pos0 > 0;
        const TI* zs = cur ? Za : Zb;
        const TI* xs = cur ? Ca : Cb;
        zp = here ? zs + seq + tok * c + ch0 : (pos0 > 0 ? pZb + off : Za + seq + ch0);
        xp = here ? xs + seq + tok * c + ch0 : (pos0 > 0 ? pCb + off : Ca + seq + ch0);
      }
      zl[u] = *reinterpret_cast<const Raw<TI, VEC>*>(zp);
      xl[u] = *reinterpret_cast<const Raw<TI, VEC>*>(xp);
      load_f32<VEC>(bias + static_cast<int64_t>(rr) * c + ch0, bl[u]);
      have[u] = in && ok;
    }
    // logits of the chunk in the log2 domain, and their per-channel max
    float lg[UC][VEC];
    float cm[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) cm[v] = -INFINITY;
#pragma unroll
    for (int u = 0; u < UC; ++u) {
      float zf[VEC];
      unpack_raw<TI, VEC>(zl[u], zf);
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        lg[u][v] = have[u] ? (zf[v] + bl[u][v]) * kLog2e : -INFINITY;
        cm[v] = fmaxf(cm[v], lg[u][v]);
      }
    }
    // fold the chunk into the running state: one rescale per chunk, one exp per row
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      if (cm[v] > st[v].m) {
        const float a = (st[v].m == -INFINITY) ? 0.f : exp2_le0(st[v].m - cm[v]);
        st[v].s *= a;
        st[v].y *= a;
        st[v].m = cm[v];
      }
    }
#pragma unroll
    for (int u = 0; u < UC; ++u) {
      float xf[VEC];
      unpack_raw<TI, VEC>(xl[u], xf);
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const float p = have[u] ? exp2_le0(lg[u][v] - st[v].m) : 0.f;
        st[v].s += p;
        st[v].y = fmaf(p, xf[v], st[v].y);
      }
    }
  }

  // Tree merge of the G row groups through LDS: at each level the upper half
  // of the remaining groups hands its states to the lower half.
  extern __shared__ float smem[];
  for (int half = G >> 1; half >= 1; half >>= 1) {
    float* base = smem + static_cast<int64_t>(g - half) * 3 * c;
    if (g >= half && g < 2 * half) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        base[ch0 + v] = st[v].m;
        base[c + ch0 + v] = st[v].s;
        base[2 * c + ch0 + v] = st[v].y;
      }
    }
    __syncthreads();
    if (g < half) {
      const float* src = smem + static_cast<int64_t>(g) * 3 * c;
#pragma unroll
      for (int v = 0; v < VEC; ++v)
        online_merge(st[v], Online{src[ch0 + v], src[c + ch0 + v], src[2 * c + ch0 + v]});
    }
    __syncthreads();
  }

  if constexpr (SPLIT) {
    // this row range's state, [entry][range][m | s | y][c], merged by compress_merge_kernel
    if (g == 0) {
      const int64_t n_ent = n_tok / RATIO;
      float* pp = part + ((b * n_ent + i) * nz + z) * 3 * c + ch0;
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        pp[v] = st[v].m;
        pp[c + v] = st[v].s;
        pp[2 * c + v] = st[v].y;
      }
    }
    return;
  }

  // RMSNorm over the c channels (group 0 threads hold them all).
  float y[VEC];
  float ss = 0.f;
  if (g == 0) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      y[v] = st[v].y / st[v].s;
      ss += y[v] * y[v];
    }
  }
  ss = wave_sum(g == 0 ? ss : 0.f);
  float* red = smem;
  const int wid = tid / 64;
  const int nw = (blockDim.x + 63) / 64;
  if ((tid & 63) == 0) red[wid] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < nw; ++w) tot += red[w];
  if constexpr (std::is_same_v<TO, E2M1x2>) {
    // Quantize-on-write to MXFP4 (OCP MX v1.0): per block of 32 channels --
    // 32 / VEC neighbouring channel threads, i.e. lanes -- the shared exponent
    // E = floor(log2 amax) - 2 read off amax's float bits (E8M0 = E + 127,
    // clipped to [0, 254]), elements o * 2^-E (exact) rounded to E2M1, two
    // per byte with the even channel in the low nibble.
    if (g != 0) return;
    const float inv = rsqrtf(tot / static_cast<float>(c) + eps);
    float o[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) o[v] = y[v] * inv * gm[v];
    if (__builtin_expect(rope_R > 0, 0) && ch0 + VEC > c - rope_R) {
#pragma unroll
      for (int v = 0; v < VEC; v += 2) {
        if (ch0 + v >= c - rope_R) {
          const float2 k = rope_tab[(ch0 + v - (c - rope_R)) / 2];
          rope_pair(o[v], o[v + 1], k.x, k.y);
        }
      }
    }
    float am = 0.f;
#pragma unroll
    for (int v = 0; v < VEC; ++v) am = fmaxf(am, fabsf(o[v]));
#pragma unroll
    for (int m = 1; m < 32 / VEC; m <<= 1) am = fmaxf(am, __shfl_xor(am, m, 64));
    int E = am > 0.f ? static_cast<int>((__float_as_uint(am) >> 23) & 0xffu) - 129 : -127;
    E = E < -127 ? -127 : (E > 127 ? 127 : E);
    uint32_t word = 0;
#pragma unroll
    for (int v = 0; v < VEC; ++v) word |= f32_to_e2m1(ldexpf(o[v], -E)) << (4 * v);
    uint8_t* dst = reinterpret_cast<uint8_t*>(out) + (b * out_stride + io * c + ch0) / 2;
    if constexpr (VEC == 8) *reinterpret_cast<uint32_t*>(dst) = word;
    else if constexpr (VEC == 4) *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>(word);
    else *dst = static_cast<uint8_t>(word);
    if (ct % (32 / VEC) == 0)
      static_cast<uint8_t*>(out_scale)[(b * scale_stride + io) * (c / 32) + ch0 / 32] = static_cast<uint8_t>(E + 127);
    return;
  }
  if constexpr (std::is_same_v<TO, uint8_t>) {
    // Quantize-on-write: E4M3 codes with one fp32 scale per entry, amax / 448
    // over the entry's normalised (and rotated) channels -- a second block
    // reduction, which every thread joins -- and each code from the fp32
    // quotient o / scale.
    float o[VEC];
    float am = 0.f;
    if (g == 0) {
      const float inv = rsqrtf(tot / static_cast<float>(c) + eps);
#pragma unroll
      for (int v = 0; v < VEC; ++v) o[v] = y[v] * inv * gm[v];
      if (__builtin_expect(rope_R > 0, 0) && ch0 + VEC > c - rope_R) {
#pragma unroll
        for (int v = 0; v < VEC; v += 2) {
          if (ch0 + v >= c - rope_R) {
            const float2 k = rope_tab[(ch0 + v - (c - rope_R)) / 2];
            rope_pair(o[v], o[v + 1], k.x, k.y);
          }
        }
      }
#pragma unroll
      for (int v = 0; v < VEC; ++v) am = fmaxf(am, fabsf(o[v]));
    }
    am = wave_max(am);
    float* red_max = smem + 32;   // red holds at most 16 wave sums
    if ((tid & 63) == 0) red_max[wid] = am;
    __syncthreads();
    float amax = 0.f;
    for (int w = 0; w < nw; ++w) amax = fmaxf(amax, red_max[w]);
    if (g != 0) return;
    const float scale = amax > 0.f ? amax / 448.f : 1.f;
    uint32_t word[(VEC + 3) / 4] = {};
#pragma unroll
    for (int v = 0; v < VEC; ++v) word[v / 4] |= f32_to_e4m3(o[v] / scale) << (8 * (v % 4));
    uint8_t* dst = reinterpret_cast<uint8_t*>(out + b * out_stride + io * c + ch0);
    if constexpr (VEC == 8) *reinterpret_cast<uint2*>(dst) = make_uint2(word[0], word[1]);
    else if constexpr (VEC == 4) *reinterpret_cast<uint32_t*>(dst) = word[0];
    else *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>(word[0]);
    if (ct == 0) static_cast<float*>(out_scale)[b * scale_stride + io] = scale;
    return;
  }
  if (g != 0) return;
  const float inv = rsqrtf(tot / static_cast<float>(c) + eps);
  float o[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) o[v] = y[v] * inv * gm[v];
  // partial RoPE at the entry's anchor position; a thread's VEC channels hold
  // whole pairs (the rotated part starts at an even channel)
  if (__builtin_expect(rope_R > 0, 0) && ch0 + VEC > c - rope_R) {
#pragma unroll
    for (int v = 0; v < VEC; v += 2) {
      if (ch0 + v >= c - rope_R) {
        const float2 k = rope_tab[(ch0 + v - (c - rope_R)) / 2];
        rope_pair(o[v], o[v + 1], k.x, k.y);
      }
    }
  }
  store_out<TO, VEC>(out + b * out_stride + io * c + ch0, o);
}

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

// Several compressions of one ratio and dtype pair in one launch (blockIdx.z
// picks the job); a job's workgroups past its own grid return at once.
struct CompressJobDev {
  const void *Ca, *Za, *Cb, *Zb, *pCb, *pZb;
  const float* bias;
  const float* gamma;
  void* out;
  int64_t n_tok, pos0, out_stride, n_ent, B;
  float eps;
  int c, G;
  int rope_R;
  double rope_l2b;
  int rope_anchor;
  void* out_scale;        // quantized output: fp32 scale per entry (fp8), E8M0 per 32 channels (fp4)
  int64_t scale_stride;
  int qfmt;               // MIXED batches: 1 fp8, 2 fp4, 0 the float type
};
constexpr int kMaxBatchJobs = 4;
struct CompressBatch {
  CompressJobDev j[kMaxBatchJobs];
};

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
