// The compressor's per-entry device code (C4A / C128A pooling, RMSNorm,
// partial RoPE and quantize-on-write), shared by the compressor kernels and
// by launches of other stages that run a decode step's compressor writes
// themselves (the MXFP4 decode indexer).  See compress.hip for the method.
#pragma once
#include <cmath>
#include <type_traits>

#include "device.h"

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
                                               int64_t scale_stride, int64_t out_i = -1, float* lds = nullptr) {
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
  // LDS for the group merge and the norm sums: the launch's dynamic LDS, or
  // `lds` when the caller lends a region of its own
  extern __shared__ float smem_dyn[];
  float* const smem = lds ? lds : smem_dyn;
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

}  // namespace
}  // namespace csa
