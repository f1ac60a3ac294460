// Hierarchical sparse indexer: scores of a per-query candidate pool.
//
// "DeepSeek Technical Reports" (DeepSeek-V4.1, CSA2: Cross-Layer KV and
// Index Reuse; Hierarchical Sparse Indexer): a full indexer pass over the whole context
// gives each query a large candidate pool; later Reindex layers score, with
// their own query, only the entries of that pool.  The score is the indexer
// equation of "DeepSeek Technical Reports" (DSA):
//   I[t, j] = sum_h w[t,h] * ReLU(q[t,h] . k[pool[t,j]]).
//
// Unlike the full indexer, every query gathers its own key rows, so nothing
// is shared between queries: the kernel is a gathered GEMV per query, bound
// by the key bytes in decode.  The 64 heads are the MFMA M dimension and 16
// gathered rows the N dimension; lane l supplies row l % 16 and the K range
// 32 (l / 16) .. + 31 of the 128 key dims in the low-precision forms (one
// v_mfma_scale_f32_16x16x128_f8f6f4 per head block: E4M3 rows of 128 bytes,
// or MXFP4 rows of 64 bytes whose E8M0 block scales go to the instruction),
// and dims 8 (l / 16) + 32 s .. + 7 of k-step s in bf16 (four
// v_mfma_f32_16x16x32_bf16).  A wave scores chunks of 64 slots (four groups
// of 16) and has every key load of a chunk in flight before its first MFMA.
// q (64 heads x 128 dims) sits in registers as the A operand.  ReLU * w is
// summed over each lane's heads in registers, then over the four lane groups
// of a row.  The fp8 forms' positive row scales come out of the ReLU: the
// query's fold into the head weights, the key row's multiplies the sum.
#include "device.h"
#include "launch.h"

namespace csa {
namespace {

constexpr int kPoolHeads = 64, kPoolDim = 128;
constexpr int kChunk = 64, kWavesPerGroup = 4;   // slots per chunk (four groups of 16)

template <typename TS> __device__ __forceinline__ TS to_score(float v);
template <> __device__ __forceinline__ float to_score<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t to_score<uint16_t>(float v) { return f32_to_bf16(v); }

// Bytes of one q / key row, and the 16-byte words of it each lane holds.
template <int QK> struct PoolRow;
template <> struct PoolRow<CSA_BF16> {
  static constexpr int kBytes = 256, kWords = 4;
  __device__ static constexpr int offset(int s, int g) { return 64 * s + 16 * g; }   // k-step s, dims 32 s + 8 g
};
template <> struct PoolRow<CSA_FP8_E4M3> {
  static constexpr int kBytes = 128, kWords = 2;
  __device__ static constexpr int offset(int s, int g) { return 32 * g + 16 * s; }   // dims 32 g .. 32 g + 31
};
template <> struct PoolRow<CSA_MXFP4> {
  static constexpr int kBytes = 64, kWords = 1;
  __device__ static constexpr int offset(int, int g) { return 16 * g; }              // MX block g
};

// C += A B for one 16-head block against one group of 16 rows.
template <int QK>
__device__ __forceinline__ f32x4 pool_qk(const uint4 (&a)[PoolRow<QK>::kWords], const uint4 (&k)[PoolRow<QK>::kWords],
                                         int sa, int sb) {
  f32x4 c = {0.f, 0.f, 0.f, 0.f};
  if constexpr (QK == CSA_BF16) {
#pragma unroll
    for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[s]), as_bf16x8(k[s]), c, 0, 0, 0);
  } else if constexpr (QK == CSA_FP8_E4M3) {
    const i32x8 av = {(int)a[0].x, (int)a[0].y, (int)a[0].z, (int)a[0].w, (int)a[1].x, (int)a[1].y, (int)a[1].z, (int)a[1].w};
    const i32x8 bv = {(int)k[0].x, (int)k[0].y, (int)k[0].z, (int)k[0].w, (int)k[1].x, (int)k[1].y, (int)k[1].z, (int)k[1].w};
    c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, 127, 0, 127);
  } else {
    const i32x8 av = {(int)a[0].x, (int)a[0].y, (int)a[0].z, (int)a[0].w, 0, 0, 0, 0};
    const i32x8 bv = {(int)k[0].x, (int)k[0].y, (int)k[0].z, (int)k[0].w, 0, 0, 0, 0};
    c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, sa, 0, sb);
  }
  return c;
}

// A wave scores NCH consecutive chunks of 64 slots.  NCH = 1 spreads a few
// queries' pools over many workgroups (decode); NCH = 8 keeps q, loaded
// once, over 512 slots when there are queries enough to fill the chip
// (prefill), with the next chunk's key rows in flight while a chunk computes.
template <typename TS, int NCH, int QK>
__global__ void __launch_bounds__(256)
index_pool_kernel(int64_t T, int64_t N, int64_t P, int64_t nblk, const uint8_t* __restrict__ q,
                  const void* __restrict__ q_scale, const float* __restrict__ w, const uint8_t* __restrict__ keys,
                  const void* __restrict__ k_scale, const int32_t* __restrict__ pool, TS* __restrict__ scores) {
  using R = PoolRow<QK>;
  constexpr int KW = R::kWords, RB = R::kBytes;
  // all slot runs of one query on one XCD: its q and its sequence's keys
  // share that XCD's L2
  const uint32_t wg = xcd_swizzle(blockIdx.x, gridDim.x);
  const int64_t gq = wg / nblk;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t j0 = (static_cast<int64_t>(wg % nblk) * kWavesPerGroup + wid) * (NCH * kChunk);
  if (j0 >= P) return;   // no barriers below
  const int r = lane & 15, g = lane >> 4;
  const int64_t b = gq / T;

  // this lane's row of every group of 16 slots of the run; empty and
  // out-of-range slots read nothing
  const int32_t* prow = pool + gq * P;
  int32_t id[NCH * 4];
#pragma unroll
  for (int u = 0; u < NCH * 4; ++u) {
    const int64_t j = j0 + 16 * u + r;
    const int32_t v = j < P ? prow[j] : -1;
    id[u] = v >= 0 && v < N ? v : -1;
  }
  const int64_t krow0 = b * N;
  uint4 kf[2][4][KW];
  float kr[2][4];   // fp8: the key rows' scales
  int ksb[2][4];    // MXFP4: this lane's E8M0 block scale of each row
  auto load_chunk = [&](int c, int slot) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int32_t e = id[4 * c + u];
      const uint8_t* row = keys + (krow0 + (e >= 0 ? e : 0)) * RB;
#pragma unroll
      for (int s = 0; s < KW; ++s)
        kf[slot][u][s] = e >= 0 ? *reinterpret_cast<const uint4*>(row + R::offset(s, g)) : make_uint4(0, 0, 0, 0);
      if constexpr (QK == CSA_FP8_E4M3) kr[slot][u] = e >= 0 ? static_cast<const float*>(k_scale)[krow0 + e] : 0.f;
      if constexpr (QK == CSA_MXFP4)
        ksb[slot][u] = e >= 0 ? static_cast<const uint8_t*>(k_scale)[(krow0 + e) * 4 + g] : 127;
    }
  };
  load_chunk(0, 0);

  // q as the A operand: head block hb -> head 16 hb + r, the same K range as the keys
  const uint8_t* qq = q + gq * kPoolHeads * RB;
  uint4 qf[4][KW];
  int qsb[4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
#pragma unroll
    for (int s = 0; s < KW; ++s) qf[hb][s] = *reinterpret_cast<const uint4*>(qq + (16 * hb + r) * RB + R::offset(s, g));
    qsb[hb] = QK == CSA_MXFP4 ? static_cast<const uint8_t*>(q_scale)[(gq * kPoolHeads + 16 * hb + r) * 4 + g] : 127;
  }
  // head weights of this lane's C rows: heads 16 hb + 4 g + i (fp8: times the query row scales)
  float4 wv[4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    wv[hb] = *reinterpret_cast<const float4*>(w + gq * kPoolHeads + 16 * hb + 4 * g);
    if constexpr (QK == CSA_FP8_E4M3) {
      const float4 s4 = *reinterpret_cast<const float4*>(static_cast<const float*>(q_scale) + gq * kPoolHeads + 16 * hb + 4 * g);
      wv[hb].x *= s4.x; wv[hb].y *= s4.y; wv[hb].z *= s4.z; wv[hb].w *= s4.w;
    }
  }

  TS* out = scores + gq * P;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (c + 1 < NCH) load_chunk(c + 1, (c + 1) & 1);   // masked past the pool: no traffic
    const int cur = c & 1;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float acc = 0.f;
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        const f32x4 cc = pool_qk<QK>(qf[hb], kf[cur][u], qsb[hb], QK == CSA_MXFP4 ? ksb[cur][u] : 127);
        // C[4 g + i][r]: head 16 hb + 4 g + i against row r
        acc += wv[hb].x * fmaxf(cc[0], 0.f) + wv[hb].y * fmaxf(cc[1], 0.f) + wv[hb].z * fmaxf(cc[2], 0.f) +
               wv[hb].w * fmaxf(cc[3], 0.f);
      }
      acc = pair_sum16(acc, acc);
      acc = pair_sum32(acc, acc);
      if constexpr (QK == CSA_FP8_E4M3) acc *= kr[cur][u];
      const int64_t j = j0 + kChunk * c + 16 * u + r;
      if (g == 0 && j < P) out[j] = to_score<TS>(id[4 * c + u] >= 0 ? acc : -INFINITY);
    }
  }
}

template <typename TS, int NCH, int QK>
void launch_pool_t(const IndexPoolArgs& a, hipStream_t s) {
  const int64_t per_wg = static_cast<int64_t>(kWavesPerGroup) * NCH * kChunk;
  const int64_t nblk = (a.P + per_wg - 1) / per_wg;
  hipLaunchKernelGGL((index_pool_kernel<TS, NCH, QK>), dim3(static_cast<uint32_t>(a.B * a.T * nblk)), dim3(256), 0, s,
                     a.T, a.N, a.P, nblk, static_cast<const uint8_t*>(a.q), a.q_scale, a.w,
                     static_cast<const uint8_t*>(a.k), a.k_scale, a.pool, static_cast<TS*>(a.scores));
}

template <typename TS, int QK>
void launch_pool_s(const IndexPoolArgs& a, hipStream_t s) {
  // long runs only when the queries alone give about four workgroups per CU
  const int64_t long_wgs = a.B * a.T * ((a.P + 2047) / 2048);
  if (long_wgs >= 1024) launch_pool_t<TS, 8, QK>(a, s);
  else launch_pool_t<TS, 1, QK>(a, s);
}

template <typename TS>
void launch_pool_d(const IndexPoolArgs& a, hipStream_t s) {
  if (a.qk_dtype == CSA_FP8_E4M3) launch_pool_s<TS, CSA_FP8_E4M3>(a, s);
  else if (a.qk_dtype == CSA_MXFP4) launch_pool_s<TS, CSA_MXFP4>(a, s);
  else launch_pool_s<TS, CSA_BF16>(a, s);
}

}  // namespace

hipError_t launch_index_pool(const IndexPoolArgs& a, hipStream_t s) {
  if (a.B == 0 || a.T == 0 || a.P == 0) return hipSuccess;
  if (a.score_dtype == CSA_F32) launch_pool_d<float>(a, s);
  else launch_pool_d<uint16_t>(a, s);
  return hipGetLastError();
}

}  // namespace csa
