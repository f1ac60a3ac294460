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
// gathered rows the N dimension (v_mfma_f32_16x16x32_bf16, four k-steps of 32
// over the 128 key dims): lane l supplies row l % 16, dims 8(l/16)..+7 of
// each k-step -- one 16-byte load per k-step, the 4 lanes of a row covering
// 64 contiguous bytes.  A wave scores chunks of 64 slots (four groups of 16)
// and has every key load of a chunk in flight before its first MFMA.  q (64
// heads x 128 dims) sits in registers as the A operand.  ReLU * w is summed
// over each lane's heads in registers, then over the four lane groups of a
// row.
#include "device.h"
#include "launch.h"

namespace csa {
namespace {

constexpr int kPoolHeads = 64, kPoolDim = 128;
constexpr int kChunk = 64, kWavesPerGroup = 4;   // slots per chunk (four groups of 16)

template <typename TS> __device__ __forceinline__ TS to_score(float v);
template <> __device__ __forceinline__ float to_score<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t to_score<uint16_t>(float v) { return f32_to_bf16(v); }

// A wave scores NCH consecutive chunks of 64 slots.  NCH = 1 spreads a few
// queries' pools over many workgroups (decode); NCH = 8 keeps q, loaded
// once, over 512 slots when there are queries enough to fill the chip
// (prefill), with the next chunk's key rows in flight while a chunk computes.
template <typename TS, int NCH>
__global__ void __launch_bounds__(256)
index_pool_kernel(int64_t T, int64_t N, int64_t P, int64_t nblk, const uint16_t* __restrict__ q,
                  const float* __restrict__ w, const uint16_t* __restrict__ keys, const int32_t* __restrict__ pool,
                  TS* __restrict__ scores) {
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
  const uint16_t* kseq = keys + b * N * kPoolDim;
  uint4 kf[2][4][4];
  auto load_chunk = [&](int c, uint4 (&dst)[4][4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        dst[u][s] = id[4 * c + u] >= 0
                        ? *reinterpret_cast<const uint4*>(kseq + static_cast<int64_t>(id[4 * c + u]) * kPoolDim +
                                                          32 * s + 8 * g)
                        : make_uint4(0, 0, 0, 0);
  };
  load_chunk(0, kf[0]);

  // q as the A operand: head block hb, k-step s -> head 16 hb + r, dims 32 s + 8 g ..
  const uint16_t* qq = q + gq * kPoolHeads * kPoolDim;
  uint4 qf[4][4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qf[hb][s] = *reinterpret_cast<const uint4*>(qq + (16 * hb + r) * kPoolDim + 32 * s + 8 * g);
  // head weights of this lane's C rows: heads 16 hb + 4 g + i
  float4 wv[4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) wv[hb] = *reinterpret_cast<const float4*>(w + gq * kPoolHeads + 16 * hb + 4 * g);

  TS* out = scores + gq * P;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (c + 1 < NCH) load_chunk(c + 1, kf[(c + 1) & 1]);   // masked past the pool: no traffic
    const uint4 (&kc)[4][4] = kf[c & 1];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float acc = 0.f;
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        f32x4 cc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
          cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qf[hb][s]), as_bf16x8(kc[u][s]), cc, 0, 0, 0);
        // C[4 g + i][r]: head 16 hb + 4 g + i against row r
        acc += wv[hb].x * fmaxf(cc[0], 0.f) + wv[hb].y * fmaxf(cc[1], 0.f) + wv[hb].z * fmaxf(cc[2], 0.f) +
               wv[hb].w * fmaxf(cc[3], 0.f);
      }
      acc += __shfl_xor(acc, 16, 64);
      acc += __shfl_xor(acc, 32, 64);
      const int64_t j = j0 + kChunk * c + 16 * u + r;
      if (g == 0 && j < P) out[j] = to_score<TS>(id[4 * c + u] >= 0 ? acc : -INFINITY);
    }
  }
}

template <typename TS, int NCH>
void launch_pool_t(const IndexPoolArgs& a, hipStream_t s) {
  const int64_t per_wg = static_cast<int64_t>(kWavesPerGroup) * NCH * kChunk;
  const int64_t nblk = (a.P + per_wg - 1) / per_wg;
  hipLaunchKernelGGL((index_pool_kernel<TS, NCH>), dim3(static_cast<uint32_t>(a.B * a.T * nblk)), dim3(256), 0, s,
                     a.T, a.N, a.P, nblk, static_cast<const uint16_t*>(a.q), a.w, static_cast<const uint16_t*>(a.k),
                     a.pool, static_cast<TS*>(a.scores));
}

template <typename TS>
void launch_pool_s(const IndexPoolArgs& a, hipStream_t s) {
  // long runs only when the queries alone give about four workgroups per CU
  const int64_t long_wgs = a.B * a.T * ((a.P + 2047) / 2048);
  if (long_wgs >= 1024) launch_pool_t<TS, 8>(a, s);
  else launch_pool_t<TS, 1>(a, s);
}

}  // namespace

hipError_t launch_index_pool(const IndexPoolArgs& a, hipStream_t s) {
  if (a.B == 0 || a.T == 0 || a.P == 0) return hipSuccess;
  if (a.score_dtype == CSA_F32) launch_pool_s<float>(a, s);
  else launch_pool_s<uint16_t>(a, s);
  return hipGetLastError();
}

}  // namespace csa
