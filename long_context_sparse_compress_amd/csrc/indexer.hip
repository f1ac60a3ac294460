// Stage 2: the lightning indexer on gfx950.
//
// "DeepSeek Technical Reports" (DSA, the indexer equation):
//   I[t,s] = sum_j w[t,j] * ReLU(q[t,j] . k[s]),  64 heads of 128 dims.
// "DeepSeek V4 结构速览" (Lightning Indexer): low-precision QK, ReLU, the
// head-weighted sum, scores stored as BF16, only the causal range s < V(t).
//
// The QK product is a GEMM with the 64 heads of one query as M, entries as N
// and d_I = 128 as K, so it runs on MFMA:
//   bf16   v_mfma_f32_16x16x32_bf16           (4 k-steps for K = 128)
//   fp8    v_mfma_scale_f32_16x16x128_f8f6f4  (E4M3, unit block scale; the
//          per-row fp32 scales are applied in the epilogue)
//   MXFP4  v_mfma_scale_f32_16x16x128_f8f6f4  (E2M1 with the E8M0 block
//          scales fed to the instruction)
// One 16-entry tile per MFMA column block; a wave owns QPW queries (their q
// fragments stay in registers) and streams TPW tiles of keys straight from
// HBM into registers (each lane reads one contiguous run of a key row).  The
// epilogue -- ReLU, multiply by w, sum over the 64 heads -- is fused: a lane
// reduces its 16 head values, two cross-lane steps finish the sum, and the
// scores of four tiles leave as one 128-byte store per query.
//
// Because K is contracted, the order of K inside a lane's fragment is free as
// long as q and k use the same order: every lane loads the same contiguous
// byte range of its q row and of its key row.
#include <cmath>
#include <type_traits>
#include <utility>

#include "compress_entry.h"
#include "device.h"
#include "launch.h"

namespace csa {
namespace {

constexpr int kH = 64;    // indexer heads
constexpr int kD = 128;   // indexer dim

// ---------------------------------------------------------------- fp32 path
// Plain fp32 arithmetic for fp32 inputs (small problems): one workgroup per
// (64-entry block, query, sequence); q[t] and w[t] are staged in LDS.
__global__ void __launch_bounds__(256)
index_f32_kernel(int64_t T, int64_t N, int64_t q_pos0, int ratio, const float* __restrict__ q,
                 const float* __restrict__ w, const float* __restrict__ k, float* __restrict__ scores) {
  __shared__ float qs[kH * kD];
  __shared__ float ws[kH];
  __shared__ float part[4][64];
  const int64_t t = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const float* qt = q + (b * T + t) * kH * kD;
  for (int i = tid; i < kH * kD; i += 256) qs[i] = qt[i];
  if (tid < kH) ws[tid] = w[(b * T + t) * kH + tid];
  __syncthreads();
  const int el = tid % 64, hq = tid / 64;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 64 + el;
  int64_t vis = (q_pos0 + t + 1) / ratio;
  if (vis > N) vis = N;
  float acc = 0.f;
  if (e < vis) {
    const float* kr = k + (b * N + e) * kD;
    for (int h = hq * 16; h < hq * 16 + 16; ++h) {
      float dot = 0.f;
      for (int d = 0; d < kD; ++d) dot = fmaf(qs[h * kD + d], kr[d], dot);
      acc = fmaf(ws[h], fmaxf(dot, 0.f), acc);
    }
  }
  part[hq][el] = acc;
  __syncthreads();
  if (hq == 0 && e < N) {
    const float s = (part[0][el] + part[1][el]) + (part[2][el] + part[3][el]);
    scores[(b * T + t) * N + e] = (e < vis) ? s : -INFINITY;
  }
}

// ---------------------------------------------------------------- MFMA path
template <int QK> struct Frag;

// bf16: rows of 256 B; for k-step i, lane (r, g) holds bytes [64i + 16g, +16),
// so the four lanes of a row read 64 contiguous bytes per load instruction
// (16 half cache lines per instruction, not 32 partial ones: about 15% more
// read bandwidth on MI355X).
template <> struct Frag<CSA_BF16> {
  static constexpr int kRowBytes = 256;
  static constexpr int kRegs = 4;  // uint4 per lane per 16-row tile
  uint4 v[kRegs];
  __device__ __forceinline__ void load(const uint8_t* row, int g) {
    const uint4* p = reinterpret_cast<const uint4*>(row + 16 * g);
#pragma unroll
    for (int i = 0; i < kRegs; ++i) v[i] = p[4 * i];
  }
  __device__ static constexpr int chunk(int i, int g) { return 4 * i + g; }
};
// fp8: rows of 128 B; lane (r, g) holds bytes [32g, 32g+32).
template <> struct Frag<CSA_FP8_E4M3> {
  static constexpr int kRowBytes = 128;
  static constexpr int kRegs = 2;
  uint4 v[kRegs];
  __device__ __forceinline__ void load(const uint8_t* row, int g) {
    const uint4* p = reinterpret_cast<const uint4*>(row + 32 * g);
    v[0] = p[0];
    v[1] = p[1];
  }
  __device__ static constexpr int chunk(int i, int g) { return 2 * g + i; }
};
// A key tile staged in LDS row by row, the 16-byte chunks of row r permuted
// by XOR with swz(r): chunk c of row r sits at r * RB + (c ^ swz(r)) * 16.
// One direct-to-LDS load then fills 1 KB of whole rows (contiguous in HBM
// too: full cache lines only), and the 16 lanes that read one chunk of the
// 16 rows hit 16 distinct 16-byte bank groups.
template <int RB>
__device__ __forceinline__ constexpr int tile_swz(int r) { return RB == 256 ? (r & 15) : ((r >> 1) & 7); }
template <typename F>
__device__ __forceinline__ void load_tile_frag(F& f, const uint8_t* tile, int col, int g) {
  constexpr int RB = F::kRowBytes;
#pragma unroll
  for (int i = 0; i < F::kRegs; ++i)
    f.v[i] = *reinterpret_cast<const uint4*>(tile + col * RB + ((F::chunk(i, g) ^ tile_swz<RB>(col)) << 4));
}

// MXFP4: rows of 64 B + 4 scale bytes; lane (r, g) holds bytes [16g, 16g+16)
// (the 32 elements of MX block g) and block g's scale.
template <> struct Frag<CSA_MXFP4> {
  static constexpr int kRowBytes = 64;
  static constexpr int kRegs = 1;
  uint4 v[kRegs];
  __device__ __forceinline__ void load(const uint8_t* row, int g) {
    v[0] = *reinterpret_cast<const uint4*>(row + 16 * g);
  }
};

// C[mt] = A[mt] x B for the four 16-head blocks of one query against one
// 16-entry key tile.  The four products are independent, so their MFMAs are
// issued interleaved (k-step outer, head block inner): no MFMA waits on the
// one before it.
template <int QK>
__device__ __forceinline__ void qk_tiles(const Frag<QK> (&a)[4], const Frag<QK>& b, const int (&sa)[4], int sb,
                                         f32x4 (&c)[4]) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) c[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (QK == CSA_BF16) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        c[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[mt].v[s]), as_bf16x8(b.v[s]), c[mt], 0, 0, 0);
  } else if constexpr (QK == CSA_FP8_E4M3) {
    const i32x8 bv = {(int)b.v[0].x, (int)b.v[0].y, (int)b.v[0].z, (int)b.v[0].w,
                      (int)b.v[1].x, (int)b.v[1].y, (int)b.v[1].z, (int)b.v[1].w};
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const i32x8 av = {(int)a[mt].v[0].x, (int)a[mt].v[0].y, (int)a[mt].v[0].z, (int)a[mt].v[0].w,
                        (int)a[mt].v[1].x, (int)a[mt].v[1].y, (int)a[mt].v[1].z, (int)a[mt].v[1].w};
      c[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c[mt], 0, 0, 0, 127, 0, 127);
    }
  } else {
    const i32x8 bv = {(int)b.v[0].x, (int)b.v[0].y, (int)b.v[0].z, (int)b.v[0].w, 0, 0, 0, 0};
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const i32x8 av = {(int)a[mt].v[0].x, (int)a[mt].v[0].y, (int)a[mt].v[0].z, (int)a[mt].v[0].w, 0, 0, 0, 0};
      c[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c[mt], 4, 4, 0, sa[mt], 0, sb);
    }
  }
}

// max(x, 0) as one integer max on the bit pattern: a float with the sign bit
// set is a negative int32 (fmaxf would add a canonicalising max per value)
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

__device__ __forceinline__ void store_score(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_score(uint16_t* p, float v) { *p = f32_to_bf16(v); }

// Paged keys (the heterogeneous cache's classical blocks): entry e of
// sequence b is row (table[b][e / 32] * 32 + e % 32) of the key pool, and the
// sequence's query sits at seq_pos[b].  A 16-entry tile never straddles a
// 32-entry block, so paging only moves a tile's base row.
struct KeyPages {
  const int32_t* table;
  int64_t max_blocks, n_pool;
  const int64_t* seq_pos;
};

// Grid: x = entry block of 4 * TPW * 16 entries (one TPW-tile run per wave),
// y = block of QPW queries, z = sequence.  256 threads = 4 waves.  Keys are
// loaded GT tiles (GT * 16 entries) at a time, one group ahead of the group
// being computed; OCC is the number of waves per SIMD the register budget is
// sized for (GT = 8 needs the whole register file: one wave per SIMD).
// PG: keys in the paged pool (decode, T = 1): a tile's block comes from the
// block table by one wave-uniform load, ids outside the pool read block 0.
template <int QK, int QPW, int TPW, int GT, typename TS, bool PG>
__device__ __forceinline__ void index_mfma_body(int64_t bx, int64_t by, int64_t bz, int64_t T, int64_t N,
                                                int64_t q_pos0, int ratio, const uint8_t* __restrict__ q,
                                                const void* __restrict__ q_scale, const float* __restrict__ w,
                                                const uint8_t* __restrict__ k, const void* __restrict__ k_scale,
                                                TS* __restrict__ scores, const KeyPages& pg) {
  static_assert(GT % 4 == 0 && TPW % GT == 0, "tiles are stored four at a time");
  static_assert(!PG || QPW == 1, "paged keys: decode shape");
  constexpr int KG = GT / 4;   // 4-tile score stores per group
  using F = Frag<QK>;
  constexpr int RB = F::kRowBytes;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar loop control
  const int col = lane & 15;   // row of a 16-row operand tile / column of the output tile
  const int g = lane >> 4;     // lane group: K sub-range, and output rows 4g..4g+3
  const int64_t b = bz;
  const int64_t t0 = by * QPW;
  const int64_t e_wave = (bx * 4 + wid) * (TPW * 16);

  // The workgroup's q rows go through LDS once (coalesced 16-byte loads)
  // instead of every wave fetching its fragments from global memory.
  __shared__ __attribute__((aligned(16))) uint8_t qs[QPW * kH * RB];
  for (int o = threadIdx.x * 16; o < QPW * kH * RB; o += 256 * 16) {
    const int qi = o / (kH * RB);
    int64_t t = t0 + qi;
    if (t >= T) t = T - 1;
    *reinterpret_cast<uint4*>(qs + o) = *reinterpret_cast<const uint4*>(q + (b * T + t) * kH * RB + o % (kH * RB));
  }
  __syncthreads();
  if (e_wave >= N) return;

  // q fragments and head weights of this wave's queries.
  F qa[QPW][4];
  int qsc[QPW][4];
  float wv[QPW][4][4];
  int64_t vis[QPW];
  int64_t vis_max = 0, vis_min = INT64_MAX;
#pragma unroll
  for (int qi = 0; qi < QPW; ++qi) {
    int64_t t = t0 + qi;
    if (t >= T) t = T - 1;
    int64_t v = ((PG ? pg.seq_pos[b] : q_pos0 + t) + 1) / ratio;
    if (v > N) v = N;
    vis[qi] = (t0 + qi < T) ? v : 0;
    vis_max = vis[qi] > vis_max ? vis[qi] : vis_max;
    if (t0 + qi < T) vis_min = vis[qi] < vis_min ? vis[qi] : vis_min;
    const int64_t qrow = (b * T + t) * kH;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      qa[qi][mt].load(qs + (qi * kH + mt * 16 + col) * RB, g);
      if constexpr (QK == CSA_MXFP4)
        qsc[qi][mt] = static_cast<const uint8_t*>(q_scale)[(qrow + mt * 16 + col) * 4 + g];
      else
        qsc[qi][mt] = 127;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = mt * 16 + 4 * g + i;
        float wt = w[qrow + h];
        if constexpr (QK == CSA_FP8_E4M3) wt *= static_cast<const float*>(q_scale)[qrow + h];
        wv[qi][mt][i] = wt;
      }
    }
  }

  const int64_t krow0 = b * N;
  // paged: lane i holds the physical block of the wave's i-th 32-entry block
  // (ids outside the pool, and blocks past the table, read block 0), so a
  // tile's block is a readlane away instead of a dependent load per tile
  [[maybe_unused]] int32_t my_blk = 0;
  if constexpr (PG) {
    static_assert(TPW % 2 == 0 && TPW / 2 <= 64, "a wave's blocks fit its lanes");
    const int64_t lb = (e_wave >> 5) + lane;
    int32_t v = 0;
    if (lane < TPW / 2 && lb < pg.max_blocks) v = pg.table[b * pg.max_blocks + lb];
    my_blk = (v >= 0 && v < pg.n_pool) ? v : 0;
  }
  // Key fragments of one group (GT tiles); the next group's loads are issued
  // before the current group's MFMAs.
  F kb[2][GT];
  int ksc[2][GT];
  float kscale[2][GT];
  const uint8_t* kseq = k + krow0 * RB + col * RB;   // this lane's row of every tile, from entry 0
  auto load_group = [&](int slot, int64_t eg) {
    const bool full = eg + GT * 16 <= N;   // wave-uniform: only the last group can run past N
#pragma unroll
    for (int tt = 0; tt < GT; ++tt) {
      int64_t row;   // this lane's key row in k
      if constexpr (PG) {
        // N is a whole number of 32-entry blocks: a tile lies wholly inside
        // or wholly past it; a tile past it (never stored) reads the last one
        int64_t e0 = eg + tt * 16;
        if (e0 >= N) e0 = N - 16;
        const int64_t blk = __builtin_amdgcn_readlane(my_blk, static_cast<int>((e0 - e_wave) >> 5));
        row = (blk << 5) + (e0 & 31) + col;
      } else {
        int64_t e = eg + tt * 16 + col;
        if (e >= N) e = N - 1;
        row = full ? krow0 + eg + tt * 16 + col : krow0 + e;
      }
      kb[slot][tt].load((PG || !full) ? k + row * RB : kseq + (eg + tt * 16) * RB, g);
      if constexpr (QK == CSA_MXFP4) ksc[slot][tt] = static_cast<const uint8_t*>(k_scale)[row * 4 + g];
      else ksc[slot][tt] = 127;
      if constexpr (QK == CSA_FP8_E4M3) kscale[slot][tt] = static_cast<const float*>(k_scale)[row];
      else kscale[slot][tt] = 1.f;
    }
  };
  load_group(0, e_wave);
#pragma unroll 2
  for (int tg = 0; tg < TPW / GT; ++tg) {
    const int cur = tg & 1;
    const int64_t eg = e_wave + tg * (GT * 16);
    if (eg >= N) break;
    if (tg + 1 < TPW / GT && eg + GT * 16 < N) load_group(cur ^ 1, eg + GT * 16);
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) {
      // four tiles: each lane's 16 head values reduced in registers, then one
      // reduce-scatter over the four lane groups (three lane exchanges for
      // four tiles) leaves lane group g with the score of tile g
      float part[QPW][4];
#pragma unroll
      for (int tq = 0; tq < 4; ++tq) {
        const int tt = kg * 4 + tq;
        const int64_t et = eg + tt * 16;
#pragma unroll
        for (int qi = 0; qi < QPW; ++qi) part[qi][tq] = 0.f;
        if (et >= vis_max) continue;   // whole tile masked for every query (wave-uniform)
        // all MFMAs of the tile first (every query, every head block), then the epilogues
        f32x4 cc[QPW][4];
#pragma unroll
        for (int qi = 0; qi < QPW; ++qi) qk_tiles<QK>(qa[qi], kb[cur][tt], qsc[qi], ksc[cur][tt], cc[qi]);
#pragma unroll
        for (int qi = 0; qi < QPW; ++qi) {
          float acc = 0.f;
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            const f32x4 c = cc[qi][mt];
            acc = fmaf(wv[qi][mt][0], relu(c[0]), acc);
            acc = fmaf(wv[qi][mt][1], relu(c[1]), acc);
            acc = fmaf(wv[qi][mt][2], relu(c[2]), acc);
            acc = fmaf(wv[qi][mt][3], relu(c[3]), acc);
          }
          part[qi][tq] = acc * kscale[cur][tt];
        }
      }
      const int64_t e = eg + kg * 64 + g * 16 + col;   // the entry this lane ends up holding
#pragma unroll
      for (int qi = 0; qi < QPW; ++qi) {
        // across the halves (g by 2): lanes g < 2 keep tiles {0, 1}, g >= 2 tiles {2, 3};
        // then across rows (g by 1): lane group g keeps tile g
        const float k0 = pair_sum32(part[qi][0], part[qi][2]), k1 = pair_sum32(part[qi][1], part[qi][3]);
        float v = pair_sum16(k0, k1);
        if (e >= vis[qi]) v = -INFINITY;
        if (e < N && t0 + qi < T) store_score(scores + (b * T + t0 + qi) * N + e, v);
      }
    }
  }
}


template <int QK, int QPW, int TPW, int GT, int OCC, typename TS, bool PG = false>
__global__ void __launch_bounds__(256, OCC)
index_mfma_kernel(int64_t T, int64_t N, int64_t q_pos0, int ratio,
                  const uint8_t* __restrict__ q, const void* __restrict__ q_scale,
                  const float* __restrict__ w, const uint8_t* __restrict__ k,
                  const void* __restrict__ k_scale, TS* __restrict__ scores, KeyPages pg) {
  index_mfma_body<QK, QPW, TPW, GT, TS, PG>(blockIdx.x, blockIdx.y, blockIdx.z, T, N, q_pos0, ratio, q, q_scale, w,
                                            k, k_scale, scores, pg);
}

// A decode step's compressor writes in the indexer's own launch (one query a
// sequence, contiguous keys).  Grid (X, 1, B).  The first B workgroups
// dispatched are, for each sequence b, the one whose key run holds the
// written entry (run x_own): it runs sequence b's share of every job -- one
// entry each, two channels a thread -- and only then reads its keys, so it
// scores the key it has just written; no other workgroup reads that entry.
// Dispatched first, its extra latency overlaps the other workgroups' key
// streams instead of adding a launch to the step.  The remaining workgroups
// take the other runs in the plain order.
template <int QK, int TPW, int GT, int OCC, typename TS>
__global__ void __launch_bounds__(256, OCC)
index_mfma_jobs_kernel(int64_t N, int64_t q_pos0, int ratio, const uint8_t* __restrict__ q,
                       const void* __restrict__ q_scale, const float* __restrict__ w,
                       const uint8_t* __restrict__ k, const void* __restrict__ k_scale, TS* __restrict__ scores,
                       CompressBatch jb, int n_jobs, int64_t x_own) {
  const int64_t X = gridDim.x, B = gridDim.z;
  const int64_t L = blockIdx.x + X * static_cast<int64_t>(blockIdx.z);
  int64_t bx, bz;
  if (L < B) {
    bx = x_own;
    bz = L;
    for (int j = 0; j < n_jobs; ++j) {
      const CompressJobDev& J = jb.j[j];
      const auto* Ca = static_cast<const uint16_t*>(J.Ca);
      const auto* Za = static_cast<const uint16_t*>(J.Za);
      const auto* Cb = static_cast<const uint16_t*>(J.Cb);
      const auto* Zb = static_cast<const uint16_t*>(J.Zb);
      const auto* pCb = static_cast<const uint16_t*>(J.pCb);
      const auto* pZb = static_cast<const uint16_t*>(J.pZb);
      if (J.qfmt == 2)
        compress_entry<uint16_t, E2M1x2, 4, false, 2, 8>(0, bz, 0, 1, J.n_tok, J.c, J.pos0, Ca, Za, Cb, Zb, pCb, pZb,
                                                         J.bias, J.gamma, J.eps, static_cast<E2M1x2*>(J.out),
                                                         J.out_stride, J.G, nullptr, J.rope_R, J.rope_l2b,
                                                         J.rope_anchor, J.out_scale, J.scale_stride);
      else if (J.qfmt == 1)
        compress_entry<uint16_t, uint8_t, 4, false, 2, 8>(0, bz, 0, 1, J.n_tok, J.c, J.pos0, Ca, Za, Cb, Zb, pCb, pZb,
                                                          J.bias, J.gamma, J.eps, static_cast<uint8_t*>(J.out),
                                                          J.out_stride, J.G, nullptr, J.rope_R, J.rope_l2b,
                                                          J.rope_anchor, J.out_scale, J.scale_stride);
      else
        compress_entry<uint16_t, uint16_t, 4, false, 2, 8>(0, bz, 0, 1, J.n_tok, J.c, J.pos0, Ca, Za, Cb, Zb, pCb,
                                                           pZb, J.bias, J.gamma, J.eps, static_cast<uint16_t*>(J.out),
                                                           J.out_stride, J.G, nullptr, J.rope_R, J.rope_l2b,
                                                           J.rope_anchor, J.out_scale, J.scale_stride);
      // the job's writes are visible to every wave of the workgroup, and
      // its LDS (norm sums, RoPE table) is free for the next one
      __syncthreads();
    }
  } else {
    const int64_t m = L - B;   // X > 1 here
    bz = m / (X - 1);
    const int64_t xi = m % (X - 1);
    bx = xi < x_own ? xi : xi + 1;
  }
  index_mfma_body<QK, 1, TPW, GT, TS, false>(bx, 0, bz, 1, N, q_pos0, ratio, q, q_scale, w, k, k_scale, scores,
                                             KeyPages{nullptr, 0, 0, nullptr});
}

// ---------------------------------------------------------------- ring path
// bf16 / fp8 keys: each wave streams its TPW tiles through a D-slot ring of
// LDS tile buffers filled by direct global->LDS loads (no registers held for
// loads in flight), D - 1 tiles ahead of the one being computed.  Each slot is
// its own LDS array, so the compiler can see that reading slot r does not
// touch the loads landing in the other slots; the waits for a tile's rows are
// explicit.  A wave only ever reads its own slots: no barriers.
typedef __attribute__((address_space(3))) void lds_void;

// Direct-to-LDS 16-byte load (lane l's bytes land at dst + 16 l) and a 4-byte
// register load, both through a buffer resource over [base, base + bytes):
// a lane whose offset is out of that range reads nothing.
constexpr int kRsrcWord3 = 0x00020000;   // 32-bit data format, no swizzle
__device__ __forceinline__ void buffer_load_lds16(const void* base, int bytes, void* dst, uint32_t off) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRsrcWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, off, 0, 0, 0);
}
__device__ __forceinline__ float buffer_load_f32(const float* base, int bytes, uint32_t off) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, bytes, kRsrcWord3);
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// f(integral_constant<I>) for I = 0 .. N-1, every index a compile-time constant
template <int I, int N, typename Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// A decode step's compressor jobs run by the ring kernel's workgroup whose
// key run x_own holds the written entry (see index_ring_kernel).
struct RingJobs {
  CompressBatch jb;
  int n;
  int64_t x_own;
};

template <int QK, int QPW, int TPW, int D, bool XS, bool PIPE, typename TS, bool PG = false, bool CJ = false>
__global__ void __launch_bounds__(256, PIPE ? 1 : 2)
index_ring_kernel(int64_t T, int64_t N, int64_t q_pos0, int ratio,
                  const uint8_t* __restrict__ q, const void* __restrict__ q_scale,
                  const float* __restrict__ w, const uint8_t* __restrict__ k,
                  const void* __restrict__ k_scale, TS* __restrict__ scores, KeyPages pg, RingJobs rj) {
  static_assert(!PG || (QPW == 1 && TPW <= 128), "paged keys: decode shape, a wave's blocks in one lane each");
  static_assert(QK == CSA_BF16 || QK == CSA_FP8_E4M3, "MXFP4 keys use index_mfma_kernel");
  static_assert(TPW % 4 == 0 && TPW >= D, "scores leave four tiles at a time");
  static_assert(D == 4 || D == 8, "ring of four or eight slots");
  using F = Frag<QK>;
  constexpr int RB = F::kRowBytes;
  constexpr int TB = 16 * RB;                               // bytes per 16-entry tile
  constexpr int NI = TB / 1024;                             // 1 KB row loads per tile
  constexpr int OPS = NI + (QK == CSA_FP8_E4M3 ? 1 : 0);    // vector memory ops issued per tile
  static_assert((D - 2) * OPS < 64, "the deepest wait must fit vmcnt");
  constexpr int QB = QPW * kH * RB;                          // query bytes staged per workgroup
  static_assert(QB % 4096 == 0, "queries are staged 4 KB (one load per wave) at a time");
  constexpr int WN = QK == CSA_FP8_E4M3 ? 2 * QPW : QPW;     // 256-byte weight / scale rows staged
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, g = lane >> 4;
  uint32_t bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
  if constexpr (XS) {
    // Each XCD takes a contiguous range of workgroups.  Decode (PIPE false):
    // key runs vary fastest, so an XCD streams one contiguous range of keys
    // from HBM (measured about 8% faster than the round-robin spread).
    // Prefill (PIPE): query blocks vary fastest, so an XCD works through one
    // or two key runs for every query and they stay in its L2.
    const uint32_t lin = bx + gridDim.x * (by + gridDim.y * bz);
    const uint32_t sw = xcd_swizzle(lin, gridDim.x * gridDim.y * gridDim.z);
    if constexpr (!PIPE) {
      bx = sw % gridDim.x;
      by = (sw / gridDim.x) % gridDim.y;
    } else {
      by = sw % gridDim.y;
      bx = (sw / gridDim.y) % gridDim.x;
    }
    bz = sw / (gridDim.x * gridDim.y);
  }
  const int64_t b = bz;
  const int64_t t0 = static_cast<int64_t>(by) * QPW;
  const int64_t e_wave = (static_cast<int64_t>(bx) * 4 + wid) * (TPW * 16);

  __shared__ __attribute__((aligned(16))) uint8_t qs[QB + WN * kH * 4];
  __shared__ __attribute__((aligned(16))) uint8_t ring0[4][TB];
  __shared__ __attribute__((aligned(16))) uint8_t ring1[4][TB];
  __shared__ __attribute__((aligned(16))) uint8_t ring2[4][TB];
  __shared__ __attribute__((aligned(16))) uint8_t ring3[4][TB];
  __shared__ __attribute__((aligned(16))) uint8_t ring4[D > 4 ? 4 : 1][D > 4 ? TB : 16];
  __shared__ __attribute__((aligned(16))) uint8_t ring5[D > 4 ? 4 : 1][D > 4 ? TB : 16];
  __shared__ __attribute__((aligned(16))) uint8_t ring6[D > 4 ? 4 : 1][D > 4 ? TB : 16];
  __shared__ __attribute__((aligned(16))) uint8_t ring7[D > 4 ? 4 : 1][D > 4 ? TB : 16];

  if constexpr (CJ) {
    // The workgroup whose key run holds the step's new entry writes it (and
    // the step's other one-entry jobs of sequence b) before it stages or
    // reads anything; ring slot 0 lends the jobs' LDS.  No other workgroup
    // reads that entry.
    if (static_cast<int64_t>(bx) == rj.x_own) {
      float* const lds = reinterpret_cast<float*>(&ring0[0][0]);
      for (int jn = 0; jn < rj.n; ++jn) {
        const CompressJobDev& J = rj.jb.j[jn];
        const auto* Ca = static_cast<const uint16_t*>(J.Ca);
        const auto* Za = static_cast<const uint16_t*>(J.Za);
        const auto* Cb = static_cast<const uint16_t*>(J.Cb);
        const auto* Zb = static_cast<const uint16_t*>(J.Zb);
        const auto* pCb = static_cast<const uint16_t*>(J.pCb);
        const auto* pZb = static_cast<const uint16_t*>(J.pZb);
        if (J.qfmt == 2)
          compress_entry<uint16_t, E2M1x2, 4, false, 2, 8>(0, b, 0, 1, J.n_tok, J.c, J.pos0, Ca, Za, Cb, Zb, pCb, pZb,
                                                           J.bias, J.gamma, J.eps, static_cast<E2M1x2*>(J.out),
                                                           J.out_stride, J.G, nullptr, J.rope_R, J.rope_l2b,
                                                           J.rope_anchor, J.out_scale, J.scale_stride, -1, lds);
        else if (J.qfmt == 1)
          compress_entry<uint16_t, uint8_t, 4, false, 2, 8>(0, b, 0, 1, J.n_tok, J.c, J.pos0, Ca, Za, Cb, Zb, pCb,
                                                            pZb, J.bias, J.gamma, J.eps, static_cast<uint8_t*>(J.out),
                                                            J.out_stride, J.G, nullptr, J.rope_R, J.rope_l2b,
                                                            J.rope_anchor, J.out_scale, J.scale_stride, -1, lds);
        else
          compress_entry<uint16_t, uint16_t, 4, false, 2, 8>(0, b, 0, 1, J.n_tok, J.c, J.pos0, Ca, Za, Cb, Zb, pCb,
                                                             pZb, J.bias, J.gamma, J.eps, static_cast<uint16_t*>(J.out),
                                                             J.out_stride, J.G, nullptr, J.rope_R, J.rope_l2b,
                                                             J.rope_anchor, J.out_scale, J.scale_stride, -1, lds);
        __syncthreads();   // the job's writes are visible and its LDS is free
      }
    }
  }

  // paged: lane i holds the physical block of the wave's i-th 32-entry
  // block, loaded before anything else (the counter of loads in flight is in
  // order, so waiting for it later does not wait for the queries); ids
  // outside the pool, and blocks past the table, read block 0
  [[maybe_unused]] int32_t my_blk = 0;
  if constexpr (PG) {
    const int64_t lb = (e_wave >> 5) + lane;
    int32_t v = 0;
    if (lane < TPW / 2 && lb < pg.max_blocks) v = pg.table[b * pg.max_blocks + lb];
    my_blk = (v >= 0 && v < pg.n_pool) ? v : 0;
  }

  // which entries each query sees (scalar arithmetic only)
  int64_t vis[QPW];
  int64_t vis_max = 0;
#pragma unroll
  for (int qi = 0; qi < QPW; ++qi) {
    int64_t t = t0 + qi;
    if (t >= T) t = T - 1;
    int64_t v = ((PG && pg.seq_pos) ? pg.seq_pos[b] : q_pos0 + t) + 1;
    v /= ratio;
    if (v > N) v = N;
    vis[qi] = (t0 + qi < T) ? v : 0;
    vis_max = vis[qi] > vis_max ? vis[qi] : vis_max;
  }
  const bool streams = e_wave < vis_max;   // wave-uniform (vis_max <= N)

  // The workgroup's queries and head weights go to LDS by direct loads, then
  // the first D - 1 key tiles follow: all of their latencies overlap.
  // Wave w's i-th query load fills bytes [(4i + w) KB, (4i + w + 1) KB) of qs.
#pragma unroll
  for (int i = 0; i < QB / 4096; ++i) {
    const int o = (4 * i + wid) * 1024;
    const int qi = o / (kH * RB);
    int64_t t = t0 + qi;
    if (t >= T) t = T - 1;
    const uint8_t* src = q + (b * T + t) * kH * RB + o % (kH * RB) + 16 * lane;
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(src), (lds_void*)(qs + o), 16, 0, 0);
  }
  // The head weights (and fp8 query scales) of query qi follow: 64 floats,
  // one 4-byte load per lane, into the same LDS array.  Every wave loads them
  // (the same values to the same place): no branch around a load into LDS.
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    const int qi = j % QPW;
    int64_t t = t0 + qi;
    if (t >= T) t = T - 1;
    const float* src = (j < QPW ? w : static_cast<const float*>(q_scale)) + (b * T + t) * kH + lane;
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(src), (lds_void*)(qs + QB + j * kH * 4), 4, 0, 0);
  }

  const int64_t krow0 = b * N;
  float ks[D];   // fp8 key row scales of the tiles in the ring
#pragma unroll
  for (int r = 0; r < D; ++r) ks[r] = 1.f;
  auto slot = [&](auto rc) -> uint8_t* {
    constexpr int r = decltype(rc)::value;
    if constexpr (r == 0) return ring0[wid];
    else if constexpr (r == 1) return ring1[wid];
    else if constexpr (r == 2) return ring2[wid];
    else if constexpr (r == 3) return ring3[wid];
    else if constexpr (r == 4) return ring4[wid];
    else if constexpr (r == 5) return ring5[wid];
    else if constexpr (r == 6) return ring6[wid];
    else return ring7[wid];
  };
  // Load j of a tile fills rows RPI j .. RPI j + RPI - 1; lane l takes chunk
  // position l % CPR of row RPI j + l / CPR, i.e. chunk (l % CPR) ^ swz(row).
  // The loads go through a buffer resource whose base is the tile's first row
  // and whose size ends at row N - 1: the lane offsets are fixed, the per-tile
  // address arithmetic is scalar, and rows past N - 1 read nothing (their
  // scores are never stored).  A wave with nothing visible reads row N - 1.
  constexpr int CPR = RB / 16, RPI = 64 / CPR;
  uint32_t voff[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int row = RPI * j + lane / CPR;
    voff[j] = static_cast<uint32_t>(row * RB + (((lane % CPR) ^ tile_swz<RB>(row)) << 4));
  }
  auto issue = [&](int t, auto rc) {
    constexpr int r = decltype(rc)::value;
    uint8_t* dst = slot(rc);
    const int64_t e0 = streams ? e_wave + 16 * t : N - 1;
    int64_t srow;   // the tile's first row in the key array
    int rows;       // rows of this tile that may be read
    if constexpr (PG) {
      const int32_t blk = __builtin_amdgcn_readlane(my_blk, streams ? (t >> 1) : 0);
      srow = (static_cast<int64_t>(blk) << 5) + (streams ? (e0 & 31) : 0);
      rows = 16;    // inside its block
    } else {
      srow = krow0 + e0;
      rows = static_cast<int>(N - e0 < 16 ? N - e0 : 16);   // rows of this tile inside [0, N)
    }
    const uint8_t* base = k + srow * RB;
    wait_lgkm0();   // this wave's reads of the slot's previous tile are done
#pragma unroll
    for (int j = 0; j < NI; ++j) buffer_load_lds16(base, rows * RB, dst + 1024 * j, voff[j]);
    if constexpr (QK == CSA_FP8_E4M3)   // the scale of this lane's key column
      ks[r] = buffer_load_f32(static_cast<const float*>(k_scale) + srow, rows * 4, col * 4);
  };
  // Every wave issues the first tiles, also one whose entries are all masked
  // or past N (its loads all read entry N - 1): with no branch around a load
  // into LDS the compiler keeps track of which LDS array each load in flight
  // fills, and reading qs below does not wait for the key tiles.  Such a
  // wave skips the tile loop below.
  static_for<0, D - 1>([&](auto rc) { issue(decltype(rc)::value, rc); });
  wait_vm<(D - 1) * OPS>();   // this wave's query and weight loads have landed ...
  // ... and every other wave's: a bare barrier (__syncthreads' release fence
  // would also wait for the key tiles still in flight)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

  F qa[QPW][4];
  float wv[QPW][4][4];   // weights of heads 16 mt + 4 g + i: this lane's accumulator rows
#pragma unroll
  for (int qi = 0; qi < QPW; ++qi)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      qa[qi][mt].load(qs + (qi * kH + mt * 16 + col) * RB, g);
      float4 wt = *reinterpret_cast<const float4*>(qs + QB + (qi * kH + mt * 16 + 4 * g) * 4);
      if constexpr (QK == CSA_FP8_E4M3) {
        const float4 s4 = *reinterpret_cast<const float4*>(qs + QB + ((QPW + qi) * kH + mt * 16 + 4 * g) * 4);
        wt.x *= s4.x; wt.y *= s4.y; wt.z *= s4.z; wt.w *= s4.w;
      }
      wv[qi][mt][0] = wt.x; wv[qi][mt][1] = wt.y; wv[qi][mt][2] = wt.z; wv[qi][mt][3] = wt.w;
    }
  const int qsc[4] = {127, 127, 127, 127};

  float sc[QPW][TPW / 4];
  float part[QPW][4];
  // four tiles' partial scores -> lane group g keeps tile u - 3 + g's score
  auto scatter4 = [&](auto uc) {
    constexpr int u = decltype(uc)::value;
    const int64_t e = e_wave + 16 * (u - 3 + g) + col;
#pragma unroll
    for (int qi = 0; qi < QPW; ++qi) {
      const float k0 = pair_sum32(part[qi][0], part[qi][2]), k1 = pair_sum32(part[qi][1], part[qi][3]);
      float v = pair_sum16(k0, k1);
      sc[qi][u / 4] = (e >= vis[qi]) ? -INFINITY : v;
    }
  };
  if (!streams) {
    // Nothing of this wave's run is visible to the workgroup's queries (a key
    // run past N, or past a short sequence): no tile to score.  Its prologue
    // tile loads are drained, so no load into LDS is left in flight, its
    // scores are -inf, and the wave ends: wave-uniform, and no barrier
    // follows the prologue's.
    wait_vm<0>();
#pragma unroll
    for (int tb = 0; tb < TPW; tb += 4) {
      const int64_t e = e_wave + 16 * (tb + g) + col;
#pragma unroll
      for (int qi = 0; qi < QPW; ++qi)
        if (e < N && t0 + qi < T) store_score(scores + (b * T + t0 + qi) * N + e, -INFINITY);
    }
    return;
  }
  if constexpr (PIPE) {
    // Software pipeline (prefill, where the MFMAs and the ReLU-weighted sums
    // both take time): tile t's MFMAs are issued before tile t - 1's sums,
    // which consume MFMA results that are already done.  Every tile is
    // computed (masked entries get -inf at the end).
    f32x4 cc[2][QPW][4];
    float kss[2];
    static_for<0, TPW + 1>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      if constexpr (t < TPW) {
        constexpr int r = t % D;
        constexpr int later = (TPW - 1 - t) < (D - 2) ? (TPW - 1 - t) : (D - 2);
        wait_vm<later * OPS>();
        if constexpr (t + D - 1 < TPW) issue(t + D - 1, std::integral_constant<int, (t + D - 1) % D>{});
        F kf;
        load_tile_frag(kf, slot(std::integral_constant<int, r>{}), col, g);
#pragma unroll
        for (int qi = 0; qi < QPW; ++qi) qk_tiles<QK>(qa[qi], kf, qsc, 127, cc[t & 1][qi]);
        kss[t & 1] = ks[r];   // the ring slot's scale is reloaded by the next issue
      }
      if constexpr (t >= 1) {
        constexpr int u = t - 1;
#pragma unroll
        for (int qi = 0; qi < QPW; ++qi) {
          float acc = 0.f;
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            acc = fmaf(wv[qi][mt][0], relu(cc[u & 1][qi][mt][0]), acc);
            acc = fmaf(wv[qi][mt][1], relu(cc[u & 1][qi][mt][1]), acc);
            acc = fmaf(wv[qi][mt][2], relu(cc[u & 1][qi][mt][2]), acc);
            acc = fmaf(wv[qi][mt][3], relu(cc[u & 1][qi][mt][3]), acc);
          }
          part[qi][u & 3] = acc * kss[u & 1];
        }
        if constexpr ((u & 3) == 3) scatter4(std::integral_constant<int, u>{});
      }
    });
  } else
  static_for<0, TPW>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    constexpr int r = t % D;
    // rows of tile t have landed once at most the ops of the (up to D - 2)
    // tiles issued after it are outstanding
    constexpr int later = (TPW - 1 - t) < (D - 2) ? (TPW - 1 - t) : (D - 2);
    wait_vm<later * OPS>();
    if constexpr (t + D - 1 < TPW) issue(t + D - 1, std::integral_constant<int, (t + D - 1) % D>{});
#pragma unroll
    for (int qi = 0; qi < QPW; ++qi) part[qi][t & 3] = 0.f;
    if (e_wave + 16 * t < vis_max) {   // else the whole tile is masked for every query (wave-uniform)
      F kf;
      load_tile_frag(kf, slot(std::integral_constant<int, r>{}), col, g);
#pragma unroll
      for (int qi = 0; qi < QPW; ++qi) {
        f32x4 cc[4];
        qk_tiles<QK>(qa[qi], kf, qsc, 127, cc);
        float acc = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          acc = fmaf(wv[qi][mt][0], relu(cc[mt][0]), acc);
          acc = fmaf(wv[qi][mt][1], relu(cc[mt][1]), acc);
          acc = fmaf(wv[qi][mt][2], relu(cc[mt][2]), acc);
          acc = fmaf(wv[qi][mt][3], relu(cc[mt][3]), acc);
        }
        part[qi][t & 3] = acc * ks[r];
      }
    }
    if constexpr ((t & 3) == 3) scatter4(std::integral_constant<int, t>{});
  });
  // scores leave after the last tile: no stores among the counted row loads
#pragma unroll
  for (int tb = 0; tb < TPW; tb += 4) {
    const int64_t e = e_wave + 16 * (tb + g) + col;
#pragma unroll
    for (int qi = 0; qi < QPW; ++qi)
      if (e < N && t0 + qi < T) store_score(scores + (b * T + t0 + qi) * N + e, sc[qi][tb / 4]);
  }
}

template <int QK, int QPW, int TPW, int D, bool XS, bool PIPE, bool PG = false>
hipError_t launch_ring(const IndexArgs& a, hipStream_t s) {
  const int64_t per_wg = 4 * TPW * 16;
  dim3 grid(static_cast<uint32_t>((a.N + per_wg - 1) / per_wg),
            static_cast<uint32_t>((a.T + QPW - 1) / QPW), static_cast<uint32_t>(a.B));
  const auto* q = static_cast<const uint8_t*>(a.q);
  const auto* k = static_cast<const uint8_t*>(a.k);
  const KeyPages pg{a.block_table, a.max_blocks, a.n_pool, a.seq_pos};
  if (a.score_dtype == CSA_BF16)
    hipLaunchKernelGGL((index_ring_kernel<QK, QPW, TPW, D, XS, PIPE, uint16_t, PG>), grid, dim3(256), 0, s, a.T,
                       a.N, a.q_pos0, a.ratio, q, a.q_scale, a.w, k, a.k_scale, static_cast<uint16_t*>(a.scores), pg,
                       RingJobs{});
  else
    hipLaunchKernelGGL((index_ring_kernel<QK, QPW, TPW, D, XS, PIPE, float, PG>), grid, dim3(256), 0, s, a.T,
                       a.N, a.q_pos0, a.ratio, q, a.q_scale, a.w, k, a.k_scale, static_cast<float*>(a.scores), pg,
                       RingJobs{});
  return hipGetLastError();
}

template <int QK, int QPW, int TPW, int GT, int OCC, bool PG = false>
hipError_t launch_mfma(const IndexArgs& a, hipStream_t s) {
  const int64_t per_wg = 4 * TPW * 16;
  dim3 grid(static_cast<uint32_t>((a.N + per_wg - 1) / per_wg),
            static_cast<uint32_t>((a.T + QPW - 1) / QPW), static_cast<uint32_t>(a.B));
  const auto* q = static_cast<const uint8_t*>(a.q);
  const auto* k = static_cast<const uint8_t*>(a.k);
  const KeyPages pg{a.block_table, a.max_blocks, a.n_pool, a.seq_pos};
  if (a.score_dtype == CSA_BF16)
    hipLaunchKernelGGL((index_mfma_kernel<QK, QPW, TPW, GT, OCC, uint16_t, PG>), grid, dim3(256), 0, s, a.T, a.N,
                       a.q_pos0, a.ratio, q, a.q_scale, a.w, k, a.k_scale,
                       static_cast<uint16_t*>(a.scores), pg);
  else
    hipLaunchKernelGGL((index_mfma_kernel<QK, QPW, TPW, GT, OCC, float, PG>), grid, dim3(256), 0, s, a.T, a.N,
                       a.q_pos0, a.ratio, q, a.q_scale, a.w, k, a.k_scale,
                       static_cast<float*>(a.scores), pg);
  return hipGetLastError();
}

template <int QK>
hipError_t launch_qk(const IndexArgs& a, hipStream_t s) {
  // Shapes from sweeps on MI355X.  Decode streams keys from HBM: one query per
  // wave, 32 tiles per wave, a 4-slot ring (an 8-slot ring was slower), each
  // XCD on a contiguous range of key runs.  Prefill is MFMA and VALU work on
  // keys that stay in cache: two queries per wave share each key tile (one
  // query per wave, at two waves per SIMD, measured 13% slower on random
  // data).
  if constexpr (QK == CSA_MXFP4) {
    if (a.block_table) return launch_mfma<QK, 1, 8, 4, 2, true>(a, s);   // paged decode (T = 1)
    if (a.T <= 2) return launch_mfma<QK, 1, 8, 4, 2>(a, s);
    return launch_mfma<QK, 2, 64, 4, 2>(a, s);
  } else {
    if (a.block_table) return launch_ring<QK, 1, 32, 4, true, false, true>(a, s);   // paged decode (T = 1)
    if (a.T <= 2) return launch_ring<QK, 1, 32, 4, true, false>(a, s);
    return launch_ring<QK, 2, 64, 4, true, true>(a, s);
  }
}

}  // namespace

hipError_t launch_index(const IndexArgs& a, hipStream_t s) {
  if (a.B == 0 || a.T == 0 || a.N == 0) return hipSuccess;
  switch (a.qk_dtype) {
    case CSA_F32: {
      dim3 grid(static_cast<uint32_t>((a.N + 63) / 64), static_cast<uint32_t>(a.T),
                static_cast<uint32_t>(a.B));
      hipLaunchKernelGGL(index_f32_kernel, grid, dim3(256), 0, s, a.T, a.N, a.q_pos0, a.ratio,
                         static_cast<const float*>(a.q), a.w, static_cast<const float*>(a.k),
                         static_cast<float*>(a.scores));
      return hipGetLastError();
    }
    case CSA_BF16: return launch_qk<CSA_BF16>(a, s);
    case CSA_FP8_E4M3: return launch_qk<CSA_FP8_E4M3>(a, s);
    case CSA_MXFP4: return launch_qk<CSA_MXFP4>(a, s);
    default: return hipErrorNotSupported;
  }
}

namespace {

// Whether launch_index_jobs may run the jobs inside the decode indexer's
// launch (MXFP4 keys: the register kernel; bf16 keys: the ring kernel): every job a one-entry C4A write from bf16 rows in the
// narrow layout (two channels a thread, at most 256 threads), and any job
// output that lands in the keys or their scales is exactly entry e_new in
// the layout the indexer reads; no job output touches q, w or the scores.
bool jobs_fusable(const IndexArgs& a, const CompressArgs* jobs, int n, int64_t e_new) {
  if ((a.qk_dtype != CSA_MXFP4 && a.qk_dtype != CSA_BF16) || a.T != 1 || a.block_table || a.N < 1 || e_new < 0 ||
      e_new >= a.N)
    return false;
  if (a.score_dtype != CSA_BF16 && a.score_dtype != CSA_F32) return false;
  auto range = [](const void* p, int64_t bytes) {
    const uintptr_t b = reinterpret_cast<uintptr_t>(p);
    return std::make_pair(b, b + static_cast<uintptr_t>(bytes));
  };
  auto overlap = [](std::pair<uintptr_t, uintptr_t> x, std::pair<uintptr_t, uintptr_t> y) {
    return x.first < y.second && y.first < x.second;
  };
  const bool bfk = a.qk_dtype == CSA_BF16;   // bf16 keys: 256-byte rows, no scales
  const auto kr = range(a.k, a.B * a.N * (bfk ? 256 : 64)), sr = range(a.k_scale, bfk ? 0 : a.B * a.N * 4);
  const auto qr = range(a.q, a.B * 64 * (bfk ? 256 : 64)), qsr = range(a.q_scale, bfk ? 0 : a.B * 64 * 4);
  const auto wr = range(a.w, a.B * 64 * 4);
  const auto scr = range(a.scores, a.B * a.N * (a.score_dtype == CSA_BF16 ? 2 : 4));
  for (int q = 0; q < n; ++q) {
    const CompressArgs& j = jobs[q];
    if (j.ratio != 4 || j.in_dtype != CSA_BF16 || j.n_tok != 4 || j.B != a.B || j.c > 512 || j.c % 64) return false;
    if (j.out_dtype != CSA_BF16 && j.out_dtype != CSA_FP8_E4M3 && j.out_dtype != CSA_MXFP4) return false;
    const int64_t stride = j.out_batch_stride ? j.out_batch_stride : j.c;   // elements a sequence
    const int64_t span = (j.B - 1) * stride + j.c;
    const int64_t ob = j.out_dtype == CSA_BF16 ? 2 * span : (j.out_dtype == CSA_FP8_E4M3 ? span : span / 2);
    const auto orr = range(j.out, ob);
    const int64_t sb = j.out_dtype == CSA_FP8_E4M3 ? ((j.B - 1) * (stride / j.c) + 1) * 4
                       : j.out_dtype == CSA_MXFP4  ? ((j.B - 1) * (stride / j.c) + 1) * (j.c / 32)
                                                   : 0;
    const auto osr = range(j.out_scale, sb);
    for (const auto& x : {qr, qsr, wr, scr})
      if (overlap(orr, x) || (sb && overlap(osr, x))) return false;
    const bool in_keys = overlap(orr, kr) || (sb && overlap(osr, kr));
    const bool in_scales = overlap(orr, sr) || (sb && overlap(osr, sr));
    if (in_keys || in_scales) {
      const bool key_entry =
          bfk ? (j.out_dtype == CSA_BF16 && j.c == 128 && stride == a.N * 128 &&
                 orr.first == kr.first + static_cast<uintptr_t>(e_new * 256))
              : (j.out_dtype == CSA_MXFP4 && j.c == 128 && stride == a.N * 128 &&
                 orr.first == kr.first + static_cast<uintptr_t>(e_new * 64) &&
                 osr.first == sr.first + static_cast<uintptr_t>(e_new * 4));
      if (!key_entry) return false;
    }
  }
  return true;
}

}  // namespace

hipError_t launch_index_jobs(const IndexArgs& a, const CompressArgs* jobs, int n, int64_t e_new, hipStream_t s) {
  if (n < 1) return launch_index(a, s);
  if (a.B == 0 || a.N == 0 || !jobs_fusable(a, jobs, n, e_new)) {
    const hipError_t e = launch_compress_batch(jobs, n, s);
    return e != hipSuccess ? e : launch_index(a, s);
  }
  CompressBatch jb{};
  for (int q = 0; q < n; ++q) {
    const CompressArgs& j = jobs[q];
    const int64_t stride = j.out_batch_stride ? j.out_batch_stride : j.c;
    const double l2b = j.rope_dims > 0 ? std::log2(static_cast<double>(j.rope_base)) : 0.0;
    jb.j[q] = CompressJobDev{j.Ca, j.Za, j.Cb, j.Zb, j.prev_Cb, j.prev_Zb, j.bias, j.gamma, j.out, j.n_tok, j.pos0,
                             stride, 1, j.B, j.eps, static_cast<int>(j.c), 1, j.rope_dims, l2b, j.rope_anchor,
                             j.out_scale, stride / j.c,
                             j.out_dtype == CSA_FP8_E4M3 ? 1 : (j.out_dtype == CSA_MXFP4 ? 2 : 0)};
  }
  const auto* q = static_cast<const uint8_t*>(a.q);
  const auto* k = static_cast<const uint8_t*>(a.k);
  if (a.qk_dtype == CSA_BF16) {
    // the bf16 decode shape of launch_qk (32 tiles a wave, a 4-slot ring):
    // the workgroup of the new entry's key run writes it first
    constexpr int TPW = 32;
    constexpr int64_t per_wg = 4 * TPW * 16;
    const dim3 grid(static_cast<uint32_t>((a.N + per_wg - 1) / per_wg), 1, static_cast<uint32_t>(a.B));
    const RingJobs rj{jb, n, e_new / per_wg};
    if (a.score_dtype == CSA_BF16)
      hipLaunchKernelGGL((index_ring_kernel<CSA_BF16, 1, TPW, 4, true, false, uint16_t, false, true>), grid, dim3(256),
                         0, s, a.T, a.N, a.q_pos0, a.ratio, q, a.q_scale, a.w, k, a.k_scale,
                         static_cast<uint16_t*>(a.scores), KeyPages{nullptr, 0, 0, nullptr}, rj);
    else
      hipLaunchKernelGGL((index_ring_kernel<CSA_BF16, 1, TPW, 4, true, false, float, false, true>), grid, dim3(256),
                         0, s, a.T, a.N, a.q_pos0, a.ratio, q, a.q_scale, a.w, k, a.k_scale,
                         static_cast<float*>(a.scores), KeyPages{nullptr, 0, 0, nullptr}, rj);
    return hipGetLastError();
  }
  // the MXFP4 decode shape of launch_qk: one query a wave, 8 tiles a wave;
  // registers for five waves a SIMD, the plain kernel's occupancy
  constexpr int TPW = 8, GT = 4, OCC = 5;
  constexpr int64_t per_wg = 4 * TPW * 16;
  const dim3 grid(static_cast<uint32_t>((a.N + per_wg - 1) / per_wg), 1, static_cast<uint32_t>(a.B));
  const int64_t x_own = e_new / per_wg;
  const size_t smem = 64 * sizeof(float);   // the jobs' RMSNorm sums and fp8 amax
  if (a.score_dtype == CSA_BF16)
    hipLaunchKernelGGL((index_mfma_jobs_kernel<CSA_MXFP4, TPW, GT, OCC, uint16_t>), grid, dim3(256), smem, s, a.N,
                       a.q_pos0, a.ratio, q, a.q_scale, a.w, k, a.k_scale, static_cast<uint16_t*>(a.scores), jb, n,
                       x_own);
  else
    hipLaunchKernelGGL((index_mfma_jobs_kernel<CSA_MXFP4, TPW, GT, OCC, float>), grid, dim3(256), smem, s, a.N,
                       a.q_pos0, a.ratio, q, a.q_scale, a.w, k, a.k_scale, static_cast<float*>(a.scores), jb, n, x_own);
  return hipGetLastError();
}

}  // namespace csa
