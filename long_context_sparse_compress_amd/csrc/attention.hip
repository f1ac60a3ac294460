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
// heads) and a contiguous run of 32-row tiles of that list; wave w computes
// the logits and softmax of heads 16w..16w+15 and the output columns
// 128w..128w+127 of every head.
//
// Per tile (bf16 path):
//  * each wave copies 8 of the tile's rows straight from global memory into a
//    row-major LDS tile (global_load_lds, 16 bytes per lane, no registers);
//    later tiles are in flight while the current one is computed;
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16, wave w taking heads
//    16w..16w+15 with their q in registers.  The C layout of S^T gives lane
//    (head j, group g) the logits of rows {4g..4g+3, 16+4g..16+4g+3};
//  * online softmax in the exp2 domain (logits pre-multiplied by log2 e) on
//    those registers, against a reference maximum that moves only when a
//    tile's maximum exceeds it by more than a factor 2^8, so O is rarely
//    rescaled.  Packed to bf16 the probabilities are already lane (j, g)'s
//    slice of the A operand of P V for that head block, so each wave
//    publishes them in LDS as one 16-byte word per lane, with its heads'
//    rescale factors;
//  * P V is split over the latent dimension instead of the heads: wave w
//    computes O[all 64 heads, 128w..128w+127] from the four published P blocks
//    and V columns it reads with transposing LDS reads (ds_read_b64_tr_b16)
//    from the same row-major tile.  Each wave then reads a quarter of V
//    instead of all of it, which cuts the tile's LDS reads by 30%;
//  * O (64 heads x 128 columns fp32 per wave) stays in registers.
// Decode has few queries, so a query's tiles are split over several
// workgroups whose partial (max, sum, O) go to the workspace; a combine
// kernel merges them in a fixed order (bit-reproducible results).
#include <type_traits>

#include <cmath>
#include <mutex>

#include "compress_entry.h"
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
constexpr float kLazyMax = 8.f;             // see the online softmax in attn_bf16_kernel

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
  int rope_R;           // inverse RoPE on the output's last rope_R dims (0: none)
  double rope_l2b;      // log2 of the rotary base
  // paged decode (heterogeneous cache): compressed entry e of sequence b is
  // row (block_table[b][e >> page_shift] << page_shift) + (e & mask) of the
  // pool kv_cmp (n_pool blocks; other block ids are padding); window position
  // p is row p % ring (ring a power of two) of sequence b's ring kv_raw;
  // sequence b's query sits at seq_pos[b] (T = 1)
  const int32_t* block_table;
  int64_t max_blocks, n_pool;
  int page_shift;
  int64_t ring;
  const int64_t* seq_pos;
  // a decode step's C128A write run inside the launch (dense lists): the
  // workgroup whose tiles include list tile job_tile first pools its
  // sequence's entry into the cache (job_tile < 0: none)
  CompressJobDev job;
  int64_t job_tile;
};

// Inverse partial RoPE of one output value held by this lane at column col,
// given the (cos, sin) of its pair's angle; the value of column col ^ 1 sits
// in lane ^ 1.  Every lane of the wave calls it (the exchange is wave-wide);
// columns outside the rotated part keep their value.
__device__ __forceinline__ float inv_rope_lane(float v, int col, float2 k, const Params& P) {
  const float other = __shfl_xor(v, 1, 64);
  if (col < kD - P.rope_R) return v;
  return (col & 1) ? other * k.y + v * k.x : v * k.x - other * k.y;
}
// (cos, sin) of the inverse rotation of the pair holding column col
__device__ __forceinline__ float2 inv_rope_cs(int col, int64_t pos, const Params& P) {
  float c = 1.f, s = 0.f;
  if (col >= kD - P.rope_R) rope_cos_sin(-pos, (col - (kD - P.rope_R)) >> 1, P.rope_R, P.rope_l2b, c, s);
  return make_float2(c, s);
}

struct List {
  int64_t n_cmp;   // compressed slots at the head of the list
  int64_t wstart;  // first window position
  int64_t L;       // list length
  int64_t pos;     // the query's position
};

// PG: the paged-decode addressing of Params may be in use (checked at run
// time); without it the kernels compile the contiguous addressing only.
template <bool PG>
__device__ __forceinline__ List make_list(const Params& P, int64_t b, int64_t t) {
  const int64_t pos = (PG && P.seq_pos) ? P.seq_pos[b] : P.q_pos0 + t;
  List l;
  l.pos = pos;
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
// The Top-k slot is read with `slot(p)`: from global memory, or from the
// query's Top-k row staged in LDS.
// Row of compressed entry e of sequence b in kv_cmp (-1: none), paged or not.
template <bool PG>
__device__ __forceinline__ int64_t cmp_row(const Params& P, int64_t b, int64_t e) {
  if (e < 0 || e >= P.N) return -1;
  if (!PG || !P.block_table) return b * P.N + e;
  const int64_t blk = P.block_table[b * P.max_blocks + (e >> P.page_shift)];
  if (blk < 0 || blk >= P.n_pool) return -1;
  return (blk << P.page_shift) + (e & ((int64_t{1} << P.page_shift) - 1));
}

// Row of raw (window) position u of sequence b in kv_raw: a ring or a run
// starting at raw_pos0.
template <bool PG>
__device__ __forceinline__ int64_t raw_row(const Params& P, int64_t b, int64_t u) {
  return (PG && P.ring) ? b * P.ring + (u & (P.ring - 1)) : b * P.n_raw + (u - P.raw_pos0);
}

template <typename E, bool PG, typename Slot>
__device__ __forceinline__ const E* row_ptr_by(const Params& P, int64_t b, const List& l, int64_t p, Slot slot) {
  if (p >= l.L) return nullptr;
  if (p < l.n_cmp) {
    const int64_t r = cmp_row<PG>(P, b, P.idx ? static_cast<int64_t>(slot(p)) : p);
    return r < 0 ? nullptr : static_cast<const E*>(P.kv_cmp) + r * kD;
  }
  return static_cast<const E*>(P.kv_raw) + raw_row<PG>(P, b, l.wstart + (p - l.n_cmp)) * kD;
}

template <typename E, bool PG>
__device__ __forceinline__ const E* row_ptr(const Params& P, int64_t b, int64_t t, const List& l, int64_t p) {
  const int32_t* idx = P.idx + (b * P.T + t) * P.k;
  return row_ptr_by<E, PG>(P, b, l, p, [&](int64_t q) { return idx[q]; });
}

// Whether list row `p` is a real row (row_ptr would not return nullptr).
template <bool PG>
__device__ __forceinline__ bool row_valid(const Params& P, int64_t b, const List& l, int64_t p,
                                          const int32_t* sidx) {
  if (p >= l.L) return false;
  if (p < l.n_cmp) {
    if (PG && P.block_table) return cmp_row<PG>(P, b, P.idx ? static_cast<int64_t>(sidx[p]) : p) >= 0;
    if (P.idx) {
      const int32_t e = sidx[p];
      return e >= 0 && e < P.N;
    }
  }
  return true;
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

// One split's partial in the workspace, in floats: O as 64 x 512 bf16 (in the
// MFMA register layout), then 64 running maxima and 64 sums in fp32.  bf16
// halves the bytes the split kernels write and the combine reads; its
// rounding (2^-9 relative) is that of the bf16 output itself.
constexpr int64_t kSplitFloats = kH * kD / 2 + 2 * kH;
static_assert(kSplitFloats * 4 == CSA_HEADS * CSA_HEAD_DIM * 2 + 2 * CSA_HEADS * 4, "matches attn_split_bytes");

__device__ __forceinline__ float4 unpack4(uint2 v) {
  return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                     __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
}

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
// Both addresses are formed as tile + one offset: a deeper chain of pointer
// arithmetic can lose the record of which LDS array a read touches, and the
// compiler then waits for every row load in flight before that read.
__device__ __forceinline__ bf16x8 v_operand(const uint8_t* tile, int n, uint32_t lane_off) {
  const uint32_t off = lane_off + n * 32;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(tile + off));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(tile + (off + 16 * kKsStride)));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Workgroup barrier that drains only this wave's LDS operations (the caller
// has already waited for its row loads).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(63 & 15 | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// Tile buffers: while tile t is computed, tile t + 1's rows arrive by DMA in
// the other buffer, requested one row at a time between the QK MFMAs, and
// every read of the tile being computed must be provably disjoint from the
// loads in flight (distinct LDS arrays), or the compiler drains them before
// each LDS read.  With two groups the buffers alternate and the loop body is
// instantiated once per buffer.  One group keeps a single body: rows land in
// tb1 and each step first copies them into tb0 (two bodies do not fit its
// registers: the spill reloads, being memory loads, wait for every row load
// in flight).
//
// TGN tile groups of four waves share a workgroup (two for long decode runs): group k
// takes tiles tile0 + k, tile0 + k + TGN, ... of the workgroup's run with its
// own buffers, so a run of n tiles takes ceil(n / TGN) steps.  The groups'
// running (max, sum, O) are merged through LDS at the end.
//
// HB head blocks of 16 heads per workgroup.  HB = 4 is the kernel above.
// HB = 1 (batch-invariant decode) gives each of a query's four head blocks
// its own workgroup over the whole row list: wave 0 computes the block's
// logits and softmax, every wave a quarter of its P V columns.  Every output
// element then goes through exactly the operations of the HB = 4 kernel with
// one split (same tiles in the same order, same MFMA operands, same per-head
// softmax arithmetic), so the two give identical bits -- the multi-workgroup
// kernel the pages pair with the one-workgroup kernel, with the work divided
// by heads instead of rows so that no cross-workgroup merge is needed.
template <int TGN, int HB, bool PG = false, bool CJ = false>
__global__ void __launch_bounds__(256 * TGN, 3 - TGN)
attn_bf16_kernel(Params P) {
  static_assert(TGN == 1 || TGN == 2, "one or two tile groups");
  static_assert(HB == 4 || (HB == 1 && TGN == 1), "one head block per workgroup runs one group");
  __shared__ __attribute__((aligned(16))) uint8_t tb0[TGN][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t tb1[TGN][kTileBytes];
  __shared__ int32_t sidx[CSA_MAX_TOPK];                                   // Top-k row of this query
  __shared__ uint4 pshare[TGN][4 * 64];   // P of each wave's 16 heads, in MFMA operand order (lane-major)
  __shared__ float4 ashare[TGN][kH / 4];  // per-head rescale factor of the current tile
  __shared__ float4 fshare[kH / 4];       // per-head output factor (epilogue)
  __shared__ uint4 rescale_any[TGN];      // per wave: some head's running max moved
  __shared__ float mlshare[TGN][2][kH];   // per group: running max and sum of each head (merge)
  __shared__ float2 rope_cs[kD / 2];      // inverse RoPE (cos, sin) of this query's output pairs

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: row addressing stays scalar
  const int tg = TGN == 1 ? 0 : (wv >> 2), wid = wv & 3;     // tile group, wave within the group
  const int j = lane & 15, g = lane >> 4;
  // transposing V reads: lane k of group g points at row 4g + k/4, columns 4(k%4)..
  const uint32_t voff = (4 * g + (j >> 2)) * kKsStride + 8 * (j & 3);
  // all splits (or head blocks) of a query -- and its q, and the combine
  // that reads its partials -- on one XCD, so they share that XCD's L2
  const uint32_t wg0 = xcd_swizzle(blockIdx.x, gridDim.x);
  const int hq = HB == 4 ? 0 : static_cast<int>(wg0 % 4);    // head block of an HB = 1 workgroup
  const uint32_t wg = HB == 4 ? wg0 : wg0 / 4;
  const int64_t gq = wg / P.splits;
  const int split = static_cast<int>(wg % P.splits);
  // the waves that compute logits and softmax, and the head block of each
  const bool qk_wave = HB == 4 || wid == 0;
  const int hb_qk = HB == 4 ? wid : hq;     // global head block
  const int hl_qk = HB == 4 ? wid : 0;      // its slot in this workgroup's LDS exchange
  const int64_t b = gq / P.T, t = gq % P.T;
  const List l = make_list<PG>(P, b, t);
  int64_t tile0, tile1;
  split_range(P, l, split, tile0, tile1);

  uint8_t* const T0 = tb0[tg];
  uint8_t* const T1 = tb1[tg];

  if constexpr (CJ) {
    // The decode step's new C128A entry of sequence b, pooled by the
    // workgroup whose tiles read it, before any of its rows are requested;
    // the tile buffers serve as the pooling's LDS.  No other workgroup reads
    // that entry.
    if (tile0 <= P.job_tile && P.job_tile < tile1) {
      const CompressJobDev& J = P.job;
      compress_entry<uint16_t, uint16_t, 128, false, 8, 4>(
          0, b, 0, 1, J.n_tok, J.c, J.pos0, static_cast<const uint16_t*>(J.Ca), static_cast<const uint16_t*>(J.Za),
          nullptr, nullptr, nullptr, nullptr, J.bias, J.gamma, J.eps, static_cast<uint16_t*>(J.out), J.out_stride,
          J.G, nullptr, J.rope_R, J.rope_l2b, J.rope_anchor, nullptr, 0, -1, reinterpret_cast<float*>(&tb0[0][0]));
      __syncthreads();   // the entry is in the cache and the tile buffers are free
    }
  }

  // The query's own raw row is always in the list: padding rows load it (and are masked).
  const uint16_t* safe_row = static_cast<const uint16_t*>(P.kv_raw) + raw_row<PG>(P, b, l.pos) * kD;
  // lane e (mod 8) of wave w: source of row 8w + e of `tile`
  auto row_source = [&](int64_t tile, auto slot) -> uint64_t {
    const uint16_t* p = row_ptr_by<uint16_t, PG>(P, b, l, tile * kTile + 8 * wid + (lane & 7), slot);
    return reinterpret_cast<uint64_t>(p ? p : safe_row);
  };
  // row 8w + e of a tile, from lane e's source, into tile buffer `dst`
  auto issue_row = [&](uint64_t src, int e, uint8_t* dst) {
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(src), e);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(src >> 32), e);
    row_to_lds(reinterpret_cast<const uint16_t*>((static_cast<uint64_t>(hi) << 32) | lo),
               dst + (8 * wid + e) * kKsStride, lane);
  };

  // The group's first tile's rows go out before anything else, their indices
  // read straight from global memory.
  if (tile0 + tg < tile1) {
    const int32_t* gidx = P.idx ? P.idx + gq * P.k : nullptr;   // only read for a Top-k list
    const uint64_t src = row_source(tile0 + tg, [&](int64_t q) { return gidx[q]; });
#pragma unroll
    for (int e = 0; e < 8; ++e) issue_row(src, e, TGN == 1 ? T1 : T0);
  }

  // q fragments of head 16*hb_qk + j, d in [g*128, g*128+128)
  uint4 qf[16];
  if (qk_wave) {
    const uint4* qp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(P.q) +
                                                     ((gq * kH) + 16 * hb_qk + j) * kD + g * 128);
#pragma unroll
    for (int s = 0; s < 16; ++s) qf[s] = qp[s];
  }

  // Stage the slice of this query's Top-k row that this workgroup's tiles use.
  if (P.idx) {
    const int64_t p0 = tile0 * kTile;
    const int64_t p1 = tile1 * kTile < l.n_cmp ? tile1 * kTile : l.n_cmp;
    const int32_t* src = P.idx + gq * P.k;
    for (int64_t p = p0 + tid; p < p1; p += 256 * TGN) sidx[p] = src[p];
    __syncthreads();
  }

  // O for the workgroup's head blocks and d in [128 w, 128 w + 128): o[8 hb + db]
  // holds heads 16 hb + 4g + i (i = 0..3) of local block hb, column 128 w + 16 db + j
  f32x4 o[8 * HB];
#pragma unroll
  for (int n = 0; n < 8 * HB; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // one step: wait for the group's tile (in buffer bc), compute it while the
  // group's next tile streams into the other buffer.  Every wave takes part in
  // the barriers; a group whose run has ended only waits.
  auto step = [&](int64_t tile, bool active, auto bc) {
    constexpr int kPipe = 2;
    // one group: compute in tb0, land in tb1; two groups: alternate
    uint8_t* const Ks = (TGN == 1 || decltype(bc)::value == 0) ? T0 : T1;
    uint8_t* const Kn = (TGN == 1 || decltype(bc)::value == 0) ? T1 : T0;
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0): this wave's rows of the tile landed
    lds_barrier();   // every wave's rows landed; nobody still reads the buffer the next rows go to
    if constexpr (TGN == 1) {
      // copy the landed tile into the compute buffer (this wave's 8 rows)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int off = (8 * wid + e) * kKsStride + lane * 16;
        *reinterpret_cast<uint4*>(T0 + off) = *reinterpret_cast<const uint4*>(T1 + off);
      }
      lds_barrier();   // tb0 holds the tile; tb1 is free
    }
    if (active && !qk_wave) {   // HB = 1, waves 1..3: only their rows of the next tile
      if (tile + TGN < tile1) {
        const uint64_t nsrc = row_source(tile + TGN, [&](int64_t q) { return sidx[q]; });
#pragma unroll
        for (int e = 0; e < 8; ++e) issue_row(nsrc, e, Kn);
      }
    }
    if (active && qk_wave) {
      const bool refill = tile + TGN < tile1;
      const uint64_t nsrc = refill ? row_source(tile + TGN, [&](int64_t q) { return sidx[q]; }) : 0;

      // S^T = K Q^T for rows 0..15 (s0) and 16..31 (s1).  LDS operands are read
      // kPipe k-steps ahead through a register ring (at this register budget
      // the scheduler keeps about one step of reads in flight; deeper rings,
      // explicit schedule groups and precise waits measured no faster).
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
      const uint8_t* ka = Ks + j * kKsStride + g * 256;
      uint4 ra[kPipe][2];
#pragma unroll
      for (int d = 0; d < kPipe; ++d) {
        ra[d][0] = *reinterpret_cast<const uint4*>(ka + d * 16);
        ra[d][1] = *reinterpret_cast<const uint4*>(ka + 16 * kKsStride + d * 16);
      }
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        // the next tile's rows go out one at a time between MFMAs: a burst of
        // row loads would stall this wave until the memory pipeline drains
        if (refill && (s & 1) == 0) issue_row(nsrc, s / 2, Kn);
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ra[s % kPipe][0]), as_bf16x8(qf[s]), s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ra[s % kPipe][1]), as_bf16x8(qf[s]), s1, 0, 0, 0);
        if (s + kPipe < 16) {
          ra[s % kPipe][0] = *reinterpret_cast<const uint4*>(ka + (s + kPipe) * 16);
          ra[s % kPipe][1] = *reinterpret_cast<const uint4*>(ka + 16 * kKsStride + (s + kPipe) * 16);
        }
      }
      // rows of this lane: 4g+i (s0) and 16+4g+i (s1); padding rows are masked
      // which of the tile's 32 rows are real: lane r (mod 32) tests row r
      const uint32_t vrows =
          static_cast<uint32_t>(__ballot(row_valid<PG>(P, b, l, tile * kTile + (lane & 31), sidx))) >> (4 * g);
      float lg[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lg[i] = (vrows >> i) & 1 ? s0[i] * P.scale_log2 : -INFINITY;
        lg[4 + i] = (vrows >> (16 + i)) & 1 ? s1[i] * P.scale_log2 : -INFINITY;
      }
      float mt = lg[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mt = fmaxf(mt, lg[i]);
      mt = pair_max16(mt);
      mt = pair_max32(mt);
      // The reference maximum moves only when the tile's exceeds it by more
      // than kLazyMax (log2 units): the exponentials stay below 2^kLazyMax,
      // and a running maximum that creeps up costs no rescale of O.  Every
      // later merge takes (max, sum, O) relative to whatever reference each
      // side used, so the result is the same up to rounding.
      const bool move = mt > m_run + kLazyMax;   // false while both are -inf
      const float m_new = move ? mt : m_run;
      const bool none = (m_new == -INFINITY);
      // (before the first real row O and the sum are zero: nothing to rescale)
      const float alpha = move && m_run != -INFINITY ? fast_exp2(m_run - m_new) : 1.f;
      float p[8], psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = none ? 0.f : fast_exp2(lg[i] - m_new);
        psum += p[i];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      // hand this wave's P and rescale factors to the other waves of the group
      pshare[tg][hl_qk * 64 + lane] = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                                 pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));
      if (g == 0) reinterpret_cast<float*>(ashare[tg])[16 * hl_qk + j] = alpha;
      const bool moved = __ballot(alpha != 1.f) != 0;
      if (lane == 0) reinterpret_cast<uint32_t*>(&rescale_any[tg])[hl_qk] = moved;
    }
    lds_barrier();
    if (active) {
      // O[:, 128 w .. 128 w + 127] = alpha O + P V over the workgroup's heads
      // (a rescale by 1 of a head whose maximum did not move is exact)
      const uint4 any = rescale_any[tg];
      if (HB == 4 ? (any.x | any.y | any.z | any.w) : any.x) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          const float4 a4 = ashare[tg][4 * hb + g];
#pragma unroll
          for (int db = 0; db < 8; ++db) {
            o[8 * hb + db][0] *= a4.x; o[8 * hb + db][1] *= a4.y;
            o[8 * hb + db][2] *= a4.z; o[8 * hb + db][3] *= a4.w;
          }
        }
      }
      bf16x8 pf[HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) pf[hb] = as_bf16x8(pshare[tg][hb * 64 + lane]);
      bf16x8 vr[kPipe];
#pragma unroll
      for (int d = 0; d < kPipe; ++d) vr[d] = v_operand(Ks, 8 * wid + d, voff);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
          o[8 * hb + db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[hb], vr[db % kPipe], o[8 * hb + db], 0, 0, 0);
        if (db + kPipe < 8) vr[db % kPipe] = v_operand(Ks, 8 * wid + db + kPipe, voff);
      }
    }
  };

  const int64_t nsteps = (tile1 - tile0 + TGN - 1) / TGN;
  if constexpr (TGN == 1) {
    for (int64_t tile = tile0; tile < tile1; ++tile) step(tile, true, std::integral_constant<int, 0>{});
  } else {
    // two steps per trip, one per buffer (an odd count ends with a step that
    // only waits: no branch around the second body)
    for (int64_t i = 0; i < nsteps; i += 2) {
      const int64_t tile = tile0 + tg + i * TGN;
      step(tile, tile < tile1, std::integral_constant<int, 0>{});
      step(tile + TGN, tile + TGN < tile1, std::integral_constant<int, 1>{});
    }
  }

  // The output's inverse RoPE angles, one pair per thread into LDS (formed in
  // the prologue they would keep values live through the loop and spill);
  // read after the epilogue's barrier.  A split run leaves this to the
  // combine.
  if (__builtin_expect(P.rope_R > 0 && P.splits == 1, 0)) {
    for (int p = tid; p < P.rope_R / 2; p += 256 * TGN)
      rope_cs[p] = inv_rope_cs(kD - P.rope_R + 2 * p, l.pos, P);
  }

  // per-head totals: lanes with (lane & 15) == h hold head 16*wid + h
  float l_tot = l_run;
  l_tot = pair_sum16(l_tot, l_tot);
  l_tot = pair_sum32(l_tot, l_tot);
  const int head_j = 16 * hb_qk + j;      // global head of this lane's logits (qk waves)
  const int hl_j = 16 * hl_qk + j;        // its slot in this workgroup's exchange

  // o[] is indexed with constants only (a run-time index would move it to
  // scratch memory): the group-dependent parts below branch on the group and
  // run code in which the group is a constant.
  if constexpr (TGN == 2) {
    // The two groups merge their (max, sum, O) through LDS.  Group k keeps the
    // head blocks 2k, 2k+1 (o[16k .. 16k+15]): it parks the other half for the
    // other group and folds that group's parked copy of its own half in.
    if (g == 0) {
      mlshare[tg][0][head_j] = m_run;
      mlshare[tg][1][head_j] = l_tot;
    }
    lds_barrier();   // every wave is past its last tile: the tile buffers are free
    auto park = [&](auto kc) {   // 16 KB per wave: group 0 parks in tb0, group 1 in tb1
      constexpr int k = decltype(kc)::value;
      float4* mine = reinterpret_cast<float4*>((k == 0 ? &tb0[0][0] : &tb1[0][0]) + wid * 16384) + lane;
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        const f32x4& v = o[16 * (1 - k) + n];
        mine[n * 64] = make_float4(v[0], v[1], v[2], v[3]);
      }
    };
    if (tg == 0) park(std::integral_constant<int, 0>{});
    else park(std::integral_constant<int, 1>{});
    lds_barrier();
    auto fold = [&](auto kc) {
      constexpr int k = decltype(kc)::value;
      const float4* theirs = reinterpret_cast<const float4*>((k == 0 ? &tb1[0][0] : &tb0[0][0]) + wid * 16384) + lane;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int hb = 2 * k + hh;
        float am[4], at[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int h = 16 * hb + 4 * g + i;
          const float mm = mlshare[k][0][h], mo = mlshare[1 - k][0][h];
          const float M = fmaxf(mm, mo);
          am[i] = mm == -INFINITY ? 0.f : fast_exp2(mm - M);
          at[i] = mo == -INFINITY ? 0.f : fast_exp2(mo - M);
        }
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const float4 v = theirs[(8 * hh + db) * 64];
          f32x4& x = o[8 * hb + db];
          x[0] = x[0] * am[0] + v.x * at[0];
          x[1] = x[1] * am[1] + v.y * at[1];
          x[2] = x[2] * am[2] + v.z * at[2];
          x[3] = x[3] * am[3] + v.w * at[3];
        }
      }
    };
    if (tg == 0) fold(std::integral_constant<int, 0>{});
    else fold(std::integral_constant<int, 1>{});
    const float m0 = mlshare[0][0][head_j], m1 = mlshare[1][0][head_j];
    const float M = fmaxf(m0, m1);
    l_tot = (m0 == -INFINITY ? 0.f : mlshare[0][1][head_j] * fast_exp2(m0 - M)) +
            (m1 == -INFINITY ? 0.f : mlshare[1][1][head_j] * fast_exp2(m1 - M));
    m_run = M;
  }
  // whether this wave writes head block hb: all four, or its group's two (uniform)
  auto writes = [&](int hb) { return TGN == 1 || (hb >> 1) == tg; };

  if (P.splits == 1) {
    if (tg == 0 && qk_wave && g == 0) {
      float M = m_run;
      float zl = -INFINITY;
      if (P.sink) {
        zl = P.sink[head_j] * kLog2e;
        M = fmaxf(M, zl);
      }
      const float em = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - M);
      const float denom = l_tot * em + (P.sink ? fast_exp2(zl - M) : 0.f);
      reinterpret_cast<float*>(fshare)[hl_j] = em / denom;
      if (P.lse) P.lse[gq * kH + head_j] = kLn2 * (M + log2f(denom));
    }
    lds_barrier();
    uint16_t* out = static_cast<uint16_t*>(P.out) + gq * kH * kD + 128 * wid + j;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      if (!writes(hb)) continue;
      const int hg = HB == 4 ? hb : hq;   // global head block
      const float4 f4 = fshare[4 * hb + g];
      const float f[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = o[8 * hb + db][i] * f[i];
        if (__builtin_expect(P.rope_R > 0, 0)) {
          const int col = 128 * wid + 16 * db + j;
          const float2 k = rope_cs[(col - (kD - P.rope_R) > 0 ? col - (kD - P.rope_R) : 0) >> 1];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = inv_rope_lane(v[i], col, k, P);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) out[(16 * hg + 4 * g + i) * kD + 16 * db] = f32_to_bf16(v[i]);
      }
    }
  } else if constexpr (HB == 4) {
    // partial O in bf16 in the MFMA's own layout, 8 bytes per lane:
    // [wave][hb][db][lane]; then the heads' running max and sum in fp32
    float* w = P.ws + (gq * P.splits + split) * kSplitFloats;
    uint2* wo = reinterpret_cast<uint2*>(w) + wid * (4 * 8 * 64) + lane;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      if (!writes(hb)) continue;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const f32x4& v = o[8 * hb + db];
        wo[(hb * 8 + db) * 64] = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
    if (tg == 0 && g == 0) {
      w[kH * kD / 2 + head_j] = m_run;
      w[kH * kD / 2 + kH + head_j] = l_tot;
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
  const List l = make_list<true>(P, b, t);
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
      const float* p = row_ptr<float, true>(P, b, t, l, base + r);
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
  for (int i = 0; i < 16; ++i) ov[i] *= f;
  if (__builtin_expect(P.rope_R > 0, 0)) {   // inverse partial RoPE at the query's position; pairs are thread-local
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const int col = part * 16 + i;
      if (col >= kD - P.rope_R) {
        float cs, sn;
        rope_cos_sin(-l.pos, (col - (kD - P.rope_R)) >> 1, P.rope_R, P.rope_l2b, cs, sn);
        rope_pair(ov[i], ov[i + 1], cs, sn);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) out[i] = ov[i];
  if (P.lse && part == 0) P.lse[gq * kH + head] = kLn2 * (M + log2f(denom));
}

// ------------------------------------------------------------ split combine
// One workgroup per (query, 16-head block hb, 128-column quarter w), which is
// one contiguous 8 KB run of every split's partial O.  Each thread owns two
// float4 of the run (heads 4g..4g+3 of the block, two columns) and folds the
// splits in order into a running (max, sum, O) of its four heads -- a single
// pass in which the loads of the next splits are already in flight.  Every
// thread of a lane group computes the same statistics in the same order, so
// the result is bit-reproducible.  The bf16 result goes through LDS so that
// each output row is written in full 16-byte pieces.
__global__ void __launch_bounds__(256)
attn_combine_kernel(Params P) {
  __shared__ __attribute__((aligned(16))) uint16_t ot[16 * 128];
  const uint32_t wg = xcd_swizzle(blockIdx.x, gridDim.x);   // the XCD its partials were written on
  const int64_t gq = wg / 16;
  const int hb = static_cast<int>(wg / 4 % 4), w = static_cast<int>(wg % 4);
  const int S = P.splits, tid = threadIdx.x;
  const float* base = P.ws + gq * S * kSplitFloats;
  const int ln = tid & 63, g = ln >> 4, j = ln & 15, db0 = tid >> 6;
  const int h0 = 16 * hb + 4 * g;   // first of this thread's four heads
  const uint2* src = reinterpret_cast<const uint2*>(base) + ((w * 4 + hb) * 8 + db0) * 64 + ln;
  // inverse RoPE (cos, sin) of this thread's two columns, formed while the
  // partials load
  const int c0 = 16 * db0 + j, c1 = c0 + 64;
  float2 k0 = make_float2(1.f, 0.f), k1 = k0;
  if (__builtin_expect(P.rope_R > 0, 0)) {
    const int64_t pos = P.seq_pos ? P.seq_pos[gq / P.T] : P.q_pos0 + gq % P.T;
    k0 = inv_rope_cs(128 * w + c0, pos, P);
    k1 = inv_rope_cs(128 * w + c1, pos, P);
  }
  float M[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY}, L[4] = {0.f, 0.f, 0.f, 0.f};
  float4 acc0 = make_float4(0.f, 0.f, 0.f, 0.f), acc1 = acc0;
#pragma unroll 4
  for (int s = 0; s < S; ++s) {
    const float* st = base + s * kSplitFloats + kH * kD / 2;
    const float4 ms = *reinterpret_cast<const float4*>(st + h0);
    const float4 ls = *reinterpret_cast<const float4*>(st + kH + h0);
    const float4 v0 = unpack4(src[s * (kSplitFloats / 2)]);
    const float4 v1 = unpack4(src[s * (kSplitFloats / 2) + 4 * 64]);   // d-block db0 + 4
    const float m4[4] = {ms.x, ms.y, ms.z, ms.w}, l4[4] = {ls.x, ls.y, ls.z, ls.w};
    float a[4], e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mn = fmaxf(M[i], m4[i]);
      a[i] = (M[i] == -INFINITY) ? 0.f : fast_exp2(M[i] - mn);   // rescale of what is folded so far
      e[i] = (m4[i] == -INFINITY) ? 0.f : fast_exp2(m4[i] - mn);  // weight of split s
      L[i] = L[i] * a[i] + l4[i] * e[i];
      M[i] = mn;
    }
    acc0.x = acc0.x * a[0] + v0.x * e[0]; acc0.y = acc0.y * a[1] + v0.y * e[1];
    acc0.z = acc0.z * a[2] + v0.z * e[2]; acc0.w = acc0.w * a[3] + v0.w * e[3];
    acc1.x = acc1.x * a[0] + v1.x * e[0]; acc1.y = acc1.y * a[1] + v1.y * e[1];
    acc1.z = acc1.z * a[2] + v1.z * e[2]; acc1.w = acc1.w * a[3] + v1.w * e[3];
  }
  float f[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float denom = L[i], Mi = M[i];
    if (P.sink) {
      const float zl = P.sink[h0 + i] * kLog2e;
      const float mn = fmaxf(Mi, zl);
      denom = (Mi == -INFINITY ? 0.f : denom * fast_exp2(Mi - mn)) + fast_exp2(zl - mn);
      f[i] = (Mi == -INFINITY ? 0.f : fast_exp2(Mi - mn)) / denom;
      Mi = mn;
    } else {
      f[i] = 1.f / denom;
    }
    if (P.lse && w == 0 && db0 == 0 && j == 0) P.lse[gq * kH + h0 + i] = kLn2 * (Mi + log2f(denom));
  }
  // heads 4g..4g+3 of the block, columns 16 db + j of the quarter
  float v0[4] = {acc0.x * f[0], acc0.y * f[1], acc0.z * f[2], acc0.w * f[3]};
  float v1[4] = {acc1.x * f[0], acc1.y * f[1], acc1.z * f[2], acc1.w * f[3]};
  if (__builtin_expect(P.rope_R > 0, 0)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v0[i] = inv_rope_lane(v0[i], 128 * w + c0, k0, P);
      v1[i] = inv_rope_lane(v1[i], 128 * w + c1, k1, P);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ot[(4 * g + i) * 128 + c0] = f32_to_bf16(v0[i]);
    ot[(4 * g + i) * 128 + c1] = f32_to_bf16(v1[i]);
  }
  __syncthreads();
  const int r = tid >> 4, c = (tid & 15) * 8;
  uint16_t* out = static_cast<uint16_t*>(P.out) + (gq * kH + 16 * hb + r) * kD + 128 * w + c;
  *reinterpret_cast<uint4*>(out) = *reinterpret_cast<const uint4*>(ot + r * 128 + c);
}

template <bool PG>
hipError_t launch_bf16(Params& P, int64_t nq, int64_t per_split, int flags, hipStream_t s) {
  if (flags & CSA_ATTN_BATCH_INVARIANT) {
    // no row split: every query's rows in order in one workgroup's chain;
    // few queries spread their four head blocks over four workgroups (the
    // same bits, see attn_bf16_kernel)
    P.splits = 1;
    if (nq < 256)
      hipLaunchKernelGGL((attn_bf16_kernel<1, 1, PG>), dim3(static_cast<uint32_t>(nq * 4)), dim3(256), 0, s, P);
    else
      hipLaunchKernelGGL((attn_bf16_kernel<1, 4, PG>), dim3(static_cast<uint32_t>(nq)), dim3(256), 0, s, P);
    return hipGetLastError();
  }
  // two tile groups for long runs: a decode split of 8 tiles or more, or a
  // whole query's list of 64 tiles or more (dense prefill: 4.8% faster on the
  // 1M-context HCA chunk; a sparse prefill query's 20 tiles run faster in one)
  if ((P.splits > 1 && per_split >= 8) || per_split >= 64)
    hipLaunchKernelGGL((attn_bf16_kernel<2, 4, PG>), dim3(static_cast<uint32_t>(nq * P.splits)), dim3(512), 0, s, P);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<1, 4, PG>), dim3(static_cast<uint32_t>(nq * P.splits)), dim3(256), 0, s, P);
  if (P.splits > 1)
    hipLaunchKernelGGL(attn_combine_kernel, dim3(static_cast<uint32_t>(nq * 16)), dim3(256), 0, s, P);
  return hipGetLastError();
}

}  // namespace

// Split partials of sparse_mqa_attn_noalloc, for callers that cannot
// allocate (graph capture, allocation-free serving loops).  Every GPU the
// library runs on holds its own copy until the process ends.  In host code
// the name is only a stand-in: the array's device address comes from
// hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[kAttnStaticScratchBytes];

hipError_t attn_static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  if (a.B == 0 || a.T == 0) return hipSuccess;
  Params P{};
  P.B = a.B; P.T = a.T; P.N = a.N; P.k = a.k; P.ratio = a.ratio; P.q_pos0 = a.q_pos0;
  P.q = a.q; P.kv_cmp = a.kv_cmp; P.idx = a.idx; P.kv_raw = a.kv_raw;
  P.raw_pos0 = a.raw_pos0; P.n_raw = a.n_raw; P.window = a.window;
  P.scale_log2 = a.scale * kLog2e; P.sink = a.sink; P.out = a.out; P.lse = a.lse;
  P.ws = static_cast<float*>(a.ws);
  P.block_table = a.block_table; P.max_blocks = a.max_blocks; P.n_pool = a.n_pool;
  P.page_shift = a.page_shift; P.ring = a.ring; P.seq_pos = a.seq_pos;
  P.rope_R = a.rope_dims;
  P.rope_l2b = a.rope_dims > 0 ? std::log2(static_cast<double>(a.rope_base)) : 0.0;
  P.job_tile = -1;
  const int64_t nq = a.B * a.T;
  if (a.io_dtype == CSA_F32) {
    P.splits = 1;
    hipLaunchKernelGGL(attn_f32_kernel, dim3(static_cast<uint32_t>(nq * 8)), dim3(256), 0, s, P);
    return hipGetLastError();
  }
  // longest list over the call's queries bounds the split count
  const int64_t last = a.seq_pos ? a.max_pos : a.q_pos0 + a.T - 1;   // the longest list bounds the split
  const int64_t wlen = last - (last - a.window + 1 > 0 ? last - a.window + 1 : 0) + 1;
  int64_t ncmp = a.idx ? a.k : (last + 1) / a.ratio;
  if (!a.idx && ncmp > a.N) ncmp = a.N;
  P.splits = attn_splits(a.B, a.T, ncmp + wlen);
  // Long runs of tiles per workgroup (decode over long lists): two tile groups
  // take two tiles per step.  Measured on MI355X a step of two groups costs
  // about 1.35 of a one-group step, and the groups' second q load and their
  // merge add about 4 us, so short runs keep one group.
  const int64_t ntiles = (ncmp + wlen + kAttnTile - 1) / kAttnTile;
  const int64_t per_split = (ntiles + P.splits - 1) / P.splits;
  if (a.block_table || a.seq_pos) return launch_bf16<true>(P, nq, per_split, a.flags, s);
  return launch_bf16<false>(P, nq, per_split, a.flags, s);
}



// The HCA decode step's C128A write and the dense attention in one launch
// where the attention's decode plan allows (bf16, one query a sequence,
// contiguous cache, a two-group split plan): the workgroup whose tiles
// include the new entry pools it first; the other splits never read it.
// Otherwise the compressor's launch, then the attention's.
hipError_t launch_attn_jobs(const AttnArgs& a, const CompressArgs& j, int64_t e_new, hipStream_t s) {
  if (a.B == 0 || a.T == 0) return launch_compress(j, s);
  const int64_t last = a.q_pos0 + a.T - 1;
  const int64_t wlen = last - (last - a.window + 1 > 0 ? last - a.window + 1 : 0) + 1;
  int64_t ncmp = (last + 1) / a.ratio;
  if (ncmp > a.N) ncmp = a.N;
  const int splits = attn_splits(a.B, a.T, ncmp + wlen);
  const int64_t ntiles = (ncmp + wlen + kAttnTile - 1) / kAttnTile;
  const int64_t per_split = (ntiles + splits - 1) / splits;
  const int64_t stride = j.out_batch_stride ? j.out_batch_stride : j.c;
  const uintptr_t kv0 = reinterpret_cast<uintptr_t>(a.kv_cmp);
  bool fuse = !a.idx && a.io_dtype == CSA_BF16 && a.T == 1 && !a.block_table && !a.seq_pos && a.flags == 0 &&
              splits > 1 && per_split >= 8 && j.ratio == 128 && j.n_tok == 128 && j.B == a.B && j.c == kD &&
              j.in_dtype == CSA_BF16 && j.out_dtype == CSA_BF16 && !j.out_scale && e_new >= 0 && e_new < ncmp &&
              stride == a.N * kD && reinterpret_cast<uintptr_t>(j.out) == kv0 + static_cast<uintptr_t>(e_new * kD * 2);
  if (fuse) {
    // the job writes only the new entries: nothing else the attention reads or writes
    auto ov = [](const void* p, int64_t bytes, uintptr_t b0, uintptr_t b1) {
      const uintptr_t x = reinterpret_cast<uintptr_t>(p);
      return p && x < b1 && b0 < x + static_cast<uintptr_t>(bytes);
    };
    const uintptr_t o0 = reinterpret_cast<uintptr_t>(j.out);
    const uintptr_t o1 = o0 + static_cast<uintptr_t>(((a.B - 1) * stride + kD) * 2);
    fuse = !ov(a.q, a.B * kH * kD * 2, o0, o1) && !ov(a.kv_raw, a.B * a.n_raw * kD * 2, o0, o1) &&
           !ov(a.out, a.B * kH * kD * 2, o0, o1) && !ov(a.sink, kH * 4, o0, o1) &&
           !ov(a.lse, a.B * kH * 4, o0, o1) &&
           !ov(a.ws, static_cast<int64_t>(attn_workspace_bytes(a.B, a.T)), o0, o1);
  }
  if (!fuse) {
    const hipError_t e = launch_compress(j, s);
    return e != hipSuccess ? e : launch_attn(a, s);
  }
  Params P{};
  P.B = a.B; P.T = a.T; P.N = a.N; P.k = 0; P.ratio = a.ratio; P.q_pos0 = a.q_pos0;
  P.q = a.q; P.kv_cmp = a.kv_cmp; P.idx = nullptr; P.kv_raw = a.kv_raw;
  P.raw_pos0 = a.raw_pos0; P.n_raw = a.n_raw; P.window = a.window;
  P.scale_log2 = a.scale * kLog2e; P.sink = a.sink; P.out = a.out; P.lse = a.lse;
  P.ws = static_cast<float*>(a.ws);
  P.rope_R = a.rope_dims;
  P.rope_l2b = a.rope_dims > 0 ? std::log2(static_cast<double>(a.rope_base)) : 0.0;
  P.splits = splits;
  // 512 threads: 64 channel threads (8 channels each) x 8 row groups of 16 rows
  const double jl2b = j.rope_dims > 0 ? std::log2(static_cast<double>(j.rope_base)) : 0.0;
  P.job = CompressJobDev{j.Ca, j.Za, nullptr, nullptr, nullptr, nullptr, j.bias, j.gamma, j.out, j.n_tok, j.pos0,
                         stride, 1, j.B, j.eps, static_cast<int>(j.c), 8, j.rope_dims, jl2b, j.rope_anchor, nullptr,
                         stride / j.c, 0};
  P.job_tile = e_new / kTile;   // a dense list: entry e is list row e
  const int64_t nq = a.B * a.T;
  hipLaunchKernelGGL((attn_bf16_kernel<2, 4, false, true>), dim3(static_cast<uint32_t>(nq * P.splits)), dim3(512), 0,
                     s, P);
  hipLaunchKernelGGL(attn_combine_kernel, dim3(static_cast<uint32_t>(nq * 16)), dim3(256), 0, s, P);
  return hipGetLastError();
}

}  // namespace csa
