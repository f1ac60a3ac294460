// Stage 3: the causal Top-k selector on gfx950.
//
// "DeepSeek Technical Reports" (DSA, the Top-k attention equation) and
// "DeepSeek V4 结构速览" (核心设计; Lightning Indexer): each query keeps the k
// entries with the highest stored indexer score among s < V(t).  Equal
// scores go to the lower index.
//
// Exact radix select on an order-preserving integer image of the stored score
// (16-bit for bf16, 32-bit for fp32).  Digits are 11 bits wide from the top
// (bf16: 11 + 5 bits; fp32: 11 + 11 + 10).  Each digit pass builds a
// histogram of the digit over the keys that match the prefix found so far,
// then the bin holding the k-th largest key extends the prefix.  After the
// last digit the prefix is the exact k-th largest key K, and `rem` says how
// many keys equal to K are taken (the lowest indices).  The output is written
// in ascending index order by an ordered compaction (block-wide exclusive
// scan of per-thread counts), so the result is deterministic.
//
// Paths:
//  * rows of up to ~36K bf16 (~18K fp32) keys: one 1024-thread workgroup per
//    row holds the whole row in registers or LDS and runs every pass there;
//  * longer bf16 rows (the 1M-context decode has 262,144 candidates): slices
//    of 16,384 keys, one workgroup each, a full 16-bit histogram per slice,
//    two launches (below);
//  * longer fp32 rows: S workgroups per row, one slice each; per-digit
//    histograms are merged in global workspace with atomics, one kernel per
//    pass, then a count kernel and an ordered write kernel.
#include <cmath>

#include "compress_entry.h"
#include "device.h"
#include "launch.h"
#include "validate.h"

namespace csa {
namespace {

constexpr int kBins = 2048;   // 11-bit digits
constexpr int kRangeBins = 8192;   // direct histogram of a narrow 16-bit key range

template <typename KT> struct Digits;
template <> struct Digits<uint16_t> {
  static constexpr int n = 2;
  __device__ static constexpr int shift(int p) { return p == 0 ? 5 : 0; }
  __device__ static constexpr int bits(int p) { return p == 0 ? 11 : 5; }
};
template <> struct Digits<uint32_t> {
  static constexpr int n = 3;
  __device__ static constexpr int shift(int p) { return p == 0 ? 21 : (p == 1 ? 10 : 0); }
  __device__ static constexpr int bits(int p) { return p == 0 ? 11 : (p == 1 ? 11 : 10); }
};

// Order-preserving image of a stored score: larger float -> larger key;
// -0.0 is mapped to +0.0 first.
__device__ __forceinline__ uint16_t key_of(uint16_t b) {
  if (b == 0x8000u) b = 0;
  return (b & 0x8000u) ? static_cast<uint16_t>(~b) : static_cast<uint16_t>(b | 0x8000u);
}
__device__ __forceinline__ uint32_t key_of(uint32_t b) {
  if (b == 0x80000000u) b = 0;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <typename KT>
__device__ __forceinline__ KT load_key(const KT* row, int64_t i) {
  return key_of(row[i]);
}

// Wave-wide inclusive scans on the DPP cross-lane paths (no LDS round trip):
// Hillis-Steele shifts inside each row of 16 lanes, then the row totals are
// carried across rows with the row broadcasts of lanes 15 and 31.
#define CSA_DPP(old, x, ctrl, rmask, bound0) \
  static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(old), static_cast<int>(x), ctrl, rmask, 0xf, bound0))
__device__ __forceinline__ uint32_t wave_incl_add(uint32_t x) {
  x += CSA_DPP(0u, x, 0x111, 0xf, true);   // row_shr:1
  x += CSA_DPP(0u, x, 0x112, 0xf, true);   // row_shr:2
  x += CSA_DPP(0u, x, 0x114, 0xf, true);   // row_shr:4
  x += CSA_DPP(0u, x, 0x118, 0xf, true);   // row_shr:8
  x += CSA_DPP(0u, x, 0x142, 0xa, false);  // row_bcast:15 into rows 1 and 3
  x += CSA_DPP(0u, x, 0x143, 0xc, false);  // row_bcast:31 into rows 2 and 3
  return x;
}
__device__ __forceinline__ uint32_t wave_total_add(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wave_incl_add(x)), 63));
}
// min / max over the wave (lanes out of a row keep the identity)
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, CSA_DPP(0xffffffffu, x, 0x111, 0xf, false));
  x = min(x, CSA_DPP(0xffffffffu, x, 0x112, 0xf, false));
  x = min(x, CSA_DPP(0xffffffffu, x, 0x114, 0xf, false));
  x = min(x, CSA_DPP(0xffffffffu, x, 0x118, 0xf, false));
  x = min(x, CSA_DPP(0xffffffffu, x, 0x142, 0xa, false));
  x = min(x, CSA_DPP(0xffffffffu, x, 0x143, 0xc, false));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, CSA_DPP(0u, x, 0x111, 0xf, false));
  x = max(x, CSA_DPP(0u, x, 0x112, 0xf, false));
  x = max(x, CSA_DPP(0u, x, 0x114, 0xf, false));
  x = max(x, CSA_DPP(0u, x, 0x118, 0xf, false));
  x = max(x, CSA_DPP(0u, x, 0x142, 0xa, false));
  x = max(x, CSA_DPP(0u, x, 0x143, 0xc, false));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
}
#undef CSA_DPP

// Find the digit whose bin holds the rem-th largest key (1-based), given the
// digit histogram `hist` of nb <= 2048 bins (LDS or global).  Runs on wave 0:
// each lane first loads its (at most 32) bins into registers, so the search
// is a register scan, not a chain of dependent loads.  Lane L of wave 0
// writes (digit, rem') to out[0..1] where rem' counts from the top of that bin.
__device__ void resolve_digit(const uint32_t* hist, int nb, uint32_t rem, uint32_t* out) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x >= 64) return;
  const int per = (nb + 63) / 64;
  const int lo = lane * per;
  uint32_t h[32];
  uint32_t sum = 0;
#pragma unroll
  for (int q = 0; q < 32; ++q) {
    h[q] = (q < per && lo + q < nb) ? hist[lo + q] : 0u;
    sum += h[q];
  }
  // inclusive suffix sums over lanes: S[l] = sum over lanes >= l
  const uint32_t incl = wave_incl_add(sum);
  const uint32_t S = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), 63)) - incl + sum;
  const uint64_t ball = __ballot(S >= rem);
  const int L = 63 - __clzll(static_cast<long long>(ball));   // highest lane with S >= rem
  if (lane == L) {
    uint32_t cum = S - sum;   // keys in higher lanes' bins
    bool found = false;
#pragma unroll
    for (int q = 31; q >= 0; --q) {
      if (!found && q < per && cum + h[q] >= rem) {
        out[0] = static_cast<uint32_t>(lo + q);
        out[1] = rem - cum;
        found = true;
      }
      cum += h[q];
    }
  }
}

// Block-wide exclusive scan of one value per thread (blockDim.x <= 1024):
// a shuffle scan inside each wave, then wave 0 scans the (at most 16) wave
// totals the same way.  `tmp` holds >= 17 words; `total` gets the block sum.
// For 64-bit values the two 32-bit halves are scanned apart: callers pack
// 16-bit counts whose sums never carry out of their field.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) { return wave_incl_add(x); }
__device__ __forceinline__ uint64_t wave_incl_scan(uint64_t x) {
  return static_cast<uint64_t>(wave_incl_add(static_cast<uint32_t>(x))) |
         (static_cast<uint64_t>(wave_incl_add(static_cast<uint32_t>(x >> 32))) << 32);
}

template <typename U>
__device__ U block_exclusive_scan_t(U v, U* tmp, U* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const U x = wave_incl_scan(v);
  if (lane == 63) tmp[wid] = x;
  __syncthreads();
  if (wid == 0) {
    const U w0 = lane < nw ? tmp[lane] : U(0);
    const U t = wave_incl_scan(w0);
    if (lane < nw) tmp[lane] = t - w0;
    if (lane == nw - 1) tmp[16] = t;
  }
  __syncthreads();
  const U r = tmp[wid] + x - v;
  *total = tmp[16];
  __syncthreads();
  return r;
}

__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
  return block_exclusive_scan_t<uint32_t>(v, tmp, total);
}

// Candidates of score row `row` (query t = row % T of sequence row / T): the
// entries visible to its position -- q_pos0 + t, or the sequence's own
// position seq_pos[row / T] in a ragged decode batch.
__device__ __forceinline__ int64_t row_visible(int64_t row, int64_t T, int64_t q_pos0, int ratio, int64_t N,
                                               const int64_t* seq_pos) {
  int64_t b, t;
  if (T == 1) {
    b = row;
    t = 0;
  } else if (((row | T) >> 31) == 0) {
    b = static_cast<uint32_t>(row) / static_cast<uint32_t>(T);
    t = static_cast<uint32_t>(row) - static_cast<uint32_t>(b) * static_cast<uint32_t>(T);
  } else {
    b = row / T;
    t = row - b * T;
  }
  const int64_t pos = seq_pos ? seq_pos[b] : q_pos0 + t;
  // ratio is a power of two: 4 or 128, or 1 for pool rows
  const int64_t v = pos < 0 ? 0 : (pos + 1) >> __builtin_ctz(static_cast<unsigned>(ratio));
  return v < N ? v : N;
}

// hist[bin] += 1 for every lane with `active`.  Indexer scores crowd into a
// few bins, so lanes of a wave that share a bin are combined into one LDS
// atomic (up to four distinct bins per call); any lanes left over add their
// own.  Must be called by all lanes of the wave.
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin, bool active) {
  const int lane = threadIdx.x & 63;
  uint64_t pending = __ballot(active);
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    if (!pending) break;
    const int leader = __ffsll(static_cast<long long>(pending)) - 1;
    const uint32_t lb = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(bin), leader));
    const uint64_t same = __ballot(active && bin == lb) & pending;
    if (lane == leader) atomicAdd(&hist[lb], static_cast<uint32_t>(__popcll(same)));
    pending &= ~same;
  }
  if ((pending >> lane) & 1ull) atomicAdd(&hist[bin], 1u);
}

// Ordered compaction of one contiguous range [lo, hi) of a row: writes every
// index whose key > K, and keys == K while the running equal-rank < rem, to
// out[pos...] in ascending order.  `key(i)` reads the key of index i.
// In pool mode (pool != NULL) the written value is the pool row's entry id
// at the selected slot, -1 for an empty slot.
__device__ __forceinline__ int32_t pool_map(const int32_t* prow, int64_t n_ent, int64_t i) {
  if (!prow) return static_cast<int32_t>(i);
  const int32_t v = prow[i];
  return v >= 0 && v < n_ent ? v : -1;
}

template <typename KT, typename F>
__device__ __forceinline__ void emit_range(int64_t lo, int64_t hi, KT K, uint32_t rem, uint32_t gt_before,
                                           uint32_t eq_before, int32_t* out, F key,
                                           const int32_t* prow = nullptr, int64_t n_ent = 0) {
  uint32_t pos = gt_before + (eq_before < rem ? eq_before : rem);
  uint32_t er = eq_before;
  for (int64_t i = lo; i < hi; ++i) {
    const KT kk = key(i);
    if (kk > K) {
      out[pos++] = pool_map(prow, n_ent, i);
    } else if (kk == K) {
      if (er < rem) out[pos++] = pool_map(prow, n_ent, i);
      ++er;
    }
  }
}

// ------------------------------------------------------------ LDS path
template <typename KT>
__global__ void __launch_bounds__(1024)
topk_lds_kernel(int64_t T, int64_t N, int64_t q_pos0, int ratio, const int64_t* __restrict__ seq_pos, int k, const KT* __restrict__ scores,
                int32_t* __restrict__ idx, const int32_t* __restrict__ pool, int64_t n_ent) {
  extern __shared__ uint8_t smem_raw[];
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem_raw);           // kRangeBins (>= kBins)
  uint32_t* tmp = hist + kRangeBins;                                  // 32 words
  KT* keys = reinterpret_cast<KT*>(tmp + 32);
  const int64_t row = blockIdx.x;
  const int64_t t = row % T;
  const int64_t V = row_visible(row, T, q_pos0, ratio, N, seq_pos);
  int32_t* out = idx + row * k;
  const int32_t* prow = pool ? pool + row * N : nullptr;
  const int tid = threadIdx.x, nt = blockDim.x;
  if (V <= k) {
    for (int i = tid; i < k; i += nt) out[i] = i < V ? pool_map(prow, n_ent, i) : -1;
    return;
  }
  if (tid == 0) {
    tmp[24] = 0xffffffffu;
    tmp[25] = 0u;
  }
  const KT* src = scores + row * N;
  constexpr int PER = 16 / sizeof(KT);
  if ((reinterpret_cast<uintptr_t>(src) & 15) == 0) {
    const int64_t nv = V / PER;
    for (int64_t vi = tid; vi < nv; vi += nt) {
      const uint4 raw = reinterpret_cast<const uint4*>(src)[vi];
      const KT* e = reinterpret_cast<const KT*>(&raw);
#pragma unroll
      for (int u = 0; u < PER; ++u) keys[vi * PER + u] = key_of(e[u]);
    }
    for (int64_t i = nv * PER + tid; i < V; i += nt) keys[i] = load_key(src, i);
  } else {
    for (int64_t i = tid; i < V; i += nt) keys[i] = load_key(src, i);
  }

  __syncthreads();   // every key (and tmp[24..25]) is in LDS
  KT K;
  uint32_t rem;
  // Indexer scores span few distinct bf16 values: when the row's key range
  // fits in kRangeBins, one exact histogram of (key - min) replaces the digit
  // passes (and spreads the LDS atomics over many bins).
  bool done = false;
  if constexpr (sizeof(KT) == 2) {
    uint32_t kmin = 0xffffu, kmax = 0u;
    for (int64_t i = tid; i < V; i += nt) {
      const uint32_t kk = keys[i];
      kmin = kk < kmin ? kk : kmin;
      kmax = kk > kmax ? kk : kmax;
    }
    kmin = wave_min_u32(kmin);
    kmax = wave_max_u32(kmax);
    if ((tid & 63) == 0) {
      atomicMin(&tmp[24], kmin);
      atomicMax(&tmp[25], kmax);
    }
    __syncthreads();
    kmin = tmp[24];
    kmax = tmp[25];
    if (kmax - kmin < static_cast<uint32_t>(kRangeBins)) {
      uint32_t* bins = hist;   // kRangeBins words
      for (int i = tid; i < kRangeBins; i += nt) bins[i] = 0;
      __syncthreads();
      for (int64_t i = tid; i < V; i += nt) atomicAdd(&bins[keys[i] - kmin], 1u);
      __syncthreads();
      // each thread owns a contiguous run of bins; find the bin holding the k-th largest key
      const int per = (kRangeBins + nt - 1) / nt;
      const int b0 = tid * per;
      uint32_t mine = 0;
      for (int q = 0; q < per; ++q) mine += (b0 + q < kRangeBins) ? bins[b0 + q] : 0u;
      uint32_t total;
      // keys in bins above this thread's run = total - inclusive prefix
      const uint32_t excl = block_exclusive_scan(mine, tmp, &total);
      const uint32_t above = total - excl - mine;
      if (above < static_cast<uint32_t>(k) && above + mine >= static_cast<uint32_t>(k)) {
        uint32_t cum = above;
        for (int q = per - 1; q >= 0; --q) {
          const uint32_t h = (b0 + q < kRangeBins) ? bins[b0 + q] : 0u;
          if (cum + h >= static_cast<uint32_t>(k)) {
            tmp[20] = kmin + static_cast<uint32_t>(b0 + q);
            tmp[21] = static_cast<uint32_t>(k) - cum;
            break;
          }
          cum += h;
        }
      }
      __syncthreads();
      K = static_cast<KT>(tmp[20]);
      rem = tmp[21];
      done = true;
    }
  }
  if (!done) {
    KT prefix = 0, mask = 0;
    rem = static_cast<uint32_t>(k);
    for (int p = 0; p < Digits<KT>::n; ++p) {
      const int sh = Digits<KT>::shift(p);
      const int nb = 1 << Digits<KT>::bits(p);
      for (int i = tid; i < nb; i += nt) hist[i] = 0;
      __syncthreads();
      for (int64_t base = 0; base < V; base += nt) {
        const int64_t i = base + tid;
        const KT kk = i < V ? keys[i] : KT(0);
        hist_add(hist, (kk >> sh) & (nb - 1), i < V && (kk & mask) == prefix);
      }
      __syncthreads();
      resolve_digit(hist, nb, rem, tmp + 20);
      __syncthreads();
      prefix |= static_cast<KT>(tmp[20] << sh);
      mask |= static_cast<KT>((nb - 1) << sh);
      rem = tmp[21];
      __syncthreads();
    }
    K = prefix;
  }

  const int64_t chunk = (V + nt - 1) / nt;
  const int64_t lo = tid * chunk < V ? tid * chunk : V;
  const int64_t hi = lo + chunk < V ? lo + chunk : V;
  uint32_t gt = 0, eq = 0;
  for (int64_t i = lo; i < hi; ++i) {
    gt += keys[i] > K;
    eq += keys[i] == K;
  }
  uint32_t total;
  const uint32_t gtb = block_exclusive_scan(gt, tmp, &total);
  const uint32_t eqb = block_exclusive_scan(eq, tmp, &total);
  emit_range<KT>(lo, hi, K, rem, gtb, eqb, out, [&](int64_t i) { return keys[i]; }, prow, n_ent);
}

// Packed 16-bit integer operations on both halves of a 32-bit word at once,
// one VALU instruction each (the compiler otherwise splits such work into
// per-half compares and selects).
__device__ __forceinline__ uint32_t min_u16x2(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_min_u16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_max_u16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ uint32_t add_u16x2(uint32_t a, uint32_t b) {   // modulo 2^16 per half
  uint32_t r;
  asm("v_pk_add_u16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ uint32_t shr_u16x2(uint32_t a, uint32_t sh2) {   // sh2: the shift in both halves
  uint32_t r;
  asm("v_pk_lshrrev_b16 %0, %1, %2" : "=v"(r) : "v"(sh2), "v"(a));
  return r;
}

// Order-preserving keys of two stored bf16 scores at once: 0x8000 + m for a
// non-negative half of magnitude bits m, 0x8000 - m for a negative one (so
// -0.0 and +0.0 share 0x8000).  The same order as key_of, one above it on
// negative scores.
__device__ __forceinline__ uint32_t key_pair(uint32_t w) {
  const uint32_t sg = (w >> 15) & 0x00010001u;               // sign of each half
  const uint32_t t = (w & 0x7fff7fffu) ^ (sg * 0xffffu);     // m, or 0xffff - m
  return add_u16x2(t, sg + 0x80008000u);                     // + 0x8000 (+ 1 for a negative half)
}

// ------------------------------------------------------------ register path
// bf16 rows of up to 1024 * 8 * CPT keys: thread t holds keys
// 8 CPT t .. 8 CPT t + 8 CPT - 1 (CPT 16-byte chunks) in registers for the
// whole selection; LDS only holds a histogram.  The key range [min, max] is
// found while the chunks load.  Pass 1 histograms (key - min) >> s over at
// most 8192 bins (s = 0..3, the smallest shift that fits the range), which
// spreads any score distribution over the bins (no pile-up of atomics on a
// few digit values); when s > 0, pass 2 histograms the low s bits of the keys
// in the chosen bin.  That gives the k-th largest key K exactly.  Since each
// thread's keys are contiguous, the ordered compaction is one block-wide scan
// of two packed 16-bit counts (keys above K, keys equal to K).
__device__ __forceinline__ uint64_t block_exclusive_scan_u64(uint64_t v, uint64_t* tmp, uint64_t* total) {
  return block_exclusive_scan_t<uint64_t>(v, tmp, total);
}

template <int CPT>
__device__ __forceinline__ void topk_reg_body(int64_t row, int64_t T, int64_t N, int64_t q_pos0, int ratio,
                                              const int64_t* __restrict__ seq_pos, int k,
                                              const uint16_t* __restrict__ scores, int32_t* __restrict__ idx,
                                              const int32_t* __restrict__ pool, int64_t n_ent,
                                              uint32_t* __restrict__ bins) {
  constexpr int NT = 1024;
  static_assert(8 * CPT * NT < 65536, "block-wide counts are packed in 16 bits");
  __shared__ uint32_t tmp[32];
  const int64_t t = row % T;
  const int64_t V = row_visible(row, T, q_pos0, ratio, N, seq_pos);
  int32_t* out = idx + row * k;
  const int32_t* prow = pool ? pool + row * N : nullptr;
  const int tid = threadIdx.x;
  if (V <= k) {
    for (int i = tid; i < k; i += NT) out[i] = i < V ? pool_map(prow, n_ent, i) : -1;
    return;
  }
  for (int i = tid; i < kRangeBins; i += NT) bins[i] = 0;
  if (tid == 0) {
    tmp[24] = 0xffffu;
    tmp[25] = 0u;
  }
  // keys in registers, two per register: key u of chunk c is KEY(c, u)
  // (after the range is known: key - min); keys at or past V are not valid
  // (valid bits 0)
  const uint4* src = reinterpret_cast<const uint4*>(scores + row * N) + static_cast<int64_t>(tid) * CPT;
  const int64_t i00 = static_cast<int64_t>(tid) * 8 * CPT;   // this thread's first key
  uint32_t kp[CPT][4];
  uint32_t valid[CPT];
#define KEY(c, u) ((kp[c][(u) >> 1] >> (16 * ((u) & 1))) & 0xffffu)
  // keys and their range two at a time; a key past V takes no part (its
  // halves enter the minimum as 0xffff and the maximum as 0)
  uint32_t mn2 = 0xffffffffu, mx2 = 0u;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int64_t i0 = i00 + 8 * c;
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (i0 < V) raw = src[c];
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    const int64_t nv = V - i0;
    valid[c] = nv >= 8 ? 0xffu : (nv > 0 ? (1u << nv) - 1u : 0u);
#pragma unroll
    for (int j = 0; j < 4; ++j) kp[c][j] = key_pair(w[j]);
    if (valid[c] == 0xffu) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        mn2 = min_u16x2(mn2, kp[c][j]);
        mx2 = max_u16x2(mx2, kp[c][j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t vm = (valid[c] >> (2 * j)) & 3u;
        const uint32_t keep = ((vm & 1u) ? 0xffffu : 0u) | ((vm & 2u) ? 0xffff0000u : 0u);
        mn2 = min_u16x2(mn2, kp[c][j] | ~keep);
        mx2 = max_u16x2(mx2, kp[c][j] & keep);
      }
    }
  }
  uint32_t kmin = min(mn2 & 0xffffu, mn2 >> 16), kmax = max(mx2 & 0xffffu, mx2 >> 16);
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if ((tid & 63) == 0) {
    atomicMin(&tmp[24], kmin);
    atomicMax(&tmp[25], kmax);
  }
  __syncthreads();   // range known, bins zeroed
  kmin = tmp[24];
  kmax = tmp[25];
  int sh = 0;
  while (((kmax - kmin) >> sh) >= static_cast<uint32_t>(kRangeBins)) ++sh;   // 0..3 for 16-bit keys
  // from here on the registers hold key - min (two 16-bit differences each)
  {
    typedef short v2i16 __attribute__((ext_vector_type(2)));
    const v2i16 m2 = {static_cast<short>(kmin), static_cast<short>(kmin)};
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        kp[c][j] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2i16, kp[c][j]) - m2);
  }

  // pass 1: bin (key - min) >> sh, both keys of a register shifted at once
  // in a whole chunk
  {
    const uint32_t sh2 = static_cast<uint32_t>(sh) * 0x10001u;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      if (valid[c] == 0xffu) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t b2 = shr_u16x2(kp[c][j], sh2);
          atomicAdd(&bins[b2 & 0xffffu], 1u);
          atomicAdd(&bins[b2 >> 16], 1u);
        }
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if ((valid[c] >> u) & 1u) atomicAdd(&bins[KEY(c, u) >> sh], 1u);
      }
    }
  }
  __syncthreads();
  // thread t owns bins 8t .. 8t+7; find the bin holding the k-th largest key
  constexpr int per = kRangeBins / NT;
  {
    const int b0 = tid * per;
    uint32_t h[per], mine = 0;
#pragma unroll
    for (int q = 0; q < per; ++q) {
      h[q] = bins[b0 + q];
      mine += h[q];
    }
    uint32_t total;
    const uint32_t excl = block_exclusive_scan(mine, tmp, &total);
    const uint32_t above = total - excl - mine;
    if (above < static_cast<uint32_t>(k) && above + mine >= static_cast<uint32_t>(k)) {
      uint32_t cum = above;
      bool found = false;
#pragma unroll
      for (int q = per - 1; q >= 0; --q) {
        if (!found && cum + h[q] >= static_cast<uint32_t>(k)) {
          tmp[20] = static_cast<uint32_t>(b0 + q);
          tmp[21] = static_cast<uint32_t>(k) - cum;
          found = true;
        }
        cum += h[q];
      }
    }
  }
  __syncthreads();
  const uint32_t bstar = tmp[20];
  uint32_t rem = tmp[21];
  uint32_t K = bstar << sh;   // as a difference from min
  if (sh > 0) {
    // pass 2: the low sh bits of the keys in bin bstar
    if (tid < (1 << sh)) bins[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t d = KEY(c, u);
        if (((valid[c] >> u) & 1u) && (d >> sh) == bstar) atomicAdd(&bins[d & ((1u << sh) - 1u)], 1u);
      }
    __syncthreads();
    if (tid == 0) {
      uint32_t cum = 0, f = 0, r = rem;
      for (int q = (1 << sh) - 1; q >= 0; --q) {
        if (cum + bins[q] >= rem) { f = static_cast<uint32_t>(q); r = rem - cum; break; }
        cum += bins[q];
      }
      tmp[22] = f;
      tmp[23] = r;
    }
    __syncthreads();
    K += tmp[22];
    rem = tmp[23];
  }

  // ordered compaction: this thread's keys above K, then the first rem equal
  // to K.  Bit 8c + u of gtm / eqm: key u of chunk c is above / equal to K.
  uint64_t gtm = 0, eqm = 0;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    uint32_t g8 = 0, e8 = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      g8 |= static_cast<uint32_t>(KEY(c, u) > K) << u;
      e8 |= static_cast<uint32_t>(KEY(c, u) == K) << u;
    }
    gtm |= static_cast<uint64_t>(g8 & valid[c]) << (8 * c);
    eqm |= static_cast<uint64_t>(e8 & valid[c]) << (8 * c);
  }
  const uint32_t gt = static_cast<uint32_t>(__popcll(gtm)), eq = static_cast<uint32_t>(__popcll(eqm));
  uint32_t tot;
  const uint32_t ex = block_exclusive_scan(gt | (eq << 16), tmp, &tot);
  // which of this thread's keys are taken (bit 8c + u): every one above K and
  // its ties in index order while fewer than rem ties come before them; then
  // one store per taken key in index order
  uint64_t take = gtm;
  for (uint32_t er = ex >> 16; eqm != 0 && er < rem; ++er) {
    take |= eqm & (0ull - eqm);
    eqm &= eqm - 1ull;
  }
  uint32_t pos = (ex & 0xffffu) + min(ex >> 16, rem);
  while (take) {
    out[pos++] = pool_map(prow, n_ent, i00 + __builtin_ctzll(take));
    take &= take - 1;
  }
#undef KEY
}

template <int CPT>
__global__ void __launch_bounds__(1024)
topk_reg_kernel(int64_t T, int64_t N, int64_t q_pos0, int ratio, const int64_t* __restrict__ seq_pos, int k,
                const uint16_t* __restrict__ scores, int32_t* __restrict__ idx, const int32_t* __restrict__ pool,
                int64_t n_ent) {
  __shared__ uint32_t bins[kRangeBins];
  topk_reg_body<CPT>(blockIdx.x, T, N, q_pos0, ratio, seq_pos, k, scores, idx, pool, n_ent, bins);
}

// Top-k with a decode step's compressor writes in the same launch: workgroups
// 0 .. rows-1 select as topk_reg_kernel; the ones after them each run one
// sequence's share of a job (one entry, two channels a thread), which no
// selection reads -- spare CUs of a launch that fills one CU a row.
template <int CPT>
__global__ void __launch_bounds__(1024)
topk_reg_jobs_kernel(int64_t rows, int64_t T, int64_t N, int64_t q_pos0, int ratio, int k,
                     const uint16_t* __restrict__ scores, int32_t* __restrict__ idx, CompressBatch jb, int64_t B) {
  __shared__ uint32_t bins[kRangeBins];
  if (static_cast<int64_t>(blockIdx.x) < rows) {
    topk_reg_body<CPT>(blockIdx.x, T, N, q_pos0, ratio, nullptr, k, scores, idx, nullptr, 0, bins);
    return;
  }
  const int64_t w = blockIdx.x - rows;
  const CompressJobDev& J = jb.j[w / B];
  const int64_t b = w % B;
  float* const lds = reinterpret_cast<float*>(bins);
  const auto* Ca = static_cast<const uint16_t*>(J.Ca);
  const auto* Za = static_cast<const uint16_t*>(J.Za);
  const auto* Cb = static_cast<const uint16_t*>(J.Cb);
  const auto* Zb = static_cast<const uint16_t*>(J.Zb);
  const auto* pCb = static_cast<const uint16_t*>(J.pCb);
  const auto* pZb = static_cast<const uint16_t*>(J.pZb);
  if (J.qfmt == 2)
    compress_entry<uint16_t, E2M1x2, 4, false, 2, 8>(0, b, 0, 1, J.n_tok, J.c, J.pos0, Ca, Za, Cb, Zb, pCb, pZb,
                                                     J.bias, J.gamma, J.eps, static_cast<E2M1x2*>(J.out), J.out_stride,
                                                     J.G, nullptr, J.rope_R, J.rope_l2b, J.rope_anchor, J.out_scale,
                                                     J.scale_stride, -1, lds);
  else if (J.qfmt == 1)
    compress_entry<uint16_t, uint8_t, 4, false, 2, 8>(0, b, 0, 1, J.n_tok, J.c, J.pos0, Ca, Za, Cb, Zb, pCb, pZb,
                                                      J.bias, J.gamma, J.eps, static_cast<uint8_t*>(J.out),
                                                      J.out_stride, J.G, nullptr, J.rope_R, J.rope_l2b,
                                                      J.rope_anchor, J.out_scale, J.scale_stride, -1, lds);
  else
    compress_entry<uint16_t, uint16_t, 4, false, 2, 8>(0, b, 0, 1, J.n_tok, J.c, J.pos0, Ca, Za, Cb, Zb, pCb, pZb,
                                                       J.bias, J.gamma, J.eps, static_cast<uint16_t*>(J.out),
                                                       J.out_stride, J.G, nullptr, J.rope_R, J.rope_l2b,
                                                       J.rope_anchor, J.out_scale, J.scale_stride, -1, lds);
}

// ------------------------------------------------------------ global path
// Workspace per row (uint32 words): hist[3][2048], counts[S][2].
constexpr int kWsHist = 3 * kBins;

__global__ void fill_zero_kernel(uint32_t* p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Re-derive (prefix, mask, rem) from the histograms of passes 0..np-1.
template <typename KT>
__device__ void derive_state(const uint32_t* rowws, int np, uint32_t k, uint32_t* sh_state, KT& prefix,
                             KT& mask, uint32_t& rem) {
  prefix = 0;
  mask = 0;
  rem = k;
  for (int p = 0; p < np; ++p) {
    const int sh = Digits<KT>::shift(p);
    const int nb = 1 << Digits<KT>::bits(p);
    resolve_digit(rowws + p * kBins, nb, rem, sh_state);
    __syncthreads();
    prefix |= static_cast<KT>(sh_state[0] << sh);
    mask |= static_cast<KT>((nb - 1) << sh);
    rem = sh_state[1];
    __syncthreads();
  }
}

template <typename KT>
__global__ void __launch_bounds__(256)
topk_hist_kernel(int pass, int64_t T, int64_t N, int64_t q_pos0, int ratio, const int64_t* __restrict__ seq_pos, int k, int S,
                 const KT* __restrict__ scores, uint32_t* __restrict__ ws) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t st[4];
  const int64_t row = blockIdx.y;
  const int64_t t = row % T;
  const int64_t V = row_visible(row, T, q_pos0, ratio, N, seq_pos);
  if (V <= k) return;
  uint32_t* rowws = ws + row * (kWsHist + 2 * S);
  KT prefix, mask;
  uint32_t rem;
  derive_state<KT>(rowws, pass, static_cast<uint32_t>(k), st, prefix, mask, rem);
  const int sh = Digits<KT>::shift(pass);
  const int nb = 1 << Digits<KT>::bits(pass);
  for (int i = threadIdx.x; i < nb; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  const int64_t L = (V + S - 1) / S;
  const int64_t lo = blockIdx.x * L, hi = lo + L < V ? lo + L : V;
  const KT* src = scores + row * N;
  for (int64_t base = lo; base < hi; base += blockDim.x) {
    const int64_t i = base + threadIdx.x;
    const KT kk = i < hi ? load_key(src, i) : KT(0);
    hist_add(hist, (kk >> sh) & (nb - 1), i < hi && (kk & mask) == prefix);
  }
  __syncthreads();
  uint32_t* gh = rowws + pass * kBins;
  for (int i = threadIdx.x; i < nb; i += blockDim.x)
    if (hist[i]) atomicAdd(&gh[i], hist[i]);
}

template <typename KT>
__global__ void __launch_bounds__(256)
topk_count_kernel(int64_t T, int64_t N, int64_t q_pos0, int ratio, const int64_t* __restrict__ seq_pos, int k, int S,
                  const KT* __restrict__ scores, uint32_t* __restrict__ ws) {
  __shared__ uint32_t st[4];
  __shared__ uint32_t red[2][4];
  const int64_t row = blockIdx.y;
  const int64_t t = row % T;
  const int64_t V = row_visible(row, T, q_pos0, ratio, N, seq_pos);
  if (V <= k) return;
  uint32_t* rowws = ws + row * (kWsHist + 2 * S);
  KT K, mask;
  uint32_t rem;
  derive_state<KT>(rowws, Digits<KT>::n, static_cast<uint32_t>(k), st, K, mask, rem);
  const int64_t L = (V + S - 1) / S;
  const int64_t lo = blockIdx.x * L, hi = lo + L < V ? lo + L : V;
  const KT* src = scores + row * N;
  uint32_t gt = 0, eq = 0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += blockDim.x) {
    const KT kk = load_key(src, i);
    gt += kk > K;
    eq += kk == K;
  }
  gt = wave_total_add(gt);
  eq = wave_total_add(eq);
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = gt;
    red[1][threadIdx.x >> 6] = eq;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t* cnt = rowws + kWsHist;
    cnt[2 * blockIdx.x] = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    cnt[2 * blockIdx.x + 1] = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  }
}

template <typename KT>
__global__ void __launch_bounds__(256)
topk_write_kernel(int64_t T, int64_t N, int64_t q_pos0, int ratio, const int64_t* __restrict__ seq_pos, int k, int S,
                  const KT* __restrict__ scores, uint32_t* __restrict__ ws, int32_t* __restrict__ idx) {
  __shared__ uint32_t st[4];
  __shared__ uint32_t tmp[32];
  const int64_t row = blockIdx.y;
  const int64_t t = row % T;
  const int64_t V = row_visible(row, T, q_pos0, ratio, N, seq_pos);
  int32_t* out = idx + row * k;
  if (V <= k) {
    if (blockIdx.x == 0)
      for (int i = threadIdx.x; i < k; i += blockDim.x) out[i] = i < V ? i : -1;
    return;
  }
  uint32_t* rowws = ws + row * (kWsHist + 2 * S);
  KT K, mask;
  uint32_t rem;
  derive_state<KT>(rowws, Digits<KT>::n, static_cast<uint32_t>(k), st, K, mask, rem);
  const uint32_t* cnt = rowws + kWsHist;
  uint32_t gt_before = 0, eq_before = 0;
  for (int s = 0; s < static_cast<int>(blockIdx.x); ++s) {
    gt_before += cnt[2 * s];
    eq_before += cnt[2 * s + 1];
  }
  const int64_t L = (V + S - 1) / S;
  const int64_t lo = blockIdx.x * L, hi = lo + L < V ? lo + L : V;
  const KT* src = scores + row * N;
  // per-thread contiguous sub-ranges of the slice
  const int nt = blockDim.x;
  const int64_t len = hi > lo ? hi - lo : 0;
  const int64_t chunk = (len + nt - 1) / nt;
  const int64_t a = lo + (threadIdx.x * chunk < len ? threadIdx.x * chunk : len);
  const int64_t b = a + chunk < hi ? a + chunk : (hi > a ? hi : a);
  uint32_t gt = 0, eq = 0;
  for (int64_t i = a; i < b; ++i) {
    const KT kk = load_key(src, i);
    gt += kk > K;
    eq += kk == K;
  }
  uint32_t total;
  const uint32_t gtb = block_exclusive_scan(gt, tmp, &total);
  const uint32_t eqb = block_exclusive_scan(eq, tmp, &total);
  emit_range<KT>(a, b, K, rem, gt_before + gtb, eq_before + eqb, out,
                 [&](int64_t i) { return load_key(src, i); });
}

// ------------------------------------------------------------ long bf16 rows
// Rows longer than one workgroup keeps in registers (the 1M-context decode
// has 262,144 candidates) are cut into slices of kFineSlice keys, one
// 1024-thread workgroup each, and selected in two launches.  A key's top 10
// bits are its coarse bin, the low 6 its fine bin inside it.
//   F1  The slice's full 65,536-bin histogram of 16-bit keys in LDS (two
//       16-bit counts per word).  From it the slice's record: per coarse bin
//       c the number of keys at or above c and the number of distinct keys at
//       or above c, then the distinct keys with their counts in descending
//       order.  The list stops after the coarse bin that holds the slice's own
//       k-th largest key: the row's k-th largest key K is at least that key
//       (the slice alone has k keys at or above it), so the coarse bin of K is
//       never below it, and the list holds at most k - 1 + 64 entries.
//   F2  Every workgroup of the row sums the slices' coarse counts to find the
//       coarse bin c* of K, sums the listed keys of c* over the slices to find
//       K and how many keys equal to K are taken (`rem`), and the same sums
//       over the slices before its own give its output offset; then an
//       ordered compaction of its slice.
// Every record is written whole by its slice, so the workspace needs no
// clearing and no global atomics are used.
constexpr int kFineSlice = 16384;   // keys per slice
constexpr int kFineThreads = 1024;  // 16 keys per thread, two 16-byte chunks
constexpr int kCoarse = 1024;       // coarse bins (top 10 key bits), one per F1 thread
static_assert(kFineSlice == kTopkFineSlice && kCoarse == kTopkFineCoarse, "shared with the workspace sizing");

template <int NC>
__device__ __forceinline__ void fine_slice_keys(const uint16_t* row, int64_t lo, int64_t hi, uint32_t (&kp)[NC][4],
                                                uint32_t (&valid)[NC]) {
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int64_t i0 = lo + 8 * (static_cast<int64_t>(c) * kFineThreads + threadIdx.x);
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (i0 < hi) raw = *reinterpret_cast<const uint4*>(row + i0);
    const int64_t nv = hi - i0;
    valid[c] = nv >= 8 ? 0xffu : (nv > 0 ? (1u << nv) - 1u : 0u);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      kp[c][j] = key_of(static_cast<uint16_t>(w[j] & 0xffffu)) |
                 (static_cast<uint32_t>(key_of(static_cast<uint16_t>(w[j] >> 16))) << 16);
  }
}
#define FKEY(c, u) ((kp[c][(u) >> 1] >> (16 * ((u) & 1))) & 0xffffu)

// Word w of the histogram (bins 2w, 2w + 1) lives at fine_slot(w): the 32
// words of coarse bin j = w / 32 are 8 quads, quad q stored at q ^ (j & 7), so
// lanes reading quad q of consecutive coarse bins hit different banks.
__host__ __device__ constexpr uint32_t fine_slot(uint32_t w) {
  return ((w >> 5) << 5) | ((((w >> 2) & 7u) ^ ((w >> 5) & 7u)) << 2) | (w & 3u);
}
// The same for both keys of a packed pair (key a in the low half, b in the
// high half) at once: the slot is w with bits 2..4 XORed by bits 5..7, so one
// shift, mask and XOR on the 32-bit pair give fine_slot(a >> 1) in the low
// half and fine_slot(b >> 1) in the high half.
__host__ __device__ constexpr uint32_t fine_slot_pair(uint32_t keys) {
  const uint32_t w = (keys >> 1) & 0x7fff7fffu;
  return w ^ ((w >> 3) & 0x001c001cu);
}
constexpr bool fine_slot_pair_ok() {
  for (uint32_t a = 0; a < 65536u; a += 3u) {
    const uint32_t b = (a * 40503u + 17u) & 0xffffu;
    if (fine_slot_pair(a | (b << 16)) != (fine_slot(a >> 1) | (fine_slot(b >> 1) << 16))) return false;
  }
  return true;
}
static_assert(fine_slot_pair_ok(), "packed slots agree with fine_slot");

__global__ void __launch_bounds__(kFineThreads)
topk_fine_record_kernel(int64_t T, int64_t N, int64_t q_pos0, int ratio, const int64_t* __restrict__ seq_pos, int k,
                        const uint16_t* __restrict__ scores, uint32_t* __restrict__ ws, int64_t rec_words,
                        int64_t row_words) {
  __shared__ uint32_t hist[32768];               // bin 2w in the low half of word w, 2w + 1 in the high half
  __shared__ uint32_t lst[CSA_MAX_TOPK + 64];    // the list, staged
  __shared__ uint32_t tmp[32];
  const int64_t row = blockIdx.y;
  const int64_t V = row_visible(row, T, q_pos0, ratio, N, seq_pos);
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * kFineSlice;
  if (V <= k || lo >= V) return;
  const int64_t hi = lo + kFineSlice < V ? lo + kFineSlice : V;
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t kp[2][4], valid[2];
  fine_slice_keys<2>(scores + row * N, lo, hi, kp, valid);
  {
    uint4* h4 = reinterpret_cast<uint4*>(hist);
#pragma unroll
    for (int q = 0; q < 8; ++q) h4[q * kFineThreads + tid] = make_uint4(0, 0, 0, 0);
  }
  if (tid == 0) tmp[20] = 0xffffffffu;
  __syncthreads();
  // A whole chunk (every slice but a row's last) takes its slots and 16-bit
  // increments from the packed key pairs; a partial one key by key.
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (valid[c] == 0xffu) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t sl = fine_slot_pair(kp[c][j]);
        const uint32_t sh = (kp[c][j] << 4) & 0x00100010u;   // 16 * (key & 1), both halves
        atomicAdd(&hist[sl & 0xffffu], 1u << (sh & 0xffffu));
        atomicAdd(&hist[sl >> 16], 1u << (sh >> 16));
      }
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if ((valid[c] >> u) & 1u) {
          const uint32_t kk = FKEY(c, u);
          atomicAdd(&hist[fine_slot(kk >> 1)], 1u << (16 * (kk & 1u)));
        }
    }
  }
  __syncthreads();
  // thread t owns coarse bin cb = 1023 - t (fine bins 64 cb .. 64 cb + 63):
  // count its distinct keys and its keys
  const uint32_t cb = static_cast<uint32_t>(kCoarse - 1 - tid);
  const uint4* hq = reinterpret_cast<const uint4*>(hist) + cb * 8;
  // Both 16-bit halves of a word are summed at once: the key counts as plain
  // 32-bit adds (a half's sum is at most the slice's 16,384 keys, so no carry
  // crosses into the other half), the non-empty bins as sums of min(count, 1)
  // per half.
  uint32_t nd2 = 0, ns2 = 0;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint4 v = hq[q ^ (cb & 7u)];
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ns2 += w4[j];
      nd2 += min_u16x2(w4[j], 0x00010001u);
    }
  }
  const uint32_t nd = (nd2 & 0xffffu) + (nd2 >> 16), ns = (ns2 & 0xffffu) + (ns2 >> 16);
  uint32_t tot;
  const uint32_t ex = block_exclusive_scan(nd | (ns << 16), tmp, &tot);   // both totals <= 16384
  const uint32_t incl = ex + (nd | (ns << 16));
  // The keys at or above a coarse bin grow as the bin falls (as tid grows):
  // the one thread where they first reach k names the slice's cut (a single
  // writer, where an atomic minimum over every thread past it would
  // serialize on one LDS word).
  if ((incl >> 16) >= static_cast<uint32_t>(k) && (ex >> 16) < static_cast<uint32_t>(k)) tmp[20] = static_cast<uint32_t>(tid);
  __syncthreads();
  // the list runs through the coarse bin of the slice's k-th largest key (all
  // of it when the slice has fewer than k keys).  Each wave stages the
  // non-empty coarse bins of its own threads, one bin at a time, a lane per
  // fine bin in descending order.
  const uint32_t last = tmp[20] == 0xffffffffu ? kFineThreads - 1 : tmp[20];
  if (tid == static_cast<int>(last)) tmp[21] = incl & 0xffffu;
  {
    const uint32_t w0 = static_cast<uint32_t>(tid & ~63);
    uint64_t todo = __ballot(nd != 0 && static_cast<uint32_t>(tid) <= last);
    while (todo) {
      const int j = __ffsll(static_cast<long long>(todo)) - 1;
      todo &= todo - 1;
      const uint32_t base = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(ex & 0xffffu), j));
      const uint32_t bin = 64 * (kCoarse - 1 - (w0 + j)) + 63 - lane;
      const uint32_t cnt = (hist[fine_slot(bin >> 1)] >> (16 * (bin & 1u))) & 0xffffu;
      const uint64_t has = __ballot(cnt != 0);
      if (cnt) lst[base + __popcll(has & ((uint64_t(1) << lane) - 1))] = (bin << 16) | cnt;
    }
  }
  __syncthreads();
  // the record's global stores come last: no barrier waits for them
  uint32_t* rec = ws + row * row_words + static_cast<int64_t>(blockIdx.x) * rec_words;
  rec[cb] = incl >> 16;                  // keys at or above coarse bin cb
  rec[kCoarse + cb] = incl & 0xffffu;    // distinct keys at or above coarse bin cb
  const uint32_t n_list = tmp[21];
  for (uint32_t e = tid; e < n_list; e += kFineThreads) rec[2 * kCoarse + e] = lst[e];
}

__global__ void __launch_bounds__(kFineThreads)
topk_fine_write_kernel(int64_t T, int64_t N, int64_t q_pos0, int ratio, const int64_t* __restrict__ seq_pos, int k,
                       const uint16_t* __restrict__ scores, const uint32_t* __restrict__ ws, int64_t rec_words,
                       int64_t row_words, int32_t* __restrict__ idx) {
  constexpr int kMaxS = kFineThreads;   // slices whose list ranges are staged in LDS at once
  __shared__ uint32_t fine[64], fine_before[64];
  __shared__ uint32_t tot_c[kCoarse + 1], before_c[kCoarse + 1];
  __shared__ uint32_t e_lo[kMaxS], e_cnt[kMaxS + 1];
  __shared__ uint32_t st[8];
  __shared__ uint64_t tmp64[17];
  __shared__ uint32_t tmp32[20];
  const int64_t row = blockIdx.y;
  const int64_t V = row_visible(row, T, q_pos0, ratio, N, seq_pos);
  int32_t* out = idx + row * k;
  const int tid = threadIdx.x;
  if (V <= k) {
    if (blockIdx.x == 0)
      for (int i = tid; i < k; i += kFineThreads) out[i] = i < V ? i : -1;
    return;
  }
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * kFineSlice;
  if (lo >= V) return;
  const int64_t hi = lo + kFineSlice < V ? lo + kFineSlice : V;
  const int S = static_cast<int>((V + kFineSlice - 1) / kFineSlice);
  const int me = static_cast<int>(blockIdx.x);
  uint32_t kp[2][4], valid[2];
  fine_slice_keys<2>(scores + row * N, lo, hi, kp, valid);
  const uint32_t* rws = ws + row * row_words;
  tot_c[tid] = 0;
  before_c[tid] = 0;
  if (tid < 64) {
    fine[tid] = 0;
    fine_before[tid] = 0;
  } else if (tid == 64) {
    tot_c[kCoarse] = 0;
    before_c[kCoarse] = 0;
  }
  __syncthreads();
  // coarse counts (keys at or above each coarse bin) summed over all slices
  // and over the slices before this one: thread t adds quad t % 256 of slices
  // t / 256, t / 256 + 4, ..., four loads in flight at a time
  {
    const int q = tid & 255, g = tid >> 8;
    uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
    for (int i0 = g; i0 < S; i0 += 16) {
      uint4 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = i0 + 4 * j;
        v[j] = i < S ? reinterpret_cast<const uint4*>(rws + static_cast<int64_t>(i) * rec_words)[q]
                     : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a.x += v[j].x; a.y += v[j].y; a.z += v[j].z; a.w += v[j].w;
        if (i0 + 4 * j < me) { b.x += v[j].x; b.y += v[j].y; b.z += v[j].z; b.w += v[j].w; }
      }
    }
    atomicAdd(&tot_c[4 * q], a.x); atomicAdd(&tot_c[4 * q + 1], a.y);
    atomicAdd(&tot_c[4 * q + 2], a.z); atomicAdd(&tot_c[4 * q + 3], a.w);
    atomicAdd(&before_c[4 * q], b.x); atomicAdd(&before_c[4 * q + 1], b.y);
    atomicAdd(&before_c[4 * q + 2], b.z); atomicAdd(&before_c[4 * q + 3], b.w);
  }
  __syncthreads();
  // c*: the highest coarse bin with at least k keys at or above it
  if (tot_c[tid] >= static_cast<uint32_t>(k) && tot_c[tid + 1] < static_cast<uint32_t>(k)) st[0] = tid;
  __syncthreads();
  const int cs = static_cast<int>(st[0]);
  const uint32_t rem1 = static_cast<uint32_t>(k) - tot_c[cs + 1];   // keys of bin c* still to take
  // the listed keys of c* in every slice: entries [distinct above c*, distinct
  // at or above c*) of its list (at most 64 per slice), four loads in flight
  for (int s0 = 0; s0 < S; s0 += kMaxS) {
    const int ns = S - s0 < kMaxS ? S - s0 : kMaxS;
    uint32_t cnt = 0;
    if (tid < ns) {
      const uint32_t* rec = rws + static_cast<int64_t>(s0 + tid) * rec_words;
      const uint32_t e0 = cs < kCoarse - 1 ? rec[kCoarse + cs + 1] : 0u;
      cnt = rec[kCoarse + cs] - e0;
      e_lo[tid] = e0;
    }
    uint32_t tot_e;
    const uint32_t ex = block_exclusive_scan(cnt, tmp32, &tot_e);
    if (tid < ns) e_cnt[tid] = ex;
    if (tid == 0) e_cnt[ns] = tot_e;
    __syncthreads();
    for (uint32_t f0 = 0; f0 < tot_e; f0 += 4 * kFineThreads) {
      uint32_t v[4];
      int sl[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t f = f0 + j * kFineThreads + tid;
        v[j] = 0;
        sl[j] = -1;
        if (f < tot_e) {
          int lo_s = 0, hi_s = ns;   // the slice whose range holds flat entry f: e_cnt[s] <= f < e_cnt[s + 1]
          while (hi_s - lo_s > 1) {
            const int mid = (lo_s + hi_s) >> 1;
            if (e_cnt[mid] <= f) lo_s = mid; else hi_s = mid;
          }
          sl[j] = lo_s;
          v[j] = rws[static_cast<int64_t>(s0 + lo_s) * rec_words + 2 * kCoarse + e_lo[lo_s] + (f - e_cnt[lo_s])];
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (sl[j] < 0) continue;
        const uint32_t fb = (v[j] >> 16) & 63u, n = v[j] & 0xffffu;
        atomicAdd(&fine[fb], n);
        if (s0 + sl[j] < me) atomicAdd(&fine_before[fb], n);
      }
    }
    __syncthreads();
  }
  resolve_digit(fine, 64, rem1, st + 2);
  __syncthreads();
  const uint32_t fs = st[2], rem = st[3];
  const uint32_t K = (static_cast<uint32_t>(cs) << 6) | fs;
  // keys above K and equal to K in the slices before this one
  if (tid < 64) {
    uint32_t g = tid > static_cast<int>(fs) ? fine_before[tid] : 0u;
    g = wave_total_add(g);
    if (tid == 0) st[4] = g + before_c[cs + 1];
  }
  __syncthreads();
  uint32_t gt_run = st[4], eq_run = fine_before[fs];
  // ordered compaction of the slice (fields gt0 | eq0 | gt1 | eq1 of the two
  // chunks): bit u of gtm[h] / eqm[h] marks key u of chunk h above / equal to K
  uint32_t gtm[2], eqm[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    gtm[h] = 0;
    eqm[h] = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      gtm[h] |= static_cast<uint32_t>(FKEY(h, u) > K) << u;
      eqm[h] |= static_cast<uint32_t>(FKEY(h, u) == K) << u;
    }
    gtm[h] &= valid[h];
    eqm[h] &= valid[h];
  }
  const uint64_t packed = static_cast<uint64_t>(__popc(gtm[0])) | (static_cast<uint64_t>(__popc(eqm[0])) << 16) |
                          (static_cast<uint64_t>(__popc(gtm[1])) << 32) |
                          (static_cast<uint64_t>(__popc(eqm[1])) << 48);
  uint64_t tot;
  const uint64_t ex = block_exclusive_scan_u64(packed, tmp64, &tot);
  const uint32_t tg0 = tot & 0xffffu, te0 = (tot >> 16) & 0xffffu;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t gb = gt_run + (h ? tg0 + ((ex >> 32) & 0xffffu) : (ex & 0xffffu));
    const uint32_t eb = eq_run + (h ? te0 + ((ex >> 48) & 0xffffu) : ((ex >> 16) & 0xffffu));
    // the keys taken: every one above K, and the ties in index order while
    // fewer than rem ties of the row come before them
    uint32_t take = gtm[h];
    uint32_t ties = eqm[h];
    for (uint32_t er = eb; ties != 0 && er < rem; ++er) {
      take |= ties & (0u - ties);
      ties &= ties - 1u;
    }
    uint32_t pos = gb + (eb < rem ? eb : rem);
    const int32_t i0 = static_cast<int32_t>(lo + 8 * (h * kFineThreads + tid));
    while (take) {
      out[pos++] = i0 + static_cast<int32_t>(__builtin_ctz(take));
      take &= take - 1u;
    }
  }
}
#undef FKEY

hipError_t launch_fine(const TopkArgs& a, hipStream_t s) {
  const int64_t rows = a.B * a.T;
  const int64_t S = (a.N + kFineSlice - 1) / kFineSlice;
  const int64_t rec = topk_fine_rec_words(a.k);
  const int64_t per_row = S * rec;
  uint32_t* ws = static_cast<uint32_t*>(a.ws);
  const auto* sc = static_cast<const uint16_t*>(a.scores);
  const dim3 grid(static_cast<uint32_t>(S), static_cast<uint32_t>(rows));
  hipLaunchKernelGGL(topk_fine_record_kernel, grid, dim3(kFineThreads), 0, s, a.T, a.N, a.q_pos0, a.ratio, a.seq_pos,
                     a.k, sc, ws, rec, per_row);
  hipLaunchKernelGGL(topk_fine_write_kernel, grid, dim3(kFineThreads), 0, s, a.T, a.N, a.q_pos0, a.ratio, a.seq_pos,
                     a.k, sc, ws, rec, per_row, a.idx);
  return hipGetLastError();
}

template <typename KT>
hipError_t launch_typed(const TopkArgs& a, hipStream_t s) {
  const KT* sc = static_cast<const KT*>(a.scores);
  const int64_t rows = a.B * a.T;
  if constexpr (sizeof(KT) == 2) {
    // rows of bf16 keys that fit 1024 threads x CPT chunks of 8, 16-byte aligned
    const int cpt = static_cast<int>((a.N + 8 * 1024 - 1) / (8 * 1024));
    if (a.N % 8 == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0 && cpt <= 5) {
      const dim3 grid(static_cast<uint32_t>(rows));
      const auto* sc16 = static_cast<const uint16_t*>(a.scores);
      switch (cpt) {
        case 1: hipLaunchKernelGGL(topk_reg_kernel<1>, grid, dim3(1024), 0, s, a.T, a.N, a.q_pos0, a.ratio, a.seq_pos, a.k, sc16, a.idx, a.pool, a.n_ent); break;
        case 2: hipLaunchKernelGGL(topk_reg_kernel<2>, grid, dim3(1024), 0, s, a.T, a.N, a.q_pos0, a.ratio, a.seq_pos, a.k, sc16, a.idx, a.pool, a.n_ent); break;
        case 3: hipLaunchKernelGGL(topk_reg_kernel<3>, grid, dim3(1024), 0, s, a.T, a.N, a.q_pos0, a.ratio, a.seq_pos, a.k, sc16, a.idx, a.pool, a.n_ent); break;
        case 4: hipLaunchKernelGGL(topk_reg_kernel<4>, grid, dim3(1024), 0, s, a.T, a.N, a.q_pos0, a.ratio, a.seq_pos, a.k, sc16, a.idx, a.pool, a.n_ent); break;
        default: hipLaunchKernelGGL(topk_reg_kernel<5>, grid, dim3(1024), 0, s, a.T, a.N, a.q_pos0, a.ratio, a.seq_pos, a.k, sc16, a.idx, a.pool, a.n_ent); break;
      }
      return hipGetLastError();
    }
  }
  if (topk_row_in_lds(a.N, a.score_dtype)) {
    const size_t smem = (kRangeBins + 32) * sizeof(uint32_t) + static_cast<size_t>(a.N) * sizeof(KT);
    hipLaunchKernelGGL((topk_lds_kernel<KT>), dim3(static_cast<uint32_t>(rows)), dim3(1024), smem, s, a.T,
                       a.N, a.q_pos0, a.ratio, a.seq_pos, a.k, sc, a.idx, a.pool, a.n_ent);
    return hipGetLastError();
  }
  if constexpr (sizeof(KT) == 2) {
    // long bf16 rows: slices of kFineSlice keys, a full 16-bit histogram each
    if (a.N % 8 == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0) return launch_fine(a, s);
  }
  const int S = kTopkSlices;
  uint32_t* ws = static_cast<uint32_t*>(a.ws);
  const int64_t words = rows * (kWsHist + 2 * S);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<uint32_t>((words + 255) / 256)), dim3(256), 0, s, ws,
                     words);
  const dim3 grid(S, static_cast<uint32_t>(rows));
  for (int p = 0; p < Digits<KT>::n; ++p)
    hipLaunchKernelGGL((topk_hist_kernel<KT>), grid, dim3(256), 0, s, p, a.T, a.N, a.q_pos0, a.ratio, a.seq_pos, a.k, S,
                       sc, ws);
  hipLaunchKernelGGL((topk_count_kernel<KT>), grid, dim3(256), 0, s, a.T, a.N, a.q_pos0, a.ratio, a.seq_pos, a.k, S, sc,
                     ws);
  hipLaunchKernelGGL((topk_write_kernel<KT>), grid, dim3(256), 0, s, a.T, a.N, a.q_pos0, a.ratio, a.seq_pos, a.k, S, sc,
                     ws, a.idx);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.B == 0 || a.T == 0) return hipSuccess;
  if (a.score_dtype == CSA_BF16) return launch_typed<uint16_t>(a, s);
  return launch_typed<uint32_t>(a, s);
}


// Top-k, with a decode step's compressor jobs in the register kernel's launch
// where it applies (bf16 rows that fit it, one-entry jobs from bf16 rows of
// at most 512 channels, outputs clear of the scores and ids); otherwise the
// jobs' launch, then Top-k's.  Same results either way.
hipError_t launch_topk_jobs(const TopkArgs& a, const CompressArgs* jobs, int n, hipStream_t s) {
  if (n < 1) return launch_topk(a, s);
  const int64_t rows = a.B * a.T;
  const int cpt = static_cast<int>((a.N + 8 * 1024 - 1) / (8 * 1024));
  bool fuse = rows > 0 && a.score_dtype == CSA_BF16 && !a.pool && !a.seq_pos && a.N % 8 == 0 &&
              (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0 && cpt <= 5;
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(a.scores), s1 = s0 + static_cast<uintptr_t>(rows * a.N * 2);
  const uintptr_t i0 = reinterpret_cast<uintptr_t>(a.idx), i1 = i0 + static_cast<uintptr_t>(rows * a.k * 4);
  for (int q = 0; q < n && fuse; ++q) {
    const CompressArgs& j = jobs[q];
    fuse = j.ratio == 4 && j.n_tok == 4 && j.B == jobs[0].B && j.c <= 512 && j.in_dtype == CSA_BF16 &&
           (j.out_dtype == CSA_BF16 || j.out_dtype == CSA_FP8_E4M3 || j.out_dtype == CSA_MXFP4);
    const int64_t stride = j.out_batch_stride ? j.out_batch_stride : j.c;
    const int64_t span = (j.B - 1) * stride + j.c;
    const int64_t ob = j.out_dtype == CSA_BF16 ? 2 * span : (j.out_dtype == CSA_FP8_E4M3 ? span : span / 2);
    const uintptr_t o0 = reinterpret_cast<uintptr_t>(j.out), o1 = o0 + static_cast<uintptr_t>(ob);
    if ((o0 < s1 && s0 < o1) || (o0 < i1 && i0 < o1)) fuse = false;
    if (j.out_scale) {
      const uintptr_t c0 = reinterpret_cast<uintptr_t>(j.out_scale);
      const uintptr_t c1 = c0 + static_cast<uintptr_t>(((j.B - 1) * (stride / j.c) + 1) * 4 * (j.c / 32 + 1));
      if ((c0 < s1 && s0 < c1) || (c0 < i1 && i0 < c1)) fuse = false;
    }
  }
  if (!fuse) {
    const hipError_t e = launch_compress_batch(jobs, n, s);
    return e != hipSuccess ? e : launch_topk(a, s);
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
  const int64_t B = jobs[0].B;
  const dim3 grid(static_cast<uint32_t>(rows + n * B));
  const auto* sc = static_cast<const uint16_t*>(a.scores);
  switch (cpt) {
    case 1: hipLaunchKernelGGL(topk_reg_jobs_kernel<1>, grid, dim3(1024), 0, s, rows, a.T, a.N, a.q_pos0, a.ratio, a.k, sc, a.idx, jb, B); break;
    case 2: hipLaunchKernelGGL(topk_reg_jobs_kernel<2>, grid, dim3(1024), 0, s, rows, a.T, a.N, a.q_pos0, a.ratio, a.k, sc, a.idx, jb, B); break;
    case 3: hipLaunchKernelGGL(topk_reg_jobs_kernel<3>, grid, dim3(1024), 0, s, rows, a.T, a.N, a.q_pos0, a.ratio, a.k, sc, a.idx, jb, B); break;
    case 4: hipLaunchKernelGGL(topk_reg_jobs_kernel<4>, grid, dim3(1024), 0, s, rows, a.T, a.N, a.q_pos0, a.ratio, a.k, sc, a.idx, jb, B); break;
    default: hipLaunchKernelGGL(topk_reg_jobs_kernel<5>, grid, dim3(1024), 0, s, rows, a.T, a.N, a.q_pos0, a.ratio, a.k, sc, a.idx, jb, B); break;
  }
  return hipGetLastError();
}

}  // namespace csa
