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
// Two paths:
//  * rows of up to ~36K bf16 (~18K fp32) keys: one 1024-thread workgroup per
//    row holds the whole row in LDS and runs every pass there;
//  * longer rows (the 1M-context decode has 262,144 candidates): S workgroups
//    per row, one slice each; per-digit histograms are merged in global
//    workspace with atomics, one kernel per pass, then a count kernel and an
//    ordered write kernel.
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
  uint32_t S = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t v = __shfl_down(S, o, 64);
    if (lane + o < 64) S += v;
  }
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
template <typename U>
__device__ U block_exclusive_scan_t(U v, U* tmp, U* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  U x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const U y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wid] = x;
  __syncthreads();
  if (wid == 0) {
    const U w0 = lane < nw ? tmp[lane] : U(0);
    U t = w0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const U y = __shfl_up(t, o, 64);
      if (lane >= o) t += y;
    }
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
  const int64_t pos = seq_pos ? seq_pos[row / T] : q_pos0 + row % T;
  const int64_t v = (pos + 1) / ratio;
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
    const uint32_t lb = __shfl(bin, leader, 64);
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
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      kmin = min(kmin, static_cast<uint32_t>(__shfl_xor(kmin, o, 64)));
      kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(kmax, o, 64)));
    }
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
__global__ void __launch_bounds__(1024)
topk_reg_kernel(int64_t T, int64_t N, int64_t q_pos0, int ratio, const int64_t* __restrict__ seq_pos, int k, const uint16_t* __restrict__ scores,
                int32_t* __restrict__ idx, const int32_t* __restrict__ pool, int64_t n_ent) {
  constexpr int NT = 1024;
  static_assert(8 * CPT * NT < 65536, "block-wide counts are packed in 16 bits");
  __shared__ uint32_t bins[kRangeBins];
  __shared__ uint32_t tmp[32];
  const int64_t row = blockIdx.x;
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
  uint32_t kmin = 0xffffu, kmax = 0u;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int64_t i0 = i00 + 8 * c;
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (i0 < V) raw = src[c];
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    const int64_t nv = V - i0;
    valid[c] = nv >= 8 ? 0xffu : (nv > 0 ? (1u << nv) - 1u : 0u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = key_of(static_cast<uint16_t>(w[j] & 0xffffu));
      const uint32_t hi = key_of(static_cast<uint16_t>(w[j] >> 16));
      kp[c][j] = lo | (hi << 16);
      if ((valid[c] >> (2 * j)) & 1u) { kmin = min(kmin, lo); kmax = max(kmax, lo); }
      if ((valid[c] >> (2 * j + 1)) & 1u) { kmin = min(kmin, hi); kmax = max(kmax, hi); }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    kmin = min(kmin, static_cast<uint32_t>(__shfl_xor(kmin, o, 64)));
    kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(kmax, o, 64)));
  }
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

  // pass 1: bin (key - min) >> sh
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if ((valid[c] >> u) & 1u) atomicAdd(&bins[KEY(c, u) >> sh], 1u);
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

  // ordered compaction: this thread's keys above K, then the first rem equal to K
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool vv = (valid[c] >> u) & 1u;
      gt += vv && KEY(c, u) > K;
      eq += vv && KEY(c, u) == K;
    }
  uint32_t tot;
  const uint32_t ex = block_exclusive_scan(gt | (eq << 16), tmp, &tot);
  // which of this thread's keys are taken (bit 8c + u), then one store per
  // taken key in index order
  uint64_t take = 0;
  uint32_t er = ex >> 16;
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool vv = (valid[c] >> u) & 1u;
      const uint32_t kk = KEY(c, u);
      const bool tie = vv && kk == K;
      if ((vv && kk > K) || (tie && er < rem)) take |= uint64_t(1) << (8 * c + u);
      er += tie;
    }
  uint32_t pos = (ex & 0xffffu) + min(ex >> 16, rem);
  while (take) {
    out[pos++] = pool_map(prow, n_ent, i00 + __builtin_ctzll(take));
    take &= take - 1;
  }
#undef KEY
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
  gt = wave_sum_u32(gt);
  eq = wave_sum_u32(eq);
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
// Rows too long for one workgroup (the 1M-context decode: 262,144 keys): S
// slices per row, one 256-thread workgroup per slice holding its keys in
// registers (thread t, chunk c: keys lo + 8 (c * 256 + t) .. + 7).
//   G1  histogram of the top 11 key bits of the slice, merged into the row's
//       histogram with one atomic per non-empty bin;
//   G2  with the top bin b* resolved: the slice's count of keys above b* and
//       its 32-bin histogram of the low 5 bits among keys in b*, kept per
//       slice and merged into the row's low histogram;
//   G3  with K resolved: each slice's output offset follows from the per-slice
//       records of the slices before it, then an ordered compaction.
// Row workspace (uint32): hist1[2048] | hist2[32] | pad | per-slice [S][33].
constexpr int kLongHist2 = kBins;                 // offset of hist2
constexpr int kLongSlices = kBins + 64;           // offset of the per-slice records
constexpr int kSliceRec = 33;                     // above, low histogram[32]

template <int CPT>
__device__ __forceinline__ void long_slice_keys(const uint16_t* row, int64_t lo, int64_t hi, uint32_t (&kp)[CPT][4],
                                                uint32_t (&valid)[CPT]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int64_t i0 = lo + 8 * (static_cast<int64_t>(c) * 256 + tid);
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (i0 < hi) raw = *reinterpret_cast<const uint4*>(row + i0);
    const int64_t nv = hi - i0;
    valid[c] = nv >= 8 ? 0xffu : (nv > 0 ? (1u << nv) - 1u : 0u);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      kp[c][j] = key_of(static_cast<uint16_t>(w[j] & 0xffffu)) | (static_cast<uint32_t>(key_of(static_cast<uint16_t>(w[j] >> 16))) << 16);
  }
}
#define LKEY(c, u) ((kp[c][(u) >> 1] >> (16 * ((u) & 1))) & 0xffffu)

__device__ __forceinline__ void long_slice_range(int64_t V, int S, int64_t& lo, int64_t& hi) {
  const int64_t L = ((V + S - 1) / S + 7) / 8 * 8;
  lo = blockIdx.x * L;
  hi = lo + L < V ? lo + L : V;
  if (lo > hi) lo = hi;
}

template <int CPT>
__global__ void __launch_bounds__(256)
topk_long_hist1_kernel(int64_t T, int64_t N, int64_t q_pos0, int ratio, const int64_t* __restrict__ seq_pos, int k, int S,
                       const uint16_t* __restrict__ scores, uint32_t* __restrict__ ws) {
  __shared__ uint32_t hist[kBins];
  const int64_t row = blockIdx.y;
  const int64_t V = row_visible(row, T, q_pos0, ratio, N, seq_pos);
  if (V <= k) return;
  for (int i = threadIdx.x; i < kBins; i += 256) hist[i] = 0;
  int64_t lo, hi;
  long_slice_range(V, S, lo, hi);
  uint32_t kp[CPT][4], valid[CPT];
  long_slice_keys<CPT>(scores + row * N, lo, hi, kp, valid);
  __syncthreads();
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int u = 0; u < 8; ++u) hist_add(hist, LKEY(c, u) >> 5, (valid[c] >> u) & 1u);
  __syncthreads();
  uint32_t* h1 = ws + row * (kLongSlices + kSliceRec * S);
  for (int i = threadIdx.x; i < kBins; i += 256)
    if (hist[i]) atomicAdd(&h1[i], hist[i]);
}

template <int CPT>
__global__ void __launch_bounds__(256)
topk_long_hist2_kernel(int64_t T, int64_t N, int64_t q_pos0, int ratio, const int64_t* __restrict__ seq_pos, int k, int S,
                       const uint16_t* __restrict__ scores, uint32_t* __restrict__ ws) {
  __shared__ uint32_t st[4];
  __shared__ uint32_t h2[32];
  __shared__ uint32_t above_s;
  const int64_t row = blockIdx.y;
  const int64_t V = row_visible(row, T, q_pos0, ratio, N, seq_pos);
  if (V <= k) return;
  uint32_t* rws = ws + row * (kLongSlices + kSliceRec * S);
  int64_t lo, hi;
  long_slice_range(V, S, lo, hi);
  uint32_t kp[CPT][4], valid[CPT];
  long_slice_keys<CPT>(scores + row * N, lo, hi, kp, valid);   // in flight while the top bin resolves
  if (threadIdx.x < 32) h2[threadIdx.x] = 0;
  if (threadIdx.x == 0) above_s = 0;
  resolve_digit(rws, kBins, static_cast<uint32_t>(k), st);
  __syncthreads();
  const uint32_t bstar = st[0];
  uint32_t above = 0;
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool v = (valid[c] >> u) & 1u;
      const uint32_t kk = LKEY(c, u);
      above += v && (kk >> 5) > bstar;
      if (v && (kk >> 5) == bstar) atomicAdd(&h2[kk & 31], 1u);
    }
  above = wave_sum_u32(above);
  if ((threadIdx.x & 63) == 0) atomicAdd(&above_s, above);
  __syncthreads();
  uint32_t* rec = rws + kLongSlices + kSliceRec * blockIdx.x;
  if (threadIdx.x == 0) rec[0] = above_s;
  if (threadIdx.x < 32) {
    rec[1 + threadIdx.x] = h2[threadIdx.x];
    if (h2[threadIdx.x]) atomicAdd(&rws[kLongHist2 + threadIdx.x], h2[threadIdx.x]);
  }
}

template <int CPT>
__global__ void __launch_bounds__(256)
topk_long_write_kernel(int64_t T, int64_t N, int64_t q_pos0, int ratio, const int64_t* __restrict__ seq_pos, int k, int S,
                       const uint16_t* __restrict__ scores, uint32_t* __restrict__ ws, int32_t* __restrict__ idx) {
  __shared__ uint32_t st[4];
  __shared__ uint32_t st2[4];
  __shared__ uint64_t tmp64[17];
  __shared__ uint32_t before[2];
  const int64_t row = blockIdx.y;
  const int64_t V = row_visible(row, T, q_pos0, ratio, N, seq_pos);
  int32_t* out = idx + row * k;
  if (V <= k) {
    if (blockIdx.x == 0)
      for (int i = threadIdx.x; i < k; i += 256) out[i] = i < V ? i : -1;
    return;
  }
  const uint32_t* rws = ws + row * (kLongSlices + kSliceRec * S);
  int64_t lo, hi;
  long_slice_range(V, S, lo, hi);
  uint32_t kp[CPT][4], valid[CPT];
  long_slice_keys<CPT>(scores + row * N, lo, hi, kp, valid);
  resolve_digit(rws, kBins, static_cast<uint32_t>(k), st);
  __syncthreads();
  const uint32_t bstar = st[0], rem1 = st[1];
  resolve_digit(rws + kLongHist2, 32, rem1, st2);
  __syncthreads();
  const uint32_t lowk = st2[0], rem = st2[1];
  const uint32_t K = (bstar << 5) | lowk;
  // keys > K and == K in the slices before this one
  if (threadIdx.x < 64) {
    uint32_t gt = 0, eq = 0;
    for (int s2 = threadIdx.x; s2 < static_cast<int>(blockIdx.x); s2 += 64) {
      const uint32_t* rec = rws + kLongSlices + kSliceRec * s2;
      gt += rec[0];
      for (int b = lowk + 1; b < 32; ++b) gt += rec[1 + b];
      eq += rec[1 + lowk];
    }
    gt = wave_sum_u32(gt);
    eq = wave_sum_u32(eq);
    if (threadIdx.x == 0) {
      before[0] = gt;
      before[1] = eq;
    }
  }
  __syncthreads();
  uint32_t gt_run = before[0], eq_run = before[1];
  // ordered compaction of the slice, two chunks per scan (fields gt0 | eq0 | gt1 | eq1)
#pragma unroll
  for (int c0 = 0; c0 < CPT; c0 += 2) {
    uint32_t cnt[2][2] = {{0, 0}, {0, 0}};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (c0 + h >= CPT) continue;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool vv = (valid[c0 + h] >> u) & 1u;
        cnt[h][0] += vv && LKEY(c0 + h, u) > K;
        cnt[h][1] += vv && LKEY(c0 + h, u) == K;
      }
    }
    const uint64_t packed = static_cast<uint64_t>(cnt[0][0]) | (static_cast<uint64_t>(cnt[0][1]) << 16) |
                            (static_cast<uint64_t>(cnt[1][0]) << 32) | (static_cast<uint64_t>(cnt[1][1]) << 48);
    uint64_t tot;
    const uint64_t ex = block_exclusive_scan_u64(packed, tmp64, &tot);
    const uint32_t tg0 = tot & 0xffffu, te0 = (tot >> 16) & 0xffffu;
    const uint32_t tg1 = (tot >> 32) & 0xffffu, te1 = (tot >> 48) & 0xffffu;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = c0 + h;
      if (c >= CPT) continue;
      const uint32_t gb = gt_run + (h ? tg0 + ((ex >> 32) & 0xffffu) : (ex & 0xffffu));
      const uint32_t eb = eq_run + (h ? te0 + ((ex >> 48) & 0xffffu) : ((ex >> 16) & 0xffffu));
      uint32_t pos = gb + (eb < rem ? eb : rem);
      uint32_t er = eb;
      const int32_t i0 = static_cast<int32_t>(lo + 8 * (c * 256 + threadIdx.x));
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (!((valid[c] >> u) & 1u)) continue;
        const uint32_t kk = LKEY(c, u);
        if (kk > K) {
          out[pos++] = i0 + u;
        } else if (kk == K) {
          if (er < rem) out[pos++] = i0 + u;
          ++er;
        }
      }
    }
    gt_run += tg0 + tg1;
    eq_run += te0 + te1;
  }
}
#undef LKEY

template <int CPT>
hipError_t launch_long(const TopkArgs& a, hipStream_t s) {
  const int S = kTopkSlices;
  const int64_t rows = a.B * a.T;
  uint32_t* ws = static_cast<uint32_t*>(a.ws);
  const auto* sc = static_cast<const uint16_t*>(a.scores);
  const int64_t per_row = kLongSlices + kSliceRec * S;
  const int64_t words = rows * per_row;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<uint32_t>((words + 255) / 256)), dim3(256), 0, s, ws, words);
  const dim3 grid(S, static_cast<uint32_t>(rows));
  hipLaunchKernelGGL(topk_long_hist1_kernel<CPT>, grid, dim3(256), 0, s, a.T, a.N, a.q_pos0, a.ratio, a.seq_pos, a.k, S, sc, ws);
  hipLaunchKernelGGL(topk_long_hist2_kernel<CPT>, grid, dim3(256), 0, s, a.T, a.N, a.q_pos0, a.ratio, a.seq_pos, a.k, S, sc, ws);
  hipLaunchKernelGGL(topk_long_write_kernel<CPT>, grid, dim3(256), 0, s, a.T, a.N, a.q_pos0, a.ratio, a.seq_pos, a.k, S, sc, ws,
                     a.idx);
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
    // long bf16 rows: slices of up to 8 * 256 * 8 keys held in registers
    const int64_t slice = ((a.N + kTopkSlices - 1) / kTopkSlices + 7) / 8 * 8;
    const int64_t cpt = (slice + 2047) / 2048;
    if (a.N % 8 == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0 && cpt <= 8) {
      if (cpt <= 1) return launch_long<1>(a, s);
      if (cpt <= 2) return launch_long<2>(a, s);
      if (cpt <= 4) return launch_long<4>(a, s);
      return launch_long<8>(a, s);
    }
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

}  // namespace csa
