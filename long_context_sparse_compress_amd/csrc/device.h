// Device helpers shared by the gfx950 kernels: bf16 conversion, vector
// types, MFMA operand types and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (low half = a), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// float -> bfloat16, round to nearest even.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Unpack 8 bf16 held in a uint4 into floats.
__device__ __forceinline__ void unpack_bf16x8(const uint4& v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return exp2f(x); }

// Sum / max over the 64 lanes of a wave.
// On the DPP cross-lane paths (no LDS round trip): shifts inside each row of
// 16 lanes, then the row results carried across rows by the row broadcasts
// of lanes 15 and 31, so lane 63 ends with the whole wave's; every lane gets
// lane 63's value.  All 64 lanes must be active.
#define CSA_FDPP(old, x, ctrl, rmask, bound0) \
  __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(x), ctrl, rmask, 0xf, bound0))
__device__ __forceinline__ float wave_sum(float v) {
  v += CSA_FDPP(0.f, v, 0x111, 0xf, true);   // row_shr:1
  v += CSA_FDPP(0.f, v, 0x112, 0xf, true);   // row_shr:2
  v += CSA_FDPP(0.f, v, 0x114, 0xf, true);   // row_shr:4
  v += CSA_FDPP(0.f, v, 0x118, 0xf, true);   // row_shr:8
  v += CSA_FDPP(0.f, v, 0x142, 0xa, false);  // row_bcast:15 into rows 1 and 3
  v += CSA_FDPP(0.f, v, 0x143, 0xc, false);  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, CSA_FDPP(-INFINITY, v, 0x111, 0xf, false));
  v = fmaxf(v, CSA_FDPP(-INFINITY, v, 0x112, 0xf, false));
  v = fmaxf(v, CSA_FDPP(-INFINITY, v, 0x114, 0xf, false));
  v = fmaxf(v, CSA_FDPP(-INFINITY, v, 0x118, 0xf, false));
  v = fmaxf(v, CSA_FDPP(-INFINITY, v, 0x142, 0xa, false));
  v = fmaxf(v, CSA_FDPP(-INFINITY, v, 0x143, 0xc, false));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
#undef CSA_FDPP

// Cross-lane read with a precomputed byte address (lane index * 4):
// ds_bpermute without the per-call lane arithmetic of __shfl*.
__device__ __forceinline__ float lane_read(int addr, float v) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(v)));
}

// Pairwise combines across the two lane halves (32) or across neighbouring
// 16-lane rows (16) on the gfx950 lane-swap instructions, with no LDS round
// trip.  v_permlane32_swap trades the upper half of a with the lower half of
// b, so the two results added give a[l] + a[l + 32] in the lower half and
// b[l - 32] + b[l] in the upper half; v_permlane16_swap does the same for the
// odd rows of a and the even rows of b (a[l] + a[l + 16] in rows 0 and 2,
// b[l - 16] + b[l] in rows 1 and 3).  With a = b that is v + v[l ^ 32] (or
// v[l ^ 16]) in every lane.  Every lane of the wave must take part.
__device__ __forceinline__ float pair_sum32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_sum16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_max32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_max16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Partial rotary embedding ("DeepSeek Technical Reports", Hybrid Attention,
// CSA; "DeepSeek V4 结构速览", the CSA operator graph; the rotation is
// RoFormer's): pair p of the last R dimensions,
// (x[2p], x[2p+1]) of that part, turns by pos * base^(-2p/R).  At a million
// tokens of context the angle reaches ~1e6 rad, so it is counted in turns in
// fp64 -- pos * theta / 2pi, whose fractional part is exact -- and only the
// reduced angle, |a| <= pi, goes to the fp32 sine and cosine (an angle error
// near 1e-9 rad; no fp64 trigonometry with its long-argument reduction).
// log2_base = log2(base), formed once on the host in fp64.
__device__ inline void rope_cos_sin(int64_t pos, int p, int R, double log2_base, float& c, float& s) {
  constexpr double kLog2TwoPi = 2.65149612947231879804;   // log2(2 pi)
  constexpr double k2Pi = 6.28318530717958647693;
  const double turns = static_cast<double>(pos) * exp2(-(2.0 * p / R) * log2_base - kLog2TwoPi);
  const double frac = turns - rint(turns);              // in [-1/2, 1/2]
  sincosf(static_cast<float>(frac * k2Pi), &s, &c);
}
// (x, y) -> (x c - y s, x s + y c)
__device__ __forceinline__ void rope_pair(float& x, float& y, float c, float s) {
  const float nx = x * c - y * s;
  const float ny = x * s + y * c;
  x = nx;
  y = ny;
}

// fp32 -> OCP E4M3 byte code: round to nearest even, magnitudes from 464 (the
// midpoint past the largest finite value, 448) up saturate to 448, the sign
// is kept.  Normal results round the float's mantissa to 3 bits on its bit
// pattern (a carry moves into the exponent, which is then rebiased from 127
// to 7); results below 2^-6 are subnormal multiples of 2^-9, rounded with
// rint (the scaling by 2^9 is exact).
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a >= 0x43e80000u) {                 // |v| >= 464 (or not finite)
    code = 0x7eu;
  } else if (a >= 0x3c800000u) {          // |v| >= 2^-6: normal
    const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
    code = r - (120u << 3);
  } else {
    code = static_cast<uint32_t>(rintf(__uint_as_float(a) * 512.f));
  }
  return sign | code;
}

// fp32 -> OCP E2M1 nibble: the nearest of {0, 0.5, 1, 1.5, 2, 3, 4, 6}, ties to
// the even mantissa (code), magnitudes past 6 to 6; a value that rounds to 0
// is written +0.
__device__ __forceinline__ uint32_t f32_to_e2m1(float v) {
  const float a = fabsf(v);
  const uint32_t code = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                      : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.f ? 6u : 7u;
  return (v < 0.f && code) ? (code | 8u) : code;
}

// Round-robin workgroup dispatch puts consecutive workgroup ids on different
// XCDs (8 on MI355X).  Remap a linear id so that ids [x*per, (x+1)*per) run on
// XCD x, keeping neighbouring tiles (and their shared data) in one L2.
__device__ __forceinline__ uint32_t xcd_swizzle(uint32_t id, uint32_t n) {
  constexpr uint32_t kXcd = 8;
  if (n % kXcd != 0) return id;
  const uint32_t per = n / kXcd;
  return (id % kXcd) * per + id / kXcd;
}

}  // namespace csa
