// Partial RoPE (or its inverse) in place on query or window rows.
//
// "DeepSeek Technical Reports" (Hybrid Attention, CSA: partial RoPE) and
// "DeepSeek V4 结构速览" (the CSA operator graph): the query and each raw latent of the sliding window are
// rotated at their own positions on their last R dimensions, pair p turning by
// pos * base^(-2p/R) (RoFormer's rotation).  The compressed entries get theirs
// in the compressor's epilogue and the output its inverse in the attention
// epilogue; this kernel serves the rows those two do not produce.
//
// Elementwise and HBM-bound (R/D of each row is read and written).  One
// workgroup per (sequence, position): the R/2 angles of the position are
// formed once into LDS and serve all H rows of that position; each
// thread then rotates 8 consecutive elements (four pairs) per step with one
// 16-byte (bf16) or two 16-byte (fp32) loads and stores.
#include <cmath>

#include "device.h"
#include "launch.h"

namespace csa {
namespace {

constexpr int kMaxRopeDims = 1024;

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* v);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* v) {
  unpack_bf16x8(*reinterpret_cast<const uint4*>(p), v);
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <typename T>
__device__ __forceinline__ void store8(T* p, const float* v);
template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t* p, const float* v) {
  *reinterpret_cast<uint4*>(p) =
      make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}
template <>
__device__ __forceinline__ void store8<float>(float* p, const float* v) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

template <typename T>
__global__ void __launch_bounds__(256) rope_rows_kernel(RopeArgs a, double log2_base) {
  __shared__ float2 cs[kMaxRopeDims / 2];
  const int64_t row = blockIdx.x;   // b * T + t
  const int64_t pos = a.pos0 + row % a.T;
  const int R = a.dims, half = R / 2, per = R / 8;
  for (int p = threadIdx.x; p < half; p += blockDim.x) {
    float c, s;
    rope_cos_sin(a.inverse ? -pos : pos, p, R, log2_base, c, s);
    cs[p] = make_float2(c, s);
  }
  __syncthreads();
  T* base = static_cast<T*>(a.x) + row * a.H * a.D + (a.D - R);
  const int64_t items = a.H * per;
  for (int64_t it = threadIdx.x; it < items; it += blockDim.x) {
    const int64_t h = it / per;
    const int ch = static_cast<int>(it % per);
    T* p = base + h * a.D + ch * 8;
    float v[8];
    load8<T>(p, v);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float2 k = cs[ch * 4 + q];
      rope_pair(v[2 * q], v[2 * q + 1], k.x, k.y);
    }
    store8<T>(p, v);
  }
}

}  // namespace

hipError_t launch_rope(const RopeArgs& a, hipStream_t s) {
  if (a.B == 0 || a.T == 0 || a.H == 0) return hipSuccess;
  const int64_t items = a.H * (a.dims / 8);
  const int threads = items >= 256 ? 256 : (items > 64 ? 128 : 64);
  const dim3 grid(static_cast<uint32_t>(a.B * a.T));
  const double l2b = std::log2(static_cast<double>(a.base));
  if (a.dtype == CSA_F32)
    hipLaunchKernelGGL(rope_rows_kernel<float>, grid, dim3(threads), 0, s, a, l2b);
  else
    hipLaunchKernelGGL(rope_rows_kernel<uint16_t>, grid, dim3(threads), 0, s, a, l2b);
  return hipGetLastError();
}

}  // namespace csa
