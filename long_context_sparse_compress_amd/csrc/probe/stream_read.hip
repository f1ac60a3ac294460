// Measurement helper, built into its own library (libcsa_probe.so) and not
// part of the C ABI of include/csa.h: a plain streaming read of a device
// buffer -- 16-byte loads, four in flight per thread, grid-stride -- that
// folds the bytes into one word per thread.  It is the reference point for
// the read bandwidth a kernel that only streams HBM attains on this machine.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ void __launch_bounds__(256) stream_read_kernel(const uint4* __restrict__ p, int64_t n4,
                                                         uint32_t* __restrict__ out) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t nt = static_cast<int64_t>(gridDim.x) * 256;
  uint32_t acc = 0;
  for (int64_t i = tid; i < n4; i += 4 * nt) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = i + u * nt;
      v[u] = j < n4 ? p[j] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  out[tid] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16) from p with `grid` workgroups of 256
// threads; out holds grid * 256 words.  Returns a hipError_t.
extern "C" int csa_probe_stream_read(const void* p, int64_t bytes, uint32_t* out, int grid, void* stream) {
  if (bytes < 0 || bytes % 16 != 0 || grid < 1 || !p || !out) return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(p), bytes / 16, out);
  return static_cast<int>(hipGetLastError());
}
