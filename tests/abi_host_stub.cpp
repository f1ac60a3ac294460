// Host-only stand-ins for the kernel launchers and the one HIP runtime call
// the C-ABI layer makes, so that its host side (capi.cpp and validate.h) can
// be built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and
// driven by the argument-validation tests on a machine without a GPU.  Every
// launcher reports success and touches no memory.
#include "launch.h"

namespace csa {
hipError_t launch_compress(const CompressArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_compress_batch(const CompressArgs*, int, hipStream_t) { return hipSuccess; }
hipError_t launch_compress_paged(const CompressPagedArgs*, int, hipStream_t) { return hipSuccess; }
hipError_t launch_index(const IndexArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_index_jobs(const IndexArgs&, const CompressArgs*, int, int64_t, hipStream_t) { return hipSuccess; }
hipError_t launch_topk(const TopkArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_topk_jobs(const TopkArgs&, const CompressArgs*, int, hipStream_t) { return hipSuccess; }
hipError_t launch_index_pool(const IndexPoolArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_attn(const AttnArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_attn_jobs(const AttnArgs&, const CompressArgs&, int64_t, hipStream_t) { return hipSuccess; }
hipError_t launch_rope(const RopeArgs&, hipStream_t) { return hipSuccess; }
hipError_t attn_static_scratch(void** ptr) {
  *ptr = nullptr;
  return hipSuccess;
}
}  // namespace csa

extern "C" const char* hipGetErrorString(hipError_t) { return "host stub"; }
