// Streaming-read probe: the HBM read rate a plain, perfectly coalesced read reaches on this device.
// It is the practical ceiling the decode's page gather is compared against (the published 8 TB/s
// is a peak no read pattern reaches).  Not part of the attention path.
#include <hip/hip_runtime.h>

#include "nvkv_launch.h"

namespace nvkv {

constexpr unsigned kProbeMagic = 0x9E3779B9u;

// Grid-stride 16-byte loads, one per thread per round; the words are folded into one per thread
// and written only if the fold equals kProbeMagic, so the loads stay live and nothing else is written.
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ p, size_t n, unsigned* sink) {
  unsigned acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == kProbeMagic) *sink = acc;
}

hipError_t launch_read_probe(const void* buf, size_t bytes, unsigned* sink, int workgroups, hipStream_t stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace nvkv
