// Block map of a cached descriptor list, filled on the device from the
// descriptors just uploaded: for every full 8-bit block, the entry of its
// sub-list that holds it (the full-block kernels read it instead of searching
// the descriptors).  Filling it here rather than on the host saves the host
// a pass over 4 bytes per block and their copy (13 MB for a 6.7B-parameter
// list) whenever a list is uploaded.
#include <algorithm>

#include "opt8_map.h"

namespace opt8 {
namespace {

// Workgroup e (and e + grid, ...) writes entry e's blocks, its threads striding over them.
__global__ void __launch_bounds__(256)
block_map_kernel(const DevTensor* __restrict__ list, int n, uint32_t* __restrict__ map) {
  for (int e = static_cast<int>(blockIdx.x); e < n; e += static_cast<int>(gridDim.x)) {
    const int64_t b0 = list[e].block_begin;
    const uint32_t nb = list[e].nblocks;
    for (uint32_t i = threadIdx.x; i < nb; i += blockDim.x) map[b0 + i] = static_cast<uint32_t>(e);
  }
}

}  // namespace

hipError_t launch_block_map(const DevTensor* list, int n, uint32_t* map, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int grid = std::min(n, 16384);
  hipLaunchKernelGGL(block_map_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, list, n, map);
  return hipGetLastError();
}

}  // namespace opt8
