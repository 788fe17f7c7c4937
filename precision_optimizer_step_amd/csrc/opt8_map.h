// The block map of a cached descriptor list, filled on the device (opt8_map.hip).
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

#include "opt8_internal.h"

namespace opt8 {

// For the n entries of the 8-bit full-block sub-list at `list` (device memory),
// writes map[b] = e for every block b of entry e (block_begin .. block_begin +
// nblocks - 1, a gap-free numbering from 0), queued on `stream` after whatever
// wrote the descriptors there.
hipError_t launch_block_map(const DevTensor* list, int n, uint32_t* map, hipStream_t stream);

}  // namespace opt8
