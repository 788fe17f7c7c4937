// Sizes of libopt8's host-side caches (opt8_host.cpp), in a header of their
// own so that the host tests use the same values.
#pragma once

#include <cstddef>

namespace opt8 {

// Tensor lists kept validated and planned, per calling thread.  A training
// loop that steps each parameter group with its own call passes one list per
// group, every step: while the groups fit here, a call costs one compare.
constexpr int kListCache = 1024;

// Descriptor slots per device: device copies of a list's descriptors and
// block map.  While a loop's lists fit, none is uploaded twice and no call
// waits for an earlier step to finish before it can rewrite a slot.
constexpr int kSlotCache = 1024;

// Byte budget of each cache (host bytes of the list cache per thread; device
// bytes of the slots per device, with as many pinned host bytes for their
// staging): beyond it the least recently used entries are dropped, whatever
// their count, so that lists whose buffers move every step cannot pile up.
// The environment variable OPT8_CACHE_MB, read at the first step, replaces it.
constexpr size_t kCacheBytesDefault = size_t{256} << 20;

}  // namespace opt8
