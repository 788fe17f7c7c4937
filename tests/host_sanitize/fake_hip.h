// State of the host-only HIP stand-in (fake_hip.cpp), read by the driver.
#pragma once

#include <cstdint>
#include <vector>

#include "opt8_internal.h"

namespace fake {

struct Launch {
  int kind = 0, algo = 0, n = 0, num_cu = 0, resident = 0;
  const void* list = nullptr;
  int64_t total_blocks = 0, numel = 0;
  opt8::StepScalars sc{};
  std::vector<uint32_t> ids;
  bool ok = true;
  bool has_map = false;
};

struct State {
  bool have_device = true;
  int device = 0;
  bool capturing = false;
  bool fail_malloc = false;
  long mallocs = 0, frees = 0, uploads = 0, events = 0, event_syncs = 0, stream_waits = 0;
  long host_mallocs = 0, scratch_queries = 0, map_fills = 0;
  std::vector<std::pair<void*, size_t>> device_live;   // hipMalloc'd buffers not yet freed
  size_t device_bytes = 0, device_bytes_peak = 0;
  const void* scratch_lo = nullptr;   // extent of the stand-in descriptor scratch
  const void* scratch_hi = nullptr;
  long table_uploads = 0;
  // stream-order model: every upload and event record takes the next
  // sequence number; synchronising on an event completes everything up to
  // its number.  An upload from a pinned staging buffer whose previous upload
  // has not completed is a reuse violation (the host would have overwritten
  // the buffer while the copy could still be reading it).
  long seq = 0, completed = 0, reuse_violations = 0;
  int fail_launch_kind = -1;   // launch_step of this kind fails
  std::vector<std::pair<const void*, long>> pinned;   // staging buffer, seq of its last upload
  uint32_t table_sum = 0;
  std::vector<Launch> launches;
};

extern State g;

}  // namespace fake
