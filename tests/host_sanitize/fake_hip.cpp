// A host-only stand-in for the HIP runtime calls and the kernel-side functions
// that opt8_host.cpp uses, so the library's host code (codebook and LUT
// construction, validation, the per-device descriptor cache, the scalar
// prologue, launch planning) can run under AddressSanitizer and UBSan on a
// machine without a GPU.  "Device" memory is host memory; launches are
// recorded and their descriptor lists checked the way the kernels walk them.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "fake_hip.h"
#include "opt8_map.h"

namespace fake {
State g;
}

using fake::g;

extern "C" {

hipError_t hipGetDevice(int* device) {
  if (!g.have_device) return hipErrorNoDevice;
  *device = g.device;
  return hipSuccess;
}

hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t, int) {
  *value = 256;
  return hipSuccess;
}

hipError_t hipDeviceSynchronize(void) { return hipSuccess; }

// an event holds the sequence number of its last record (0: never recorded)
hipError_t hipEventCreateWithFlags(hipEvent_t* event, unsigned) {
  *event = reinterpret_cast<hipEvent_t>(new long(0));
  ++g.events;
  return hipSuccess;
}

hipError_t hipEventRecord(hipEvent_t event, hipStream_t) {
  *reinterpret_cast<long*>(event) = ++g.seq;
  return hipSuccess;
}

hipError_t hipEventSynchronize(hipEvent_t event) {
  g.completed = std::max(g.completed, *reinterpret_cast<long*>(event));
  ++g.event_syncs;
  return hipSuccess;
}

hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t event, unsigned) {
  (void)*reinterpret_cast<long*>(event);
  ++g.stream_waits;
  return hipSuccess;
}

hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus* status) {
  *status = g.capturing ? hipStreamCaptureStatusActive : hipStreamCaptureStatusNone;
  return hipSuccess;
}

hipError_t hipMalloc(void** ptr, size_t size) {
  if (g.fail_malloc) return hipErrorOutOfMemory;
  *ptr = std::malloc(size);
  ++g.mallocs;
  g.device_live.emplace_back(*ptr, size);
  g.device_bytes += size;
  g.device_bytes_peak = std::max(g.device_bytes_peak, g.device_bytes);
  return hipSuccess;
}

hipError_t hipFree(void* ptr) {
  for (size_t i = 0; i < g.device_live.size(); ++i)
    if (g.device_live[i].first == ptr) {
      g.device_bytes -= g.device_live[i].second;
      g.device_live.erase(g.device_live.begin() + static_cast<long>(i));
      break;
    }
  std::free(ptr);
  ++g.frees;
  return hipSuccess;
}

hipError_t hipHostMalloc(void** ptr, size_t size, unsigned) {
  *ptr = std::malloc(size);
  ++g.host_mallocs;
  g.pinned.emplace_back(*ptr, 0L);
  return hipSuccess;
}

hipError_t hipHostFree(void* ptr) {
  for (size_t i = 0; i < g.pinned.size(); ++i)
    if (g.pinned[i].first == ptr) {
      if (g.pinned[i].second > g.completed) ++g.reuse_violations;   // freed under a copy
      g.pinned.erase(g.pinned.begin() + static_cast<long>(i));
      break;
    }
  std::free(ptr);
  return hipSuccess;
}

hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind, hipStream_t) {
  std::memcpy(dst, src, bytes);
  ++g.uploads;
  for (auto& p : g.pinned)
    if (p.first == src) {
      if (p.second > g.completed) ++g.reuse_violations;
      p.second = ++g.seq;
    }
  return hipSuccess;
}

const char* hipGetErrorString(hipError_t) { return "error from the host-only HIP stand-in"; }

}  // extern "C"

namespace opt8 {

hipError_t upload_tables(const uint8_t* host_tables) {
  // read every byte of the image the kernels would stage (ASan checks the extent)
  uint32_t sum = 0;
  for (int i = 0; i < kTableBytesSR; ++i) sum += host_tables[i];
  g.table_sum = sum;
  ++g.table_uploads;
  return hipSuccess;
}

hipError_t launch_step(Kind kind, int algo, const DevTensor* list, int n, int64_t total_blocks,
                       const StepScalars& sc, hipStream_t, int num_cu, int resident, const uint32_t* map) {
  if (static_cast<int>(kind) == g.fail_launch_kind) return hipErrorInvalidValue;
  fake::Launch L;
  L.list = list;
  L.kind = static_cast<int>(kind);
  L.algo = algo;
  L.n = n;
  L.total_blocks = total_blocks;
  L.sc = sc;
  L.num_cu = num_cu;
  L.resident = resident;
  // the kernels find a block's tensor from block_begin and walk nblocks: the
  // numbering must be a gap-free prefix sum ending at total_blocks
  int64_t b = 0;
  for (int i = 0; i < n; ++i) {
    if (list[i].block_begin != b) L.ok = false;
    if (list[i].nblocks == 0) L.ok = false;
    // the last-partial-block kernels read entry b for block b; the short-block
    // kernel takes the partial blocks of at most kShortTail elements, the
    // other the rest
    if ((kind == Kind::k8bitTail || kind == Kind::k8bitShort) && list[i].nblocks != 1) L.ok = false;
    const int64_t rest = list[i].numel % kBlock;
    if (kind == Kind::k8bitShort && (rest < 1 || rest > kShortTail)) L.ok = false;
    if (kind == Kind::k8bitTail && rest <= kShortTail) L.ok = false;
    b += list[i].nblocks;
    L.numel += list[i].numel;
    L.ids.push_back(list[i].tensor_id);
  }
  if (b != total_blocks) L.ok = false;
  // the block map, where given (8-bit full blocks only): block -> the entry holding it
  L.has_map = map != nullptr;
  if (map) {
    if (kind != Kind::k8bit) L.ok = false;
    int64_t blk = 0;
    for (int i = 0; i < n; ++i)
      for (uint32_t k = 0; k < list[i].nblocks; ++k, ++blk)
        if (map[blk] != static_cast<uint32_t>(i)) L.ok = false;
  }
  g.launches.push_back(L);
  return hipSuccess;
}

int occupancy_per_cu(Kind, int, bool) { return 3; }

// The block-map fill, on the host: the stand-in's device memory is host memory, so ASan
// checks that the map fits the slot the library reserved for it.
hipError_t launch_block_map(const DevTensor* list, int n, uint32_t* map, hipStream_t) {
  ++g.map_fills;
  for (int e = 0; e < n; ++e)
    for (uint32_t i = 0; i < list[e].nblocks; ++i) map[list[e].block_begin + i] = static_cast<uint32_t>(e);
  return hipSuccess;
}

// The stand-in for the device's descriptor scratch: a static host array of
// the same size, so ASan checks every descriptor written into it.
hipError_t scratch_address(DevTensor** out) {
  static DevTensor fake_scratch[kScratchDescs];
  *out = fake_scratch;
  g.scratch_lo = fake_scratch;
  g.scratch_hi = fake_scratch + kScratchDescs;
  ++g.scratch_queries;
  return hipSuccess;
}

}  // namespace opt8
