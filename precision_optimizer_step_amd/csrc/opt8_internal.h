// Internal interface between the host side (opt8_host.cpp) and the gfx950
// kernels (opt8_kernels.hip) of libopt8.  Not part of the public ABI.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace opt8 {

constexpr int kBlock = 2048;        // elements per quantisation block
constexpr int kCodes = 256;

// One tensor as the kernels see it.  block_begin is the prefix sum of block
// counts over the list of one launch, so a launch walks blocks 0..total-1.
struct DevTensor {
  uint16_t* param;
  const uint16_t* grad;
  void* m;
  void* v;
  float* amax_m;
  float* amax_v;
  int64_t numel;
  int64_t index_base;
  int64_t block_begin;
  uint32_t tensor_id;
  uint32_t nblocks;
};
static_assert(sizeof(DevTensor) == 80, "descriptor layout");

// Scalars of one step, computed on the host in double and rounded once to fp32.
struct StepScalars {
  float beta1, beta2, w1, w2, eps, step_size, rbc2, lrwd, lr;
  uint32_t seed_lo, seed_hi, step_lo;
  int32_t param_round;   // 0 stochastic, 1 nearest-even
};

// Update rules sharing the state machinery.
enum Algo : int { kAdamW = 0, kLion = 1, kMomentum = 2 };

// Host-built lookup tables, uploaded once per device and staged by every
// workgroup into LDS with the same byte layout:
//   [0, 1024)      signed codebook (fp32[256], ascending)
//   [1024, 2048)   signed midpoints (fp32[255], then +inf)
//   [2048, 3072)   unsigned codebook
//   [3072, 4096)   unsigned midpoints (fp32[255], then +inf)
//   signed code LUT (u8) at byte k for the key k = sortable(n) >> 17, where
//                  sortable(n) flips the sign bit of n >= 0 and every bit of
//                  n < 0, so keys grow with n; keys of |n| < 2 span
//                  [kKeySLo, kKeySHi].
//   unsigned code LUT (u8) at byte k + kOffLutU for the key
//                  k = max(bits(n) >> 16, kKeyLo) of n >= 0 (magnitudes below
//                  2^-27 share the lowest bucket); keys of n < 2 end at kKeyHi.
// Each entry is the code of the smallest value of its bucket (the values
// sharing a key).  No bucket holds more than one midpoint (checked when the
// tables are built), so code = lut + (mid[lut] < n) exactly.
constexpr uint32_t kKeySLo = 0x1FFFu;       // sortable(-2) >> 17
constexpr uint32_t kKeySHi = 0x6000u;       // sortable(+2) >> 17
constexpr uint32_t kKeyLo = 100u << 7;      // |n| < 2^-27 share the lowest bucket
constexpr uint32_t kKeyHi = 0x3FFFu;        // last key below 2.0
constexpr int kLutSN = static_cast<int>(kKeySHi - kKeySLo + 1);
constexpr int kLutN = static_cast<int>(kKeyHi - kKeyLo + 1);
constexpr int kOffCbS = 0, kOffMidS = 1024, kOffCbU = 2048, kOffMidU = 3072;
constexpr int kOffLutSBytes = static_cast<int>(kKeySLo);   // first byte of the signed LUT
constexpr int kOffLutUBytes = (kOffLutSBytes + kLutSN + 15) / 16 * 16;
constexpr int kOffLutU = kOffLutUBytes - static_cast<int>(kKeyLo);   // address = key + kOffLutU
constexpr int kTableBytes = (kOffLutUBytes + kLutN + 15) / 16 * 16;

enum class Kind : int { k8bit = 0, kBf16 = 1, kFp32 = 2, k8bitTail = 3 };

// Kernel side (opt8_kernels.hip).
hipError_t upload_tables(const uint8_t* host_tables);   // kTableBytes, to the current device
hipError_t launch_step(Kind kind, int algo, const DevTensor* dev_list, int ntensors,
                       int64_t total_blocks, const StepScalars& sc, hipStream_t stream, int grid_cap);
// Workgroups per CU that the kernel of this kind and algorithm can keep resident.
int occupancy_per_cu(Kind kind, int algo);

}  // namespace opt8
