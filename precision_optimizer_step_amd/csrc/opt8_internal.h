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
  int32_t state_round;   // 8-bit state: 0 nearest entry, 1 stochastic between neighbours
};

// Update rules sharing the state machinery.
enum Algo : int { kAdamW = 0, kLion = 1, kMomentum = 2 };

// Host-built lookup tables, uploaded once per device and staged by every
// workgroup into LDS with the same byte layout (every address below is a
// constant, so each lookup is one LDS read with an immediate offset):
//   [0x0000, 0x2000)  signed code LUT (u8) for 0 <= n < 2, at byte bits(n) >> 17
//   [0x2000, 0x2400)  signed codebook (fp32[256], ascending)
//   [0x2400, 0x2800)  signed midpoints (fp32[255], then +inf)
//   [0x2800, 0x2C00)  unsigned codebook
//   [0x2C00, 0x3000)  unsigned midpoints (fp32[255], then +inf)
//   [0x3200, 0x4000)  unsigned code LUT (u8) for 0 <= n < 2, at byte
//                     max(bits(n) >> 16, kKeyLo) (magnitudes below 2^-27
//                     share the lowest bucket)
//   [0x4000, 0x6000)  signed code LUT (u8) for -2 < n <= -0, at byte bits(n) >> 17
// A bucket is the set of values sharing a key (a contiguous interval of
// fp32 values); its entry is the code of its smallest value.  No bucket
// holds more than one midpoint (checked when the tables are built), so
// code = lut + (mid[lut] < n) exactly.
constexpr uint32_t kKeyLo = 100u << 7;      // unsigned key floor: |n| < 2^-27
constexpr uint32_t kKeyHi = 0x3FFFu;        // last unsigned key below 2.0
constexpr uint32_t kKeySPosEnd = 0x2000u;   // signed keys of +0 <= n < 2: [0, kKeySPosEnd)
constexpr uint32_t kKeySNeg = 0x4000u;      // signed keys of -2 < n <= -0: [kKeySNeg, kKeySNegEnd)
constexpr uint32_t kKeySNegEnd = 0x6000u;
constexpr int kOffCbS = 0x2000, kOffMidS = 0x2400, kOffCbU = 0x2800, kOffMidU = 0x2C00;
constexpr int kTableBytes = 0x6000;
static_assert(kKeyLo == 0x3200u && kOffMidU + 1024 <= static_cast<int>(kKeyLo),
              "the unsigned LUT sits at its own keys, after the codebooks");
static_assert(kOffCbS >= static_cast<int>(kKeySPosEnd) && kKeyHi < kKeySNeg, "LUT regions overlap");

// Second half, staged only by the kernels that round the 8-bit state
// stochastically (the same keys, shifted by kOffFloor):
//   [0x6000, 0x8000)  signed floor LUT for 0 <= n < 2 at kOffFloor + (bits(n) >> 17)
//   [0x8000, 0x8800)  signed pairs (C[k], W[k]), k = 0..255, fp32 each
//   [0x8800, 0x9000)  unsigned pairs
//   [0x9200, 0xA000)  unsigned floor LUT at kOffFloor + max(bits(n) >> 16, kKeyLo)
//   [0xA000, 0xC000)  signed floor LUT for -2 < n <= -0 at kOffFloor + (bits(n) >> 17)
// A floor entry is the index of the largest codebook entry at or below the
// bucket's smallest value, clamped to [0, 254]; no bucket holds more than one
// entry (checked), so the entry at or below n is floor + (C[floor + 1] <= n).
// Pair k holds (C[k], W[k]), W[k] = 65536 / (C[k+1] - C[k]) in double rounded
// once to fp32; pair 255 holds (+inf, 0), so k never passes 254.
constexpr int kOffFloor = 0x6000;
constexpr int kOffPairS = 0x8000, kOffPairU = 0x8800;
constexpr int kTableBytesSR = 0xC000;
static_assert(kOffPairU + 2048 <= kOffFloor + static_cast<int>(kKeyLo) &&
              kOffFloor + static_cast<int>(kKeyHi) < kOffFloor + static_cast<int>(kKeySNeg),
              "floor LUT regions overlap the pairs");

// k8bitTail: the last partial blocks of 8-bit tensors longer than kShortTail
// elements, a wave per block; k8bitShort: those of at most kShortTail
// elements, eight blocks per wave (one 8-lane run each).
enum class Kind : int { k8bit = 0, kBf16 = 1, kFp32 = 2, k8bitTail = 3, k8bitShort = 4 };
constexpr int kShortTail = 64;

// Descriptor scratch of the entry point that allocates nothing: a fixed
// device array in opt8_kernels.hip, one copy per device, holding the
// per-kernel descriptor lists of one call (a tensor is at most two entries:
// its full 8-bit blocks and its partial last block).
constexpr int kNoAllocMaxTensors = 4096;
constexpr int kScratchDescs = 2 * kNoAllocMaxTensors;

// Host side (opt8_tables.cpp): fills the kTableBytesSR-byte table image;
// false if a construction check fails (a bucket holding two midpoints).
bool build_table_image(uint8_t* bytes);

// Kernel side (opt8_kernels.hip).
hipError_t upload_tables(const uint8_t* host_tables);   // kTableBytesSR, to the current device
// Device address of the descriptor scratch on the current device (taken once per device).
hipError_t scratch_address(DevTensor** out);
// The 8-bit kinds take the stochastic-state kernels when sc.state_round is set.
// resident: workgroups of that kernel that fit on the device at once (CUs x
// occupancy); the launch size itself is the kernel side's choice.  map: for the
// 8-bit full blocks, block b -> the entry of dev_list holding it (device
// memory, total_blocks entries), or NULL to have the kernels search.
hipError_t launch_step(Kind kind, int algo, const DevTensor* dev_list, int ntensors,
                       int64_t total_blocks, const StepScalars& sc, hipStream_t stream, int num_cu, int resident,
                       const uint32_t* map);
// Workgroups per CU that the kernel of this kind, algorithm and state rounding can keep resident.
int occupancy_per_cu(Kind kind, int algo, bool state_sr);

}  // namespace opt8
