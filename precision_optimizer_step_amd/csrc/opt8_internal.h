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
  float beta1, beta2, w1, w2, eps, step_size, rbc2, lrwd;
  uint32_t seed_lo, seed_hi, step_lo;
  int32_t param_round;   // 0 stochastic, 1 nearest-even
};

// Host-built lookup tables uploaded once per device.  Layout (fp32 words):
// [0,256) signed codebook, [256,512) signed midpoints (255 + padding),
// [512,768) unsigned codebook, [768,1024) unsigned midpoints.
constexpr int kTableWords = 4 * kCodes;

enum class Kind : int { k8bit = 0, kBf16 = 1, kFp32 = 2 };

// Kernel side (opt8_kernels.hip).
hipError_t upload_tables(const float* host_tables);   // to the current device
hipError_t launch_step(Kind kind, const DevTensor* dev_list, int ntensors, int64_t total_blocks,
                       const StepScalars& sc, hipStream_t stream, int grid_cap);
// Workgroups per CU that the kernel of this kind can keep resident.
int occupancy_per_cu(Kind kind);

}  // namespace opt8
