// Test-only GPU checks of the library's fast paths against their plain forms:
// the short correctly rounded sequences (opt8_exact.h: sqrt_rn, div_rn)
// against the IEEE operations the compiler emits for sqrtf and '/' (correctly
// rounded under hipcc's defaults, which the Python test confirms on a sample
// of the inputs with numpy), and the bucket-LUT code lookups (opt8_codes.h)
// against the binary searches, on the library's own table image
// (opt8_tables.cpp).  Built in-tree into libexact_check.so; nothing in the
// library loads it.
//
// Every kernel is a grid-stride loop over a 64-bit index range, run to a
// multiple of the grid so that every lane of a wave takes the same iterations
// (the counts are wave ballots); it touches no memory but a mismatch counter
// and a small sample array, whose index is bounds-checked.
#include <cstdint>

#include <hip/hip_runtime.h>

#include "../../precision_optimizer_step_amd/csrc/opt8_codes.h"
#include "../../precision_optimizer_step_amd/csrc/opt8_exact.h"
#include "../../precision_optimizer_step_amd/csrc/opt8_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kGrid = 256 * 16;

// One atomic per wave: lane 0 adds the wave's mismatch count.
__device__ __forceinline__ void count_bad(bool bad, unsigned long long* counter) {
  const uint64_t m = __builtin_amdgcn_ballot_w64(bad);
  if ((threadIdx.x & 63) == 0 && m != 0) atomicAdd(counter, static_cast<unsigned long long>(__popcll(m)));
}

// x = the fp32 with bits lo + i, i < count.
__global__ void __launch_bounds__(kThreads)
sqrt_kernel(uint32_t lo, uint64_t count, unsigned long long* bad, float* sample, uint64_t every, int nsample) {
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  const uint64_t end = (count + stride - 1) / stride * stride;   // whole waves to the end
  for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < end; i += stride) {
    bool mismatch = false;
    if (i < count) {
      const float x = __uint_as_float(lo + static_cast<uint32_t>(i));
      const float got = opt8::sqrt_rn(x);
      const float want = sqrtf(x);
      mismatch = __float_as_uint(got) != __float_as_uint(want);
      if (i % every == 0 && i / every < static_cast<uint64_t>(nsample)) {
        sample[2 * (i / every)] = x;
        sample[2 * (i / every) + 1] = got;
      }
    }
    count_bad(mismatch, bad);
  }
}

// a = 1.f with significand a_first + k * a_stride (k < a_count, mod 2^23),
// d = 1.f with significand j (every j < 2^23): index i = k * 2^23 + j.
__global__ void __launch_bounds__(kThreads)
div_sig_kernel(uint32_t a_first, uint32_t a_stride, uint64_t count, unsigned long long* bad, float* sample,
               uint64_t every, int nsample) {
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  const uint64_t end = (count + stride - 1) / stride * stride;   // whole waves to the end
  for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < end; i += stride) {
    bool mismatch = false;
    if (i < count) {
      const uint32_t k = static_cast<uint32_t>(i >> 23), j = static_cast<uint32_t>(i & 0x7FFFFFu);
      const float a = __uint_as_float(0x3F800000u | ((a_first + k * a_stride) & 0x7FFFFFu));
      const float d = __uint_as_float(0x3F800000u | j);
      const float got = opt8::div_rn(a, d);
      const float want = a / d;
      mismatch = __float_as_uint(got) != __float_as_uint(want);
      if (i % every == 0 && i / every < static_cast<uint64_t>(nsample)) {
        sample[3 * (i / every)] = a;
        sample[3 * (i / every) + 1] = d;
        sample[3 * (i / every) + 2] = got;
      }
    }
    count_bad(mismatch, bad);
  }
}

__device__ __forceinline__ uint64_t splitmix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Random pairs over the ranges the step's range check admits: d = den in
// [2^-60, 2^101), the quotient's exponent in [-99, 100], |a| = |m2| in
// [2^ea_min, 2^127) (the step's check sends a block with a non-zero moment
// below 2^-89 to the plain path), random signs and significands.  Pairs
// outside are skipped and not counted.
__global__ void __launch_bounds__(kThreads)
div_random_kernel(uint64_t seed, uint64_t count, int ea_min, unsigned long long* bad, unsigned long long* checked,
                  float* sample, uint64_t every, int nsample) {
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  const uint64_t end = (count + stride - 1) / stride * stride;   // whole waves to the end
  for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < end; i += stride) {
    bool mismatch = false, in_range = false;
    if (i < count) {
      const uint64_t h0 = splitmix64(seed ^ (i * 0xD1B54A32D192ED03ull));
      const uint64_t h1 = splitmix64(h0);
      const int ed = -60 + static_cast<int>((h0 >> 32) % 161u);   // [-60, 100]
      const int eq = -99 + static_cast<int>((h0 & 0xFFFFFFFFu) % 200u);   // [-99, 100]
      const int ea = ed + eq;
      in_range = ea >= ea_min && ea <= 126;
      if (in_range) {
        const uint32_t sa = static_cast<uint32_t>(h1) & 0x807FFFFFu;   // sign and significand
        const uint32_t sd = static_cast<uint32_t>(h1 >> 32) & 0x007FFFFFu;
        const float a = __uint_as_float(sa | (static_cast<uint32_t>(ea + 127) << 23));
        const float d = __uint_as_float(sd | (static_cast<uint32_t>(ed + 127) << 23));
        const float got = opt8::div_rn(a, d);
        const float want = a / d;
        mismatch = __float_as_uint(got) != __float_as_uint(want);
        if (i % every == 0 && i / every < static_cast<uint64_t>(nsample)) {
          sample[3 * (i / every)] = a;
          sample[3 * (i / every) + 1] = d;
          sample[3 * (i / every) + 2] = got;
        }
      }
    }
    count_bad(mismatch, bad);
    const uint64_t m = __builtin_amdgcn_ballot_w64(in_range);
    if ((threadIdx.x & 63) == 0 && m != 0) atomicAdd(checked, static_cast<unsigned long long>(__popcll(m)));
  }
}

// Code lookups for every n with bits lo + i (i < count), on the table image
// staged in LDS as the step kernels stage it.  which: 0 signed nearest (LUT vs
// binary search), 1 unsigned nearest, 2 signed stochastic, 3 unsigned
// stochastic (random 16-bit draw per n from a hash of (seed, i)).  Samples are
// (bits(n), draw, code) triples.
__global__ void __launch_bounds__(kThreads)
codes_kernel(const uint4* image, int which, uint32_t lo, uint64_t count, uint64_t seed, unsigned long long* bad,
             uint32_t* sample, uint64_t every, int nsample) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[opt8::kTableBytesSR];
  for (int k = threadIdx.x; k < opt8::kTableBytesSR / 16; k += blockDim.x) reinterpret_cast<uint4*>(lds)[k] = image[k];
  __syncthreads();
  const float* mid_s = reinterpret_cast<const float*>(lds + opt8::kOffMidS);
  const float* mid_u = reinterpret_cast<const float*>(lds + opt8::kOffMidU);
  const float* pair_s = reinterpret_cast<const float*>(lds + opt8::kOffPairS);
  const float* pair_u = reinterpret_cast<const float*>(lds + opt8::kOffPairU);
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  const uint64_t end = (count + stride - 1) / stride * stride;   // whole waves to the end
  for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < end; i += stride) {
    bool mismatch = false;
    if (i < count) {
      const uint32_t bits = lo + static_cast<uint32_t>(i);
      const float n = __uint_as_float(bits);
      const uint32_t r16 = static_cast<uint32_t>(splitmix64(seed ^ i) >> 48);
      uint32_t got = 0, want = 0;
      if (which == 0) {
        got = opt8::code_s(n, lds, mid_s);
        want = opt8::code_search(n, mid_s);
      } else if (which == 1) {
        got = opt8::code_u(n, lds, mid_u);
        want = opt8::code_search(n, mid_u);
      } else if (which == 2) {
        got = opt8::code_sr<true>(n, lds, r16);
        want = opt8::code_sr_search(n, pair_s, r16);
      } else {
        got = opt8::code_sr<false>(n, lds, r16);
        want = opt8::code_sr_search(n, pair_u, r16);
      }
      mismatch = got != want;
      if (i % every == 0 && i / every < static_cast<uint64_t>(nsample)) {
        sample[3 * (i / every)] = bits;
        sample[3 * (i / every) + 1] = r16;
        sample[3 * (i / every) + 2] = got;
      }
    }
    count_bad(mismatch, bad);
  }
}

struct Device {
  unsigned long long* counters = nullptr;   // [0] mismatches, [1] pairs checked
  float* sample = nullptr;
  int nsample = 0;
  int width = 0;
  bool ok = false;

  Device(int n, int w) : nsample(n), width(w) {
    ok = hipMalloc(&counters, 2 * sizeof(unsigned long long)) == hipSuccess &&
         hipMemset(counters, 0, 2 * sizeof(unsigned long long)) == hipSuccess &&
         hipMalloc(&sample, sizeof(float) * static_cast<size_t>(w) * (n > 0 ? n : 1)) == hipSuccess &&
         hipMemset(sample, 0, sizeof(float) * static_cast<size_t>(w) * (n > 0 ? n : 1)) == hipSuccess;
  }
  ~Device() {
    if (counters) (void)hipFree(counters);
    if (sample) (void)hipFree(sample);
  }
  // copies the results back; -1 on any HIP error
  int64_t finish(float* sample_out, unsigned long long* checked_out) {
    unsigned long long c[2] = {0, 0};
    if (hipGetLastError() != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(c, counters, sizeof c, hipMemcpyDeviceToHost) != hipSuccess)
      return -1;
    if (sample_out && nsample > 0 &&
        hipMemcpy(sample_out, sample, sizeof(float) * static_cast<size_t>(width) * nsample, hipMemcpyDeviceToHost) !=
            hipSuccess)
      return -1;
    if (checked_out) *checked_out = c[1];
    return static_cast<int64_t>(c[0]);
  }
};

uint64_t every_of(uint64_t count, int nsample) {
  const uint64_t e = nsample > 0 ? count / static_cast<uint64_t>(nsample) : count;
  return e > 0 ? e : 1;
}

}  // namespace

// Mismatches of sqrt_rn against sqrtf over the fp32 bit patterns lo..hi
// (inclusive); sample_out receives nsample (x, sqrt_rn(x)) pairs evenly spaced
// over the range.  -1 on a HIP error.
extern "C" int64_t exact_check_sqrt(uint32_t lo, uint32_t hi, float* sample_out, int nsample) {
  if (hi < lo || nsample < 0) return -1;
  const uint64_t count = static_cast<uint64_t>(hi) - lo + 1;
  Device dev(nsample, 2);
  if (!dev.ok) return -1;
  hipLaunchKernelGGL(sqrt_kernel, dim3(kGrid), dim3(kThreads), 0, 0, lo, count, dev.counters, dev.sample,
                     every_of(count, nsample), nsample);
  return dev.finish(sample_out, nullptr);
}

// Mismatches of div_rn against '/' for a_count dividend significands
// (a_first + k * a_stride) times every divisor significand, both in [1, 2);
// sample_out receives nsample (a, d, div_rn(a, d)) triples.
extern "C" int64_t exact_check_div_significands(uint32_t a_first, uint32_t a_stride, uint32_t a_count,
                                                float* sample_out, int nsample) {
  if (nsample < 0) return -1;
  const uint64_t count = static_cast<uint64_t>(a_count) << 23;
  Device dev(nsample, 3);
  if (!dev.ok) return -1;
  hipLaunchKernelGGL(div_sig_kernel, dim3(kGrid), dim3(kThreads), 0, 0, a_first, a_stride, count, dev.counters,
                     dev.sample, every_of(count, nsample), nsample);
  return dev.finish(sample_out, nullptr);
}

// Mismatches of div_rn against '/' over `count` random pairs in the step's
// ranges, dividends down to 2^ea_min; *checked receives the number of pairs
// inside the ranges.
extern "C" int64_t exact_check_div_random(uint64_t seed, uint64_t count, int ea_min, unsigned long long* checked,
                                          float* sample_out, int nsample) {
  if (nsample < 0) return -1;
  Device dev(nsample, 3);
  if (!dev.ok) return -1;
  if (ea_min < -126 || ea_min > 126) return -1;
  hipLaunchKernelGGL(div_random_kernel, dim3(kGrid), dim3(kThreads), 0, 0, seed, count, ea_min, dev.counters,
                     dev.counters + 1, dev.sample, every_of(count, nsample), nsample);
  return dev.finish(sample_out, checked);
}

// Mismatches of the LUT code lookup against the binary search over the fp32
// bit patterns lo..hi (which: 0 signed, 1 unsigned, 2 signed stochastic, 3
// unsigned stochastic); the table image is built by the library's own builder.
// sample_out receives nsample (bits(n), draw, code) triples.  -1 on a HIP
// error, -2 if the table image fails its construction check.
extern "C" int64_t exact_check_codes(int which, uint32_t lo, uint32_t hi, uint64_t seed, uint32_t* sample_out,
                                     int nsample) {
  if (hi < lo || nsample < 0 || which < 0 || which > 3) return -1;
  static uint8_t image[opt8::kTableBytesSR] __attribute__((aligned(16)));
  if (!opt8::build_table_image(image)) return -2;
  uint4* dimage = nullptr;
  if (hipMalloc(&dimage, sizeof image) != hipSuccess) return -1;
  if (hipMemcpy(dimage, image, sizeof image, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(dimage);
    return -1;
  }
  const uint64_t count = static_cast<uint64_t>(hi) - lo + 1;
  int64_t rc = -1;
  {
    Device dev(nsample, 3);
    if (dev.ok) {
      hipLaunchKernelGGL(codes_kernel, dim3(kGrid), dim3(kThreads), 0, 0, dimage, which, lo, count, seed,
                         dev.counters, reinterpret_cast<uint32_t*>(dev.sample), every_of(count, nsample), nsample);
      rc = dev.finish(reinterpret_cast<float*>(sample_out), nullptr);
    }
  }
  (void)hipFree(dimage);
  return rc;
}
