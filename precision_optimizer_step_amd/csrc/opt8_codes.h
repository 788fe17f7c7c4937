// Requantisation of a normalised moment n to its 8-bit code, on the device:
// the nearest codebook entry (ties to the lower code) or, with stochastic
// state rounding, one of the two entries around n.  The plain forms are
// binary searches over the sorted tables; the fast forms read the bucket LUTs
// of the table image (layout in opt8_internal.h) and are equal to the plain
// ones for every finite -2 < n < 2 (checked exhaustively by the GPU tests).
// A header of its own so that the test-only check runs these very functions.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

#include "opt8_internal.h"

namespace opt8 {

// Number of midpoints strictly below n (255 sorted midpoints): the nearest
// codebook entry, ties to the lower code; NaN sorts above everything.
__device__ __forceinline__ uint32_t code_search(float n, const float* mid) {
  uint32_t idx = 0;
#pragma unroll
  for (uint32_t s = 128; s >= 1; s >>= 1) idx += (mid[idx + s - 1] < n) ? s : 0u;
  return (n != n) ? 255u : idx;
}

// Stochastic state rounding, plain path: k = the entry at or below n (binary
// search over the (entry, gap weight) pairs, clamped to [0, 254]), then the
// upper entry iff fp32(fp32(n - C[k]) * W[k]) > r16; NaN stores 255.
__device__ __forceinline__ uint32_t code_sr_search(float n, const float* pair, uint32_t r16) {
  uint32_t pos = 0;   // #{k <= 254 : C[k] <= n}
#pragma unroll
  for (uint32_t s = 128; s >= 1; s >>= 1) pos += (pair[2 * (pos + s - 1)] <= n) ? s : 0u;
  const uint32_t k = pos > 0 ? pos - 1 : 0u;
  const float f = (n - pair[2 * k]) * pair[2 * k + 1];
  const uint32_t code = k + ((f > static_cast<float>(r16)) ? 1u : 0u);
  return (n != n) ? 255u : code;
}

// Codes through the bucket LUTs: code = lut[key] + (mid[lut[key]] < n).
__device__ __forceinline__ uint32_t code_u(float n, const uint8_t* lds, const float* mid) {
  const uint32_t key = max(__float_as_uint(n) >> 16, kKeyLo);    // 0 <= n < 2
  const uint32_t c = lds[key];
  return c + ((mid[c] < n) ? 1u : 0u);
}

__device__ __forceinline__ uint32_t code_s(float n, const uint8_t* lds, const float* mid) {
  const uint32_t c = lds[__float_as_uint(n) >> 17];              // -2 < n < 2
  return c + ((mid[c] < n) ? 1u : 0u);
}

// Stochastic state rounding through the floor LUTs (finite -2 < n < 2): the
// entry at or below n is floor + (C[floor + 1] <= n); floors stop at 254 and
// the last pair's entry is +inf, so k stays in [0, 254].  With kKeepK the
// compiler is kept from rebuilding k for the final sum as floor + the first
// compare + the second, which keeps a 0/1 copy of the first compare and costs
// one more instruction per code (the two-moment kernels measured 1.3% faster
// with k kept, the one-moment ones 0.9% slower).
template <bool kSigned, bool kKeepK = false>
__device__ __forceinline__ uint32_t code_sr(float n, const uint8_t* lds, uint32_t r16) {
  const uint32_t b = __float_as_uint(n);
  const uint32_t key = kSigned ? (b >> 17) : max(b >> 16, kKeyLo);
  const float* pair = reinterpret_cast<const float*>(lds + (kSigned ? kOffPairS : kOffPairU));
  const uint32_t c = lds[kOffFloor + key];
  uint32_t k = c + ((pair[2 * c + 2] <= n) ? 1u : 0u);
  if constexpr (kKeepK) asm("" : "+v"(k));
  const float f = (n - pair[2 * k]) * pair[2 * k + 1];
  return k + ((f > static_cast<float>(r16)) ? 1u : 0u);
}

}  // namespace opt8
