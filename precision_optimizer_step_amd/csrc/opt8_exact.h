// Correctly rounded fp32 square root and division in short gfx950 instruction
// sequences, valid on stated input ranges (the step kernels check each block
// against them and fall back to the IEEE operations outside).  A header of its
// own so that the exhaustive GPU check in the tests runs these very functions.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace opt8 {

// Correctly rounded sqrt for x == +0 or 2^-96 <= x < inf: one Newton step
// from the hardware reciprocal square root, s = s0 + (x - s0^2) * y/2 with
// s0 = x*y, the residual exact in an fma.  Checked against the correctly
// rounded root for every fp32 in [2^-96, inf) on gfx950 (v_sqrt_f32 alone is
// one ulp off for about 15% of them).  Below 2^-96 the residual can underflow;
// the input floor 2^-126 (an integer max on the bits, equal to the float max
// for x >= +0) keeps y finite so that x = 0 gives 0, and a negative x keeps its
// bits, so its root is NaN as the IEEE one.  Outside that range the plain
// sqrtf is used.
__device__ __forceinline__ float sqrt_rn(float x) {
  const float y = __builtin_amdgcn_rsqf(__uint_as_float(max(__float_as_uint(x), 0x00800000u)));
  const float s0 = x * y;
  const float h = 0.5f * y;
  const float r = __builtin_fmaf(-s0, s0, x);
  return __builtin_fmaf(r, h, s0);
}

// Correctly rounded a / d by a refined reciprocal and one residual
// correction, valid when a == +-0, or 2^-100 < |a/d| and |a| >= 2^-89 with d
// normal and nothing near overflow (no operand or residual leaves the normal
// range; for |a| near 2^-126 the residual would).  Checked against IEEE
// division on gfx950 for every pair of significands (a, d in [1, 2), 2^46
// pairs) and for 1.7e10 random pairs across the exponent ranges of the step;
// the unrefined reciprocal fails both.  The residual is kept negated so a
// zero quotient keeps the sign of a.
__device__ __forceinline__ float div_rn(float a, float d) {
  const float r0 = __builtin_amdgcn_rcpf(d);
  const float e = __builtin_fmaf(-d, r0, 1.0f);
  const float r = __builtin_fmaf(e, r0, r0);
  const float q0 = a * r;
  const float t0 = __builtin_fmaf(d, q0, -a);
  return __builtin_fmaf(-t0, r, q0);
}

}  // namespace opt8
