// The table image every step kernel stages in LDS: the signed and unsigned
// codebooks, their midpoints, the code LUTs of the nearest-rounding path and the
// floor LUTs and (entry, gap weight) pairs of the stochastic-state path (layout in
// opt8_internal.h).  Host code, built from the definitions in exact integer
// arithmetic; every LUT is checked against the sorted tables as it is built.
// Compiled into libopt8.so and into the test-only GPU check of the code lookups.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "opt8_internal.h"

namespace opt8 {
namespace {

// Nearest fp32 to num/den (num, den > 0), ties to even, in exact integer
// arithmetic: scale so the quotient has 24 significant bits, round on the
// remainder.
float nearest_f32(uint64_t num, uint64_t den) {
  if (num == 0) return 0.0f;
  using u128 = unsigned __int128;
  const u128 n = num, d = den;
  int s = 0;                                   // value = q * 2^-s
  while ((n << s) < (static_cast<u128>(d) << 23)) ++s;
  while ((n << s) >= (static_cast<u128>(d) << 24)) --s;   // only for values >= 2^24 (never)
  const u128 scaled = n << s;
  u128 q = scaled / d;
  const u128 rem = scaled % d;
  if (2 * rem > d || (2 * rem == d && (q & 1))) ++q;
  if (q == (static_cast<u128>(1) << 24)) { q >>= 1; --s; }
  return std::ldexp(static_cast<float>(static_cast<uint64_t>(q)), -s);
}

uint64_t pow10u(int e) {
  uint64_t r = 1;
  while (e-- > 0) r *= 10;
  return r;
}

// Dynamic tree code, read as: decade E of the magnitude (10^-(E+1), 10^-E] is
// split into 2^F equal steps, F = magnitude_bits - 1 - E, and level k
// (k = 0..2^F-1) is the upper end of step k:
//   (2^F + 9 (k + 1)) / (10^(E+1) 2^F).
// The signed code spends one bit on the sign (magnitude_bits 7) and the
// unsigned code does not (magnitude_bits 8).  Source: "8-bit Optimizers via
// Block-wise Quantization", innovations list (dynamic tree quantization
// extended to unipolar data) and method bullets (non-linear 8-bit code).
void tree_levels(int magnitude_bits, bool negative_too, std::vector<float>& out) {
  for (int e = 0; e < magnitude_bits; ++e) {
    const int f = magnitude_bits - 1 - e;
    const uint64_t steps = 1ull << f;
    for (uint64_t k = 0; k < steps; ++k) {
      const float x = nearest_f32(steps + 9 * (k + 1), pow10u(e + 1) * steps);
      out.push_back(x);
      if (negative_too) out.push_back(-x);
    }
  }
}


// #{k : mid[k] < x} over the 255 midpoints.
int count_below(const float* mid, float x) {
  int c = 0;
  while (c < kCodes - 1 && mid[c] < x) ++c;
  return c;
}

float bits_f32(uint32_t b) {
  float f;
  std::memcpy(&f, &b, 4);
  return f;
}

// #{k : mid[k] < x} is constant on a bucket except at most one step; the LUT
// entry is its value at the bucket's smallest member.  Returns false if a
// bucket holds two midpoints (the lookup would then be wrong).
bool lut_entry(const float* mid, float least, float most, uint8_t& out) {
  const int base = count_below(mid, least);
  const int top = count_below(mid, most);   // the largest count is at the largest member
  out = static_cast<uint8_t>(base);
  return top - base <= 1;
}

// Code LUTs: the signed table keyed by bits(n) >> 17 (a bucket of n >= +0
// grows with its bits, one of n <= -0 shrinks), the unsigned table keyed by
// bits(n) >> 16, clamped below at kKeyLo.
bool build_luts(uint8_t* bytes) {
  const float* mid_s = reinterpret_cast<const float*>(bytes + kOffMidS);
  const float* mid_u = reinterpret_cast<const float*>(bytes + kOffMidU);
  for (uint32_t key = 0; key < kKeySPosEnd; ++key)
    if (!lut_entry(mid_s, bits_f32(key << 17), bits_f32((key << 17) | 0x1FFFFu), bytes[key])) return false;
  for (uint32_t key = kKeySNeg; key < kKeySNegEnd; ++key)
    if (!lut_entry(mid_s, bits_f32((key << 17) | 0x1FFFFu), bits_f32(key << 17), bytes[key])) return false;
  for (uint32_t key = kKeyLo; key <= kKeyHi; ++key) {
    const float least = key == kKeyLo ? 0.0f : bits_f32(key << 16);
    const float most = bits_f32((key << 16) | 0xFFFFu);
    if (!lut_entry(mid_u, least, most, bytes[key])) return false;
  }
  return true;
}

// #{k : table[k] <= x} over the 256 entries.
int count_at_or_below(const float* table, float x) {
  int c = 0;
  while (c < kCodes && table[c] <= x) ++c;
  return c;
}

// Floor LUT entry: the largest entry at or below the bucket's smallest value,
// clamped to [0, 254] (the lower end of the last gap); false if a bucket holds
// two entries.
bool floor_entry(const float* table, float least, float most, uint8_t& out) {
  const int base = std::min(std::max(count_at_or_below(table, least) - 1, 0), kCodes - 2);
  const int top = std::min(std::max(count_at_or_below(table, most) - 1, 0), kCodes - 2);
  out = static_cast<uint8_t>(base);
  return top - base <= 1;
}

// The stochastic-state half of the image: floor LUTs and (entry, gap weight) pairs.
bool build_sr_tables(uint8_t* bytes) {
  const float* cb_s = reinterpret_cast<const float*>(bytes + kOffCbS);
  const float* cb_u = reinterpret_cast<const float*>(bytes + kOffCbU);
  for (uint32_t key = 0; key < kKeySPosEnd; ++key)
    if (!floor_entry(cb_s, bits_f32(key << 17), bits_f32((key << 17) | 0x1FFFFu), bytes[kOffFloor + key]))
      return false;
  for (uint32_t key = kKeySNeg; key < kKeySNegEnd; ++key)
    if (!floor_entry(cb_s, bits_f32((key << 17) | 0x1FFFFu), bits_f32(key << 17), bytes[kOffFloor + key]))
      return false;
  for (uint32_t key = kKeyLo; key <= kKeyHi; ++key) {
    const float least = key == kKeyLo ? 0.0f : bits_f32(key << 16);
    if (!floor_entry(cb_u, least, bits_f32((key << 16) | 0xFFFFu), bytes[kOffFloor + key])) return false;
  }
  // the last pair holds +inf as its entry, so the comparison with the entry
  // after a floor of 254 never moves k past 254
  auto pairs = [&](const float* table, int off) {
    float pr[2 * kCodes];
    for (int k = 0; k < kCodes; ++k) {
      pr[2 * k] = k + 1 < kCodes ? table[k] : INFINITY;
      pr[2 * k + 1] = k + 1 < kCodes
          ? static_cast<float>(65536.0 / (static_cast<double>(table[k + 1]) - static_cast<double>(table[k])))
          : 0.0f;
    }
    std::memcpy(bytes + off, pr, sizeof pr);
  };
  pairs(cb_s, kOffPairS);
  pairs(cb_u, kOffPairU);
  return true;
}

}  // namespace

bool build_table_image(uint8_t* bytes) {
  std::vector<float> s, u;
  tree_levels(7, true, s);
  s.push_back(0.0f);
  s.push_back(nearest_f32(1, 10000000));   // the spare signed string: the 1e-7 level
  tree_levels(8, false, u);
  u.push_back(0.0f);
  std::sort(s.begin(), s.end());
  std::sort(u.begin(), u.end());
  std::memset(bytes, 0, kTableBytesSR);
  auto fill = [&](const std::vector<float>& c, int off_tab, int off_mid) {
    float tab[kCodes], mid[kCodes];
    for (int k = 0; k < kCodes; ++k) tab[k] = c[k];
    for (int k = 0; k + 1 < kCodes; ++k)   // neighbours sum exactly in double
      mid[k] = static_cast<float>((static_cast<double>(c[k]) + static_cast<double>(c[k + 1])) * 0.5);
    mid[kCodes - 1] = INFINITY;
    std::memcpy(bytes + off_tab, tab, sizeof tab);
    std::memcpy(bytes + off_mid, mid, sizeof mid);
  };
  fill(s, kOffCbS, kOffMidS);
  fill(u, kOffCbU, kOffMidU);
  return s.size() == kCodes && u.size() == kCodes && build_luts(bytes) && build_sr_tables(bytes);
}

}  // namespace opt8
