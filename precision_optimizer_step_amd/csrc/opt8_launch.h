// Launch size of the step kernels (host code, kept apart so that the host
// tests check it).  kWavesPerGroup waves per workgroup.
#pragma once

#include <algorithm>
#include <cstdint>

#include "opt8_internal.h"

namespace opt8 {

constexpr int kWavesPerGroup = 4;

// Launch size.  A grid of only the workgroups that fit at once would give each
// wave a fixed share of the blocks; a SIMD issues from its oldest wave first,
// so its waves finish their shares far apart (on the 6.7B list the first
// third of the waves is done at 62% of the kernel's time, the second at 80%)
// and the SIMD runs the rest with one or two waves instead of three.  The
// grid is therefore several times the resident count: the dispatcher starts a
// new workgroup on a CU as soon as one finishes, and every SIMD keeps its
// full set of waves until the last few hundred microseconds.  Each new
// workgroup pays for staging the tables and finding its first tensor, so the
// count per CU is the measured best of sweeps from 6 to 768 per CU for each
// family on the 6.7B, 2.7B, 1.5B and 350M lists and a list of 30,000 small
// tensors (two-state 8-bit 192, Lion 96, momentum 384 but 96 with the state
// rounded stochastically, bf16 and fp32 state 384; the last partial blocks,
// one short block per tensor, keep the resident grid), and a wave gets at
// least two blocks (one in the fp32-state kernels, whose tensors have one or
// two blocks).
template <Kind K, int A, bool SS = false>
constexpr int groups_per_cu() {
  if constexpr (K == Kind::k8bit) return A == kLion ? 96 : (A == kMomentum ? (SS ? 96 : 384) : 192);
  else if constexpr (K == Kind::kBf16 || K == Kind::kFp32) return 384;
  else return 0;
}

template <Kind K, int A, bool SS = false>
int64_t launch_groups(int64_t total_blocks, int num_cu, int resident) {
  const int64_t one_block_per_wave = (total_blocks + kWavesPerGroup - 1) / kWavesPerGroup;
  int64_t grid = std::min<int64_t>(one_block_per_wave, resident);
  if (groups_per_cu<K, A, SS>() > 0) {
    const int64_t min_blocks = K == Kind::kFp32 ? 1 : 2;
    const int64_t by_work = (total_blocks + kWavesPerGroup * min_blocks - 1) / (kWavesPerGroup * min_blocks);
    grid = std::max(grid, std::min<int64_t>(static_cast<int64_t>(num_cu) * groups_per_cu<K, A, SS>(), by_work));
  }
  if (grid >= 64) grid &= ~int64_t{31};   // a multiple of 32 keeps the XCD-aware wave numbering
  return std::max<int64_t>(grid, 1);
}

}  // namespace opt8
