// gfx950 kernels of the fused optimizer steps: AdamW, Lion and SGD with
// momentum over 8-bit block-wise, bf16 (stochastically rounded) or fp32 state.
//
// Work unit: one 2048-element quantisation block per wave64 ("8-bit Optimizers
// via Block-wise Quantization", method bullets: 2048-element blocks normalised
// by their own absolute maximum).  Lane l of the wave owns elements
// r*512 + 8l .. r*512 + 8l + 7 for r = 0..3, so every global access of a wave
// is one contiguous 1 KiB (bf16, 16 B per lane) or 512 B (codes, 8 B per lane)
// segment, and one Philox call per lane, r and stream yields the 8 random
// 16-bit words of those 8 elements.  A block's absmax is a max, reduced across
// the wave with cross-lane (DPP or shuffle) steps, so it is exact and
// independent of order; no workgroup barrier is needed inside the block loop.
//
// The waves of the grid stride over the blocks of the whole tensor list (wave
// w takes blocks w, w + W, w + 2W, ... for W waves in the grid, the waves
// numbered so that runs of 16 lie on one XCD); the grid is several times what
// fits on the device at once, so finished workgroups are replaced until the
// end (launch_groups); each workgroup stages the codebooks, midpoints and
// code LUTs in LDS once.
//
// Arithmetic is the step exactly as the oracle states it: fp32, one rounding
// per operation (built with -ffp-contract=off), IEEE sqrt and divide,
// denormals kept.  The fast paths reach the same bits with cheaper instruction
// sequences whose exactness holds inside a range the block is checked
// against; a block outside it takes the plain path.
#include "opt8_codes.h"
#include "opt8_exact.h"
#include "opt8_internal.h"
#include "opt8_launch.h"

namespace opt8 {
namespace {

constexpr int kWaves = kWavesPerGroup;      // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kGroups = kBlock / (64 * 8);  // 8-element groups per lane per block (4)
constexpr float kMinNormal = 1.17549435e-38f;  // 2^-126

__device__ uint4 g_tables[kTableBytesSR / 16];

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): two 32x32->64 products per
// round, the words permuted and xored with the round key, key bumped by the
// Weyl constants.
constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

struct Rand4 {
  uint32_t w[4];
};

// The key is uniform across the wave: it lives in scalar registers and is
// bumped on the scalar unit round by round (the empty asm keeps the compiler
// from precomputing all twenty round keys, which would spill).
__device__ __forceinline__ Rand4 philox10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                          uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    asm volatile("" : "+s"(k0), "+s"(k1));
    const uint64_t p0 = static_cast<uint64_t>(kPhiloxM0) * c0;
    const uint64_t p1 = static_cast<uint64_t>(kPhiloxM1) * c2;
    // three-input xor in one instruction (truth table 0x96)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(p1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(p0 >> 32), c3, k1, 0x96);
    c1 = static_cast<uint32_t>(p1);
    c3 = static_cast<uint32_t>(p0);
    c0 = n0;
    c2 = n2;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  return Rand4{{c0, c1, c2, c3}};
}

// Random words of the 8-element group `grp` (global element index / 8).
__device__ __forceinline__ Rand4 group_bits(uint64_t grp, uint32_t stream, uint32_t tensor_id,
                                            const StepScalars& sc) {
  return philox10(static_cast<uint32_t>(grp), static_cast<uint32_t>(grp >> 32) | (stream << 30),
                  sc.step_lo, tensor_id, sc.seed_lo, sc.seed_hi);
}

__device__ __forceinline__ uint32_t r16_of(const Rand4& r, int j) {
  return (r.w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
}

// Philox for N counters at once (four 8-element groups, or the streams of
// one group), round by round, so each round key is computed once on the
// scalar unit and used by all N.
template <int N>
__device__ __forceinline__ void philox10_n(uint32_t (&c0)[N], uint32_t (&c1)[N], uint32_t (&c2)[N],
                                           uint32_t (&c3)[N], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
#pragma unroll
    for (int g = 0; g < N; ++g) {
      const uint64_t p0 = static_cast<uint64_t>(kPhiloxM0) * c0[g];
      const uint64_t p1 = static_cast<uint64_t>(kPhiloxM1) * c2[g];
      const uint32_t n0 = __builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(p1 >> 32), c1[g], k0, 0x96);
      const uint32_t n2 = __builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(p0 >> 32), c3[g], k1, 0x96);
      c1[g] = static_cast<uint32_t>(p1);
      c3[g] = static_cast<uint32_t>(p0);
      c0[g] = n0;
      c2[g] = n2;
    }
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
}

// Random words of the first and second moment (streams 1 and 2) of group grp.
__device__ __forceinline__ void state_bits(uint64_t grp, uint32_t tensor_id, const StepScalars& sc, Rand4& rm,
                                           Rand4& rv) {
  uint32_t c0[2], c1[2], c2[2], c3[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    c0[s] = static_cast<uint32_t>(grp);
    c1[s] = static_cast<uint32_t>(grp >> 32) | (static_cast<uint32_t>(s + 1) << 30);
    c2[s] = sc.step_lo;
    c3[s] = tensor_id;
  }
  philox10_n<2>(c0, c1, c2, c3, sc.seed_lo, sc.seed_hi);
  rm = Rand4{{c0[0], c1[0], c2[0], c3[0]}};
  rv = Rand4{{c0[1], c1[1], c2[1], c3[1]}};
}

// Random words of the parameter, first and second moment (streams 0, 1, 2) of
// group grp in one call, so their shared products are computed once.
__device__ __forceinline__ void all_bits(uint64_t grp, uint32_t tensor_id, const StepScalars& sc, Rand4& rp,
                                         Rand4& rm, Rand4& rv) {
  uint32_t c0[3], c1[3], c2[3], c3[3];
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    c0[s] = static_cast<uint32_t>(grp);
    c1[s] = static_cast<uint32_t>(grp >> 32) | (static_cast<uint32_t>(s) << 30);
    c2[s] = sc.step_lo;
    c3[s] = tensor_id;
  }
  philox10_n<3>(c0, c1, c2, c3, sc.seed_lo, sc.seed_hi);
  rp = Rand4{{c0[0], c1[0], c2[0], c3[0]}};
  rm = Rand4{{c0[1], c1[1], c2[1], c3[1]}};
  rv = Rand4{{c0[2], c1[2], c2[2], c3[2]}};
}

// fp32 -> bf16 bits: stochastic (add 16 random bits below the kept half, then
// truncate) or nearest-even; NaN becomes the quiet NaN with its sign.
__device__ __forceinline__ uint32_t to_bf16(float x, uint32_t r16, bool nearest) {
  const uint32_t b = __float_as_uint(x);
  const uint32_t add = nearest ? (0x7FFFu + ((b >> 16) & 1u)) : r16;
  const uint32_t rounded = (b + add) >> 16;
  const uint32_t qnan = 0x7FC0u | ((b >> 16) & 0x8000u);
  return (x != x) ? qnan : rounded;
}

// Streaming global accesses: every byte of the step is read once and written
// once, so loads and stores are non-temporal (no reuse to keep in the caches).
// The pointers are cast to the global address space so the accesses are
// global_* instructions (scalar base + 32-bit lane offset) rather than flat
// ones, which would also count against the LDS wait counter.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) u32x4_t g_u32x4_t;
typedef __attribute__((address_space(1))) u32x2_t g_u32x2_t;
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load((const g_u32x4_t*)(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_stream8(const void* p) {
  const u32x2_t v = __builtin_nontemporal_load((const g_u32x2_t*)(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void st_stream16(void* p, const uint4& q) {
  u32x4_t v;
  v.x = q.x; v.y = q.y; v.z = q.z; v.w = q.w;
  __builtin_nontemporal_store(v, (g_u32x4_t*)(p));
}
__device__ __forceinline__ void st_stream8(void* p, const uint2& q) {
  u32x2_t v;
  v.x = q.x; v.y = q.y;
  __builtin_nontemporal_store(v, (g_u32x2_t*)(p));
}

// A block's absmax through the scalar cache (the address is uniform across the
// wave).  Each wave reads its block's absmax before writing it back and no
// other wave touches that word, and the scalar cache starts every dispatch
// empty, so the read sees the value the step began with.  A scalar load waits
// on its own counter; a generic (flat) load here would count against the
// vector-memory loads of the block's data and make the first use of the
// absmax wait for all of them.
__device__ __forceinline__ float ld_absmax(const float* p, int64_t blk) {
  typedef const __attribute__((address_space(4))) float c_f32_t;
  return ((c_f32_t*)p)[blk];
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t word_of(const uint4& q, int k) {
  return (k == 0) ? q.x : (k == 1) ? q.y : (k == 2) ? q.z : q.w;
}
__device__ __forceinline__ float bf16_at(const uint4& q, int j) {
  const uint32_t w = word_of(q, j >> 1);
  return (j & 1) ? bf16_hi(w) : bf16_lo(w);
}
__device__ __forceinline__ uint32_t byte_at(const uint2& q, int j) {
  return (((j < 4) ? q.x : q.y) >> (8 * (j & 3))) & 0xFFu;
}

// Max that keeps NaN once seen (the oracle's numpy max propagates NaN).
__device__ __forceinline__ float nan_max(float acc, float x) {
  return (x > acc || x != x) ? x : acc;
}

// AdamW on one element with IEEE sqrt and divide; returns the new fp32 parameter.
__device__ __forceinline__ float adamw(float p, float g, float m1, float v1, const StepScalars& sc,
                                       float& m2, float& v2) {
  m2 = sc.beta1 * m1 + sc.w1 * g;
  v2 = sc.beta2 * v1 + sc.w2 * (g * g);
  const float den = sqrtf(v2) * sc.rbc2 + sc.eps;
  return (p - sc.lrwd * p) - sc.step_size * (m2 / den);
}

__device__ __forceinline__ float wave_nan_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = nan_max(x, __shfl_xor(x, o, 64));
  return x;
}

// Wave max of values that are +0, positive or NaN, returned as a uniform
// value: the unsigned max of the bit patterns (which orders such floats as
// their values) through DPP quad, half-row, row and row-broadcast steps, read
// from lane 63.  Unlike the shuffle reduction above it moves nothing through
// LDS.
__device__ __forceinline__ float wave_max_nonneg(float x) {
  uint32_t u = __float_as_uint(x);
  u = max(u, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(u), 0xB1, 0xF, 0xF, false)));
  u = max(u, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(u), 0x4E, 0xF, 0xF, false)));
  u = max(u, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(u), 0x141, 0xF, 0xF, false)));
  u = max(u, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(u), 0x140, 0xF, 0xF, false)));
  u = max(u, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(u), 0x142, 0xA, 0xF, false)));
  u = max(u, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(u), 0x143, 0xC, 0xF, false)));
  return __uint_as_float(__builtin_amdgcn_readlane(static_cast<int>(u), 63));
}

// The same maximum over each run of eight lanes (0-7, 8-15, ...), every lane
// of a run getting its run's value: quad steps, then the half-row mirror.
__device__ __forceinline__ float group8_max_nonneg(float x) {
  uint32_t u = __float_as_uint(x);
  u = max(u, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(u), 0xB1, 0xF, 0xF, false)));
  u = max(u, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(u), 0x4E, 0xF, 0xF, false)));
  u = max(u, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(u), 0x141, 0xF, 0xF, false)));
  return __uint_as_float(u);
}

// ----------------------------------------------------------------------------- 8-bit, plain path
// Every block whose values leave the fast path's range, every partial block,
// and every non-finite case: IEEE operations, binary search over the
// midpoints, NaN-propagating block max.
template <bool kFull, bool kSS>
__device__ __forceinline__ void block_8bit_plain(const DevTensor& d, int64_t blk, int lane, int valid,
                                              const StepScalars& sc, const uint8_t* lds) {
  const float* cb_s = reinterpret_cast<const float*>(lds + kOffCbS);
  const float* mid_s = reinterpret_cast<const float*>(lds + kOffMidS);
  const float* cb_u = reinterpret_cast<const float*>(lds + kOffCbU);
  const float* mid_u = reinterpret_cast<const float*>(lds + kOffMidU);
  const int64_t e0 = blk * kBlock;
  const uint16_t* gp = d.grad + e0;
  uint16_t* pp = d.param + e0;
  uint8_t* mp = static_cast<uint8_t*>(d.m) + e0;
  uint8_t* vp = static_cast<uint8_t*>(d.v) + e0;
  const float am = ld_absmax(d.amax_m, blk);
  const float av = ld_absmax(d.amax_v, blk);
  const bool nearest = sc.param_round != 0;

  float M2[kGroups * 8], V2[kGroups * 8];
  float mxm = 0.0f, mxv = 0.0f;
  const uint64_t grp0 = static_cast<uint64_t>(d.index_base + e0) >> 3;
#pragma unroll
  for (int r = 0; r < kGroups; ++r) {
    const int off = r * 512 + lane * 8;
    uint4 G, P;
    uint2 QM, QV;
    if (kFull) {
      G = *reinterpret_cast<const uint4*>(gp + off);
      P = *reinterpret_cast<const uint4*>(pp + off);
      QM = *reinterpret_cast<const uint2*>(mp + off);
      QV = *reinterpret_cast<const uint2*>(vp + off);
    } else {
      uint32_t g32[4] = {0, 0, 0, 0}, p32[4] = {0, 0, 0, 0}, m32[2] = {0, 0}, v32[2] = {0, 0};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (off + j < valid) {
          g32[j >> 1] |= static_cast<uint32_t>(gp[off + j]) << (16 * (j & 1));
          p32[j >> 1] |= static_cast<uint32_t>(pp[off + j]) << (16 * (j & 1));
          m32[j >> 2] |= static_cast<uint32_t>(mp[off + j]) << (8 * (j & 3));
          v32[j >> 2] |= static_cast<uint32_t>(vp[off + j]) << (8 * (j & 3));
        }
      }
      G = make_uint4(g32[0], g32[1], g32[2], g32[3]);
      P = make_uint4(p32[0], p32[1], p32[2], p32[3]);
      QM = make_uint2(m32[0], m32[1]);
      QV = make_uint2(v32[0], v32[1]);
    }
    Rand4 rnd{{0, 0, 0, 0}};
    if (!nearest) rnd = group_bits(grp0 + (off >> 3), 0u, d.tensor_id, sc);
    uint32_t outw[4] = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float m1 = cb_s[byte_at(QM, j)] * am;
      const float v1 = cb_u[byte_at(QV, j)] * av;
      float m2, v2;
      const float pn = adamw(bf16_at(P, j), bf16_at(G, j), m1, v1, sc, m2, v2);
      outw[j >> 1] |= to_bf16(pn, r16_of(rnd, j), nearest) << (16 * (j & 1));
      const bool ok = kFull || (off + j < valid);
      M2[r * 8 + j] = ok ? m2 : 0.0f;
      V2[r * 8 + j] = ok ? v2 : 0.0f;
      mxm = nan_max(mxm, fabsf(M2[r * 8 + j]));
      mxv = nan_max(mxv, fabsf(V2[r * 8 + j]));   // |v2|: a negative v2 is possible from a negative absmax_v
    }
    if (kFull) {
      *reinterpret_cast<uint4*>(pp + off) = make_uint4(outw[0], outw[1], outw[2], outw[3]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (off + j < valid) pp[off + j] = static_cast<uint16_t>(outw[j >> 1] >> (16 * (j & 1)));
    }
  }

  mxm = wave_nan_max(mxm);
  mxv = wave_nan_max(mxv);
  const bool live_m = mxm >= kMinNormal;
  const bool live_v = mxv >= kMinNormal;
  const float inv_m = live_m ? 1.0f / mxm : 0.0f;
  const float inv_v = live_v ? 1.0f / mxv : 0.0f;
#pragma unroll
  for (int r = 0; r < kGroups; ++r) {
    const int off = r * 512 + lane * 8;
    uint32_t cm[2] = {0, 0}, cv[2] = {0, 0};
    Rand4 rm{{0, 0, 0, 0}}, rv{{0, 0, 0, 0}};
    if constexpr (kSS) state_bits(grp0 + (off >> 3), d.tensor_id, sc, rm, rv);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float nm = M2[r * 8 + j] * inv_m;
      const float nv = V2[r * 8 + j] * inv_v;
      uint32_t qm, qv;
      if constexpr (kSS) {
        qm = live_m ? code_sr_search(nm, reinterpret_cast<const float*>(lds + kOffPairS), r16_of(rm, j)) : 127u;
        qv = live_v ? code_sr_search(nv, reinterpret_cast<const float*>(lds + kOffPairU), r16_of(rv, j)) : 0u;
      } else {
        qm = live_m ? code_search(nm, mid_s) : 127u;
        qv = live_v ? code_search(nv, mid_u) : 0u;
      }
      cm[j >> 2] |= qm << (8 * (j & 3));
      cv[j >> 2] |= qv << (8 * (j & 3));
    }
    if (kFull) {
      *reinterpret_cast<uint2*>(mp + off) = make_uint2(cm[0], cm[1]);
      *reinterpret_cast<uint2*>(vp + off) = make_uint2(cv[0], cv[1]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (off + j < valid) {
          mp[off + j] = static_cast<uint8_t>(cm[j >> 2] >> (8 * (j & 3)));
          vp[off + j] = static_cast<uint8_t>(cv[j >> 2] >> (8 * (j & 3)));
        }
      }
    }
  }
  if (lane == 0) {
    d.amax_m[blk] = mxm;
    d.amax_v[blk] = mxv;
  }
}

// ----------------------------------------------------------------------------- 8-bit, fast path
// A full block, or with kPartial the last block of a tensor holding `valid`
// elements; returns false (having written nothing) when the block must take
// the plain path instead.  Everything that could make a result NaN or leave
// the range of the fast sequences is checked after pass 1, so pass 2 stores
// each group's parameters and codes as soon as they are formed.  In a partial
// block a lane reads only valid elements (element by element in the one group
// that straddles the end) and fills the rest with a zero gradient, a zero
// parameter and the zero codes, whose moments are +0: they leave every block
// maximum and range check to the valid elements, and are never stored.
template <bool kNearest, bool kSS, bool kPartial = false>
__device__ __forceinline__ bool block_8bit_fast(const DevTensor& d, int64_t blk, int lane,
                                                const StepScalars& sc, const uint8_t* lds, bool range_ok,
                                                int valid = kBlock) {
  const int64_t e0 = blk * kBlock;
  const uint16_t* gp = d.grad + e0;
  uint16_t* pp = d.param + e0;
  uint8_t* mp = static_cast<uint8_t*>(d.m) + e0;
  uint8_t* vp = static_cast<uint8_t*>(d.v) + e0;
  const float am = ld_absmax(d.amax_m, blk);
  const float av = ld_absmax(d.amax_v, blk);

  uint4 G[kGroups], P[kGroups];
  uint2 QM[kGroups], QV[kGroups];
  if constexpr (kPartial) {
#pragma unroll
    for (int r = 0; r < kGroups; ++r) {
      const int off = r * 512 + lane * 8;
      if (off + 8 <= valid) {
        G[r] = ld_stream16(gp + off);
        P[r] = ld_stream16(pp + off);
        QM[r] = ld_stream8(mp + off);
        QV[r] = ld_stream8(vp + off);
      } else {
        uint32_t gw[4] = {0, 0, 0, 0}, pw[4] = {0, 0, 0, 0};
        uint32_t mw[2] = {0x7F7F7F7Fu, 0x7F7F7F7Fu}, vw[2] = {0, 0};
        for (int j = 0; j < 8 && off + j < valid; ++j) {
          const int sh16 = 16 * (j & 1), sh8 = 8 * (j & 3);
          gw[j >> 1] |= static_cast<uint32_t>(gp[off + j]) << sh16;
          pw[j >> 1] |= static_cast<uint32_t>(pp[off + j]) << sh16;
          mw[j >> 2] = (mw[j >> 2] & ~(0xFFu << sh8)) | (static_cast<uint32_t>(mp[off + j]) << sh8);
          vw[j >> 2] |= static_cast<uint32_t>(vp[off + j]) << sh8;
        }
        G[r] = make_uint4(gw[0], gw[1], gw[2], gw[3]);
        P[r] = make_uint4(pw[0], pw[1], pw[2], pw[3]);
        QM[r] = make_uint2(mw[0], mw[1]);
        QV[r] = make_uint2(vw[0], vw[1]);
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < kGroups; ++r) {
      const int off = r * 512 + lane * 8;
      G[r] = ld_stream16(gp + off);
      QM[r] = ld_stream8(mp + off);
      QV[r] = ld_stream8(vp + off);
    }
#pragma unroll
    for (int r = 0; r < kGroups; ++r)
      P[r] = ld_stream16(pp + r * 512 + lane * 8);
  }

  // pass 1: moments, block maxima (NaN-propagating), smallest exponents, and
  // the largest parameter magnitude
  const float* cb_s = reinterpret_cast<const float*>(lds + kOffCbS);
  const float* cb_u = reinterpret_cast<const float*>(lds + kOffCbU);
  float M2[kGroups * 8], V2[kGroups * 8];
  float mxm = 0.0f, mxv = 0.0f, mxp = 0.0f;
  int emin = 0;
#pragma unroll
  for (int r = 0; r < kGroups; ++r) {
    if (kPartial && r * 512 >= valid) continue;   // no lane has an element left
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float g = bf16_at(G[r], j);
      const float m1 = cb_s[byte_at(QM[r], j)] * am;
      const float v1 = cb_u[byte_at(QV[r], j)] * av;
      const float m2 = sc.beta1 * m1 + sc.w1 * g;
      const float v2 = sc.beta2 * v1 + sc.w2 * (g * g);
      M2[r * 8 + j] = m2;
      V2[r * 8 + j] = v2;
      mxm = __builtin_elementwise_maximum(mxm, fabsf(m2));
      mxv = __builtin_elementwise_maximum(mxv, v2);
      mxp = __builtin_elementwise_maximum(mxp, fabsf(bf16_at(P[r], j)));
      // smallest exponent of any non-zero m2 or v2 (frexp gives 0 for zero)
      emin = min(min(emin, __builtin_amdgcn_frexp_expf(m2)), __builtin_amdgcn_frexp_expf(v2));
    }
  }
  // finite parameters and moments (NaN fails every comparison)
  const bool lane_finite = (mxm <= 3.0e38f) && (mxv <= 3.0e38f) && (mxp <= 3.4028235e38f);
  mxm = wave_max_nonneg(mxm);
  mxv = wave_max_nonneg(mxv);

  // range check (uniform): finite inputs and moments; every non-zero v2 >=
  // 2^-89 (sqrt_rn) and every non-zero m2 / den quotient far above 2^-126
  // (div_rn).  With range_ok (eps in [2^-60, 2^60], rbc2 <= 2^20, lrwd <= 1,
  // step_size <= 2^26) no step of pass 2 can then produce a NaN or overflow
  // an intermediate: den >= eps, |u| <= 2^101, |p - lrwd p| <= |p|.
  const int e_den = __builtin_amdgcn_frexp_expf(sqrtf(mxv) * sc.rbc2 + sc.eps);
  const int e_mmax = __builtin_amdgcn_frexp_expf(mxm);
  const int e_eps = __builtin_amdgcn_frexp_expf(sc.eps);
  const int floor_e = max(-88, e_den - 98);
  const bool lane_bad = !lane_finite || emin < floor_e;
  // a negative (or NaN) absmax_v could make v2 negative, whose root is NaN
  if (!range_ok || !(av >= 0.0f) || e_den > 100 || e_mmax - e_eps > 100 ||
      __builtin_amdgcn_ballot_w64(lane_bad) != 0)
    return false;

  // pass 2, group by group: parameter update, its rounding and store, then the
  // requantised moments (a block with absmax below 2^-126 stores the zero code:
  // its multiplier is 0, so with finite moments every n is +-0, whose code under
  // either rounding rule is the zero code, 127 signed and 0 unsigned)
  const float* mid_s = reinterpret_cast<const float*>(lds + kOffMidS);
  const float* mid_u = reinterpret_cast<const float*>(lds + kOffMidU);
  const bool live_m = mxm >= kMinNormal;
  const bool live_v = mxv >= kMinNormal;
  const float inv_m = live_m ? 1.0f / mxm : 0.0f;
  const float inv_v = live_v ? 1.0f / mxv : 0.0f;
  const uint64_t grp0 = (static_cast<uint64_t>(d.index_base + e0) >> 3) + static_cast<uint64_t>(lane);
#pragma unroll
  for (int r = 0; r < kGroups; ++r) {
    if (kPartial && r * 512 >= valid) continue;   // no lane has an element left
    const int off = r * 512 + lane * 8;
    const uint64_t grp = grp0 + static_cast<uint64_t>(r * 64);
    Rand4 rnd{{0, 0, 0, 0}};
    Rand4 rm{{0, 0, 0, 0}}, rv{{0, 0, 0, 0}};
    if constexpr (kSS && !kNearest) all_bits(grp, d.tensor_id, sc, rnd, rm, rv);
    else if (!kNearest) rnd = group_bits(grp, 0u, d.tensor_id, sc);
    uint32_t sums[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = bf16_at(P[r], j);
      const float den = sqrt_rn(V2[r * 8 + j]) * sc.rbc2 + sc.eps;
      const float u = div_rn(M2[r * 8 + j], den);
      const float pn = (p - sc.lrwd * p) - sc.step_size * u;
      const uint32_t b = __float_as_uint(pn);
      sums[j] = b + (kNearest ? (0x7FFFu + ((b >> 16) & 1u)) : r16_of(rnd, j));
    }
    // keep the upper halves: bf16 pairs (element 2k in the low half)
    if (!kPartial || off + 8 <= valid) {
      st_stream16(pp + off, make_uint4(__builtin_amdgcn_perm(sums[1], sums[0], 0x07060302u),
                                       __builtin_amdgcn_perm(sums[3], sums[2], 0x07060302u),
                                       __builtin_amdgcn_perm(sums[5], sums[4], 0x07060302u),
                                       __builtin_amdgcn_perm(sums[7], sums[6], 0x07060302u)));
    } else {
      for (int j = 0; j < 8 && off + j < valid; ++j) pp[off + j] = static_cast<uint16_t>(sums[j] >> 16);
    }
    uint32_t cm[2] = {0, 0}, cv[2] = {0, 0};
    if constexpr (kSS && kNearest) state_bits(grp, d.tensor_id, sc, rm, rv);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t qm, qv;
      if constexpr (kSS) {
        qm = code_sr<true, true>(M2[r * 8 + j] * inv_m, lds, r16_of(rm, j));
        qv = code_sr<false, true>(V2[r * 8 + j] * inv_v, lds, r16_of(rv, j));
      } else {
        qm = code_s(M2[r * 8 + j] * inv_m, lds, mid_s);
        qv = code_u(V2[r * 8 + j] * inv_v, lds, mid_u);
      }
      cm[j >> 2] |= qm << (8 * (j & 3));
      cv[j >> 2] |= qv << (8 * (j & 3));
    }
    if (!kPartial || off + 8 <= valid) {
      st_stream8(mp + off, make_uint2(cm[0], cm[1]));
      st_stream8(vp + off, make_uint2(cv[0], cv[1]));
    } else {
      for (int j = 0; j < 8 && off + j < valid; ++j) {
        mp[off + j] = static_cast<uint8_t>(cm[j >> 2] >> (8 * (j & 3)));
        vp[off + j] = static_cast<uint8_t>(cv[j >> 2] >> (8 * (j & 3)));
      }
    }
  }
  if (lane == 0) {
    d.amax_m[blk] = mxm;
    d.amax_v[blk] = mxv;
  }
  return true;
}

// ----------------------------------------------------------------------------- 8-bit, short last blocks
// Last partial blocks of at most kShortTail (64) elements: such a block fits
// one 8-element group per lane in eight lanes, so a wave takes eight of them at
// once, lane run t (lanes 8t .. 8t+7) the entry first + t, its lane i holding
// elements 8i .. 8i+7 as lane i of the one-block layout.  The arithmetic is the
// fast path's; the block maxima are reduced within the run, the range check
// decides per run, and the blocks of runs that fail it are then stepped one at
// a time by the whole wave on the plain path.  (A wave per short block would
// issue a whole wave's instructions for a few elements.)
template <bool kNearest, bool kSS>
__device__ __forceinline__ void blocks_8bit_short(const DevTensor* __restrict__ list, int64_t first, int64_t count,
                                                  int lane, const StepScalars& sc, const uint8_t* lds,
                                                  bool range_ok) {
  const int t = lane >> 3, i = lane & 7;
  const int64_t entry = first + t;
  const bool has = entry < count;
  DevTensor d{};
  if (has) d = list[entry];
  const int64_t blk = has ? (d.numel - 1) / kBlock : 0;
  const int valid = has ? static_cast<int>(d.numel - blk * kBlock) : 0;
  const int off = 8 * i;
  const int64_t e0 = blk * kBlock;
  const uint16_t* gp = d.grad + e0;
  uint16_t* pp = d.param + e0;
  uint8_t* mp = static_cast<uint8_t*>(d.m) + e0;
  uint8_t* vp = static_cast<uint8_t*>(d.v) + e0;

  // a run's lanes past its block's end (and runs with no block) hold a zero
  // gradient and parameter and the zero codes, whose moments are +0
  uint4 G = make_uint4(0u, 0u, 0u, 0u), P = G;
  uint2 QM = make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu), QV = make_uint2(0u, 0u);
  float am = 0.0f, av = 0.0f;
  if (has) {
    am = d.amax_m[blk];
    av = d.amax_v[blk];
    if (off + 8 <= valid) {
      G = ld_stream16(gp + off);
      P = ld_stream16(pp + off);
      QM = ld_stream8(mp + off);
      QV = ld_stream8(vp + off);
    } else if (off < valid) {
      uint32_t gw[4] = {0, 0, 0, 0}, pw[4] = {0, 0, 0, 0};
      uint32_t mw[2] = {0x7F7F7F7Fu, 0x7F7F7F7Fu}, vw[2] = {0, 0};
      for (int j = 0; j < 8 && off + j < valid; ++j) {
        const int sh16 = 16 * (j & 1), sh8 = 8 * (j & 3);
        gw[j >> 1] |= static_cast<uint32_t>(gp[off + j]) << sh16;
        pw[j >> 1] |= static_cast<uint32_t>(pp[off + j]) << sh16;
        mw[j >> 2] = (mw[j >> 2] & ~(0xFFu << sh8)) | (static_cast<uint32_t>(mp[off + j]) << sh8);
        vw[j >> 2] |= static_cast<uint32_t>(vp[off + j]) << sh8;
      }
      G = make_uint4(gw[0], gw[1], gw[2], gw[3]);
      P = make_uint4(pw[0], pw[1], pw[2], pw[3]);
      QM = make_uint2(mw[0], mw[1]);
      QV = make_uint2(vw[0], vw[1]);
    }
  }

  // pass 1 (every lane, so the run reductions see all eight)
  const float* cb_s = reinterpret_cast<const float*>(lds + kOffCbS);
  const float* cb_u = reinterpret_cast<const float*>(lds + kOffCbU);
  float M2[8], V2[8];
  float mxm = 0.0f, mxv = 0.0f, mxp = 0.0f;
  int emin = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float g = bf16_at(G, j);
    const float m1 = cb_s[byte_at(QM, j)] * am;
    const float v1 = cb_u[byte_at(QV, j)] * av;
    const float m2 = sc.beta1 * m1 + sc.w1 * g;
    const float v2 = sc.beta2 * v1 + sc.w2 * (g * g);
    M2[j] = m2;
    V2[j] = v2;
    mxm = __builtin_elementwise_maximum(mxm, fabsf(m2));
    mxv = __builtin_elementwise_maximum(mxv, v2);
    mxp = __builtin_elementwise_maximum(mxp, fabsf(bf16_at(P, j)));
    emin = min(min(emin, __builtin_amdgcn_frexp_expf(m2)), __builtin_amdgcn_frexp_expf(v2));
  }
  const bool lane_finite = (mxm <= 3.0e38f) && (mxv <= 3.0e38f) && (mxp <= 3.4028235e38f);
  mxm = group8_max_nonneg(mxm);
  mxv = group8_max_nonneg(mxv);
  // the fast path's range check, per run
  const int e_den = __builtin_amdgcn_frexp_expf(sqrtf(mxv) * sc.rbc2 + sc.eps);
  const int e_mmax = __builtin_amdgcn_frexp_expf(mxm);
  const int e_eps = __builtin_amdgcn_frexp_expf(sc.eps);
  const int floor_e = max(-88, e_den - 98);
  const bool lane_bad = !lane_finite || emin < floor_e;
  const bool run_bad = ((__builtin_amdgcn_ballot_w64(lane_bad) >> (8 * t)) & 0xFFu) != 0;
  const bool fast = has && range_ok && av >= 0.0f && e_den <= 100 && e_mmax - e_eps <= 100 && !run_bad;

  if (fast) {
    const float* mid_s = reinterpret_cast<const float*>(lds + kOffMidS);
    const float* mid_u = reinterpret_cast<const float*>(lds + kOffMidU);
    const float inv_m = mxm >= kMinNormal ? 1.0f / mxm : 0.0f;
    const float inv_v = mxv >= kMinNormal ? 1.0f / mxv : 0.0f;
    const uint64_t grp = (static_cast<uint64_t>(d.index_base + e0) >> 3) + static_cast<uint64_t>(i);
    Rand4 rnd{{0, 0, 0, 0}};
    Rand4 rm{{0, 0, 0, 0}}, rv{{0, 0, 0, 0}};
    if constexpr (kSS && !kNearest) all_bits(grp, d.tensor_id, sc, rnd, rm, rv);
    else if (!kNearest) rnd = group_bits(grp, 0u, d.tensor_id, sc);
    if constexpr (kSS && kNearest) state_bits(grp, d.tensor_id, sc, rm, rv);
    uint32_t sums[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = bf16_at(P, j);
      const float den = sqrt_rn(V2[j]) * sc.rbc2 + sc.eps;
      const float u = div_rn(M2[j], den);
      const float pn = (p - sc.lrwd * p) - sc.step_size * u;
      const uint32_t b = __float_as_uint(pn);
      sums[j] = b + (kNearest ? (0x7FFFu + ((b >> 16) & 1u)) : r16_of(rnd, j));
    }
    uint32_t cm[2] = {0, 0}, cv[2] = {0, 0};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t qm, qv;
      if constexpr (kSS) {
        qm = code_sr<true, true>(M2[j] * inv_m, lds, r16_of(rm, j));
        qv = code_sr<false, true>(V2[j] * inv_v, lds, r16_of(rv, j));
      } else {
        qm = code_s(M2[j] * inv_m, lds, mid_s);
        qv = code_u(V2[j] * inv_v, lds, mid_u);
      }
      cm[j >> 2] |= qm << (8 * (j & 3));
      cv[j >> 2] |= qv << (8 * (j & 3));
    }
    if (off + 8 <= valid) {
      st_stream16(pp + off, make_uint4(__builtin_amdgcn_perm(sums[1], sums[0], 0x07060302u),
                                       __builtin_amdgcn_perm(sums[3], sums[2], 0x07060302u),
                                       __builtin_amdgcn_perm(sums[5], sums[4], 0x07060302u),
                                       __builtin_amdgcn_perm(sums[7], sums[6], 0x07060302u)));
      st_stream8(mp + off, make_uint2(cm[0], cm[1]));
      st_stream8(vp + off, make_uint2(cv[0], cv[1]));
    } else {
      for (int j = 0; j < 8 && off + j < valid; ++j) {
        pp[off + j] = static_cast<uint16_t>(sums[j] >> 16);
        mp[off + j] = static_cast<uint8_t>(cm[j >> 2] >> (8 * (j & 3)));
        vp[off + j] = static_cast<uint8_t>(cv[j >> 2] >> (8 * (j & 3)));
      }
    }
    if (i == 0) {
      d.amax_m[blk] = mxm;
      d.amax_v[blk] = mxv;
    }
  }

  // the blocks whose run failed the check, one at a time by the whole wave
  uint64_t slow = __builtin_amdgcn_ballot_w64(has && !fast && i == 0);
  while (slow) {
    const int src = __builtin_ctzll(slow);   // lane 8t of such a run
    slow &= slow - 1;
    DevTensor u;
    const uint32_t* w = reinterpret_cast<const uint32_t*>(&d);
    uint32_t* uw = reinterpret_cast<uint32_t*>(&u);
#pragma unroll
    for (int k = 0; k < static_cast<int>(sizeof(DevTensor) / 4); ++k)
      uw[k] = __builtin_amdgcn_readlane(static_cast<int>(w[k]), src);
    const int64_t ublk = (u.numel - 1) / kBlock;
    block_8bit_plain<false, kSS>(u, ublk, lane, static_cast<int>(u.numel - ublk * kBlock), sc, lds);
  }
}

// ----------------------------------------------------------------------------- bf16 state (SR)
// Plain path: IEEE operations, every rounding with its NaN rule.  Used for the
// partial last block of a tensor and for any 8-element group of a full block
// whose values leave the fast path's range.
__device__ __forceinline__ void group_bf16_plain(const uint4& G, const uint4& P, const uint4& M,
                                                 const uint4& V, const Rand4& rp, const Rand4& rm,
                                                 const Rand4& rv, bool nearest, const StepScalars& sc,
                                                 uint32_t (&po)[4], uint32_t (&mo)[4], uint32_t (&vo)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) po[k] = mo[k] = vo[k] = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float m2, v2;
    const float pn = adamw(bf16_at(P, j), bf16_at(G, j), bf16_at(M, j), bf16_at(V, j), sc, m2, v2);
    const int s = 16 * (j & 1);
    po[j >> 1] |= to_bf16(pn, r16_of(rp, j), nearest) << s;
    mo[j >> 1] |= to_bf16(m2, r16_of(rm, j), false) << s;
    vo[j >> 1] |= to_bf16(v2, r16_of(rv, j), false) << s;
  }
}

// Upper halves of two 32-bit sums as one bf16 pair (element 2k in the low half).
__device__ __forceinline__ uint32_t hi_pair(uint32_t even, uint32_t odd) {
  return __builtin_amdgcn_perm(odd, even, 0x07060302u);
}

// A full block.  Each group takes the fast sequences (sqrt_rn, div_rn, the
// plain add-and-truncate rounding) when every element of the wave's group is
// in their range -- no NaN result, and non-zero m2, v2 and m2/den all at or
// above 2^-88 -- and otherwise recomputes the group on the plain path.
// With kPartial, the last block of a tensor holding `valid` elements: groups
// wholly past the end are skipped, the group that straddles it is read and
// written element by element with zeros in the rest (a zero gradient,
// parameter and moments give den = eps and u = 0, so they decide nothing),
// and every other group takes the same path as in a full block.
template <bool kNearest, bool kPartial = false>
__device__ __forceinline__ void block_bf16_full(const DevTensor& d, int64_t blk, int lane,
                                                const StepScalars& sc, bool range_ok, int valid = kBlock) {
  const int64_t e0 = blk * kBlock;
  const uint16_t* gp = d.grad + e0;
  uint16_t* pp = d.param + e0;
  uint16_t* mp = static_cast<uint16_t*>(d.m) + e0;
  uint16_t* vp = static_cast<uint16_t*>(d.v) + e0;
  const uint64_t grp0 = (static_cast<uint64_t>(d.index_base + e0) >> 3) + static_cast<uint64_t>(lane);
#pragma unroll 1
  for (int r = 0; r < kGroups; ++r) {
    if (kPartial && r * 512 >= valid) break;       // no lane has an element left
    const int off = r * 512 + lane * 8;
    const bool whole = !kPartial || off + 8 <= valid;
    uint4 G, P, M, V;
    if (whole) {
      G = ld_stream16(gp + off);
      P = ld_stream16(pp + off);
      M = ld_stream16(mp + off);
      V = ld_stream16(vp + off);
    } else {
      uint32_t a[4] = {0, 0, 0, 0}, b[4] = {0, 0, 0, 0}, c[4] = {0, 0, 0, 0}, e[4] = {0, 0, 0, 0};
      for (int j = 0; j < 8 && off + j < valid; ++j) {
        const int sh = 16 * (j & 1);
        a[j >> 1] |= static_cast<uint32_t>(gp[off + j]) << sh;
        b[j >> 1] |= static_cast<uint32_t>(pp[off + j]) << sh;
        c[j >> 1] |= static_cast<uint32_t>(mp[off + j]) << sh;
        e[j >> 1] |= static_cast<uint32_t>(vp[off + j]) << sh;
      }
      G = make_uint4(a[0], a[1], a[2], a[3]);
      P = make_uint4(b[0], b[1], b[2], b[3]);
      M = make_uint4(c[0], c[1], c[2], c[3]);
      V = make_uint4(e[0], e[1], e[2], e[3]);
    }
    const uint64_t grp = grp0 + static_cast<uint64_t>(r * 64);
    uint32_t c0[3], c1[3], c2[3], c3[3];
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      c0[s] = static_cast<uint32_t>(grp);
      c1[s] = static_cast<uint32_t>(grp >> 32) | (static_cast<uint32_t>(s) << 30);
      c2[s] = sc.step_lo;
      c3[s] = d.tensor_id;
    }
    philox10_n<3>(c0, c1, c2, c3, sc.seed_lo, sc.seed_hi);
    const Rand4 rp{{c0[0], c1[0], c2[0], c3[0]}};
    const Rand4 rm{{c0[1], c1[1], c2[1], c3[1]}};
    const Rand4 rv{{c0[2], c1[2], c2[2], c3[2]}};

    uint32_t ps[8], ms[8], vs[8];
    int emin = 0;
    bool nan = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float g = bf16_at(G, j);
      const float p = bf16_at(P, j);
      const float m2 = sc.beta1 * bf16_at(M, j) + sc.w1 * g;
      const float v2 = sc.beta2 * bf16_at(V, j) + sc.w2 * (g * g);
      const float den = sqrt_rn(v2) * sc.rbc2 + sc.eps;
      const float u = div_rn(m2, den);
      const float pn = (p - sc.lrwd * p) - sc.step_size * u;
      nan |= (pn != pn);
      emin = min(min(emin, __builtin_amdgcn_frexp_expf(u)),
                 min(__builtin_amdgcn_frexp_expf(m2), __builtin_amdgcn_frexp_expf(v2)));
      const uint32_t b = __float_as_uint(pn);
      ps[j] = b + (kNearest ? (0x7FFFu + ((b >> 16) & 1u)) : r16_of(rp, j));
      ms[j] = __float_as_uint(m2) + r16_of(rm, j);
      vs[j] = __float_as_uint(v2) + r16_of(rv, j);
    }
    uint32_t po[4], mo[4], vo[4];
    if (range_ok && __builtin_amdgcn_ballot_w64(nan || emin < -88) == 0) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        po[k] = hi_pair(ps[2 * k], ps[2 * k + 1]);
        mo[k] = hi_pair(ms[2 * k], ms[2 * k + 1]);
        vo[k] = hi_pair(vs[2 * k], vs[2 * k + 1]);
      }
    } else {
      group_bf16_plain(G, P, M, V, rp, rm, rv, kNearest, sc, po, mo, vo);
    }
    if (whole) {
      st_stream16(pp + off, make_uint4(po[0], po[1], po[2], po[3]));
      st_stream16(mp + off, make_uint4(mo[0], mo[1], mo[2], mo[3]));
      st_stream16(vp + off, make_uint4(vo[0], vo[1], vo[2], vo[3]));
    } else {
      for (int j = 0; j < 8 && off + j < valid; ++j) {
        const int sh = 16 * (j & 1);
        pp[off + j] = static_cast<uint16_t>(po[j >> 1] >> sh);
        mp[off + j] = static_cast<uint16_t>(mo[j >> 1] >> sh);
        vp[off + j] = static_cast<uint16_t>(vo[j >> 1] >> sh);
      }
    }
  }
}

// ----------------------------------------------------------------------------- fp32 state
// The fallback for small tensors.  Lane l of a group of 512 elements takes two
// quads, elements 4l..4l+3 and 256+4l..256+4l+3, so every access instruction
// of the wave covers one contiguous segment: 8-byte accesses of the bf16
// gradient and parameter (512 B per instruction) and 16-byte accesses of the
// fp32 moments (1 KiB).  The random words follow the global element index: a
// quad is half of an 8-element Philox group, so lane pair (2m, 2m+1) needs
// groups m and m+32 of the 512; the even lane computes the first, the odd lane
// the second, and each hands its neighbour the two words of the other's quad.
// Each group of a lane takes the fast exact sequences under the same check as
// the bf16-state kernel (no NaN result, non-zero m2, v2 and m2/den at or above
// 2^-89, the host's range for eps and the corrections), else the plain IEEE
// operations; the moments are stored as computed.  With kPartial (the last
// block of a tensor holding `valid` elements) the groups past the end are
// skipped; in the one that straddles it, every quad wholly inside the tensor
// still moves with vector accesses, and the one quad that crosses the end is
// read and written element by element with zeros in the rest.
__device__ __forceinline__ uint32_t word2_of(const uint2& q, int k) { return k == 0 ? q.x : q.y; }

template <bool kNearest, bool kPartial>
__device__ __forceinline__ void block_fp32(const DevTensor& d, int64_t blk, int lane, const StepScalars& sc,
                                           bool range_ok, int valid = kBlock) {
  const int64_t e0 = blk * kBlock;
  const uint16_t* gp = d.grad + e0;
  uint16_t* pp = d.param + e0;
  float* mp = static_cast<float*>(d.m) + e0;
  float* vp = static_cast<float*>(d.v) + e0;
  const uint64_t grp0 = static_cast<uint64_t>(d.index_base + e0) >> 3;
  const bool odd = (lane & 1) != 0;
#pragma unroll 1
  for (int r = 0; r < kGroups; ++r) {
    if (kPartial && r * 512 >= valid) break;       // no lane has an element left
    const int o[2] = {r * 512 + 4 * lane, r * 512 + 256 + 4 * lane};   // the lane's two quads
    const bool whole = !kPartial || r * 512 + 512 <= valid;
    // random words of the two quads (element i of quad q: word wq[q][i >> 1], half i & 1)
    uint32_t wq[2][2] = {{0, 0}, {0, 0}};
    if (!kNearest) {
      const Rand4 x = group_bits(grp0 + static_cast<uint64_t>(r * 64 + (odd ? 32 : 0) + (lane >> 1)), 0u,
                                 d.tensor_id, sc);
      const uint32_t t0 = __shfl_xor(odd ? x.w[0] : x.w[2], 1, 64);
      const uint32_t t1 = __shfl_xor(odd ? x.w[1] : x.w[3], 1, 64);
      wq[0][0] = odd ? t0 : x.w[0];
      wq[0][1] = odd ? t1 : x.w[1];
      wq[1][0] = odd ? x.w[2] : t0;
      wq[1][1] = odd ? x.w[3] : t1;
    }
    // a quad wholly inside the tensor moves with vector accesses (in the group that
    // straddles the end too); only the quad that crosses the end goes element by element
    uint2 G[2], P[2];
    float M[8], V[8];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (whole || o[q] + 4 <= valid) {
        G[q] = ld_stream8(gp + o[q]);
        P[q] = ld_stream8(pp + o[q]);
        const uint4 m4 = ld_stream16(mp + o[q]), v4 = ld_stream16(vp + o[q]);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          M[4 * q + k] = __uint_as_float(word_of(m4, k));
          V[4 * q + k] = __uint_as_float(word_of(v4, k));
        }
      } else {
        uint32_t a[2] = {0, 0}, b[2] = {0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = o[q] + i < valid;
          a[i >> 1] |= (ok ? static_cast<uint32_t>(gp[o[q] + i]) : 0u) << (16 * (i & 1));
          b[i >> 1] |= (ok ? static_cast<uint32_t>(pp[o[q] + i]) : 0u) << (16 * (i & 1));
          M[4 * q + i] = ok ? mp[o[q] + i] : 0.0f;
          V[4 * q + i] = ok ? vp[o[q] + i] : 0.0f;
        }
        G[q] = make_uint2(a[0], a[1]);
        P[q] = make_uint2(b[0], b[1]);
      }
    }
    uint32_t ps[8];
    float M2[8], V2[8];
    int emin = 0;
    bool nan = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = j >> 2, i = j & 3;
      const uint32_t gw = word2_of(G[q], i >> 1), pw = word2_of(P[q], i >> 1);
      const float g = (i & 1) ? bf16_hi(gw) : bf16_lo(gw);
      const float p = (i & 1) ? bf16_hi(pw) : bf16_lo(pw);
      const float m2 = sc.beta1 * M[j] + sc.w1 * g;
      const float v2 = sc.beta2 * V[j] + sc.w2 * (g * g);
      const float den = sqrt_rn(v2) * sc.rbc2 + sc.eps;
      const float u = div_rn(m2, den);
      const float pn = (p - sc.lrwd * p) - sc.step_size * u;
      nan |= (pn != pn);
      emin = min(min(emin, __builtin_amdgcn_frexp_expf(u)),
                 min(__builtin_amdgcn_frexp_expf(m2), __builtin_amdgcn_frexp_expf(v2)));
      const uint32_t bits = __float_as_uint(pn);
      const uint32_t r16 = (wq[q][i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      ps[j] = bits + (kNearest ? (0x7FFFu + ((bits >> 16) & 1u)) : r16);
      M2[j] = m2;
      V2[j] = v2;
    }
    uint32_t po[4];
    if (range_ok && __builtin_amdgcn_ballot_w64(nan || emin < -88) == 0) {
#pragma unroll
      for (int k = 0; k < 4; ++k) po[k] = hi_pair(ps[2 * k], ps[2 * k + 1]);
    } else {
      po[0] = po[1] = po[2] = po[3] = 0u;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int q = j >> 2, i = j & 3;
        const uint32_t gw = word2_of(G[q], i >> 1), pw = word2_of(P[q], i >> 1);
        const float g = (i & 1) ? bf16_hi(gw) : bf16_lo(gw);
        const float p = (i & 1) ? bf16_hi(pw) : bf16_lo(pw);
        const uint32_t r16 = (wq[q][i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
        const float pn = adamw(p, g, M[j], V[j], sc, M2[j], V2[j]);
        po[j >> 1] |= to_bf16(pn, r16, kNearest) << (16 * (j & 1));
      }
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (whole || o[q] + 4 <= valid) {
        st_stream8(pp + o[q], make_uint2(po[2 * q], po[2 * q + 1]));
        st_stream16(mp + o[q], make_uint4(__float_as_uint(M2[4 * q]), __float_as_uint(M2[4 * q + 1]),
                                          __float_as_uint(M2[4 * q + 2]), __float_as_uint(M2[4 * q + 3])));
        st_stream16(vp + o[q], make_uint4(__float_as_uint(V2[4 * q]), __float_as_uint(V2[4 * q + 1]),
                                          __float_as_uint(V2[4 * q + 2]), __float_as_uint(V2[4 * q + 3])));
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = o[q] + i;
          if (e < valid) {
            pp[e] = static_cast<uint16_t>(po[2 * q + (i >> 1)] >> (16 * (i & 1)));
            mp[e] = M2[4 * q + i];
            vp[e] = V2[4 * q + i];
          }
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------- Lion, momentum
// One-state rules on the same machinery (readings: Lion as in "Symbolic
// Discovery of Optimization Algorithms", SGD momentum with dampening 0, weight
// decay decoupled as for AdamW; the pages name both, "8-bit Optimizers via
// Block-wise Quantization", motivation, and "Stochastic rounding support for
// 8-bit optimizers", motivation).  Returns the new fp32 parameter.
template <int A>
__device__ __forceinline__ float update1(float p, float g, float m1, const StepScalars& sc, float& m2) {
  if constexpr (A == kLion) {
    const float c = sc.beta1 * m1 + sc.w1 * g;          // direction from the old moment
    m2 = sc.beta2 * m1 + sc.w2 * g;
    // lr * sign(c): +-lr, +0 for a zero c, NaN for a NaN c
    const float t = (c > 0.0f) ? sc.lr : (c < 0.0f) ? -sc.lr : (c == c) ? 0.0f : c;
    return (p - sc.lrwd * p) - t;
  } else {
    m2 = sc.beta1 * m1 + g;
    return (p - sc.lrwd * p) - sc.lr * m2;
  }
}

// 8-bit state, plain path: partial blocks and any block with a NaN result or a
// non-finite moment.
template <int A, bool kFull, bool kSS>
__device__ __forceinline__ void block_1s_8bit_plain(const DevTensor& d, int64_t blk, int lane, int valid,
                                                    const StepScalars& sc, const uint8_t* lds) {
  const float* cb_s = reinterpret_cast<const float*>(lds + kOffCbS);
  const float* mid_s = reinterpret_cast<const float*>(lds + kOffMidS);
  const int64_t e0 = blk * kBlock;
  const uint16_t* gp = d.grad + e0;
  uint16_t* pp = d.param + e0;
  uint8_t* mp = static_cast<uint8_t*>(d.m) + e0;
  const float am = ld_absmax(d.amax_m, blk);
  const bool nearest = sc.param_round != 0;
  float M2[kGroups * 8];
  float mxm = 0.0f;
  const uint64_t grp0 = static_cast<uint64_t>(d.index_base + e0) >> 3;
#pragma unroll
  for (int r = 0; r < kGroups; ++r) {
    const int off = r * 512 + lane * 8;
    uint4 G, P;
    uint2 QM;
    if (kFull) {
      G = *reinterpret_cast<const uint4*>(gp + off);
      P = *reinterpret_cast<const uint4*>(pp + off);
      QM = *reinterpret_cast<const uint2*>(mp + off);
    } else {
      uint32_t g32[4] = {0, 0, 0, 0}, p32[4] = {0, 0, 0, 0}, m32[2] = {0, 0};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (off + j < valid) {
          g32[j >> 1] |= static_cast<uint32_t>(gp[off + j]) << (16 * (j & 1));
          p32[j >> 1] |= static_cast<uint32_t>(pp[off + j]) << (16 * (j & 1));
          m32[j >> 2] |= static_cast<uint32_t>(mp[off + j]) << (8 * (j & 3));
        }
      }
      G = make_uint4(g32[0], g32[1], g32[2], g32[3]);
      P = make_uint4(p32[0], p32[1], p32[2], p32[3]);
      QM = make_uint2(m32[0], m32[1]);
    }
    Rand4 rnd{{0, 0, 0, 0}};
    if (!nearest) rnd = group_bits(grp0 + (off >> 3), 0u, d.tensor_id, sc);
    uint32_t outw[4] = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float m2;
      const float pn = update1<A>(bf16_at(P, j), bf16_at(G, j), cb_s[byte_at(QM, j)] * am, sc, m2);
      outw[j >> 1] |= to_bf16(pn, r16_of(rnd, j), nearest) << (16 * (j & 1));
      const bool ok = kFull || (off + j < valid);
      M2[r * 8 + j] = ok ? m2 : 0.0f;
      mxm = nan_max(mxm, fabsf(M2[r * 8 + j]));
    }
    if (kFull) {
      *reinterpret_cast<uint4*>(pp + off) = make_uint4(outw[0], outw[1], outw[2], outw[3]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (off + j < valid) pp[off + j] = static_cast<uint16_t>(outw[j >> 1] >> (16 * (j & 1)));
    }
  }
  mxm = wave_nan_max(mxm);
  const bool live = mxm >= kMinNormal;
  const float inv = live ? 1.0f / mxm : 0.0f;
#pragma unroll
  for (int r = 0; r < kGroups; ++r) {
    const int off = r * 512 + lane * 8;
    uint32_t cm[2] = {0, 0};
    Rand4 rm{{0, 0, 0, 0}};
    if constexpr (kSS) rm = group_bits(grp0 + (off >> 3), 1u, d.tensor_id, sc);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float nm = M2[r * 8 + j] * inv;
      uint32_t q;
      if constexpr (kSS)
        q = live ? code_sr_search(nm, reinterpret_cast<const float*>(lds + kOffPairS), r16_of(rm, j)) : 127u;
      else
        q = live ? code_search(nm, mid_s) : 127u;
      cm[j >> 2] |= q << (8 * (j & 3));
    }
    if (kFull) {
      *reinterpret_cast<uint2*>(mp + off) = make_uint2(cm[0], cm[1]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (off + j < valid) mp[off + j] = static_cast<uint8_t>(cm[j >> 2] >> (8 * (j & 3)));
    }
  }
  if (lane == 0) d.amax_m[blk] = mxm;
}

// 8-bit state, full block: LUT requantisation and the plain add-and-truncate
// rounding; returns false (nothing written) on a NaN parameter or moment, or
// an infinite block maximum.
// With kPartial, the last block of a tensor holding `valid` elements, filled as
// in block_8bit_fast (a zero gradient, parameter and moment leave a zero
// moment and parameter under either rule, never stored).
template <int A, bool kNearest, bool kSS, bool kPartial = false>
__device__ __forceinline__ bool block_1s_8bit_fast(const DevTensor& d, int64_t blk, int lane,
                                                   const StepScalars& sc, const uint8_t* lds,
                                                   int valid = kBlock) {
  const float* cb_s = reinterpret_cast<const float*>(lds + kOffCbS);
  const float* mid_s = reinterpret_cast<const float*>(lds + kOffMidS);
  const int64_t e0 = blk * kBlock;
  const uint16_t* gp = d.grad + e0;
  uint16_t* pp = d.param + e0;
  uint8_t* mp = static_cast<uint8_t*>(d.m) + e0;
  const float am = ld_absmax(d.amax_m, blk);
  uint4 G[kGroups], P[kGroups];
  uint2 QM[kGroups];
#pragma unroll
  for (int r = 0; r < kGroups; ++r) {
    if (kPartial && r * 512 >= valid) continue;   // no lane has an element left
    const int off = r * 512 + lane * 8;
    if (!kPartial || off + 8 <= valid) {
      G[r] = ld_stream16(gp + off);
      P[r] = ld_stream16(pp + off);
      QM[r] = ld_stream8(mp + off);
    } else {
      uint32_t gw[4] = {0, 0, 0, 0}, pw[4] = {0, 0, 0, 0};
      uint32_t mw[2] = {0x7F7F7F7Fu, 0x7F7F7F7Fu};
      for (int j = 0; j < 8 && off + j < valid; ++j) {
        const int sh16 = 16 * (j & 1), sh8 = 8 * (j & 3);
        gw[j >> 1] |= static_cast<uint32_t>(gp[off + j]) << sh16;
        pw[j >> 1] |= static_cast<uint32_t>(pp[off + j]) << sh16;
        mw[j >> 2] = (mw[j >> 2] & ~(0xFFu << sh8)) | (static_cast<uint32_t>(mp[off + j]) << sh8);
      }
      G[r] = make_uint4(gw[0], gw[1], gw[2], gw[3]);
      P[r] = make_uint4(pw[0], pw[1], pw[2], pw[3]);
      QM[r] = make_uint2(mw[0], mw[1]);
    }
  }
  uint32_t c0[4] = {0, 0, 0, 0}, c1[4] = {0, 0, 0, 0}, c2[4] = {0, 0, 0, 0}, c3[4] = {0, 0, 0, 0};
  if (!kNearest) {
    const uint64_t grp0 = (static_cast<uint64_t>(d.index_base + e0) >> 3) + static_cast<uint64_t>(lane);
#pragma unroll
    for (int r = 0; r < kGroups; ++r) {
      const uint64_t grp = grp0 + static_cast<uint64_t>(r * 64);
      c0[r] = static_cast<uint32_t>(grp);
      c1[r] = static_cast<uint32_t>(grp >> 32);
      c2[r] = sc.step_lo;
      c3[r] = d.tensor_id;
    }
    philox10_n<4>(c0, c1, c2, c3, sc.seed_lo, sc.seed_hi);
  }
  float M2[kGroups * 8];
  float mxm = 0.0f;
  uint64_t nan_lanes = 0;
#pragma unroll
  for (int r = 0; r < kGroups; ++r) {
    if (kPartial && r * 512 >= valid) continue;   // no lane has an element left
    const Rand4 rnd{{c0[r], c1[r], c2[r], c3[r]}};
    uint32_t sums[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float m2;
      const float pn = update1<A>(bf16_at(P[r], j), bf16_at(G[r], j), cb_s[byte_at(QM[r], j)] * am, sc, m2);
      M2[r * 8 + j] = m2;
      mxm = fmaxf(mxm, fabsf(m2));
      // a NaN moment need not make a NaN parameter (Lion with beta2 = 0 and an
      // infinite old moment), and fmaxf would drop it from the maximum
      nan_lanes |= __builtin_amdgcn_ballot_w64(__builtin_isunordered(pn, m2));
      const uint32_t b = __float_as_uint(pn);
      sums[j] = b + (kNearest ? (0x7FFFu + ((b >> 16) & 1u)) : r16_of(rnd, j));
    }
    P[r] = make_uint4(__builtin_amdgcn_perm(sums[1], sums[0], 0x07060302u),
                      __builtin_amdgcn_perm(sums[3], sums[2], 0x07060302u),
                      __builtin_amdgcn_perm(sums[5], sums[4], 0x07060302u),
                      __builtin_amdgcn_perm(sums[7], sums[6], 0x07060302u));
  }
  mxm = wave_max_nonneg(mxm);
  if (nan_lanes != 0 || !(mxm <= 3.0e38f)) return false;
#pragma unroll
  for (int r = 0; r < kGroups; ++r) {
    if (kPartial && r * 512 >= valid) continue;   // no lane has an element left
    const int off = r * 512 + lane * 8;
    if (!kPartial || off + 8 <= valid) {
      st_stream16(pp + off, P[r]);
    } else {
      for (int j = 0; j < 8 && off + j < valid; ++j)
        pp[off + j] = static_cast<uint16_t>(word_of(P[r], j >> 1) >> (16 * (j & 1)));
    }
  }
  // absmax below 2^-126: the multiplier is 0, every n is +-0 (the moments are
  // finite here) and takes the zero code, 127, under either rounding rule
  const float inv = mxm >= kMinNormal ? 1.0f / mxm : 0.0f;
#pragma unroll
  for (int r = 0; r < kGroups; ++r) {
    if (kPartial && r * 512 >= valid) continue;   // no lane has an element left
    uint32_t cm[2] = {0, 0};
    if constexpr (kSS) {
      const Rand4 rm = group_bits((static_cast<uint64_t>(d.index_base + e0) >> 3) +
                                      static_cast<uint64_t>(lane + r * 64), 1u, d.tensor_id, sc);
#pragma unroll
      for (int j = 0; j < 8; ++j) cm[j >> 2] |= code_sr<true>(M2[r * 8 + j] * inv, lds, r16_of(rm, j)) << (8 * (j & 3));
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) cm[j >> 2] |= code_s(M2[r * 8 + j] * inv, lds, mid_s) << (8 * (j & 3));
    }
    const int off = r * 512 + lane * 8;
    if (!kPartial || off + 8 <= valid) {
      st_stream8(mp + off, make_uint2(cm[0], cm[1]));
    } else {
      for (int j = 0; j < 8 && off + j < valid; ++j) mp[off + j] = static_cast<uint8_t>(cm[j >> 2] >> (8 * (j & 3)));
    }
  }
  if (lane == 0) d.amax_m[blk] = mxm;
  return true;
}

// Short last blocks of the one-state rules, eight to a wave as in
// blocks_8bit_short: the fast path's arithmetic per lane, the run's block
// maximum reduced in the run, and a run with a NaN result or a non-finite
// moment stepped afterwards by the whole wave on the plain path.
template <int A, bool kNearest, bool kSS>
__device__ __forceinline__ void blocks_1s_8bit_short(const DevTensor* __restrict__ list, int64_t first,
                                                     int64_t count, int lane, const StepScalars& sc,
                                                     const uint8_t* lds) {
  const int t = lane >> 3, i = lane & 7;
  const int64_t entry = first + t;
  const bool has = entry < count;
  DevTensor d{};
  if (has) d = list[entry];
  const int64_t blk = has ? (d.numel - 1) / kBlock : 0;
  const int valid = has ? static_cast<int>(d.numel - blk * kBlock) : 0;
  const int off = 8 * i;
  const int64_t e0 = blk * kBlock;
  const uint16_t* gp = d.grad + e0;
  uint16_t* pp = d.param + e0;
  uint8_t* mp = static_cast<uint8_t*>(d.m) + e0;

  uint4 G = make_uint4(0u, 0u, 0u, 0u), P = G;
  uint2 QM = make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
  float am = 0.0f;
  if (has) {
    am = d.amax_m[blk];
    if (off + 8 <= valid) {
      G = ld_stream16(gp + off);
      P = ld_stream16(pp + off);
      QM = ld_stream8(mp + off);
    } else if (off < valid) {
      uint32_t gw[4] = {0, 0, 0, 0}, pw[4] = {0, 0, 0, 0};
      uint32_t mw[2] = {0x7F7F7F7Fu, 0x7F7F7F7Fu};
      for (int j = 0; j < 8 && off + j < valid; ++j) {
        const int sh16 = 16 * (j & 1), sh8 = 8 * (j & 3);
        gw[j >> 1] |= static_cast<uint32_t>(gp[off + j]) << sh16;
        pw[j >> 1] |= static_cast<uint32_t>(pp[off + j]) << sh16;
        mw[j >> 2] = (mw[j >> 2] & ~(0xFFu << sh8)) | (static_cast<uint32_t>(mp[off + j]) << sh8);
      }
      G = make_uint4(gw[0], gw[1], gw[2], gw[3]);
      P = make_uint4(pw[0], pw[1], pw[2], pw[3]);
      QM = make_uint2(mw[0], mw[1]);
    }
  }
  const float* cb_s = reinterpret_cast<const float*>(lds + kOffCbS);
  const float* mid_s = reinterpret_cast<const float*>(lds + kOffMidS);
  const uint64_t grp = (static_cast<uint64_t>(d.index_base + e0) >> 3) + static_cast<uint64_t>(i);
  Rand4 rnd{{0, 0, 0, 0}};
  if (!kNearest) rnd = group_bits(grp, 0u, d.tensor_id, sc);
  float M2[8];
  float mxm = 0.0f;
  bool nan = false;
  uint32_t sums[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float m2;
    const float pn = update1<A>(bf16_at(P, j), bf16_at(G, j), cb_s[byte_at(QM, j)] * am, sc, m2);
    M2[j] = m2;
    mxm = fmaxf(mxm, fabsf(m2));
    nan |= __builtin_isunordered(pn, m2);
    const uint32_t b = __float_as_uint(pn);
    sums[j] = b + (kNearest ? (0x7FFFu + ((b >> 16) & 1u)) : r16_of(rnd, j));
  }
  mxm = group8_max_nonneg(mxm);
  const bool run_bad = ((__builtin_amdgcn_ballot_w64(nan) >> (8 * t)) & 0xFFu) != 0;
  const bool fast = has && !run_bad && mxm <= 3.0e38f;

  if (fast) {
    const float inv = mxm >= kMinNormal ? 1.0f / mxm : 0.0f;
    uint32_t cm[2] = {0, 0};
    if constexpr (kSS) {
      const Rand4 rm = group_bits(grp, 1u, d.tensor_id, sc);
#pragma unroll
      for (int j = 0; j < 8; ++j) cm[j >> 2] |= code_sr<true>(M2[j] * inv, lds, r16_of(rm, j)) << (8 * (j & 3));
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) cm[j >> 2] |= code_s(M2[j] * inv, lds, mid_s) << (8 * (j & 3));
    }
    if (off + 8 <= valid) {
      st_stream16(pp + off, make_uint4(__builtin_amdgcn_perm(sums[1], sums[0], 0x07060302u),
                                       __builtin_amdgcn_perm(sums[3], sums[2], 0x07060302u),
                                       __builtin_amdgcn_perm(sums[5], sums[4], 0x07060302u),
                                       __builtin_amdgcn_perm(sums[7], sums[6], 0x07060302u)));
      st_stream8(mp + off, make_uint2(cm[0], cm[1]));
    } else {
      for (int j = 0; j < 8 && off + j < valid; ++j) {
        pp[off + j] = static_cast<uint16_t>(sums[j] >> 16);
        mp[off + j] = static_cast<uint8_t>(cm[j >> 2] >> (8 * (j & 3)));
      }
    }
    if (i == 0) d.amax_m[blk] = mxm;
  }

  // the blocks whose run failed the check, one at a time by the whole wave
  uint64_t slow = __builtin_amdgcn_ballot_w64(has && !fast && i == 0);
  while (slow) {
    const int src = __builtin_ctzll(slow);   // lane 8t of such a run
    slow &= slow - 1;
    DevTensor u;
    const uint32_t* w = reinterpret_cast<const uint32_t*>(&d);
    uint32_t* uw = reinterpret_cast<uint32_t*>(&u);
#pragma unroll
    for (int k = 0; k < static_cast<int>(sizeof(DevTensor) / 4); ++k)
      uw[k] = __builtin_amdgcn_readlane(static_cast<int>(w[k]), src);
    const int64_t ublk = (u.numel - 1) / kBlock;
    block_1s_8bit_plain<A, false, kSS>(u, ublk, lane, static_cast<int>(u.numel - ublk * kBlock), sc, lds);
  }
}

// bf16 state of the one-state rules: plain operations with every rounding's NaN
// rule.  Full blocks move whole 8-element groups with 16-byte accesses (the
// random words of the parameter and the state come from one two-stream Philox
// call); in the group that straddles the end of a partial block, elements go
// one by one.
template <int A, bool kFull>
__device__ __forceinline__ void block_1s_bf16(const DevTensor& d, int64_t blk, int lane, int valid,
                                              const StepScalars& sc) {
  const int64_t e0 = blk * kBlock;
  const uint16_t* gp = d.grad + e0;
  uint16_t* pp = d.param + e0;
  uint16_t* mp = static_cast<uint16_t*>(d.m) + e0;
  const bool nearest = sc.param_round != 0;
  const uint64_t grp0 = static_cast<uint64_t>(d.index_base + e0) >> 3;
#pragma unroll 1
  for (int r = 0; r < kGroups; ++r) {
    if (!kFull && r * 512 >= valid) break;         // no lane has an element left
    const int off = r * 512 + lane * 8;
    // a whole group moves with 16-byte accesses; only the one that straddles the
    // end of a partial block goes element by element
    const bool whole = kFull || off + 8 <= valid;
    float g[8], p[8], m1[8];
    if (whole) {
      const uint4 G = ld_stream16(gp + off);
      const uint4 P = ld_stream16(pp + off);
      const uint4 M = ld_stream16(mp + off);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        g[j] = bf16_at(G, j);
        p[j] = bf16_at(P, j);
        m1[j] = bf16_at(M, j);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool ok = off + j < valid;
        g[j] = ok ? __uint_as_float(static_cast<uint32_t>(gp[off + j]) << 16) : 0.0f;
        p[j] = ok ? __uint_as_float(static_cast<uint32_t>(pp[off + j]) << 16) : 0.0f;
        m1[j] = ok ? __uint_as_float(static_cast<uint32_t>(mp[off + j]) << 16) : 0.0f;
      }
    }
    // streams 0 (parameter) and 1 (state) in one call
    const uint64_t grp = grp0 + (off >> 3);
    uint32_t c0[2], c1[2], c2[2], c3[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      c0[s] = static_cast<uint32_t>(grp);
      c1[s] = static_cast<uint32_t>(grp >> 32) | (static_cast<uint32_t>(s) << 30);
      c2[s] = sc.step_lo;
      c3[s] = d.tensor_id;
    }
    philox10_n<2>(c0, c1, c2, c3, sc.seed_lo, sc.seed_hi);
    const Rand4 rp{{c0[0], c1[0], c2[0], c3[0]}};
    const Rand4 rm{{c0[1], c1[1], c2[1], c3[1]}};
    uint32_t po[4] = {0, 0, 0, 0}, mo[4] = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float m2;
      const float pn = update1<A>(p[j], g[j], m1[j], sc, m2);
      po[j >> 1] |= to_bf16(pn, r16_of(rp, j), nearest) << (16 * (j & 1));
      mo[j >> 1] |= to_bf16(m2, r16_of(rm, j), false) << (16 * (j & 1));
    }
    if (whole) {
      st_stream16(pp + off, make_uint4(po[0], po[1], po[2], po[3]));
      st_stream16(mp + off, make_uint4(mo[0], mo[1], mo[2], mo[3]));
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (off + j < valid) {
          pp[off + j] = static_cast<uint16_t>(po[j >> 1] >> (16 * (j & 1)));
          mp[off + j] = static_cast<uint16_t>(mo[j >> 1] >> (16 * (j & 1)));
        }
      }
    }
  }
}

// fp32 state of the one-state rules: the quad layout of block_fp32 (lane l
// takes elements 4l..4l+3 and 256+4l..256+4l+3 of each group, so every access
// instruction covers one contiguous segment; lane pairs share the Philox work
// of their two groups), plain operations with every rounding's NaN rule.
// Partial blocks skip the groups past the end; in the group that straddles it
// only the quad that crosses the end goes element by element.
template <int A>
__device__ __forceinline__ void block_1s_fp32(const DevTensor& d, int64_t blk, int lane, int valid,
                                              const StepScalars& sc) {
  const int64_t e0 = blk * kBlock;
  const uint16_t* gp = d.grad + e0;
  uint16_t* pp = d.param + e0;
  float* mp = static_cast<float*>(d.m) + e0;
  const bool nearest = sc.param_round != 0;
  const uint64_t grp0 = static_cast<uint64_t>(d.index_base + e0) >> 3;
  const bool odd = (lane & 1) != 0;
#pragma unroll 1
  for (int r = 0; r < kGroups; ++r) {
    if (r * 512 >= valid) break;                   // no lane has an element left
    const int o[2] = {r * 512 + 4 * lane, r * 512 + 256 + 4 * lane};
    const bool whole = r * 512 + 512 <= valid;
    uint32_t wq[2][2] = {{0, 0}, {0, 0}};
    if (!nearest) {
      const Rand4 x = group_bits(grp0 + static_cast<uint64_t>(r * 64 + (odd ? 32 : 0) + (lane >> 1)), 0u,
                                 d.tensor_id, sc);
      const uint32_t t0 = __shfl_xor(odd ? x.w[0] : x.w[2], 1, 64);
      const uint32_t t1 = __shfl_xor(odd ? x.w[1] : x.w[3], 1, 64);
      wq[0][0] = odd ? t0 : x.w[0];
      wq[0][1] = odd ? t1 : x.w[1];
      wq[1][0] = odd ? x.w[2] : t0;
      wq[1][1] = odd ? x.w[3] : t1;
    }
    // a quad wholly inside the tensor moves with vector accesses; only the quad that
    // crosses the end goes element by element
    float g[8], p[8], m1[8];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (whole || o[q] + 4 <= valid) {
        const uint2 G = ld_stream8(gp + o[q]), P = ld_stream8(pp + o[q]);
        const uint4 M = ld_stream16(mp + o[q]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t gw = word2_of(G, i >> 1), pw = word2_of(P, i >> 1);
          g[4 * q + i] = (i & 1) ? bf16_hi(gw) : bf16_lo(gw);
          p[4 * q + i] = (i & 1) ? bf16_hi(pw) : bf16_lo(pw);
          m1[4 * q + i] = __uint_as_float(word_of(M, i));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = o[q] + i;
          const bool ok = e < valid;
          g[4 * q + i] = ok ? __uint_as_float(static_cast<uint32_t>(gp[e]) << 16) : 0.0f;
          p[4 * q + i] = ok ? __uint_as_float(static_cast<uint32_t>(pp[e]) << 16) : 0.0f;
          m1[4 * q + i] = ok ? mp[e] : 0.0f;
        }
      }
    }
    uint32_t po[4] = {0, 0, 0, 0};
    float M2[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = j >> 2, i = j & 3;
      const uint32_t r16 = (wq[q][i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      const float pn = update1<A>(p[j], g[j], m1[j], sc, M2[j]);
      po[j >> 1] |= to_bf16(pn, r16, nearest) << (16 * (j & 1));
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (whole || o[q] + 4 <= valid) {
        st_stream8(pp + o[q], make_uint2(po[2 * q], po[2 * q + 1]));
        st_stream16(mp + o[q], make_uint4(__float_as_uint(M2[4 * q]), __float_as_uint(M2[4 * q + 1]),
                                          __float_as_uint(M2[4 * q + 2]), __float_as_uint(M2[4 * q + 3])));
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = o[q] + i;
          if (e < valid) {
            pp[e] = static_cast<uint16_t>(po[2 * q + (i >> 1)] >> (16 * (i & 1)));
            mp[e] = M2[4 * q + i];
          }
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------- driver
// Index of the tensor holding block b: the last i in [lo, hi] whose first
// block is <= b, given that list[lo] starts at or before b (blocks are
// numbered by a prefix sum, so the predicate holds on a prefix of the list).
// Each round the 64 lanes test 64 evenly spaced candidates at once and a
// ballot keeps the last that passes, so the range shrinks 64-fold per round
// trip: one round for up to 64 tensors, two for 4,096, three for 262,144.
__device__ __forceinline__ int find_tensor(const DevTensor* __restrict__ list, int lo, int hi, int64_t b,
                                           int lane) {
  while (true) {
    const int step = (hi - lo + 64) >> 6;          // ceil((hi - lo + 1) / 64)
    const int cand = lo + lane * step;
    const bool ok = cand <= hi && list[cand].block_begin <= b;
    const uint64_t m = __builtin_amdgcn_ballot_w64(ok);   // lane 0 always passes
    lo = __builtin_amdgcn_readfirstlane(lo + (63 - __builtin_clzll(m)) * step);
    if (step == 1) return lo;
    hi = min(hi, lo + step - 1);
  }
}

template <int kBytes>
__device__ __forceinline__ void stage_tables(uint8_t* lds) {
  uint4* dst = reinterpret_cast<uint4*>(lds);
  for (int i = threadIdx.x; i < kBytes / 16; i += kThreads) dst[i] = g_tables[i];
  __syncthreads();
}

// SS: the 8-bit state is rounded stochastically between neighbouring entries
// (only the 8-bit kinds are instantiated with it).
template <Kind K, int A, bool SS>
__global__ void __launch_bounds__(kThreads)
step_kernel(const DevTensor* __restrict__ list, int ntensors, int64_t total_blocks, StepScalars sc,
            int range_ok, const uint32_t* __restrict__ map) {
  constexpr bool kQ8 = (K == Kind::k8bit || K == Kind::k8bitTail);
  // the block map (block -> entry) replaces the descriptor search in the 8-bit
  // full-block kernels of AdamW and Lion; the others keep the search, which
  // measured faster for them (see launch_groups for how they are launched)
  constexpr bool kMap = K == Kind::k8bit && A != kMomentum;
  if constexpr (!kMap) map = nullptr;
  constexpr int kLds = kQ8 ? (SS ? kTableBytesSR : kTableBytes) : 16;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
  if constexpr (kQ8) stage_tables<kLds>(lds);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  // workgroups are dispatched to the 8 XCDs round-robin (workgroup i on XCD
  // i mod 8); the waves are renumbered so that each run of 16 consecutive
  // numbers (four workgroups) lies on one XCD, so 16 adjacent blocks, and
  // with them most 64-byte lines of absmax values, go through one XCD's L2
  // (any grid size that is a multiple of 32 keeps the numbering a bijection)
  int64_t gw = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  if ((gridDim.x & 31u) == 0) {
    const int64_t x = blockIdx.x & 7u, i = blockIdx.x >> 3;   // XCD, workgroup within it
    gw = (((i >> 2) * 8 + x) * 4 + (i & 3)) * kWaves + wave;
  }
  const int64_t nw = static_cast<int64_t>(gridDim.x) * kWaves;
  // wave gw takes blocks gw, gw + nw, gw + 2 nw, ...: the waves in flight
  // (consecutive workgroups) stream through one window of adjacent blocks,
  // which the memory system serves faster than as many separate runs
  int64_t b = gw;
  if (b >= total_blocks) return;

  // the list of last partial blocks has one block per entry, so block b is
  // entry b: no search, and the next entry's descriptor is read while the
  // current block is processed
  int t = 0;
  DevTensor d;
  DevTensor d_next;
  uint32_t t_next = 0;   // with a block map: the entry of the wave's next block, read one block ahead
  if constexpr (K == Kind::k8bitTail) {
    d_next = list[b];
  } else {
    t = map ? static_cast<int>(map[b]) : find_tensor(list, 0, ntensors - 1, b, lane);
    d = list[t];
    if (map && b + nw < total_blocks) t_next = map[b + nw];
  }
  for (; b < total_blocks; b += nw) {
    if constexpr (K == Kind::k8bitTail) {
      d = d_next;
      if (b + nw < total_blocks) d_next = list[b + nw];
    } else if (map) {
      if (b != gw && static_cast<int>(t_next) != t) {
        t = static_cast<int>(t_next);
        d = list[t];
      }
      if (b + nw < total_blocks) t_next = map[b + nw];
    } else if (b >= d.block_begin + static_cast<int64_t>(d.nblocks)) {
      // past the current tensor: the next one starts at or before b, and a later
      // one holds it (b < total_blocks); a wave strides over many blocks, which
      // for lists of small tensors crosses many descriptors at once
      t = find_tensor(list, t + 1, ntensors - 1, b, lane);
      d = list[t];
    }
    const int64_t blk = b - d.block_begin;
    if constexpr (A != kAdamW) {
      if constexpr (K == Kind::k8bit) {
        const bool done = sc.param_round ? block_1s_8bit_fast<A, true, SS>(d, blk, lane, sc, lds)
                                         : block_1s_8bit_fast<A, false, SS>(d, blk, lane, sc, lds);
        if (!done) block_1s_8bit_plain<A, true, SS>(d, blk, lane, kBlock, sc, lds);
      } else if constexpr (K == Kind::k8bitTail) {
        const int64_t tail = (d.numel - 1) / kBlock;
        const int valid = static_cast<int>(d.numel - tail * kBlock);
        const bool done = sc.param_round ? block_1s_8bit_fast<A, true, SS, true>(d, tail, lane, sc, lds, valid)
                                         : block_1s_8bit_fast<A, false, SS, true>(d, tail, lane, sc, lds, valid);
        if (!done) block_1s_8bit_plain<A, false, SS>(d, tail, lane, valid, sc, lds);
      } else if constexpr (K == Kind::kBf16) {
        const int64_t left = d.numel - blk * kBlock;
        if (left >= kBlock) block_1s_bf16<A, true>(d, blk, lane, kBlock, sc);
        else block_1s_bf16<A, false>(d, blk, lane, static_cast<int>(left), sc);
      } else {
        const int64_t left = d.numel - blk * kBlock;
        block_1s_fp32<A>(d, blk, lane, left >= kBlock ? kBlock : static_cast<int>(left), sc);
      }
    } else if constexpr (K == Kind::k8bit) {
      // this list holds the full blocks of 8-bit tensors only
      const bool done = sc.param_round ? block_8bit_fast<true, SS>(d, blk, lane, sc, lds, range_ok != 0)
                                       : block_8bit_fast<false, SS>(d, blk, lane, sc, lds, range_ok != 0);
      if (!done) block_8bit_plain<true, SS>(d, blk, lane, kBlock, sc, lds);
    } else if constexpr (K == Kind::k8bitTail) {
      // this list holds the last, partial block of 8-bit tensors (one per entry)
      const int64_t tail = (d.numel - 1) / kBlock;
      const int valid = static_cast<int>(d.numel - tail * kBlock);
      const bool done = sc.param_round
                            ? block_8bit_fast<true, SS, true>(d, tail, lane, sc, lds, range_ok != 0, valid)
                            : block_8bit_fast<false, SS, true>(d, tail, lane, sc, lds, range_ok != 0, valid);
      if (!done) block_8bit_plain<false, SS>(d, tail, lane, valid, sc, lds);
    } else {
      const int64_t left = d.numel - blk * kBlock;
      const bool full = left >= kBlock;
      const int valid = full ? kBlock : static_cast<int>(left);
      if constexpr (K == Kind::kBf16) {
        if (!full) {
          if (sc.param_round) block_bf16_full<true, true>(d, blk, lane, sc, range_ok != 0, valid);
          else block_bf16_full<false, true>(d, blk, lane, sc, range_ok != 0, valid);
        } else if (sc.param_round) block_bf16_full<true>(d, blk, lane, sc, range_ok != 0);
        else block_bf16_full<false>(d, blk, lane, sc, range_ok != 0);
      } else {
        const bool ro = range_ok != 0;
        if (full) {
          if (sc.param_round) block_fp32<true, false>(d, blk, lane, sc, ro);
          else block_fp32<false, false>(d, blk, lane, sc, ro);
        } else if (sc.param_round) {
          block_fp32<true, true>(d, blk, lane, sc, ro, valid);
        } else {
          block_fp32<false, true>(d, blk, lane, sc, ro, valid);
        }
      }
    }
  }
}

// The short last blocks of 8-bit tensors (one entry each), eight to a wave;
// the grid is the resident count or fewer, each wave taking every nw-th set
// of eight.
template <int A, bool SS>
__global__ void __launch_bounds__(kThreads)
short_kernel(const DevTensor* __restrict__ list, int64_t count, StepScalars sc, int range_ok) {
  constexpr int kLds = SS ? kTableBytesSR : kTableBytes;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
  stage_tables<kLds>(lds);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t nw = static_cast<int64_t>(gridDim.x) * kWaves;
  for (int64_t w = static_cast<int64_t>(blockIdx.x) * kWaves + wave; w * 8 < count; w += nw) {
    if constexpr (A == kAdamW) {
      if (sc.param_round) blocks_8bit_short<true, SS>(list, w * 8, count, lane, sc, lds, range_ok != 0);
      else blocks_8bit_short<false, SS>(list, w * 8, count, lane, sc, lds, range_ok != 0);
    } else {
      if (sc.param_round) blocks_1s_8bit_short<A, true, SS>(list, w * 8, count, lane, sc, lds);
      else blocks_1s_8bit_short<A, false, SS>(list, w * 8, count, lane, sc, lds);
    }
  }
}

template <int A, bool SS>
hipError_t launch_short(const DevTensor* list, int n, const StepScalars& sc, hipStream_t stream, int resident,
                        int range_ok) {
  const int64_t sets = (static_cast<int64_t>(n) + 7) / 8;
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>((sets + kWaves - 1) / kWaves, resident));
  hipLaunchKernelGGL((short_kernel<A, SS>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream, list,
                     static_cast<int64_t>(n), sc, range_ok);
  return hipGetLastError();
}

template <bool SS>
hipError_t launch_short_algo(int algo, const DevTensor* list, int n, const StepScalars& sc, hipStream_t stream,
                             int resident, int range_ok) {
  switch (algo) {
    case kAdamW: return launch_short<kAdamW, SS>(list, n, sc, stream, resident, range_ok);
    case kLion: return launch_short<kLion, SS>(list, n, sc, stream, resident, range_ok);
    case kMomentum: return launch_short<kMomentum, SS>(list, n, sc, stream, resident, range_ok);
  }
  return hipErrorInvalidValue;
}

template <int A, bool SS>
int occupancy_short() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, short_kernel<A, SS>, kThreads, 0) != hipSuccess) return 1;
  return n > 0 ? n : 1;
}

template <bool SS>
int occupancy_short_algo(int algo) {
  switch (algo) {
    case kAdamW: return occupancy_short<kAdamW, SS>();
    case kLion: return occupancy_short<kLion, SS>();
    case kMomentum: return occupancy_short<kMomentum, SS>();
  }
  return 1;
}

template <Kind K, int A, bool SS>
hipError_t launch_kind(const DevTensor* list, int n, int64_t total_blocks, const StepScalars& sc,
                       hipStream_t stream, int num_cu, int resident, int range_ok, const uint32_t* map) {
  const int64_t grid = launch_groups<K, A, SS>(total_blocks, num_cu, resident);
  hipLaunchKernelGGL((step_kernel<K, A, SS>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream,
                     list, n, total_blocks, sc, range_ok, map);
  return hipGetLastError();
}

template <Kind K, int A, bool SS>
int occupancy_kind() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, step_kernel<K, A, SS>, kThreads, 0) != hipSuccess)
    return 1;
  return n > 0 ? n : 1;
}

// Kernel of (kind, algorithm, state rounding): the bf16 and fp32 kinds have
// no 8-bit state and always take SS = false.
template <Kind K, bool SS>
hipError_t launch_algo(int algo, const DevTensor* list, int n, int64_t total_blocks, const StepScalars& sc,
                       hipStream_t stream, int num_cu, int resident, int range_ok, const uint32_t* map) {
  switch (algo) {
    case kAdamW: return launch_kind<K, kAdamW, SS>(list, n, total_blocks, sc, stream, num_cu, resident, range_ok, map);
    case kLion: return launch_kind<K, kLion, SS>(list, n, total_blocks, sc, stream, num_cu, resident, range_ok, map);
    case kMomentum:
      return launch_kind<K, kMomentum, SS>(list, n, total_blocks, sc, stream, num_cu, resident, range_ok, map);
  }
  return hipErrorInvalidValue;
}

template <Kind K, bool SS>
int occupancy_algo(int algo) {
  switch (algo) {
    case kAdamW: return occupancy_kind<K, kAdamW, SS>();
    case kLion: return occupancy_kind<K, kLion, SS>();
    case kMomentum: return occupancy_kind<K, kMomentum, SS>();
  }
  return 1;
}

}  // namespace

// Descriptor lists of the entry point that allocates nothing: 8192
// descriptors of 80 bytes (640 KiB) per device, held until the process ends.
// In host code the array's name is only a host-side stand-in; kernels get
// its device address, taken below with hipGetSymbolAddress.
static __device__ __align__(256) DevTensor scratch[kScratchDescs];

hipError_t upload_tables(const uint8_t* host_tables) {
  return hipMemcpyToSymbol(HIP_SYMBOL(g_tables), host_tables, kTableBytesSR, 0, hipMemcpyHostToDevice);
}

hipError_t scratch_address(DevTensor** out) {
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  *out = e == hipSuccess ? static_cast<DevTensor*>(ptr) : nullptr;
  return e;
}

hipError_t launch_step(Kind kind, int algo, const DevTensor* list, int n, int64_t total_blocks,
                       const StepScalars& sc, hipStream_t stream, int num_cu, int resident,
                       const uint32_t* map) {
  if (n <= 0 || total_blocks <= 0) return hipSuccess;
  // the fast AdamW paths need eps well inside the normal range, a bounded
  // second-moment correction, decay and step size (they then check each
  // block's own values)
  const int range_ok = (sc.eps >= 0x1p-60f && sc.eps <= 0x1p+60f && sc.rbc2 <= 0x1p+20f &&
                        sc.lrwd <= 1.0f && sc.step_size <= 0x1p+26f) ? 1 : 0;
  const bool ss = sc.state_round != 0;
  switch (kind) {
    case Kind::k8bit:
      return ss ? launch_algo<Kind::k8bit, true>(algo, list, n, total_blocks, sc, stream, num_cu, resident, range_ok, map)
                : launch_algo<Kind::k8bit, false>(algo, list, n, total_blocks, sc, stream, num_cu, resident, range_ok, map);
    case Kind::k8bitTail:
      // its kernel reads entry b for block b: one block per entry
      if (total_blocks != n) return hipErrorInvalidValue;
      return ss ? launch_algo<Kind::k8bitTail, true>(algo, list, n, total_blocks, sc, stream, num_cu, resident, range_ok, map)
                : launch_algo<Kind::k8bitTail, false>(algo, list, n, total_blocks, sc, stream, num_cu, resident, range_ok, map);
    case Kind::k8bitShort:
      // one block per entry
      if (total_blocks != n) return hipErrorInvalidValue;
      return ss ? launch_short_algo<true>(algo, list, n, sc, stream, resident, range_ok)
                : launch_short_algo<false>(algo, list, n, sc, stream, resident, range_ok);
    case Kind::kBf16:
      return launch_algo<Kind::kBf16, false>(algo, list, n, total_blocks, sc, stream, num_cu, resident, range_ok, map);
    case Kind::kFp32:
      return launch_algo<Kind::kFp32, false>(algo, list, n, total_blocks, sc, stream, num_cu, resident, range_ok, map);
  }
  return hipErrorInvalidValue;
}

int occupancy_per_cu(Kind kind, int algo, bool state_sr) {
  switch (kind) {
    case Kind::k8bit:
      return state_sr ? occupancy_algo<Kind::k8bit, true>(algo) : occupancy_algo<Kind::k8bit, false>(algo);
    case Kind::k8bitTail:
      return state_sr ? occupancy_algo<Kind::k8bitTail, true>(algo) : occupancy_algo<Kind::k8bitTail, false>(algo);
    case Kind::k8bitShort: return state_sr ? occupancy_short_algo<true>(algo) : occupancy_short_algo<false>(algo);
    case Kind::kBf16: return occupancy_algo<Kind::kBf16, false>(algo);
    case Kind::kFp32: return occupancy_algo<Kind::kFp32, false>(algo);
  }
  return 1;
}

}  // namespace opt8
