// Attainable-bandwidth probes: plain streaming kernels with a chosen number of
// read and write streams of 16-byte words and no arithmetic beyond a xor
// (each thread moves four words per stream and iteration, a wave touching 4
// contiguous 1 KiB segments per stream, non-temporal loads and stores, a
// grid-stride loop), and a kernel with the 8-bit step's own access pattern and
// no arithmetic.  They give the practical HBM ceilings the step kernels are
// compared with.  Measurement infrastructure only: not part of the
// optimizer's C ABI.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kThreads)
stream_kernel(const u32x4* __restrict__ in, u32x4* __restrict__ out, int64_t n, int nin, int nout) {
  const int64_t chunk = static_cast<int64_t>(kThreads) * kUnroll;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * chunk;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * chunk; base < n; base += stride) {
    u32x4 acc[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc[u] = static_cast<u32x4>(0u);
    for (int s = 0; s < nin; ++s) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = base + u * kThreads + threadIdx.x;
        if (i < n) acc[u] ^= __builtin_nontemporal_load(&in[s * n + i]);
      }
    }
    for (int s = 0; s < nout; ++s) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = base + u * kThreads + threadIdx.x;
        if (i < n) __builtin_nontemporal_store(acc[u], &out[s * n + i]);
      }
    }
  }
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) u32x4 g_u32x4;
typedef __attribute__((address_space(1))) u32x2 g_u32x2;

// The 8-bit step's memory traffic without its arithmetic: lane l holding
// elements r*512 + 8l .. +7 (r = 0..3) of a 2048-element block; per block it
// reads 4 KiB of bf16 gradient, 4 KiB of bf16 parameter and 2 KiB each of m
// and v codes, and writes the parameter and both code arrays back (a xor of
// what it read), non-temporally, through the global address space.  Each wave
// takes kB adjacent blocks per iteration (1 as the step kernel does; 2 moves
// more bytes per wave and is faster without arithmetic) and the waves stride
// over the blocks.
template <int kB>
__global__ void __launch_bounds__(kThreads)
pattern_kernel(const uint16_t* __restrict__ g, uint16_t* __restrict__ p, uint8_t* __restrict__ m,
               uint8_t* __restrict__ v, int64_t nblocks) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = static_cast<int64_t>(gridDim.x) * (kThreads / 64);
  const int64_t w = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  for (int64_t b = w * kB; b + kB <= nblocks; b += nw * kB) {
    u32x4 G[4 * kB], P[4 * kB];
    u32x2 M[4 * kB], V[4 * kB];
#pragma unroll
    for (int i = 0; i < 4 * kB; ++i) {
      const int64_t e = (b + i / 4) * 2048 + (i % 4) * 512 + lane * 8;
      G[i] = __builtin_nontemporal_load((const g_u32x4*)(g + e));
      M[i] = __builtin_nontemporal_load((const g_u32x2*)(m + e));
      V[i] = __builtin_nontemporal_load((const g_u32x2*)(v + e));
      P[i] = __builtin_nontemporal_load((const g_u32x4*)(p + e));
    }
#pragma unroll
    for (int i = 0; i < 4 * kB; ++i) {
      const int64_t e = (b + i / 4) * 2048 + (i % 4) * 512 + lane * 8;
      __builtin_nontemporal_store(P[i] ^ G[i], (g_u32x4*)(p + e));
      __builtin_nontemporal_store(M[i] ^ G[i].xy, (g_u32x2*)(m + e));
      __builtin_nontemporal_store(V[i] ^ G[i].zw, (g_u32x2*)(v + e));
    }
  }
}

}  // namespace

// in: nin streams of `words` 16-byte words back to back; out: nout streams likewise.
extern "C" int opt8_probe_stream(const void* in, void* out, int64_t words, int nin, int nout,
                                 int grid, void* stream) {
  if (!in || !out || words <= 0 || nin < 1 || nout < 1 || nin > 8 || nout > 8 || grid < 1) return -1;
  hipLaunchKernelGGL(stream_kernel, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(in), static_cast<u32x4*>(out), words, nin, nout);
  return hipGetLastError() == hipSuccess ? 0 : -9;
}

// g, p: bf16[nblocks * 2048]; m, v: u8[nblocks * 2048]; p, m and v are rewritten.
// blocks_per_wave: 1 or 2 adjacent blocks per wave and iteration (nblocks must
// then be a multiple of it).
extern "C" int opt8_probe_pattern(const void* g, void* p, void* m, void* v, int64_t nblocks, int grid,
                                  int blocks_per_wave, void* stream) {
  if (!g || !p || !m || !v || nblocks <= 0 || grid < 1) return -1;
  if (blocks_per_wave != 1 && blocks_per_wave != 2) return -1;
  if (nblocks % blocks_per_wave) return -1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (blocks_per_wave == 1)
    hipLaunchKernelGGL(pattern_kernel<1>, dim3(grid), dim3(kThreads), 0, st, static_cast<const uint16_t*>(g),
                       static_cast<uint16_t*>(p), static_cast<uint8_t*>(m), static_cast<uint8_t*>(v), nblocks);
  else
    hipLaunchKernelGGL(pattern_kernel<2>, dim3(grid), dim3(kThreads), 0, st, static_cast<const uint16_t*>(g),
                       static_cast<uint16_t*>(p), static_cast<uint8_t*>(m), static_cast<uint8_t*>(v), nblocks);
  return hipGetLastError() == hipSuccess ? 0 : -9;
}
