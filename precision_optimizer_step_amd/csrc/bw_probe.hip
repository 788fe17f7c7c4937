// Attainable-bandwidth probe: plain streaming kernels with a chosen number of
// read and write streams of 16-byte words and no arithmetic beyond a xor.
// Each thread moves four words per stream and iteration (a wave touches 4
// contiguous 1 KiB segments per stream), with non-temporal loads and stores,
// over a grid-stride loop.  It gives the practical HBM ceiling the step
// kernels are compared with.  Measurement infrastructure only: not part of
// the optimizer's C ABI.
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

}  // namespace

// in: nin streams of `words` 16-byte words back to back; out: nout streams likewise.
extern "C" int opt8_probe_stream(const void* in, void* out, int64_t words, int nin, int nout,
                                 int grid, void* stream) {
  if (!in || !out || words <= 0 || nin < 1 || nout < 1 || nin > 8 || nout > 8 || grid < 1) return -1;
  hipLaunchKernelGGL(stream_kernel, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(in), static_cast<u32x4*>(out), words, nin, nout);
  return hipGetLastError() == hipSuccess ? 0 : -9;
}
