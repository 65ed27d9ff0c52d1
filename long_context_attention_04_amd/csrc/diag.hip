// Measurement helper: the HBM streaming-read ceiling of this device, against which
// the hot path's bandwidth-bound kernels are judged (their algorithmic bytes over
// their time, beside the nominal 8 TB/s).
#include "common.h"
#include "kernels.h"

namespace csa {

namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;

// Every 16-byte word of [p, p + n16) read once (non-temporally), grid-stride, eight
// loads in flight per thread; one word per workgroup written so nothing is elided.
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const v4i* __restrict__ p, size_t n16,
                                                                     uint32_t* __restrict__ sink) {
  int acc = 0;
  const size_t stride = (size_t)gridDim.x * kStreamThreads * kStreamUnroll;
  for (size_t base = (size_t)blockIdx.x * kStreamThreads * kStreamUnroll + threadIdx.x; base < n16; base += stride) {
    v4i v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const size_t i = base + (size_t)u * kStreamThreads;
      v[u] = i < n16 ? __builtin_nontemporal_load(p + i) : (v4i){0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  acc = (int)wave_reduce_u32<true>((uint32_t)acc);  // any combine works: the value is never used
  if (threadIdx.x == 0) sink[blockIdx.x] = (uint32_t)acc;
}

}  // namespace

hipError_t launch_stream_read(const void* data, size_t bytes, uint32_t* sink, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamReadBlocks), dim3(kStreamThreads), 0, s, (const v4i*)data, n16,
                     sink);
  return hipGetLastError();
}

}  // namespace csa
