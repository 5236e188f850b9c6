// Measurement aid: a plain streaming read, used to measure the HBM read
// rate this GPU actually reaches on a buffer the size of one decode step's
// latents (the ceiling the attention kernels are compared with).
#include "common.h"
#include "kernels.h"

namespace starkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int SR_UNROLL = 8;

// Each thread reads SR_UNROLL 16-byte words spaced one block-stride apart,
// all issued before any is used, then moves on by the grid stride.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const size_t chunk = (size_t)256 * SR_UNROLL;
  for (size_t base = (size_t)blockIdx.x * chunk; base < n16; base += (size_t)gridDim.x * chunk) {
    u32x4 v[SR_UNROLL];
#pragma unroll
    for (int u = 0; u < SR_UNROLL; ++u) {
      const size_t i = base + (size_t)u * 256 + threadIdx.x;
      v[u] = (i < n16) ? src[i] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < SR_UNROLL; ++u) acc ^= v[u];
  }
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == 0x9e3779b9u) sink[blockIdx.x & 1023] = x;  // practically never taken; keeps the loads live
}

hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  // enough work groups for every CU, each sweeping 32 KiB per trip
  const size_t chunks = (n16 + 256 * SR_UNROLL - 1) / (256 * SR_UNROLL);
  const unsigned grid = (unsigned)(chunks < 2048 ? chunks : 2048);
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, st, (const u32x4*)src, n16,
                     (uint32_t*)sink);
  return hipGetLastError();
}

}  // namespace starkv
