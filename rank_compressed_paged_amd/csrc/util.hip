// Measurement aid: a plain streaming read, used to measure the HBM read
// rate this GPU actually reaches on a buffer the size of one decode step's
// latents (the ceiling the attention kernels are compared with).
#include "common.h"
#include "kernels.h"

namespace starkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Each thread keeps SR_UNROLL 16-byte non-temporal loads in flight (each
// request spaced one work-group width apart, so a wave's loads cover whole
// contiguous KiB), then moves on by the grid stride.  512-thread work groups,
// at most 2048 of them.  Of the configurations swept on MI355X (256-1024
// threads, 8 or 16 loads in flight, plain or non-temporal loads, 256-4096
// work groups) this one read fastest: 5.9 TB/s over 168 MB and 7.0 TB/s
// over 2 GB, flushed.
constexpr int SR_BLOCK = 512;
constexpr int SR_UNROLL = 16;

__global__ __launch_bounds__(SR_BLOCK) void stream_read_kernel(const u32x4* __restrict__ src,
                                                               size_t n16,
                                                               uint32_t* __restrict__ sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const size_t chunk = (size_t)SR_BLOCK * SR_UNROLL;
  for (size_t base = (size_t)blockIdx.x * chunk; base < n16; base += (size_t)gridDim.x * chunk) {
    u32x4 v[SR_UNROLL];
#pragma unroll
    for (int u = 0; u < SR_UNROLL; ++u) {
      const size_t i = base + (size_t)u * SR_BLOCK + threadIdx.x;
      v[u] = (i < n16) ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < SR_UNROLL; ++u) acc ^= v[u];
  }
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == 0x9e3779b9u) sink[blockIdx.x & 1023] = x;  // practically never taken; keeps the loads live
}

// One-wave kernel that does nothing: the dispatch the timing hook's start
// event is bound to, so the timed span of the read starts where a decode
// split kernel's does (at the end of the dispatch just before it).
__global__ void stream_anchor_kernel() {}

hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const size_t chunks = (n16 + SR_BLOCK * SR_UNROLL - 1) / (SR_BLOCK * SR_UNROLL);
  const unsigned grid = (unsigned)(chunks < 2048 ? chunks : 2048);
  if (g_timing.which == TIME_STREAM_READ)
    launch_hooked(TIME_NONE, TIME_STREAM_READ, stream_anchor_kernel, dim3(1), dim3(64), st);
  launch_hooked(TIME_STREAM_READ, TIME_NONE, stream_read_kernel, dim3(grid), dim3(SR_BLOCK), st,
                (const u32x4*)src, n16, (uint32_t*)sink);
  return hipGetLastError();
}

}  // namespace starkv
