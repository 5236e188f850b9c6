// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
// Nothing here is exported from the shared library.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace starkv {

// One compiled shape instance: heads, head size, key rank, value rank.
struct ShapeKey {
  int H, d, rk, rv;
};

// Split plan of one decode call: pages_per_split consecutive pages per work
// group, num_splits work groups per sequence.
struct DecodePlan {
  int pages_per_split;
  int num_splits;
  int variant;  // split-kernel variant (0 = default)
};

// Byte offsets of the decode workspace regions.
struct DecodeWorkspace {
  size_t qt_off, ml_off, acc_off, z_off, total;
};

struct PrefillWorkspace {
  size_t qt_off, z_off, total;
};

bool shape_supported(const ShapeKey& s);
DecodePlan plan_decode(const ShapeKey& s, int batch, int max_seq_len, int block_size);
DecodeWorkspace decode_workspace_layout(const ShapeKey& s, int batch, const DecodePlan& p);
PrefillWorkspace prefill_workspace_layout(const ShapeKey& s, int total_q);

// Timing hook: events recorded around one kernel of a call (profiling aid).
struct TimingHook {
  hipEvent_t start = nullptr, stop = nullptr;
  int which = 0;
};
extern TimingHook g_timing;
enum { TIME_NONE = 0, TIME_DECODE_SPLIT = 1, TIME_PREFILL_ATTN = 2, TIME_APPEND = 3 };

// Launch `kernel` on `st`.  When the timing hook selects `which`, the launch
// goes through hipExtLaunchKernelGGL so that the hook's two events carry the
// dispatch's own begin and end timestamps (no event packets around it).
template <typename... KArgs, typename... Args>
inline void launch_hooked(int which, void (*kernel)(KArgs...), dim3 grid, dim3 block,
                          hipStream_t st, Args... args) {
  if (g_timing.which == which && g_timing.start && g_timing.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, g_timing.start, g_timing.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
}

hipError_t launch_qproj(const ShapeKey& s, const void* q, const void* U, int n_tokens,
                        float scale, void* qt, hipStream_t st);

hipError_t launch_decode(const ShapeKey& s, const DecodePlan& p, const void* qt,
                         const void* k_cache, const void* v_cache, const void* W,
                         const int32_t* block_tables, int max_blocks, const int32_t* seq_lens,
                         int num_blocks, int batch, float* ml, float* acc, float* z, void* out,
                         hipStream_t st);

// out[n, h, :] = W_h z[n, h, :]; wide_rows picks the prefill tiling (one
// work group per head and 64 tokens) over the decode tiling (16 rows).
hipError_t launch_upproj(const ShapeKey& s, const void* W, const float* z, int n_tokens,
                         bool wide_rows, void* out, hipStream_t st);

// Measurement aid: read `bytes` (a multiple of 16) with 16-byte loads and
// fold them into one word per work group, so nothing is optimised away.
hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, hipStream_t st);

hipError_t launch_append(const ShapeKey& s, const void* k, const void* v, const void* U,
                         const void* W, const int64_t* slots, int n_tokens, int num_blocks,
                         void* k_cache, void* v_cache, hipStream_t st);

hipError_t launch_prefill(const ShapeKey& s, const void* qt, const int32_t* qsl, int total_q,
                          int max_query_len, const void* k_cache, const void* v_cache,
                          const void* W, const int32_t* block_tables, int max_blocks,
                          const int32_t* seq_lens, int num_blocks, int batch, float* z,
                          void* out, hipStream_t st);

}  // namespace starkv
