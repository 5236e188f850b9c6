// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
// Nothing here is exported from the shared library.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace starkv {

// One compiled shape instance: query heads, head size, key rank, value rank,
// key/value heads (H for multi-head attention; H / Hkv query heads share one
// key/value head under grouped-query attention).
struct ShapeKey {
  int H, d, rk, rv, Hkv;
};

// Split plan of one decode call: pages_per_split consecutive pages per work
// group, num_splits work groups per sequence.
struct DecodePlan {
  int pages_per_split;
  int num_splits;
  int finish_tb;     // sequences per work group of the merge + up-projection (1, 2, 4, 8)
  int finish_cb;     // splits per request round of each merging thread (4, 8, 16)
  int finish_nt;     // threads per work group of the merge (256, 512)
  int split_stride;  // split slots per sequence and head in the workspace: num_splits
                     // rounded up to a multiple of finish_cb times the split groups
  bool generic = false;  // the generic kernels (generic.hip), which use the first two fields
  bool fused = false;    // the split pass and the merge in one launch (finish_cb is then 4
                         // and finish_nt the split kernel's thread count)
};

// Split groups of the merge: when a work group has more threads than
// four-feature units (TB * RV / 4), the threads form up to 8 groups that
// merge disjoint, interleaved sets of splits, combined through LDS.
constexpr int finish_split_groups(int nt, int tb, int rv) {
  return (tb * rv / 4 >= nt) ? 1 : (nt / (tb * rv / 4) > 8 ? 8 : nt / (tb * rv / 4));
}

// The first bytes of every decode, prefill and append workspace are
// reserved: the few-token append keeps its arrival counters there, which
// must be zero when a workspace is first used and which every call leaves
// zero (no other call writes them).
constexpr size_t kWorkspaceHeaderBytes = 256;

// Byte offsets of the decode workspace regions.
struct DecodeWorkspace {
  size_t qt_off, ml_off, zp_off, sync_off, total;
};

// Threads per work group of the tuned decode split kernel of a shape.
int decode_threads(const ShapeKey& s);

struct PrefillWorkspace {
  size_t qt_off, z_off, total;
};

// Byte offsets of the workspace of the bases fit: the Gram matrices (fp32),
// two n x r fp32 buffers per side (Y = G Q and the orthonormalised Q), the
// fp64 row-slice partials of S = Y^T Y, the Schur-complement matrix A that
// the Cholesky factorisation updates in place, its factor L and the inverses
// of L's 64x64 diagonal blocks.
struct FitWorkspace {
  size_t gv_off, gk_off, qv_off[2], qk_off[2], sv_off, sk_off, av_off, ak_off, lv_off, lk_off,
      dv_off, dk_off, total;
};

// Storage of the latents: fp16, or FP8 E4M3 codes of latent / scale with one
// scale per tensor (keys, values).
struct LatentFormat {
  bool fp8 = false;
  float k_scale = 1.f, v_scale = 1.f;
};

bool shape_supported(const ShapeKey& s);
// force_pps > 0 fixes the pages per split, force_tb in {1, 2, 4, 8} the
// sequences per merge work group; 0 leaves either to the planner
// launches: 2 fuses the split pass and the merge into one kernel; anything
// else (the library's choice) keeps them in launches of their own
DecodePlan plan_decode(const ShapeKey& s, int batch, int max_seq_len, int block_size,
                       int force_pps = 0, int force_tb = 0, bool generic = false,
                       int launches = 0);
DecodeWorkspace decode_workspace_layout(const ShapeKey& s, int batch, const DecodePlan& p);
PrefillWorkspace prefill_workspace_layout(const ShapeKey& s, int total_q);

// Timing hook: events recorded around one kernel of a call (profiling aid).
struct TimingHook {
  hipEvent_t start = nullptr, stop = nullptr;
  int which = 0;
};
extern TimingHook g_timing;
enum {
  TIME_NONE = 0,
  TIME_DECODE_SPLIT = 1,
  TIME_PREFILL_ATTN = 2,
  TIME_APPEND = 3,
  TIME_FIT_GRAM = 4,
  TIME_STREAM_READ = 5
};

// Launch `kernel` on `st`.  Timing hook: when the hook selects `which`, its
// stop event is bound to this dispatch (hipExtLaunchKernelGGL), so it takes
// the dispatch's end timestamp; when it selects `precedes` (the kernel this
// launch comes immediately before in the same call), its start event is bound
// to this dispatch instead.  The timed span is then end-of-predecessor to
// end-of-kernel with no event packets between the two dispatches.
template <typename... KArgs, typename... Args>
inline void launch_hooked(int which, int precedes, void (*kernel)(KArgs...), dim3 grid,
                          dim3 block, hipStream_t st, Args... args) {
  hipEvent_t ev = nullptr;
  if (g_timing.start && g_timing.stop) {
    if (g_timing.which == which)
      ev = g_timing.stop;
    else if (precedes != TIME_NONE && g_timing.which == precedes)
      ev = g_timing.start;
  }
  if (ev)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, nullptr, ev, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
}

// launch_hooked with `lds` bytes of dynamic LDS.
template <typename... KArgs, typename... Args>
inline void launch_hooked_lds(int which, int precedes, void (*kernel)(KArgs...), dim3 grid,
                              dim3 block, size_t lds, hipStream_t st, Args... args) {
  hipEvent_t ev = nullptr;
  if (g_timing.start && g_timing.stop) {
    if (g_timing.which == which)
      ev = g_timing.stop;
    else if (precedes != TIME_NONE && g_timing.which == precedes)
      ev = g_timing.start;
  }
  if (ev)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, st, nullptr, ev, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
}

// Generic instances (any shape within their limits; see generic.hip).
bool generic_shape_ok(const ShapeKey& s);
int generic_head_groups(const ShapeKey& s);
hipError_t launch_generic_qproj(const ShapeKey& s, const void* q, const void* U, int n_tokens,
                                float scale, void* qt, int precedes, hipStream_t st);
// rows: decode sequences (qsl null) or prefill chunk queries (qsl the
// query start locations of `batch` requests); num_splits 1 fuses the merge
hipError_t launch_generic_attn(const ShapeKey& s, const void* qt, const int32_t* qsl, int rows,
                               const void* k_cache, const void* v_cache, const void* W,
                               const int32_t* block_tables, int max_blocks,
                               const int32_t* seq_lens, int num_blocks, int batch,
                               int pages_per_split, int num_splits, float* ml, float* zpart,
                               void* out, const LatentFormat& fmt, int which, hipStream_t st);

// Chunked prefill on the generic kernels for r_k up to 128 and r_v up to 1024
// (generic_prefill_tiled; table rows of at most 8192 pages, whose block ids
// the kernel stages in LDS): 64 chunk queries of one head per work group, the
// up-projection in the kernel's epilogue.
bool generic_prefill_tiled(const ShapeKey& s, int max_blocks);
hipError_t launch_generic_prefill(const ShapeKey& s, const void* qt, const int32_t* qsl,
                                  int total_q, int max_query_len, const void* k_cache,
                                  const void* v_cache, const void* W,
                                  const int32_t* block_tables, int max_blocks,
                                  const int32_t* seq_lens, int num_blocks, int batch, void* out,
                                  const LatentFormat& fmt, int which, hipStream_t st);

// `precedes`: the hooked kernel that follows this launch in the call.
// w_prefetch: the W that the step's merge will read (decode), fetched into
// the L2 of the XCD that will use each head's block; null for none
// zero / n_zero: words that the launch clears (the fused decode step's
// counters), or none
hipError_t launch_qproj(const ShapeKey& s, const void* q, const void* U, int n_tokens,
                        float scale, void* qt, int precedes, hipStream_t st,
                        const void* w_prefetch = nullptr, uint32_t* zero = nullptr,
                        int n_zero = 0);

hipError_t launch_decode(const ShapeKey& s, const DecodePlan& p, const void* qt,
                         const void* k_cache, const void* v_cache, const void* W,
                         const int32_t* block_tables, int max_blocks, const int32_t* seq_lens,
                         int num_blocks, int batch, float* ml, void* zpart, void* out,
                         const LatentFormat& fmt, uint32_t* sync, hipStream_t st);

// out[n, h, :] = W_h z[n, h, :] for the many tokens of a prefill call: z is
// fp16, tiled in the A-operand order of the up-projection's 32x32x16
// products, [H][ceil(n/32)][RV/16][64][8], where lane l of 16-feature chunk
// kc of a 32-token block holds token l%32, features 16*kc + 8*(l/32) .. +7
// (prefill writes it that way).
hipError_t launch_upproj_tiled(const ShapeKey& s, const void* W, const void* z_tiled,
                               int n_tokens, void* out, hipStream_t st);

// Scratch of the no-allocation decode entry point: a device array of the
// library, one per GPU; *ptr receives its device address on the current
// device (taken once per device).
constexpr size_t kNoallocScratchBytes = (size_t)32 << 20;
hipError_t noalloc_scratch(void** ptr);

// Index checks (debugging aid): scan block tables, lengths and slots, write
// the four-word report described with starkv_check_indices.
hipError_t launch_check_indices(const int32_t* block_tables, int max_blocks,
                                const int32_t* seq_lens, int batch, int max_seq_len,
                                int num_blocks, const int64_t* slots, int n_slots,
                                uint32_t* report, hipStream_t st);

// Measurement aid: read `bytes` (a multiple of 16) with 16-byte loads and
// fold them into one word per work group, so nothing is optimised away.
hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, hipStream_t st);

// Workspace bytes of an append of n_tokens tokens (the few-token path's
// value partials; 0 above that path's token limit).
size_t append_workspace_bytes(const ShapeKey& s, int n_tokens);

hipError_t launch_append(const ShapeKey& s, const void* k, const void* v, const void* U,
                         const void* W, const int64_t* slots, int n_tokens, int num_blocks,
                         void* k_cache, void* v_cache, const LatentFormat& fmt, void* workspace,
                         hipStream_t st);

FitWorkspace fit_workspace_layout(const ShapeKey& s);

// Top-r_k eigenspaces of each head's key second-moment matrix and the top-r_v
// eigenspace of the joint value one, by subspace iteration from u0 / w0.
// residual_out (optional, 2 floats): the relative invariant-subspace residual
// of the returned bases, keys (largest over heads) then values.
hipError_t launch_fit(const ShapeKey& s, const void* k, const void* v, int n_samples,
                      const float* u0, const float* w0, int iters, void* U, void* W,
                      void* workspace, int* info, float* residual_out, hipStream_t st);

hipError_t launch_prefill(const ShapeKey& s, const void* qt, const int32_t* qsl, int total_q,
                          int max_query_len, const void* k_cache, const void* v_cache,
                          const void* W, const int32_t* block_tables, int max_blocks,
                          const int32_t* seq_lens, int num_blocks, int batch, void* z,
                          void* out, const LatentFormat& fmt, hipStream_t st);

}  // namespace starkv
