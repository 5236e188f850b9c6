// Host-side validation of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer: every entry point with good and bad arguments
// that fail (or finish) before any kernel launch, plus the size queries over
// a sweep of shapes and sizes (integer overflow in the planners or workspace
// layouts would be undefined behaviour).  No GPU is needed.  Exits non-zero
// on the first status that differs from the expected one; a sanitizer error
// aborts the program.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <initializer_list>

#include "starkv.h"

static int failures = 0;

#define EXPECT(call, want)                                                              \
  do {                                                                                  \
    const int got_ = (int)(call);                                                       \
    if (got_ != (int)(want)) {                                                          \
      std::fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call,   \
                   got_, (int)(want));                                                  \
      ++failures;                                                                       \
    }                                                                                   \
  } while (0)

static starkv_dims dims(int H, int d, int rk, int rv, int nb, int bs = 16, int hkv = 0) {
  starkv_dims x;
  x.num_heads = H;
  x.head_dim = d;
  x.rank_k = rk;
  x.rank_v = rv;
  x.block_size = bs;
  x.num_blocks = nb;
  x.num_kv_heads = hkv;
  return x;
}

int main() {
  void* const F = (void*)(uintptr_t)0x10000;  // aligned, never dereferenced
  void* const M = (void*)(uintptr_t)0x10008;  // misaligned
  const int32_t* Fi = (const int32_t*)F;
  const int64_t* Fl = (const int64_t*)F;

  EXPECT(starkv_abi_version(), STARKV_ABI_VERSION);
  for (int s = -3; s < 12; ++s)
    if (!starkv_status_string(s)) ++failures;

  // shapes: tuned, generic, and outside every limit
  const starkv_dims main_d = dims(32, 128, 64, 512, 8);
  EXPECT(starkv_shape_supported(nullptr), 0);
  EXPECT(starkv_shape_supported(&main_d), 1);
  starkv_dims odd = dims(28, 96, 48, 640, 8);
  EXPECT(starkv_shape_supported(&odd), 1);
  starkv_dims bad = dims(32, 100, 64, 512, 8);
  EXPECT(starkv_shape_supported(&bad), 0);
  starkv_dims neg = dims(-1, 128, 64, 512, 8);
  EXPECT(starkv_shape_supported(&neg), 0);

  // size queries over a sweep: no overflow, no out-of-range plan
  const int Hs[] = {1, 4, 28, 32, 64};
  const int ds[] = {32, 64, 96, 128, 256};
  const int batches[] = {0, 1, 3, 16, 64, 1000, 65535};
  const int lens[] = {0, 1, 15, 16, 17, 2048, 32768, 1 << 20, 1 << 28};
  size_t bytes = 0;
  for (int H : Hs)
    for (int d : ds) {
      const starkv_dims x = dims(H, d, (d / 2) & ~7, H * d < 1024 ? H * d : 1024, 8);
      for (int B : batches)
        for (int L : lens) {
          const starkv_status st = starkv_decode_workspace_size(&x, B, L, &bytes);
          if (st != STARKV_OK && st != STARKV_ERR_UNSUPPORTED) ++failures;
          int32_t pps = 0, ns = 0;
          (void)starkv_decode_plan(&x, B, L, &pps, &ns);
          (void)starkv_prefill_workspace_size(&x, B, B * 16, L, &bytes);
        }
      for (int n : {0, 1, 16, 64, 65, 1792, 1793, 2816, 2817, 4096, 1 << 20})
        (void)starkv_append_workspace_size(&x, n, &bytes);
      (void)starkv_fit_workspace_size(&x, &bytes);
    }
  for (int pps : {0, 1, 7, 256})
    for (int m : {0, 1, 2, 4, 8})
      for (int l : {0, 2, 3}) {
        starkv_decode_config cfg = {pps, m, l};
        EXPECT(starkv_decode_workspace_size_cfg(&main_d, 16, 2048, &cfg, &bytes), STARKV_OK);
      }
  starkv_decode_config badcfg = {257, 0, 0};
  EXPECT(starkv_decode_workspace_size_cfg(&main_d, 16, 2048, &badcfg, &bytes), STARKV_ERR_ARG);
  EXPECT(starkv_decode_workspace_size(&main_d, 16, 2048, nullptr), STARKV_ERR_NULL);

  // decode: each failure before any launch
  size_t need = 0;
  EXPECT(starkv_decode_workspace_size(&main_d, 16, 2048, &need), STARKV_OK);
  EXPECT(starkv_decode_attn(&main_d, F, F, F, F, F, Fi, 128, Fi, 16, 2048, 0.088f, F, F, need - 1,
                            nullptr),
         STARKV_ERR_WORKSPACE);
  EXPECT(starkv_decode_attn(&main_d, nullptr, F, F, F, F, Fi, 128, Fi, 16, 2048, 0.088f, F, F,
                            need, nullptr),
         STARKV_ERR_NULL);
  EXPECT(starkv_decode_attn(&main_d, M, F, F, F, F, Fi, 128, Fi, 16, 2048, 0.088f, F, F, need,
                            nullptr),
         STARKV_ERR_ALIGN);
  EXPECT(starkv_decode_attn(&main_d, F, F, F, F, F, Fi, 100, Fi, 16, 2048, 0.088f, F, F, need,
                            nullptr),
         STARKV_ERR_DIMS);
  EXPECT(starkv_decode_attn(&main_d, F, F, F, F, F, Fi, 128, Fi, 16, 2048, 0.f, F, F, need,
                            nullptr),
         STARKV_ERR_ARG);
  EXPECT(starkv_decode_attn(&bad, F, F, F, F, F, Fi, 128, Fi, 16, 2048, 0.088f, F, F, need,
                            nullptr),
         STARKV_ERR_UNSUPPORTED);
  EXPECT(starkv_decode_attn(nullptr, F, F, F, F, F, Fi, 128, Fi, 16, 2048, 0.088f, F, F, need,
                            nullptr),
         STARKV_ERR_NULL);
  EXPECT(starkv_decode_attn(&main_d, F, F, F, F, F, Fi, 128, Fi, 0, 2048, 0.088f, F, F, 0,
                            nullptr),
         STARKV_OK);
  starkv_decode_config cfg5 = {0, 5, 0};
  EXPECT(starkv_decode_attn_cfg(&main_d, F, F, F, F, F, Fi, 128, Fi, 16, 2048, 0.088f, &cfg5, F,
                                F, need, nullptr),
         STARKV_ERR_ARG);
  EXPECT(starkv_decode_attn_fp8(&main_d, F, F, F, F, F, Fi, 128, Fi, 16, 2048, 0.088f, -1.f, 1.f,
                                F, F, need, nullptr),
         STARKV_ERR_ARG);
  EXPECT(starkv_decode_attn_noalloc(&main_d, F, F, F, F, F, Fi, 256, Fi, 256, 4096, 0.088f, F,
                                    nullptr),
         STARKV_ERR_WORKSPACE);
  EXPECT(starkv_decode_attn_noalloc(&main_d, nullptr, F, F, F, F, Fi, 128, Fi, 16, 2048, 0.088f,
                                    F, nullptr),
         STARKV_ERR_NULL);

  // append
  size_t aws = 0;
  EXPECT(starkv_append_workspace_size(&main_d, 16, &aws), STARKV_OK);
  EXPECT(starkv_append(&main_d, F, F, F, F, Fl, -1, F, F, F, aws, nullptr), STARKV_ERR_DIMS);
  EXPECT(starkv_append(&main_d, F, nullptr, F, F, Fl, 16, F, F, F, aws, nullptr), STARKV_ERR_NULL);
  EXPECT(starkv_append(&main_d, F, F, F, M, Fl, 16, F, F, F, aws, nullptr), STARKV_ERR_ALIGN);
  EXPECT(starkv_append(&main_d, F, F, F, F, Fl, 16, F, F, F, aws - 1, nullptr),
         STARKV_ERR_WORKSPACE);
  EXPECT(starkv_append(&main_d, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr,
                       nullptr, 0, nullptr),
         STARKV_OK);
  EXPECT(starkv_append_fp8(&main_d, F, F, F, F, Fl, 16, 0.f, 1.f, F, F, F, aws, nullptr),
         STARKV_ERR_ARG);

  // prefill
  size_t pws = 0;
  EXPECT(starkv_prefill_workspace_size(&main_d, 16, 4096, 4352, &pws), STARKV_OK);
  EXPECT(starkv_prefill_attn(&main_d, F, Fi, 4096, 256, F, F, F, F, Fi, 272, Fi, 16, 4352, 0.088f,
                             F, F, pws - 1, nullptr),
         STARKV_ERR_WORKSPACE);
  EXPECT(starkv_prefill_attn(&main_d, F, Fi, 4096, 0, F, F, F, F, Fi, 272, Fi, 16, 4352, 0.088f,
                             F, F, pws, nullptr),
         STARKV_ERR_DIMS);
  EXPECT(starkv_prefill_attn(&main_d, F, Fi, 4096, 5000, F, F, F, F, Fi, 272, Fi, 16, 4352,
                             0.088f, F, F, pws, nullptr),
         STARKV_ERR_DIMS);
  EXPECT(starkv_prefill_attn_fp8(&main_d, F, Fi, 4096, 256, F, F, F, F, Fi, 272, Fi, 16, 4352,
                                 0.088f, 1.f, 0.f, F, F, pws, nullptr),
         STARKV_ERR_ARG);

  // fit
  size_t fws = 0;
  EXPECT(starkv_fit_workspace_size(&main_d, &fws), STARKV_OK);
  EXPECT(starkv_fit_bases(&main_d, F, F, 4096, (const float*)F, (const float*)F, 4, F, F, F,
                          fws - 1, nullptr, nullptr, nullptr),
         STARKV_ERR_WORKSPACE);
  EXPECT(starkv_fit_bases(&main_d, F, F, 4096, (const float*)F, (const float*)F, 0, F, F, F, fws,
                          nullptr, nullptr, nullptr),
         STARKV_ERR_ARG);
  EXPECT(starkv_fit_bases(&main_d, F, F, 4096, (const float*)F, (const float*)F, 4, F, F, F, fws,
                          (int32_t*)((char*)F + 2), nullptr, nullptr),
         STARKV_ERR_ALIGN);
  EXPECT(starkv_fit_bases(&main_d, F, F, 4096, (const float*)F, (const float*)F, 4, F, F, F, fws,
                          nullptr, (float*)((char*)F + 2), nullptr),
         STARKV_ERR_ALIGN);

  // index checks
  const int64_t* Fs = (const int64_t*)F;
  uint32_t* Fu = (uint32_t*)F;
  starkv_dims nb100 = dims(1, 32, 8, 8, 100);
  EXPECT(starkv_check_indices(&nb100, Fi, 8, Fi, 4, 128, Fs, 16, nullptr, nullptr), STARKV_ERR_NULL);
  EXPECT(starkv_check_indices(nullptr, Fi, 8, Fi, 4, 128, Fs, 16, Fu, nullptr), STARKV_ERR_NULL);
  EXPECT(starkv_check_indices(&nb100, Fi, 8, Fi, 4, 129, Fs, 16, Fu, nullptr), STARKV_ERR_DIMS);
  EXPECT(starkv_check_indices(&nb100, Fi, 8, Fi, 4, 128, nullptr, 16, Fu, nullptr),
         STARKV_ERR_NULL);
  EXPECT(starkv_check_indices(&nb100, Fi, 8, Fi, 4, 128, Fs, -3, Fu, nullptr), STARKV_ERR_DIMS);
  EXPECT(starkv_check_indices(&nb100, Fi, 8, Fi, 4, 128, Fs, 16, (uint32_t*)M, nullptr),
         STARKV_ERR_ALIGN);

  // measurement hooks
  EXPECT(starkv_set_timing_events(nullptr, nullptr, 0), STARKV_OK);
  EXPECT(starkv_set_timing_events(nullptr, nullptr, 1), STARKV_ERR_NULL);
  EXPECT(starkv_set_timing_events(F, F, 9), STARKV_ERR_ARG);
  EXPECT(starkv_util_stream_read(nullptr, 16, F, nullptr), STARKV_ERR_NULL);
  EXPECT(starkv_util_stream_read(M, 16, F, nullptr), STARKV_ERR_ALIGN);

  if (failures) {
    std::fprintf(stderr, "%d unexpected statuses\n", failures);
    return 1;
  }
  std::printf("abi sanitize: all statuses as expected\n");
  return 0;
}
