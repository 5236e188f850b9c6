// C ABI of libstarkv: host-side validation, split planning, workspace
// layout and kernel launches.  Every check runs before the first HIP call,
// so a rejected call enqueues nothing; no C++ exception crosses the ABI.
#include <cmath>
#include <initializer_list>

#include "../../include/starkv.h"
#include "kernels.h"

namespace starkv {

static_assert(kNoallocScratchBytes == STARKV_NOALLOC_SCRATCH_BYTES, "one scratch size");

TimingHook g_timing;

// Tuned instances: the main shape at two rank profiles (r_k, r_v) =
// (64, 512) and (32, 256), the former also with 8 key/value heads, and the
// tiny shape with 4 or 2 key/value heads.
static bool tuned_shape(const ShapeKey& s) {
  return (s.H == 32 && s.d == 128 && s.rk == 64 && s.rv == 512 && (s.Hkv == 32 || s.Hkv == 8)) ||
         (s.H == 32 && s.d == 128 && s.rk == 32 && s.rv == 256 && s.Hkv == 32) ||
         (s.H == 4 && s.d == 64 && s.rk == 16 && s.rv == 64 && (s.Hkv == 4 || s.Hkv == 2));
}

// Tuned instances over FP8 latents: the main shape (both head layouts) and
// the tiny one.
static bool tuned_fp8(const ShapeKey& s) {
  return (s.H == 32 && s.d == 128 && s.rk == 64 && s.rv == 512 && (s.Hkv == 32 || s.Hkv == 8)) ||
         (s.H == 4 && s.d == 64 && s.rk == 16 && s.rv == 64 && s.Hkv == 4);
}

// Every other shape within the generic kernels' limits runs on them (fp16
// and FP8 alike).
bool shape_supported(const ShapeKey& s) { return tuned_shape(s) || generic_shape_ok(s); }
static bool fp8_decode_supported(const ShapeKey& s) { return tuned_fp8(s) || generic_shape_ok(s); }
static bool use_generic(const ShapeKey& s, bool fp8) {
  return fp8 ? !tuned_fp8(s) : !tuned_shape(s);
}

// The append sees only the key/value heads: the key/value view (Hkv, d, r_k,
// r_v) of a tuned shape, or any view within the generic limits (the tiled
// append kernel takes every size at run time).
static bool kv_shape_supported(const ShapeKey& s) {
  return (s.d == 128 && s.rk == 64 && s.rv == 512 && (s.Hkv == 32 || s.Hkv == 8)) ||
         (s.d == 128 && s.rk == 32 && s.rv == 256 && s.Hkv == 32) ||
         (s.d == 64 && s.rk == 16 && s.rv == 64 && (s.Hkv == 4 || s.Hkv == 2)) ||
         generic_shape_ok(ShapeKey{s.Hkv, s.d, s.rk, s.rv, s.Hkv});
}

static inline int cdiv(long a, long b) { return (int)((a + b - 1) / b); }

// Number of compute units of the current device (queried once per device;
// 256, the MI355X count, when no device answers).
static int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// The merge + up-projection tile.  TB sequences per work group: 1 when the
// batch is too small to give every CU a (head, sequence) pair, else the
// widest of 2, 4, 8 that still gives a work group per CU (each work group
// reads all of W_h, so wide groups cut that traffic at large batch), unless
// the caller fixes TB.  The merge requests CB splits per round and
// thread; with many splits (small batch, long sequences) the work group
// grows to 512 threads whose split groups take disjoint sets of splits, so
// the partials are requested in fewer rounds (1024 threads would leave 128
// registers per thread, too few for the operands in flight).
static DecodePlan with_finish(DecodePlan p, const ShapeKey& s, int batch, int force_tb,
                              bool fused) {
  const int cus = device_cus();
  int tb = force_tb;
  if (tb != 1 && tb != 2 && tb != 4 && tb != 8) {
    tb = (long)s.H * batch < cus ? 1 : 2;
    while (tb >= 2 && tb < 8 && (long)s.H * cdiv(batch, 2 * tb) >= cus) tb *= 2;
  }
  if (fused) {
    // the merge runs in the split kernel's work groups: their thread count,
    // four splits per request round
    p.fused = true;
    p.finish_tb = tb;
    p.finish_cb = 4;
    p.finish_nt = decode_threads(s);
    const int per_round = 4 * finish_split_groups(p.finish_nt, tb, s.rv);
    p.split_stride = cdiv(p.num_splits, per_round) * per_round;
    return p;
  }
  int nt = 256, cb = 4;
  if (tb >= 4) {
    cb = 32 / tb;  // a thread holds TB/2 units of CB partial rows
  } else {
    while (nt < 512 && finish_split_groups(nt, tb, s.rv) * 16 < p.num_splits) nt *= 2;
    const int sg = finish_split_groups(nt, tb, s.rv);
    while (cb < 16 && cb * sg < p.num_splits) cb *= 2;
  }
  p.finish_tb = tb;
  p.finish_cb = cb;
  p.finish_nt = nt;
  const int per_round = cb * finish_split_groups(nt, tb, s.rv);
  p.split_stride = cdiv(p.num_splits, per_round) * per_round;
  return p;
}

// Split-K plan.  The split-K kernel runs one work group per compute unit,
// so B*S groups execute in ceil(B*S / CUs) rounds, each as long as its
// pages plus a start-up of about three page times (first-page latency),
// and every split adds partials that are written and merged back.  Pick the
// number of splits S that minimises
//     rounds * (3 + pages_per_split) + 6 * B * S / CUs,
// preferring fewer splits on ties; pages_per_split <= 256 (block ids are
// staged in LDS).  The weight 6 of the per-split term comes from sweeps at
// batch 1-64 (2K-32K tokens), where it picks the fastest plan or one within
// a few percent of it.  A caller may fix pages_per_split (force_pps > 0,
// at most 256) and the merge tile (force_tb in {1, 2, 4, 8}); the plan is
// otherwise a function of the shape, batch, length bound and device only.
constexpr double kSplitCost = 6.0;

// Split plan of the generic kernels: about one work group (eight waves) per
// CU over the batch, its head groups and the splits, at most 4096 splits; a
// caller's pages_per_split is kept unless it would exceed that.
static DecodePlan plan_generic(const ShapeKey& s, int batch, int max_seq_len, int bs,
                               int force_pps) {
  DecodePlan p{1, 1, 1, 4, 256, 1};
  p.generic = true;
  const int pages = cdiv(max_seq_len, bs);
  if (pages <= 0 || batch <= 0) return p;
  int pps;
  if (force_pps > 0) {
    pps = force_pps;
  } else {
    const long per_split = (long)batch * generic_head_groups(s);
    const int want = cdiv((long)device_cus(), per_split);
    pps = cdiv(pages, want < 1 ? 1 : (want > pages ? pages : want));
  }
  if (cdiv(pages, pps) > 4096) pps = cdiv(pages, 4096);
  p.pages_per_split = pps;
  p.num_splits = cdiv(pages, pps);
  p.split_stride = p.num_splits;
  return p;
}

DecodePlan plan_decode(const ShapeKey& s, int batch, int max_seq_len, int bs, int force_pps,
                       int force_tb, bool generic, int launches) {
  if (generic) return plan_generic(s, batch, max_seq_len, bs, force_pps);
  const bool fused = launches == 2;
  const int pages = cdiv(max_seq_len, bs);
  if (pages <= 0 || batch <= 0)
    return with_finish(DecodePlan{1, 1, 0, 0, 0, 0}, s, batch, force_tb, fused);
  if (force_pps > 0) {
    const int pps = force_pps < 256 ? force_pps : 256;
    return with_finish(DecodePlan{pps, cdiv(pages, pps), 0, 0, 0, 0}, s, batch, force_tb, fused);
  }
  const int cus = device_cus();
  double best = 1e300;
  int best_pps = pages < 256 ? pages : 256;
  for (int ns = cdiv(pages, 256); ns <= pages; ++ns) {
    const int pps = cdiv(pages, ns);
    const int nsr = cdiv(pages, pps);  // splits actually used at this length
    if (nsr != ns) continue;
    const double rounds = (double)cdiv((long)batch * ns, cus);
    const double cost = rounds * (3.0 + pps) + kSplitCost * (double)batch * ns / cus;
    if (cost < best - 1e-9) {
      best = cost;
      best_pps = pps;
    }
    if (ns > 4 * cus) break;
  }
  return with_finish(DecodePlan{best_pps, cdiv(pages, best_pps), 0, 0, 0, 0}, s, batch, force_tb,
                     fused);
}

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

DecodeWorkspace decode_workspace_layout(const ShapeKey& s, int batch, const DecodePlan& p) {
  const size_t r16 = (size_t)((s.H + 15) / 16) * 16;
  DecodeWorkspace w;
  size_t off = kWorkspaceHeaderBytes;
  if (p.generic) {  // q~ fp32, fp32 statistics [B][H][2][S] and unnormalised z [B][H][S][r_v]
    w.qt_off = off;
    off = align256(off + (size_t)batch * s.H * s.rk * 4);
    w.ml_off = off;
    off = align256(off + (size_t)batch * s.H * 2 * p.num_splits * 4);
    w.zp_off = off;
    off = align256(off + (size_t)batch * s.H * p.num_splits * s.rv * 4);
    w.sync_off = off;
    w.total = off;
    return w;
  }
  w.qt_off = off;
  off = align256(off + (size_t)batch * s.H * s.rk * 4);  // q~, fp32
  w.ml_off = off;
  off = align256(off + (size_t)batch * p.split_stride * 2 * r16 * 4);
  w.zp_off = off;  // per-split z rows, fp16
  off = align256(off + (size_t)batch * p.split_stride * r16 * s.rv * 2);
  w.sync_off = off;  // the fused step's counters: one per sequence, then an error word
  if (p.fused) off = align256(off + ((size_t)batch + 1) * 4);
  w.total = off;
  return w;
}

PrefillWorkspace prefill_workspace_layout(const ShapeKey& s, int total_q) {
  PrefillWorkspace w;
  size_t off = kWorkspaceHeaderBytes;
  w.qt_off = off;
  off = align256(off + (size_t)total_q * s.H * s.rk * 4);  // q~, fp32
  w.z_off = off;  // fp16 z tiled by 32-token blocks, see launch_upproj_tiled
  off = align256(off + (size_t)((total_q + 31) / 32) * 32 * s.H * s.rv * 2);
  w.total = off;
  return w;
}

}  // namespace starkv

using namespace starkv;

namespace {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Key/value heads: num_kv_heads, or num_heads when it is 0; it must divide
// num_heads.  Returns 0 when invalid.
int kv_heads(const starkv_dims* d) {
  const int hkv = d->num_kv_heads == 0 ? d->num_heads : d->num_kv_heads;
  if (hkv <= 0 || d->num_heads <= 0 || d->num_heads % hkv != 0) return 0;
  return hkv;
}

starkv_status check_dims(const starkv_dims* d, ShapeKey* key, bool kv_view = false) {
  if (!d) return STARKV_ERR_NULL;
  if (d->num_heads <= 0 || d->head_dim <= 0 || d->rank_k <= 0 || d->rank_v <= 0 ||
      d->block_size <= 0 || d->num_blocks <= 0 || d->num_kv_heads < 0)
    return STARKV_ERR_DIMS;
  const int hkv = kv_heads(d);
  if (hkv == 0) return STARKV_ERR_DIMS;
  if (d->rank_k > d->head_dim || (long)d->rank_v > (long)hkv * d->head_dim)
    return STARKV_ERR_DIMS;
  const ShapeKey k{d->num_heads, d->head_dim, d->rank_k, d->rank_v, hkv};
  if (d->block_size != 16 || !(kv_view ? kv_shape_supported(k) : shape_supported(k)))
    return STARKV_ERR_UNSUPPORTED;
  *key = k;
  return STARKV_OK;
}

starkv_status check_ptrs(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (!p) return STARKV_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return STARKV_ERR_ALIGN;
  return STARKV_OK;
}

bool scale_ok(float s) { return std::isfinite(s) && s > 0.f; }

// The bases fit has its own limits: d a multiple of 64 (Gram tiles), ranks
// up to 512 (the triangular solve keeps a row block of Q in LDS); the page
// size and page count do not enter.  The samples carry the key/value heads,
// so the fit's head count is Hkv.
starkv_status check_fit_dims(const starkv_dims* d, ShapeKey* key) {
  if (!d) return STARKV_ERR_NULL;
  if (d->num_heads <= 0 || d->head_dim <= 0 || d->rank_k <= 0 || d->rank_v <= 0 ||
      d->num_kv_heads < 0)
    return STARKV_ERR_DIMS;
  const int hkv = kv_heads(d);
  if (hkv == 0) return STARKV_ERR_DIMS;
  if (d->rank_k > d->head_dim || (long)d->rank_v > (long)hkv * d->head_dim)
    return STARKV_ERR_DIMS;
  if (d->head_dim % 64 != 0 || d->rank_k > 512 || d->rank_v > 512 || hkv > 65535 ||
      (long)hkv * d->head_dim > 65536)
    return STARKV_ERR_UNSUPPORTED;
  *key = ShapeKey{hkv, d->head_dim, d->rank_k, d->rank_v, hkv};
  return STARKV_OK;
}

starkv_status check_paging(int32_t batch, int32_t max_seq_len, int32_t max_blocks, int bs) {
  if (batch < 0 || max_seq_len < 0 || max_blocks < 0) return STARKV_ERR_DIMS;
  if (batch > 65535) return STARKV_ERR_DIMS;
  if ((long)max_blocks * bs < (long)max_seq_len) return STARKV_ERR_DIMS;
  return STARKV_OK;
}

}  // namespace

extern "C" {

int32_t starkv_abi_version(void) { return STARKV_ABI_VERSION; }

const char* starkv_status_string(int32_t status) {
  switch (status) {
    case STARKV_OK: return "ok";
    case STARKV_ERR_NULL: return "required pointer is NULL";
    case STARKV_ERR_DIMS: return "invalid or inconsistent sizes";
    case STARKV_ERR_UNSUPPORTED: return "no kernel instance for this shape";
    case STARKV_ERR_WORKSPACE: return "workspace too small";
    case STARKV_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case STARKV_ERR_LAUNCH: return "kernel launch failed";
    case STARKV_ERR_ARG: return "invalid argument";
    default: return "unknown status";
  }
}

int32_t starkv_shape_supported(const starkv_dims* dims) {
  ShapeKey k;
  return check_dims(dims, &k) == STARKV_OK ? 1 : 0;
}

starkv_status starkv_append_workspace_size(const starkv_dims* dims, int32_t num_tokens,
                                           size_t* bytes) {
  ShapeKey key;
  starkv_status st = check_dims(dims, &key, /*kv_view=*/true);
  if (st != STARKV_OK) return st;
  if (!bytes) return STARKV_ERR_NULL;
  if (num_tokens < 0) return STARKV_ERR_DIMS;
  const ShapeKey kv_key{key.Hkv, key.d, key.rk, key.rv, key.Hkv};
  *bytes = append_workspace_bytes(kv_key, num_tokens);
  return STARKV_OK;
}

// the workspace that an append of num_tokens tokens needs is present
static starkv_status check_append_workspace(const ShapeKey& kv_key, int32_t num_tokens,
                                            const void* workspace, size_t workspace_bytes) {
  const size_t need = append_workspace_bytes(kv_key, num_tokens);
  if (need == 0) return STARKV_OK;
  if (!workspace) return STARKV_ERR_NULL;
  if (workspace_bytes < need) return STARKV_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 15) != 0) return STARKV_ERR_ALIGN;
  return STARKV_OK;
}

starkv_status starkv_append(const starkv_dims* dims, const void* k, const void* v, const void* U,
                            const void* W, const int64_t* slot_mapping, int32_t num_tokens,
                            void* k_cache, void* v_cache, void* workspace, size_t workspace_bytes,
                            void* stream) {
  ShapeKey key;
  starkv_status st = check_dims(dims, &key, /*kv_view=*/true);
  if (st != STARKV_OK) return st;
  if (num_tokens < 0) return STARKV_ERR_DIMS;
  if (num_tokens == 0) return STARKV_OK;
  st = check_ptrs({k, v, U, W, slot_mapping, k_cache, v_cache});
  if (st != STARKV_OK) return st;
  // the append only sees key/value heads
  const ShapeKey kv_key{key.Hkv, key.d, key.rk, key.rv, key.Hkv};
  st = check_append_workspace(kv_key, num_tokens, workspace, workspace_bytes);
  if (st != STARKV_OK) return st;
  const hipError_t e = launch_append(kv_key, k, v, U, W, slot_mapping, num_tokens,
                                     dims->num_blocks, k_cache, v_cache, LatentFormat{},
                                     workspace, (hipStream_t)stream);
  return e == hipSuccess ? STARKV_OK : STARKV_ERR_LAUNCH;
}

starkv_status starkv_append_fp8(const starkv_dims* dims, const void* k, const void* v,
                                const void* U, const void* W, const int64_t* slot_mapping,
                                int32_t num_tokens, float k_scale, float v_scale,
                                void* k_cache8, void* v_cache8, void* workspace,
                                size_t workspace_bytes, void* stream) {
  ShapeKey key;
  starkv_status st = check_dims(dims, &key, /*kv_view=*/true);
  if (st != STARKV_OK) return st;
  if (num_tokens < 0) return STARKV_ERR_DIMS;
  if (!scale_ok(k_scale) || !scale_ok(v_scale)) return STARKV_ERR_ARG;
  if (num_tokens == 0) return STARKV_OK;
  st = check_ptrs({k, v, U, W, slot_mapping, k_cache8, v_cache8});
  if (st != STARKV_OK) return st;
  const ShapeKey kv_key{key.Hkv, key.d, key.rk, key.rv, key.Hkv};
  st = check_append_workspace(kv_key, num_tokens, workspace, workspace_bytes);
  if (st != STARKV_OK) return st;
  LatentFormat fmt;
  fmt.fp8 = true;
  fmt.k_scale = k_scale;
  fmt.v_scale = v_scale;
  const hipError_t e = launch_append(kv_key, k, v, U, W, slot_mapping, num_tokens,
                                     dims->num_blocks, k_cache8, v_cache8, fmt, workspace,
                                     (hipStream_t)stream);
  return e == hipSuccess ? STARKV_OK : STARKV_ERR_LAUNCH;
}

}  // extern "C"

namespace {

// A caller's plan override: each field 0 (the planner's choice) or in range.
starkv_status check_config(const starkv_decode_config* cfg) {
  if (!cfg) return STARKV_OK;
  if (cfg->pages_per_split < 0 || cfg->pages_per_split > 256) return STARKV_ERR_ARG;
  const int m = cfg->merge_seqs;
  if (m != 0 && m != 1 && m != 2 && m != 4 && m != 8) return STARKV_ERR_ARG;
  if (cfg->launches != 0 && cfg->launches != 2 && cfg->launches != 3) return STARKV_ERR_ARG;
  return STARKV_OK;
}

DecodePlan plan_for(const ShapeKey& key, int batch, int max_seq_len, int bs,
                    const starkv_decode_config* cfg, bool fp8) {
  return plan_decode(key, batch, max_seq_len, bs, cfg ? cfg->pages_per_split : 0,
                     cfg ? cfg->merge_seqs : 0, use_generic(key, fp8), cfg ? cfg->launches : 0);
}

// The workspace of a decode call over fp16 latents and of one over FP8
// latents may differ (one may run on the generic kernels): the size query
// covers both.
size_t decode_need(const ShapeKey& key, int batch, int max_seq_len, int bs,
                   const starkv_decode_config* cfg) {
  size_t need = decode_workspace_layout(key, batch, plan_for(key, batch, max_seq_len, bs, cfg,
                                                             false)).total;
  if (fp8_decode_supported(key)) {
    const size_t n8 = decode_workspace_layout(key, batch, plan_for(key, batch, max_seq_len, bs,
                                                                   cfg, true)).total;
    if (n8 > need) need = n8;
  }
  return need;
}

starkv_status workspace_size(const starkv_dims* dims, int32_t batch, int32_t max_seq_len,
                             const starkv_decode_config* cfg, size_t* bytes) {
  ShapeKey key;
  starkv_status st = check_dims(dims, &key);
  if (st != STARKV_OK) return st;
  if (!bytes) return STARKV_ERR_NULL;
  if (batch < 0 || max_seq_len < 0 || batch > 65535) return STARKV_ERR_DIMS;
  st = check_config(cfg);
  if (st != STARKV_OK) return st;
  *bytes = decode_need(key, batch, max_seq_len, dims->block_size, cfg);
  return STARKV_OK;
}

// Every decode entry point: host checks, then the q projection (the key
// scale, FP8 only, folds into q~), the split-K pass and the merge.
// noalloc: the library's own scratch replaces the caller's workspace (which
// is then ignored), and a plan whose workspace exceeds it is rejected.
starkv_status decode_common(const starkv_dims* dims, const void* q, const void* k_cache,
                            const void* v_cache, const void* U, const void* W,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                            float scale, const LatentFormat& fmt, const starkv_decode_config* cfg,
                            void* out, void* workspace, size_t workspace_bytes, void* stream,
                            bool noalloc = false) {
  ShapeKey key;
  starkv_status st = check_dims(dims, &key);
  if (st != STARKV_OK) return st;
  if (fmt.fp8 && !fp8_decode_supported(key)) return STARKV_ERR_UNSUPPORTED;
  st = check_paging(batch, max_seq_len, max_blocks_per_seq, dims->block_size);
  if (st != STARKV_OK) return st;
  if (!scale_ok(scale) || !scale_ok(fmt.k_scale) || !scale_ok(fmt.v_scale)) return STARKV_ERR_ARG;
  st = check_config(cfg);
  if (st != STARKV_OK) return st;
  if (batch == 0) return STARKV_OK;
  st = check_ptrs({q, k_cache, v_cache, U, W, block_tables, seq_lens, out,
                   noalloc ? (const void*)q : workspace});
  if (st != STARKV_OK) return st;
  const DecodePlan p = plan_for(key, batch, max_seq_len, dims->block_size, cfg, fmt.fp8);
  const DecodeWorkspace ws = decode_workspace_layout(key, batch, p);
  if (noalloc) {
    if (ws.total > kNoallocScratchBytes) return STARKV_ERR_WORKSPACE;
    if (noalloc_scratch(&workspace) != hipSuccess) return STARKV_ERR_LAUNCH;
  } else if (workspace_bytes < ws.total) {
    return STARKV_ERR_WORKSPACE;
  }
  char* wb = (char*)workspace;
  const hipStream_t s = (hipStream_t)stream;
  const float qscale = scale * (fmt.fp8 ? fmt.k_scale : 1.f);
  if (p.generic) {
    hipError_t e = launch_generic_qproj(key, q, U, batch, qscale, wb + ws.qt_off,
                                        TIME_DECODE_SPLIT, s);
    if (e != hipSuccess) return STARKV_ERR_LAUNCH;
    e = launch_generic_attn(key, wb + ws.qt_off, nullptr, batch, k_cache, v_cache, W,
                            block_tables, max_blocks_per_seq, seq_lens, dims->num_blocks, batch,
                            p.pages_per_split, p.num_splits, (float*)(wb + ws.ml_off),
                            (float*)(wb + ws.zp_off), out, fmt, TIME_DECODE_SPLIT, s);
    return e == hipSuccess ? STARKV_OK : STARKV_ERR_LAUNCH;
  }
  uint32_t* sync = (uint32_t*)(wb + ws.sync_off);
  hipError_t e = launch_qproj(key, q, U, batch, qscale, wb + ws.qt_off, TIME_DECODE_SPLIT, s, W,
                              p.fused ? sync : nullptr, p.fused ? batch + 1 : 0);
  if (e != hipSuccess) return STARKV_ERR_LAUNCH;
  e = launch_decode(key, p, wb + ws.qt_off, k_cache, v_cache, W, block_tables,
                    max_blocks_per_seq, seq_lens, dims->num_blocks, batch,
                    (float*)(wb + ws.ml_off), wb + ws.zp_off, out, fmt, sync, s);
  return e == hipSuccess ? STARKV_OK : STARKV_ERR_LAUNCH;
}

LatentFormat fp8_format(float k_scale, float v_scale) {
  LatentFormat fmt;
  fmt.fp8 = true;
  fmt.k_scale = k_scale;
  fmt.v_scale = v_scale;
  return fmt;
}

}  // namespace

extern "C" {

starkv_status starkv_decode_workspace_size(const starkv_dims* dims, int32_t batch,
                                           int32_t max_seq_len, size_t* bytes) {
  return workspace_size(dims, batch, max_seq_len, nullptr, bytes);
}

starkv_status starkv_decode_workspace_size_cfg(const starkv_dims* dims, int32_t batch,
                                               int32_t max_seq_len,
                                               const starkv_decode_config* cfg, size_t* bytes) {
  return workspace_size(dims, batch, max_seq_len, cfg, bytes);
}

starkv_status starkv_decode_plan(const starkv_dims* dims, int32_t batch, int32_t max_seq_len,
                                 int32_t* pages_per_split, int32_t* num_splits) {
  ShapeKey key;
  starkv_status st = check_dims(dims, &key);
  if (st != STARKV_OK) return st;
  if (!pages_per_split || !num_splits) return STARKV_ERR_NULL;
  if (batch < 0 || max_seq_len < 0) return STARKV_ERR_DIMS;
  const DecodePlan p = plan_decode(key, batch, max_seq_len, dims->block_size);
  *pages_per_split = p.pages_per_split;
  *num_splits = p.num_splits;
  return STARKV_OK;
}

starkv_status starkv_decode_attn(const starkv_dims* dims, const void* q, const void* k_cache,
                                 const void* v_cache, const void* U, const void* W,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                 float scale, void* out, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return decode_common(dims, q, k_cache, v_cache, U, W, block_tables, max_blocks_per_seq,
                       seq_lens, batch, max_seq_len, scale, LatentFormat{}, nullptr, out,
                       workspace, workspace_bytes, stream);
}

starkv_status starkv_decode_attn_cfg(const starkv_dims* dims, const void* q, const void* k_cache,
                                     const void* v_cache, const void* U, const void* W,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* seq_lens, int32_t batch,
                                     int32_t max_seq_len, float scale,
                                     const starkv_decode_config* cfg, void* out, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return decode_common(dims, q, k_cache, v_cache, U, W, block_tables, max_blocks_per_seq,
                       seq_lens, batch, max_seq_len, scale, LatentFormat{}, cfg, out, workspace,
                       workspace_bytes, stream);
}

starkv_status starkv_decode_attn_noalloc(const starkv_dims* dims, const void* q,
                                         const void* k_cache, const void* v_cache, const void* U,
                                         const void* W, const int32_t* block_tables,
                                         int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                         int32_t batch, int32_t max_seq_len, float scale,
                                         void* out, void* stream) {
  return decode_common(dims, q, k_cache, v_cache, U, W, block_tables, max_blocks_per_seq,
                       seq_lens, batch, max_seq_len, scale, LatentFormat{}, nullptr, out, nullptr,
                       0, stream, /*noalloc=*/true);
}

starkv_status starkv_decode_attn_fp8(const starkv_dims* dims, const void* q,
                                     const void* k_cache8, const void* v_cache8, const void* U,
                                     const void* W, const int32_t* block_tables,
                                     int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                     int32_t batch, int32_t max_seq_len, float scale,
                                     float k_scale, float v_scale, void* out, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return decode_common(dims, q, k_cache8, v_cache8, U, W, block_tables, max_blocks_per_seq,
                       seq_lens, batch, max_seq_len, scale, fp8_format(k_scale, v_scale),
                       nullptr, out, workspace, workspace_bytes, stream);
}

starkv_status starkv_prefill_workspace_size(const starkv_dims* dims, int32_t batch,
                                            int32_t total_q, int32_t max_seq_len, size_t* bytes) {
  ShapeKey key;
  starkv_status st = check_dims(dims, &key);
  if (st != STARKV_OK) return st;
  if (!bytes) return STARKV_ERR_NULL;
  if (batch < 0 || total_q < 0 || max_seq_len < 0) return STARKV_ERR_DIMS;
  *bytes = prefill_workspace_layout(key, total_q).total;
  return STARKV_OK;
}

}  // extern "C"

namespace {

// Both prefill entry points: host checks, the q projection (the key scale,
// FP8 only, folds into q~), then the chunk attention with the up-projection:
// the tuned kernels, or the generic ones (one row per chunk query, one split).
starkv_status prefill_common(const starkv_dims* dims, const void* q,
                             const int32_t* query_start_loc, int32_t total_q,
                             int32_t max_query_len, const void* k_cache, const void* v_cache,
                             const void* U, const void* W, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                             int32_t max_seq_len, float scale, const LatentFormat& fmt, void* out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  ShapeKey key;
  starkv_status st = check_dims(dims, &key);
  if (st != STARKV_OK) return st;
  if (fmt.fp8 && !fp8_decode_supported(key)) return STARKV_ERR_UNSUPPORTED;
  st = check_paging(batch, max_seq_len, max_blocks_per_seq, dims->block_size);
  if (st != STARKV_OK) return st;
  if (total_q < 0 || max_query_len < 0) return STARKV_ERR_DIMS;
  if (total_q > 0 && max_query_len == 0) return STARKV_ERR_DIMS;
  if (max_query_len > max_seq_len) return STARKV_ERR_DIMS;
  if (!scale_ok(scale) || !scale_ok(fmt.k_scale) || !scale_ok(fmt.v_scale)) return STARKV_ERR_ARG;
  if (batch == 0 || total_q == 0) return STARKV_OK;
  st = check_ptrs({q, query_start_loc, k_cache, v_cache, U, W, block_tables, seq_lens, out,
                   workspace});
  if (st != STARKV_OK) return st;
  const PrefillWorkspace ws = prefill_workspace_layout(key, total_q);
  if (workspace_bytes < ws.total) return STARKV_ERR_WORKSPACE;
  char* wb = (char*)workspace;
  const hipStream_t s = (hipStream_t)stream;
  const float qscale = scale * (fmt.fp8 ? fmt.k_scale : 1.f);
  hipError_t e;
  if (use_generic(key, fmt.fp8)) {
    e = launch_generic_qproj(key, q, U, total_q, qscale, wb + ws.qt_off, TIME_PREFILL_ATTN, s);
    if (e != hipSuccess) return STARKV_ERR_LAUNCH;
    if (generic_prefill_tiled(key, max_blocks_per_seq))  // 64 chunk queries per work group
      e = launch_generic_prefill(key, wb + ws.qt_off, query_start_loc, total_q, max_query_len,
                                 k_cache, v_cache, W, block_tables, max_blocks_per_seq, seq_lens,
                                 dims->num_blocks, batch, out, fmt, TIME_PREFILL_ATTN, s);
    else  // r_k > 128, r_v > 1024 or table rows past 8192 pages: one row per chunk query
      e = launch_generic_attn(key, wb + ws.qt_off, query_start_loc, total_q, k_cache, v_cache,
                              W, block_tables, max_blocks_per_seq, seq_lens, dims->num_blocks,
                              batch, max_blocks_per_seq, 1, nullptr, nullptr, out, fmt,
                              TIME_PREFILL_ATTN, s);
    return e == hipSuccess ? STARKV_OK : STARKV_ERR_LAUNCH;
  }
  e = launch_qproj(key, q, U, total_q, qscale, wb + ws.qt_off, TIME_PREFILL_ATTN, s);
  if (e != hipSuccess) return STARKV_ERR_LAUNCH;
  e = launch_prefill(key, wb + ws.qt_off, query_start_loc, total_q, max_query_len, k_cache,
                     v_cache, W, block_tables, max_blocks_per_seq, seq_lens, dims->num_blocks,
                     batch, (void*)(wb + ws.z_off), out, fmt, s);
  return e == hipSuccess ? STARKV_OK : STARKV_ERR_LAUNCH;
}

}  // namespace

extern "C" {

starkv_status starkv_prefill_attn(const starkv_dims* dims, const void* q,
                                  const int32_t* query_start_loc, int32_t total_q,
                                  int32_t max_query_len, const void* k_cache, const void* v_cache,
                                  const void* U, const void* W, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                  int32_t batch, int32_t max_seq_len, float scale, void* out,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_common(dims, q, query_start_loc, total_q, max_query_len, k_cache, v_cache, U, W,
                        block_tables, max_blocks_per_seq, seq_lens, batch, max_seq_len, scale,
                        LatentFormat{}, out, workspace, workspace_bytes, stream);
}

starkv_status starkv_prefill_attn_fp8(const starkv_dims* dims, const void* q,
                                      const int32_t* query_start_loc, int32_t total_q,
                                      int32_t max_query_len, const void* k_cache8,
                                      const void* v_cache8, const void* U, const void* W,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* seq_lens, int32_t batch,
                                      int32_t max_seq_len, float scale, float k_scale,
                                      float v_scale, void* out, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  return prefill_common(dims, q, query_start_loc, total_q, max_query_len, k_cache8, v_cache8, U,
                        W, block_tables, max_blocks_per_seq, seq_lens, batch, max_seq_len, scale,
                        fp8_format(k_scale, v_scale), out, workspace, workspace_bytes, stream);
}

starkv_status starkv_fit_workspace_size(const starkv_dims* dims, size_t* bytes) {
  ShapeKey key;
  const starkv_status st = check_fit_dims(dims, &key);
  if (st != STARKV_OK) return st;
  if (!bytes) return STARKV_ERR_NULL;
  *bytes = fit_workspace_layout(key).total;
  return STARKV_OK;
}

starkv_status starkv_fit_bases(const starkv_dims* dims, const void* k, const void* v,
                               int32_t num_samples, const float* u0, const float* w0,
                               int32_t iters, void* U, void* W, void* workspace,
                               size_t workspace_bytes, int32_t* info, float* residual,
                               void* stream) {
  ShapeKey key;
  starkv_status st = check_fit_dims(dims, &key);
  if (st != STARKV_OK) return st;
  if (num_samples < key.rk || num_samples < key.rv) return STARKV_ERR_DIMS;
  if (iters < 1 || iters > 1000) return STARKV_ERR_ARG;
  st = check_ptrs({k, v, u0, w0, U, W, workspace});
  if (st != STARKV_OK) return st;
  if (info && ((uintptr_t)info & 3u) != 0) return STARKV_ERR_ALIGN;
  if (residual && ((uintptr_t)residual & 3u) != 0) return STARKV_ERR_ALIGN;
  if (workspace_bytes < fit_workspace_layout(key).total) return STARKV_ERR_WORKSPACE;
  const hipError_t e = launch_fit(key, k, v, num_samples, u0, w0, iters, U, W, workspace,
                                  (int*)info, residual, (hipStream_t)stream);
  return e == hipSuccess ? STARKV_OK : STARKV_ERR_LAUNCH;
}

starkv_status starkv_check_indices(const starkv_dims* dims, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                   int32_t batch, int32_t max_seq_len,
                                   const int64_t* slot_mapping, int32_t num_tokens,
                                   uint32_t* report, void* stream) {
  if (!dims || !report) return STARKV_ERR_NULL;
  if (dims->block_size != 16 || dims->num_blocks < 0 || num_tokens < 0) return STARKV_ERR_DIMS;
  starkv_status st = check_paging(batch, max_seq_len, max_blocks_per_seq, dims->block_size);
  if (st != STARKV_OK) return st;
  if (batch > 0 && (!seq_lens || (max_blocks_per_seq > 0 && !block_tables))) return STARKV_ERR_NULL;
  if (num_tokens > 0 && !slot_mapping) return STARKV_ERR_NULL;
  for (const void* p : {(const void*)block_tables, (const void*)seq_lens,
                        (const void*)slot_mapping, (const void*)report})
    if (p && !aligned16(p)) return STARKV_ERR_ALIGN;
  return launch_check_indices(block_tables, max_blocks_per_seq, seq_lens, batch, max_seq_len,
                              dims->num_blocks, slot_mapping, num_tokens, report,
                              (hipStream_t)stream) == hipSuccess
             ? STARKV_OK
             : STARKV_ERR_LAUNCH;
}

starkv_status starkv_util_stream_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (bytes == 0) return STARKV_OK;
  if (!src || !sink) return STARKV_ERR_NULL;
  if (!aligned16(src) || (bytes & 15) != 0) return STARKV_ERR_ALIGN;
  return launch_stream_read(src, bytes, sink, (hipStream_t)stream) == hipSuccess ? STARKV_OK
                                                                                 : STARKV_ERR_LAUNCH;
}

starkv_status starkv_set_timing_events(void* start, void* stop, int32_t which) {
  if (which < 0 || which > 5) return STARKV_ERR_ARG;
  if (which != 0 && (!start || !stop)) return STARKV_ERR_NULL;
  g_timing.start = (hipEvent_t)start;
  g_timing.stop = (hipEvent_t)stop;
  g_timing.which = which;
  return STARKV_OK;
}

starkv_status starkv_util_event_create(void** event) {
  if (!event) return STARKV_ERR_NULL;
  *event = nullptr;
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return STARKV_ERR_LAUNCH;
  *event = (void*)e;
  return STARKV_OK;
}

starkv_status starkv_util_event_destroy(void* event) {
  if (!event) return STARKV_OK;
  return hipEventDestroy((hipEvent_t)event) == hipSuccess ? STARKV_OK : STARKV_ERR_LAUNCH;
}

starkv_status starkv_util_event_elapsed_ms(void* start, void* stop, float* ms) {
  if (!start || !stop || !ms) return STARKV_ERR_NULL;
  return hipEventElapsedTime(ms, (hipEvent_t)start, (hipEvent_t)stop) == hipSuccess
             ? STARKV_OK
             : STARKV_ERR_LAUNCH;
}

}  // extern "C"
