/*
 * starkv.h -- C ABI of libstarkv, attention over a paged KV cache stored in
 * low-rank compressed form, for AMD Instinct MI355X (gfx950).
 *
 * The method (Proxima README, introduction): each layer keeps a low-rank
 * projection of its KV cache -- head-wise for keys, joint across heads for
 * values -- in a compressed paged format.  With U_h in R^{d x r_k} per head
 * and one W in R^{(H*d) x r_v}:
 *
 *     key latent    c_k[t, h] = U_h^T k[t, h]           (r_k values per head)
 *     value latent  c_v[t]    = W^T vec(v[t])           (r_v values per token)
 *
 * where vec() flattens [H, d] head-major (row h*d + i of W pairs with
 * v[t, h, i]) and W_h denotes rows h*d .. h*d+d-1 of W.  Attention runs on the
 * latents without rebuilding K or V:
 *
 *     q~_h = U_h^T q_h,  s_t = scale * q~_h . c_k[t, h],  p = softmax(s),
 *     z_h = sum_t p_t c_v[t],  out_h = W_h z_h.
 *
 * This equals softmax attention over the rebuilt K^ = U c_k, V^ = W c_v for
 * any U and W.  Pages hold 16 tokens (README, "KV-cache capacity": block
 * size 16); token t of sequence b lives in block block_tables[b][t / 16] at
 * offset t % 16.
 *
 * Grouped-query attention (Hkv key/value heads shared by groups of H / Hkv
 * query heads) keeps the same scheme per key/value head g: U_g and the key
 * latents are per key/value head, W has Hkv*d rows and vec() flattens the
 * [Hkv, d] values, and query head h reads key/value head g = h / (H / Hkv):
 * q~_h = U_g^T q_h, scores on c_k[t, g], out_h = W_g z_h.
 *
 * Layouts (all fp16 = IEEE binary16, little-endian, dense, row-major):
 *   k_cache  [num_blocks][Hkv][16][r_k]
 *   v_cache  [num_blocks][r_v][16]      (feature-major within a page)
 *   U        [Hkv][d][r_k]
 *   W        [Hkv*d][r_v]
 *   q, out   [tokens][H][d]
 *   k, v     [tokens][Hkv][d]
 * (Hkv = H for multi-head attention.)
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns all
 *     memory, including workspaces; the library allocates nothing and keeps
 *     no per-call state.  `stream` is a hipStream_t (NULL = default stream).
 *     Calls are asynchronous on `stream`; nothing synchronises the host.
 *   - Workspaces (decode, prefill, append).  Their first 256 bytes are
 *     reserved: the few-token append keeps arrival counters there.  They
 *     must be zero when a workspace is first used (allocate it zero-filled
 *     or clear it once); every call leaves them zero and no call writes
 *     anything else there, so one buffer may serve all three kinds of call.
 *     The rest of a workspace needs no initialisation.  Calls that overlap in
 *     time must not share a workspace.
 *   - Arguments are validated on the host BEFORE any HIP call: on failure the
 *     call returns a non-zero status and enqueues nothing.  Device pointers
 *     must be 16-byte aligned.  A launch failure maps to STARKV_ERR_LAUNCH.
 *   - Contents of device index arrays (block tables, seq_lens, slots,
 *     query_start_loc) are trusted.  Block ids outside [0, num_blocks) and
 *     slots outside the cache are skipped rather than dereferenced;
 *     starkv_check_indices reports them on request.
 *   - Shapes.  Tuned instances of the attention and append calls:
 *     (H, d, r_k, r_v) = (32, 128, 64, 512) with Hkv 32 or 8,
 *     (32, 128, 32, 256) with Hkv 32, and (4, 64, 16, 64) with Hkv 4 or 2
 *     (FP8 caches: the first and the last, Hkv 32/8 and 4).  Every other
 *     shape within the generic limits -- d a multiple of 32 up to 256, r_k a
 *     multiple of 8 up to min(d, 256), r_v a multiple of 8 up to
 *     min(2048, Hkv * d), Hkv dividing H -- runs on generic kernels that take
 *     the sizes at run time (fp16 and FP8 caches alike: per-layer rank
 *     profiles, other head counts, sizes and grouped-query groups).  Block
 *     size 16.  Other shapes return STARKV_ERR_UNSUPPORTED.  The bases fit
 *     takes any shape within the limits stated at its declaration.
 */
#ifndef STARKV_H_
#define STARKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define STARKV_ABI_VERSION 8

typedef enum {
  STARKV_OK = 0,
  STARKV_ERR_NULL = 1,        /* a required pointer is NULL */
  STARKV_ERR_DIMS = 2,        /* a size is negative, zero where it must not be, or inconsistent */
  STARKV_ERR_UNSUPPORTED = 3, /* no compiled kernel instance for this shape */
  STARKV_ERR_WORKSPACE = 4,   /* workspace smaller than the size query returned */
  STARKV_ERR_ALIGN = 5,       /* a device pointer is not 16-byte aligned */
  STARKV_ERR_LAUNCH = 6,      /* a kernel launch failed (hipGetLastError) */
  STARKV_ERR_ARG = 7          /* another invalid argument (scale, timing selector) */
} starkv_status;

/* Model and cache dimensions (host struct). */
typedef struct {
  int32_t num_heads;  /* H */
  int32_t head_dim;   /* d */
  int32_t rank_k;     /* r_k, key latent size per head (<= d) */
  int32_t rank_v;     /* r_v, joint value latent size (<= Hkv*d) */
  int32_t block_size; /* tokens per page; must be 16 */
  int32_t num_blocks; /* pages in k_cache / v_cache (> 0) */
  int32_t num_kv_heads; /* Hkv, key/value heads; 0 means H (multi-head attention);
                           must divide H.  Query head h uses key/value head
                           h / (H / Hkv) (grouped-query attention). */
} starkv_dims;

/* Version of this ABI (STARKV_ABI_VERSION). */
int32_t starkv_abi_version(void);

/* Static, NUL-terminated description of a status code; never NULL. */
const char* starkv_status_string(int32_t status);

/* 1 if a kernel instance exists for these dims, else 0 (dims may be NULL -> 0). */
int32_t starkv_shape_supported(const starkv_dims* dims);

/*
 * Workspace bytes (host out-parameter *bytes) that starkv_append and
 * starkv_append_fp8 need for num_tokens tokens: 0, or the reserved 256
 * bytes (the arrival counters, see the workspace convention above) followed
 * by fp32 partial products of the value projection:
 *   num_tokens <= 64 (a decode step's tokens) at the tuned shapes: over
 *     S slices of W's Hkv*d rows, S = Hkv*d / R with
 *     R = max(64, Hkv*d * (r_v/32) / 256) rows per slice,
 *     256 + S * num_tokens * r_v * 4 bytes (S = 16 at 32 key/value heads of
 *     d 128 with r_v 512);
 *   65..1792 tokens at 32 key/value heads of d 128 with r_k 64 and r_v 512:
 *     over four equal parts of the contraction, 256 + 4 * num_tokens * r_v * 4
 *     bytes; 1793..2816 tokens there: two parts, 256 + 2 * num_tokens * r_v * 4;
 *   other token counts and shapes: 0.
 * The size is not monotonic in num_tokens: a workspace reused for several
 * token counts takes the largest of their sizes.  Returns a status.
 */
starkv_status starkv_append_workspace_size(const starkv_dims* dims, int32_t num_tokens,
                                           size_t* bytes /* (host) */);

/*
 * Append (README, "Kernel profiling breakdown": the write kernel's low-rank
 * projection and paged write).  For each n < num_tokens with
 * slot_mapping[n] >= 0, writes
 *     k_cache[slot / 16][h][slot % 16][:] = fp16(U_h^T k[n, h, :])   for all h
 *     v_cache[slot / 16][:][slot % 16]    = fp16(W^T vec(v[n]))
 * rounded to nearest even from an fp32 accumulation.  Negative slots are
 * skipped (padding); slots at or beyond num_blocks*16 are skipped.  Slots
 * must be distinct.  num_tokens == 0 is a no-op.
 *   k, v          [num_tokens][Hkv][d] fp16
 *   U, W          fp16, layouts above
 * Only the key/value heads enter: num_heads may be any multiple of Hkv
 * (dims with num_heads = Hkv and num_kv_heads 0 describe the same append).
 *   slot_mapping  [num_tokens] int64
 *   k_cache, v_cache  updated in place
 *   workspace     device scratch of at least starkv_append_workspace_size
 *                 bytes, 16-byte aligned, owned by the caller, its first 256
 *                 bytes zero (workspace convention above); may be NULL
 *                 (with workspace_bytes 0) when that size is 0.  A missing
 *                 or short workspace returns STARKV_ERR_NULL or
 *                 STARKV_ERR_WORKSPACE before anything is launched.
 * Up to 64 tokens (tuned shapes) run as one launch: slices of the value
 * projection write their partial products to the workspace and the last
 * slice of each block of 32 outputs to finish sums them in slice order,
 * rounds and writes the slots (nothing waits on another work group).
 */
starkv_status starkv_append(const starkv_dims* dims, const void* k, const void* v, const void* U,
                            const void* W, const int64_t* slot_mapping, int32_t num_tokens,
                            void* k_cache, void* v_cache, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * FP8 latents (the quantised-latent variant that adjacent KV-cache work
 * measures; half the bytes of fp16).  The caches keep the layouts above
 * with one-byte elements: OCP FP8 E4M3 codes (sign, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent 0 subnormal; S.1111.111 NaN; largest
 * value 448).  A latent c is stored as the code of c / scale, clamped to
 * +-448 and rounded to nearest with ties to the even mantissa, with one
 * scale per tensor (k_scale for keys, v_scale for values, finite and > 0),
 * and reads back as scale * value(code).
 *
 * starkv_append_fp8: starkv_append writing FP8 codes (the projection is
 * accumulated in fp32 and divided by the scale in fp32 before rounding).
 */
starkv_status starkv_append_fp8(const starkv_dims* dims, const void* k, const void* v,
                                const void* U, const void* W, const int64_t* slot_mapping,
                                int32_t num_tokens, float k_scale, float v_scale,
                                void* k_cache8, void* v_cache8, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Workspace bytes (host out-parameter *bytes) that starkv_decode_attn and
 * starkv_decode_attn_fp8 need for `batch` sequences of at most max_seq_len
 * tokens (the larger of the two).  Returns a status.
 */
starkv_status starkv_decode_workspace_size(const starkv_dims* dims, int32_t batch,
                                           int32_t max_seq_len, size_t* bytes /* (host) */);

/*
 * Decode attention (README, "Per-decode-step attention"): one query per
 * sequence attends to all seq_lens[b] cached tokens (append the step's token
 * first).  out[b, h, :] = W_h sum_t softmax_t(scale * q~_h . c_k[t, h]) c_v[t].
 *   q             [batch][H][d] fp16
 *   block_tables  [batch][max_blocks_per_seq] int32; entries past
 *                 ceil(seq_lens[b] / 16) are never read
 *   seq_lens      [batch] int32, each in [0, max_seq_len]; 0 gives zeros
 *   max_seq_len   (host) upper bound used to plan the split-K work; requires
 *                 max_blocks_per_seq >= ceil(max_seq_len / 16)
 *   scale         (host) softmax scale, normally 1/sqrt(d); finite, > 0
 *   out           [batch][H][d] fp16
 *   workspace     >= starkv_decode_workspace_size(...) bytes, 256-byte aligned
 *                 preferred; its first 256 bytes zero (workspace convention
 *                 above), the rest needs no initialisation
 * Three kernels run on `stream`: q projection, split-K latent attention,
 * and the merge of the splits fused with the W_h up-projection.
 */
starkv_status starkv_decode_attn(const starkv_dims* dims, const void* q, const void* k_cache,
                                 const void* v_cache, const void* U, const void* W,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                 float scale, void* out, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * Split plan of a decode call (host struct).  The decode step splits each
 * sequence's pages over work groups (split-K, README "Kernel profiling
 * breakdown": split-K attention plus a combine) and merges the splits' partial
 * softmax states; the plan fixes how.  Each field is 0 for the library's
 * choice (what starkv_decode_attn uses) or a value in range:
 *   pages_per_split  1..256 consecutive 16-token pages per work group
 *   merge_seqs       sequences per work group of the merge: 1, 2, 4 or 8
 *   launches         3: q projection, split pass and merge as three kernels
 *                    (the library's choice); 2: the split pass and the merge
 *                    in one kernel whose work groups merge once their
 *                    sequences' splits have signalled (tuned shapes only)
 * Any plan gives the same attention up to rounding order.
 */
typedef struct {
  int32_t pages_per_split;
  int32_t merge_seqs;
  int32_t launches;
} starkv_decode_config;

/*
 * starkv_decode_workspace_size and starkv_decode_attn with the caller's plan
 * (cfg may be NULL: the library's plan).  A field out of range returns
 * STARKV_ERR_ARG.  The workspace must be sized with the same cfg.
 */
starkv_status starkv_decode_workspace_size_cfg(const starkv_dims* dims, int32_t batch,
                                               int32_t max_seq_len,
                                               const starkv_decode_config* cfg /* (host) */,
                                               size_t* bytes /* (host) */);
starkv_status starkv_decode_attn_cfg(const starkv_dims* dims, const void* q, const void* k_cache,
                                     const void* v_cache, const void* U, const void* W,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* seq_lens, int32_t batch,
                                     int32_t max_seq_len, float scale,
                                     const starkv_decode_config* cfg /* (host) */, void* out,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * starkv_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  The call allocates nothing:
 * its scratch (q~, the split partials) is a device array of the library,
 * STARKV_NOALLOC_SCRATCH_BYTES per GPU, held from the library's first use on
 * that GPU until the process ends.  A batch / length whose plan needs more
 * scratch than that (starkv_decode_workspace_size reports the need) returns
 * STARKV_ERR_WORKSPACE before anything is launched; e.g. 64 sequences of up
 * to 8192 tokens, or 20 of 32768, at the main shape fit.  Every call on one
 * GPU shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, other host threads) race on it and must be serialised by the
 * caller.  Nothing in the scratch needs to start at zero.  Same arguments
 * and result as starkv_decode_attn otherwise (the library's plan).
 */
#define STARKV_NOALLOC_SCRATCH_BYTES (32u << 20)
starkv_status starkv_decode_attn_noalloc(const starkv_dims* dims, const void* q,
                                         const void* k_cache, const void* v_cache, const void* U,
                                         const void* W, const int32_t* block_tables,
                                         int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                         int32_t batch, int32_t max_seq_len, float scale,
                                         void* out, void* stream);

/*
 * starkv_decode_attn over FP8 caches (see starkv_append_fp8): the same
 * attention on the latents scale * value(code); k_scale folds into q~ and
 * v_scale into the split partials, so the kernels do the same work on half
 * the bytes (codes become fp16 matrix-core operands as they are used).
 * Shapes as for starkv_decode_attn (tuned FP8 instances: (32, 128, 64, 512)
 * with Hkv 32 or 8, and (4, 64, 16, 64); the generic kernels otherwise).
 * Workspace as for starkv_decode_attn (starkv_decode_workspace_size covers
 * both caches' needs).
 */
starkv_status starkv_decode_attn_fp8(const starkv_dims* dims, const void* q,
                                     const void* k_cache8, const void* v_cache8, const void* U,
                                     const void* W, const int32_t* block_tables,
                                     int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                     int32_t batch, int32_t max_seq_len, float scale,
                                     float k_scale, float v_scale, void* out, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * Workspace bytes for starkv_prefill_attn with total_q chunk queries.
 */
starkv_status starkv_prefill_workspace_size(const starkv_dims* dims, int32_t batch,
                                            int32_t total_q, int32_t max_seq_len,
                                            size_t* bytes /* (host) */);

/*
 * Chunked-prefill attention (README, "Per-prefill-chunk attention").
 * Request b owns query rows query_start_loc[b] .. query_start_loc[b+1]-1,
 * the last C_b = query_start_loc[b+1] - query_start_loc[b] of its
 * seq_lens[b] cached tokens (append the chunk first).  Chunk query j sits at
 * position P0 + j, P0 = seq_lens[b] - C_b, and sees keys 0 .. P0 + j.
 *   q                [total_q][H][d] fp16
 *   query_start_loc  [batch + 1] int32, non-decreasing, [0] = 0, [batch] = total_q
 *   max_query_len    (host) >= every C_b
 *   block_tables, seq_lens, max_seq_len, scale: as for decode; C_b <= seq_lens[b]
 *   out              [total_q][H][d] fp16
 */
starkv_status starkv_prefill_attn(const starkv_dims* dims, const void* q,
                                  const int32_t* query_start_loc, int32_t total_q,
                                  int32_t max_query_len, const void* k_cache, const void* v_cache,
                                  const void* U, const void* W, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                  int32_t batch, int32_t max_seq_len, float scale, void* out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * starkv_prefill_attn over FP8 caches (see starkv_append_fp8): the same
 * chunked-prefill attention on the latents scale * value(code), k_scale
 * folded into q~ and v_scale into z; key codes become fp16 as they enter
 * the kernel's LDS key ring, value codes before their products.  Instances
 * and workspace as for starkv_decode_attn_fp8 / starkv_prefill_attn.
 */
starkv_status starkv_prefill_attn_fp8(const starkv_dims* dims, const void* q,
                                      const int32_t* query_start_loc, int32_t total_q,
                                      int32_t max_query_len, const void* k_cache8,
                                      const void* v_cache8, const void* U, const void* W,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* seq_lens, int32_t batch,
                                      int32_t max_seq_len, float scale, float k_scale,
                                      float v_scale, void* out, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * Profiling aid: time one kernel of later calls with the hipEvent_t pair
 * `start` / `stop`.  `stop` is bound to the selected kernel's dispatch and
 * `start` to the dispatch just before it in the same call (the q projection),
 * both through hipExtLaunchKernelGGL, so the elapsed time runs from the end
 * of that predecessor to the end of the selected kernel with nothing
 * enqueued between them.  Append and the Gram kernel have no predecessor:
 * `start` is recorded on the stream just before their launch.
 *   which = 0 none (clears), 1 decode split-K attention, 2 prefill attention,
 *   3 append, 4 the Gram-matrix kernel of the bases fit (no predecessor
 *   either), 5 the streaming read of starkv_util_stream_read (which then
 *   launches an empty one-wave kernel first, for `start`).  Events are owned
 *   by the caller and must outlive the calls.
 * Process-wide setting; not for concurrent use from several threads.
 */
starkv_status starkv_set_timing_events(void* start, void* stop, int32_t which);

/*
 * Split plan the decode call will use (host out-parameters), for reports.
 */
starkv_status starkv_decode_plan(const starkv_dims* dims, int32_t batch, int32_t max_seq_len,
                                 int32_t* pages_per_split, int32_t* num_splits);

/*
 * Bases from samples (the step before the path).  The pages calibrate U_h
 * and W offline by a short knowledge distillation (README, introduction and
 * "Quick start"); this is an unlearned stand-in that returns the
 * least-squares optimal bases of K/V samples:
 *     U_h spans the top-r_k eigenspace of K_h^T K_h   (head-wise for keys)
 *     W   spans the top-r_v eigenspace of V^T V       (joint for values)
 * where row n of K_h is k[n, h, :] and row n of V is vec(v[n]) (head-major,
 * as in the append).  The second moments are uncentred, as the compression
 * is linear with no offset.  Columns come out orthonormal (to fp16
 * rounding); within the subspace the basis is arbitrary.
 * Method: subspace iteration from u0 / w0, `iters` products with the Gram
 * matrix, each followed by a Cholesky QR orthonormalisation (fp64 normal
 * equations), two on the last.  The result is the top eigenspace when the
 * start is not deficient in it and the r-th and (r+1)-th eigenvalues are
 * apart: the error falls as (lambda_{r+1} / lambda_r)^iters.
 *   dims          head_dim a multiple of 64; rank_k, rank_v <= 512;
 *                 Hkv * head_dim <= 65536; block_size and num_blocks unused
 *   k, v          [num_samples][Hkv][d] fp16; num_samples >= rank_k, rank_v
 *   u0            [Hkv][d][r_k] fp32 starting matrices (e.g. Gaussian)
 *   w0            [Hkv*d][r_v] fp32
 *   iters         1 .. 1000
 *   U             [Hkv][d][r_k] fp16 out (the layout append/decode take)
 *   W             [Hkv*d][r_v] fp16 out
 *   workspace     >= starkv_fit_workspace_size(...) bytes; no initialisation
 *                 (about (Hkv*d)^2 * 4 bytes: the value Gram matrix in fp32)
 *   info          optional (NULL = not reported), int32 device word: set to
 *                 the number of non-positive pivots the Cholesky steps met
 *                 (0 on success; > 0 means rank-deficient samples or start,
 *                 and the output is then not orthonormal)
 *   residual      optional (NULL = not computed), 2 fp32 device words: the
 *                 convergence of the returned bases (before their fp16
 *                 rounding) as the relative invariant-subspace residual
 *                 ||G B - B (B^T G B)||_F / ||G B||_F, G the second-moment
 *                 matrix; [0] keys (largest over the heads), [1] values.
 *                 0 for an exact eigenspace.  By the Davis-Kahan sin-theta
 *                 theorem the sine of the largest angle between span(B) and
 *                 the top eigenspace is at most residual * ||G B||_F /
 *                 (lambda_r - lambda_{r+1}) when that gap is positive.  Costs
 *                 one more product with G per side.
 * Asynchronous on `stream`; about 20 kernels per iteration.
 */
starkv_status starkv_fit_workspace_size(const starkv_dims* dims, size_t* bytes /* (host) */);
starkv_status starkv_fit_bases(const starkv_dims* dims, const void* k, const void* v,
                               int32_t num_samples, const float* u0, const float* w0,
                               int32_t iters, void* U, void* W, void* workspace,
                               size_t workspace_bytes, int32_t* info, float* residual,
                               void* stream);

/*
 * Index checks (a debugging aid, not part of the attention path).  Decode,
 * prefill and append trust the contents of their device index arrays: they
 * skip block ids outside [0, num_blocks) and slots outside the cache, and
 * plan the split-K work for lengths up to max_seq_len, so a bad index shows
 * up as silently missing tokens rather than as an error.  This call scans the
 * arrays those calls would read (the paged cache of README "KV-cache
 * capacity": 16-token blocks reached through a block table, and the slots of
 * the new tokens) and reports what lies outside those ranges:
 *   block_tables  [batch][max_blocks_per_seq] int32; entry (b, j) is checked
 *                 for j < ceil(min(max(seq_lens[b], 0), max_seq_len) / 16)
 *   seq_lens      [batch] int32, each expected in [0, max_seq_len]
 *   slot_mapping  [num_tokens] int64 (may be NULL when num_tokens is 0);
 *                 each expected below num_blocks * 16 (negative = padding)
 *   report        [4] uint32 (device, 16-byte aligned), written by the call:
 *                 report[0]  bit 0: a block id out of range,
 *                            bit 1: a length out of range,
 *                            bit 2: a slot at or beyond the cache
 *                 report[1]  the first sequence with a bad block id,
 *                 report[2]  the first sequence with a bad length,
 *                 report[3]  the first token with a bad slot
 *                 (0xFFFFFFFF where there is none)
 * dims supplies num_blocks and block_size (16); its other fields are not
 * used.  Host checks as for decode (batch, max_seq_len, max_blocks_per_seq),
 * num_tokens >= 0.  One work group scans everything, so the call takes time
 * linear in batch * max_blocks_per_seq + num_tokens; asynchronous on stream.
 */
starkv_status starkv_check_indices(const starkv_dims* dims, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                   int32_t batch, int32_t max_seq_len,
                                   const int64_t* slot_mapping, int32_t num_tokens,
                                   uint32_t* report, void* stream);

/*
 * Measurement utility (not part of the attention path): read `bytes` bytes
 * at `src` (16-byte aligned, bytes a multiple of 16) with 16-byte loads, as a
 * streaming-read ceiling for the HBM rate.  `sink` is a device buffer of at
 * least 1024 uint32 that may be written.  Asynchronous on `stream`.
 */
starkv_status starkv_util_stream_read(const void* src, size_t bytes, void* sink, void* stream);

/*
 * Measurement utilities (not part of the attention path): a timing event
 * created with hipEventDisableSystemFence, so recording it adds no
 * system-scope cache write-back to the timed work and its timestamps match a
 * kernel trace; for use with starkv_set_timing_events.  Such an event does
 * not make device writes visible to the host: synchronise the device before
 * reading results or elapsed times.
 *   starkv_util_event_create      *event (host out) receives a hipEvent_t
 *   starkv_util_event_destroy     NULL is a no-op
 *   starkv_util_event_elapsed_ms  *ms (host out) = stop - start, both recorded
 *                                 and complete (hipEventElapsedTime)
 */
starkv_status starkv_util_event_create(void** event /* (host) */);
starkv_status starkv_util_event_destroy(void* event);
starkv_status starkv_util_event_elapsed_ms(void* start, void* stop, float* ms /* (host) */);

#ifdef __cplusplus
}
#endif

#endif /* STARKV_H_ */
