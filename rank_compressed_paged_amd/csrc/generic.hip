// Generic instances: decode and chunked-prefill attention on the latents for
// any shape within the limits below, fp16 or FP8 caches.  The method is the
// one of the tuned kernels (Proxima README, introduction: head-wise key
// latents, one joint value latent; "Per-decode-step attention": split-K
// attention, a combine and the up-projection matmul):
//   q~ = U_g^T q (pre-scaled by scale * log2 e, and k_scale for FP8),
//   s_t = q~ . c_k[t, g], p = softmax(s), z = sum_t p_t c_v[t],
//   out = W_g z (times v_scale for FP8).
// These kernels take every size at run time, so a model whose layers use
// other ranks (the README's rank profiles and learned per-layer ranks), other
// head counts or head sizes, or other grouped-query groups, runs without a
// compiled instance of its own.  They trade speed for generality where
// the tuned kernels do not: the decode scores run on the vector ALU in fp32,
// a decode work group covers at most 16 heads (so a value page is read once
// per group of 16 heads), a prefill work group 64 queries of one head, and a
// prefill beyond the tiled kernel's limits (r_k > 128, r_v > 1024) runs each
// chunk query as a row of its own that walks its causal prefix.  P.c_v, the
// prefill scores, the q projection and the up-projections run on the matrix
// cores.
//
// Limits (checked on the host): d a multiple of 32 up to 256; r_k a multiple
// of 8 up to min(d, 256); r_v a multiple of 8 up to min(2048, Hkv * d).
//
// Rows: decode row b is sequence b (seq_lens[b] tokens, block-table row b);
// prefill row n is chunk query n of request b (query_start_loc[b] <= n <
// query_start_loc[b+1]), which sees the first P0 + j + 1 tokens of request b,
// j = n - query_start_loc[b], P0 = seq_lens[b] - C_b.
//
// Work group (split s, row, group of 16 heads), eight waves: it streams its
// pages one at a time, the next page's requests in flight.  Per 16-token page, two neighbouring threads per
// (head hh, token t) form one score from fp32 q~ in LDS and the key row; the
// 16 lanes of head h run its online-softmax update (running max, rescale
// factor, sum) with cross-lane reductions and write the page's weights to
// LDS in fp16; then P.c_v runs as v_mfma_f32_16x16x16_f16 with the
// feature-major value page as A (4 tokens of one feature per lane) and the
// weights as B (tokens x heads), wave w owning feature tiles w, w + 8, ...
// With one split the work group also normalises z and applies W_g;
// otherwise it writes its running max and sum (fp32) and its unnormalised z
// (fp32) for the merge.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace starkv {

constexpr int kGenThreads = 256;
constexpr int kGenSHG = 16;        // heads per split work group
constexpr int kGenSThreads = 512;  // split work group: eight waves
constexpr int kGenFT = 16;         // 16-feature tiles per wave of the split: r_v <= 2048
constexpr int kGenBS = 16;  // tokens per page
constexpr int kGenSB = 8;   // key-row chunks a thread requests together
constexpr float kGPRaise = 8.f;  // lazy softmax reference: threshold (log2 units)

struct GenArgs {
  int H, Hkv, D, RK, RV, QG;
  const float* qt;            // [rows][H][RK] fp32, pre-scaled
  const void* k_cache;        // [NB][Hkv][16][RK], fp16 or E4M3 codes
  const void* v_cache;        // [NB][RV][16]
  const half_t* W;            // [Hkv*D][RV]
  const int32_t* block_tables;
  int max_blocks, num_blocks;
  const int32_t* seq_lens;
  const int32_t* qsl;         // prefill: [batch + 1]; decode: null
  int batch, rows;
  int pages_per_split, num_splits;
  float v_scale;              // FP8 value scale (1 for fp16)
  float* ml;                  // [rows][H][2][num_splits]: running max, then sum
  float* zpart;               // [rows][H][num_splits][RV] unnormalised z
  half_t* out;                // [rows][H][D]
};

// Block-table row and visible length of a row.
__device__ __forceinline__ void gen_row(const GenArgs& a, int row, int& tb, int& L) {
  if (a.qsl == nullptr) {
    tb = row;
    L = a.seq_lens[row];
    return;
  }
  int lo = 0, hi = a.batch;  // largest b with qsl[b] <= row
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.qsl[mid] <= row)
      lo = mid;
    else
      hi = mid;
  }
  tb = lo;
  L = a.seq_lens[lo] - (a.qsl[lo + 1] - row) + 1;
}

// Eight latents as loaded (fp16, or E4M3 codes), and their float values:
// the loads of a batch are requested as raw registers and widened when used.
template <bool FP8>
struct Raw8 {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  std::conditional_t<FP8, u32x2, half8> r;
  __device__ __forceinline__ void load(const void* base, size_t idx) {
    if constexpr (FP8)
      r = *(const u32x2*)((const uint8_t*)base + idx);
    else
      r = *(const half8*)((const half_t*)base + idx);
  }
  __device__ __forceinline__ void widen(float (&x)[8]) const {
    if constexpr (FP8) {
      typedef _Float16 half2v __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const half2v lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r[k], 1.0f, false);
        const half2v hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r[k], 1.0f, true);
        x[4 * k + 0] = (float)lo[0];
        x[4 * k + 1] = (float)lo[1];
        x[4 * k + 2] = (float)hi[0];
        x[4 * k + 3] = (float)hi[1];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (float)r[e];
    }
  }
};

// Sum over the 64 lanes of a wave.
__device__ __forceinline__ float gen_wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}
__device__ __forceinline__ float gen_wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

// z of one head (LDS, fp32, RV values) -> out[row, h, :] = scale * W_g z.
// Wave w takes output rows w, w + 4, ...; its lanes split each W row into
// 16-byte pieces (lane l: features 8l + 512j), so a load instruction reads
// 1 KiB of one row, and a row's products are summed across the wave.  Four
// rows' loads are requested together; z stays in registers (zero past RV).
constexpr int kGenUpRows = 4;   // rows whose loads are in flight together
constexpr int kGenUpParts = 4;  // 512-feature parts of a row: RV <= 2048
__device__ __forceinline__ void gen_upproject(const GenArgs& a, const float* z, int row, int h,
                                              float scale) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  constexpr int NWV = kGenSThreads / 64;  // called by the split kernel's work groups
  const int g = h / a.QG;
  float zr[kGenUpParts][8];
#pragma unroll
  for (int j = 0; j < kGenUpParts; ++j) {
    const int f = 8 * lane + 512 * j;
#pragma unroll
    for (int e = 0; e < 8; ++e) zr[j][e] = f < a.RV ? z[f + e] : 0.f;
  }
  const half_t* Wg = a.W + (size_t)g * a.D * a.RV;
  for (int i0 = w; i0 < a.D; i0 += NWV * kGenUpRows) {  // uniform
    half8 wv[kGenUpRows][kGenUpParts];
#pragma unroll
    for (int k = 0; k < kGenUpRows; ++k) {
      const int i = min(i0 + NWV * k, a.D - 1);
#pragma unroll
      for (int j = 0; j < kGenUpParts; ++j)
        wv[k][j] = *(const half8*)(Wg + (size_t)i * a.RV + min(8 * lane + 512 * j, a.RV - 8));
    }
#pragma unroll
    for (int k = 0; k < kGenUpRows; ++k) {
      float o = 0.f;
#pragma unroll
      for (int j = 0; j < kGenUpParts; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) o = __builtin_fmaf((float)wv[k][j][e], zr[j][e], o);
      o = gen_wave_sum(o);
      const int i = i0 + NWV * k;
      if (lane == 0 && i < a.D) a.out[((size_t)row * a.H + h) * a.D + i] = (half_t)(o * scale);
    }
  }
}

template <bool FP8, int NFT, bool IDS, bool RKW>
__global__ __launch_bounds__(kGenSThreads) void generic_split_kernel(GenArgs a) {
  static_assert(NFT == kGenFT || NFT == kGenFT / 2, "feature tiles per wave: r_v <= 128 * NFT");
  extern __shared__ __attribute__((aligned(16))) float gsm[];
  const int n_hg = (a.H + kGenSHG - 1) / kGenSHG;
  const int row = blockIdx.x / n_hg, hg = blockIdx.x % n_hg;
  const int s = blockIdx.y;
  const int h0 = hg * kGenSHG;
  const int nh = min(kGenSHG, a.H - h0);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, quad = lane >> 4;
  int tb, L;
  gen_row(a, row, tb, L);
  const int n_pages = min((L + kGenBS - 1) / kGenBS, a.max_blocks);
  const int p0 = s * a.pages_per_split;
  const int p1 = min(p0 + a.pages_per_split, n_pages);
  const bool fused = a.num_splits == 1;
  if (!fused && p0 >= n_pages) return;  // whole work group, before any barrier

  float* sq = gsm;                           // [16][RK] q~ of the group's heads
  float* sS = sq + kGenSHG * a.RK;           // [2][16 heads][16 tokens] scores
  float* sA = sS + 2 * kGenSHG * kGenBS;     // [2][16] rescale factors
  half_t* sPh = (half_t*)(sA + 2 * kGenSHG);  // [2][16 heads][16 tokens] weights, fp16
  int* sBlk = (int*)(sPh + 2 * kGenSHG * kGenBS);  // [kGenSThreads] block ids of the split
  float* sZ = (float*)(sBlk + kGenSThreads);  // [RV] normalised z of one head (one split only)

  for (int i = tid; i < kGenSHG * a.RK; i += kGenSThreads) {
    const int hh = i / a.RK, r = i % a.RK;
    sq[i] = hh < nh ? a.qt[((size_t)row * a.H + h0 + hh) * a.RK + r] : 0.f;
  }
  // the split's block ids: staged once (one vector load per thread) when a
  // split has at most kGenSThreads pages (IDS), else read from the table page
  // by page
  const int32_t* bt = a.block_tables + (size_t)tb * a.max_blocks;
  if constexpr (IDS) sBlk[tid] = p0 + tid < p1 ? bt[p0 + tid] : 0;
  // softmax state of head sh = 4w + lane/16 (waves 0-3), kept by its 16 lanes
  const int sh = 4 * w + (lane >> 4), st = lane & 15;
  float m_run = -INFINITY, l_run = 0.f;
  // z^T accumulators: feature tile ft = w + 8i holds features 16 ft + 4 quad
  // .. +3 of head col (the 16x16 product's layout)
  const int ntv = (a.RV + 15) / 16;
  float4v acc[NFT];
#pragma unroll
  for (int i = 0; i < NFT; ++i) acc[i] = zero4();
  __syncthreads();

  auto block_at = [&](int p) {
    if constexpr (IDS)
      return __builtin_amdgcn_readfirstlane(sBlk[p - p0]);
    else
      return bt[p];
  };
  // scores of (head hh, token t): two neighbouring threads per pair, each
  // taking every other 8-rank chunk of the key row; a batch's chunks are
  // requested together (addresses clamped into the row, so no branch
  // separates the loads) and summed afterwards
  const int pair = tid >> 1, half = tid & 1;
  const int hh_s = pair / kGenBS, t_s = pair % kGenBS;
  const int g_s = min(h0 + hh_s, a.H - 1) / a.QG;
  const int nch = a.RK / 8;
  const float* qv = sq + hh_s * a.RK;
  auto load_keys = [&](Raw8<FP8> (&x)[kGenSB], int blk, int c0) {
    const size_t kb = (((size_t)blk * a.Hkv + g_s) * kGenBS + t_s) * a.RK;
#pragma unroll
    for (int i = 0; i < kGenSB; ++i) x[i].load(a.k_cache, kb + (size_t)min(c0 + half + 2 * i, nch - 1) * 8);
  };
  auto dot_keys = [&](const Raw8<FP8> (&x)[kGenSB], int c0, float sc) {
#pragma unroll
    for (int i = 0; i < kGenSB; ++i) {
      const int c = c0 + half + 2 * i;
      if (c < nch) {
        float xf[8];
        x[i].widen(xf);
#pragma unroll
        for (int e = 0; e < 8; ++e) sc = __builtin_fmaf(qv[c * 8 + e], xf[e], sc);
      }
    }
    return sc;
  };
  auto loadable = [&](int blk) { return (unsigned)blk < (unsigned)a.num_blocks ? blk : 0; };
  // a lane's value operand: tokens 4 quad .. +3 of feature 16 ft + col
  typedef std::conditional_t<FP8, uint32_t, half4> VRaw;
  auto load_val = [&](int blk, int ft) {
    const int f = min(16 * ft + col, a.RV - 1);
    const size_t idx = ((size_t)blk * a.RV + f) * kGenBS + 4 * quad;
    if constexpr (FP8)
      return *(const uint32_t*)((const uint8_t*)a.v_cache + idx);
    else
      return *(const half4*)((const half_t*)a.v_cache + idx);
  };
  auto to_half4 = [&](VRaw v) {
    if constexpr (FP8) {
      typedef _Float16 half2v __attribute__((ext_vector_type(2)));
      const half2v lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, false);
      const half2v hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, true);
      return half4{lo[0], lo[1], hi[0], hi[1]};
    } else {
      return v;
    }
  };

  // Pages run as a software pipeline: at the top of page p, the first
  // 2*kGenSB key chunks and the value operands of page p+1 are requested
  // into the other of two operand slots (the loop is unrolled by two, so no
  // operand is copied), and the barriers order LDS only, so these requests
  // stay in flight while page p is processed.  Every page issues the same
  // requests with no branch around them (addresses clamped into the page,
  // the last page requests itself again), so each use waits only for its own
  // page.  Scores, weights and factors alternate between two LDS buffers, so
  // two barriers a page suffice.  An invalid block id reads block 0 and
  // masks its page.  (fp16 values at r_v > 1024 have no registers for two
  // pages: they are requested at their own page's top.)
  constexpr bool VLA = FP8 || NFT < kGenFT;
  Raw8<FP8> kr[2][kGenSB];
  VRaw vr[VLA ? 2 : 1][NFT];
  auto load_vals = [&](VRaw (&dst)[NFT], int blk) {
#pragma unroll
    for (int i = 0; i < NFT; ++i) dst[i] = load_val(blk, w + 8 * i);
  };
  if (p0 < p1) {
    const int blk0 = loadable(block_at(p0));
    load_keys(kr[0], blk0, 0);
    if constexpr (VLA) load_vals(vr[0], blk0);
  }
  auto page = [&](auto phase, int p) {
    constexpr int PH = decltype(phase)::value;
    VRaw (&vc)[NFT] = vr[VLA ? PH : 0];
    const int buf = (p - p0) & 1;
    const int blk_c = block_at(p);
    const int nv = ((unsigned)blk_c < (unsigned)a.num_blocks) ? min(kGenBS, L - p * kGenBS) : 0;
    const int blk = loadable(blk_c);
    const int blk_n = loadable(block_at(min(p + 1, p1 - 1)));
    if constexpr (!VLA) load_vals(vc, blk);
    load_keys(kr[PH ^ 1], blk_n, 0);
    if constexpr (VLA) load_vals(vr[PH ^ 1], blk_n);
    float sc = dot_keys(kr[PH], 0, 0.f);
    if constexpr (RKW) {  // r_k > 128: the rest of the key row in place
      for (int c0 = 2 * kGenSB; c0 < nch; c0 += 2 * kGenSB) {
        Raw8<FP8> x[kGenSB];
        load_keys(x, blk, c0);
        sc = dot_keys(x, c0, sc);
      }
    }
    // an invalid block id masks its page: no scores (-inf), zero value
    // operands; the page still runs, so each page waits the same way
    {
      sc += __shfl_xor(sc, 1);
      if (half == 0)
        sS[(buf * kGenSHG + hh_s) * kGenBS + t_s] = (hh_s < nh && t_s < nv) ? sc : -INFINITY;
      block_sync_lds();
      // online softmax (log2 domain): head sh on the 16 lanes of its group,
      // lane st = token; the weights are rounded to fp16 for the products
      // and summed as rounded
      if (w < 4) {  // uniform
        const float sv = sS[(buf * kGenSHG + sh) * kGenBS + st];
        float pm = sv;
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) pm = fmaxf(pm, __shfl_xor(pm, m));
        // lazy reference: it moves only when the page's max passes it by
        // more than 2^kGPRaise (P <= 2^kGPRaise in fp16); the merge combines
        // the splits' (reference, sum, z) whatever each reference is
        const float mx = pm > m_run + kGPRaise ? pm : m_run;
        const float alpha = (mx == m_run) ? 1.f : exp2f(m_run - mx);  // 0 on the first page
        const half_t ph = (half_t)(sv == -INFINITY ? 0.f : exp2f(sv - mx));
        sPh[(buf * kGenSHG + sh) * kGenBS + st] = ph;
        float ps = (float)ph;
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) ps += __shfl_xor(ps, m);
        l_run = l_run * alpha + ps;
        m_run = mx;
        if (st == 0) sA[buf * kGenSHG + sh] = alpha;
      }
      block_sync_lds();
      // P.c_v on the matrix cores: A = value operands (feature x token), B =
      // weights (token x head), column = head col
      const half4 pb = *(const half4*)&sPh[(buf * kGenSHG + col) * kGenBS + 4 * quad];
      const float al = sA[buf * kGenSHG + col];
      if (__builtin_amdgcn_ballot_w64(al != 1.f) != 0) {  // uniform; no request inside
#pragma unroll
        for (int i = 0; i < NFT; ++i) acc[i] = acc[i] * al;
      }
      const bool part = nv < kGenBS;  // uniform: tokens past the end may hold NaN
#pragma unroll
      for (int i = 0; i < NFT; ++i) {
        if (w + 8 * i < ntv) {  // uniform
          half4 av = to_half4(vc[i]);
          if (part) {
#pragma unroll
            for (int e = 0; e < 4; ++e) av[e] = 4 * quad + e < nv ? av[e] : (half_t)0.f;
          }
          acc[i] = mfma16x16x16(av, pb, acc[i]);
        }
      }
    }
  };
  int p = p0;
  for (; p + 2 <= p1; p += 2) {
    page(std::integral_constant<int, 0>{}, p);
    page(std::integral_constant<int, 1>{}, p + 1);
  }
  if (p < p1) page(std::integral_constant<int, 0>{}, p);
  __syncthreads();  // the loop's LDS buffers are reused below

  if (!fused) {
    // partial state of this split: running max and sum per head, and the
    // unnormalised z rows
    if (w < 4 && st == 0 && sh < nh) {
      float* mp = a.ml + ((size_t)row * a.H + h0 + sh) * 2 * a.num_splits + s;
      mp[0] = m_run;
      mp[a.num_splits] = l_run;
    }
    if (col < nh) {
      float* zp = a.zpart + (((size_t)row * a.H + h0 + col) * a.num_splits + s) * a.RV;
#pragma unroll
      for (int i = 0; i < NFT; ++i) {
        const int f0 = 16 * (w + 8 * i) + 4 * quad;
        if (w + 8 * i < ntv && f0 < a.RV) *(float4v*)(zp + f0) = acc[i];
      }
    }
    return;
  }
  // one split: per head, z = acc / l (zero for an empty row) to LDS, then
  // out = W_g z
  if (w < 4 && st == 0) sA[sh] = l_run;
  __syncthreads();
  for (int hh = 0; hh < nh; ++hh) {  // uniform
    if (col == hh) {
      const float l = sA[hh];
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int i = 0; i < NFT; ++i) {
        const int f0 = 16 * (w + 8 * i) + 4 * quad;
        if (w + 8 * i < ntv && f0 < a.RV) *(float4v*)(sZ + f0) = acc[i] * inv;
      }
    }
    __syncthreads();
    gen_upproject(a, sZ, row, h0 + hh, a.v_scale);
    __syncthreads();  // the next head rewrites sZ
  }
}

// Merge of the splits and the up-projection for TB rows (TB <= kGenMT) of one
// head, so each W_g row is fetched once per TB rows:
//  1. wave t < TB takes row t: M = max_s m_s and the weights w_s = 2^(m_s -
//     M) of its written splits (splits past the row's pages are never written
//     and never read), the denominator sum_s w_s l_s, by cross-lane sums;
//  2. z[t, f] = sum_s w_s z_s[f] / denominator into LDS (fp32), kGenSB
//     splits' values of four (row, feature) pairs requested together;
//  3. out[t, h, :] = v_scale * W_g z[t] on the matrix cores:
//     v_mfma_f32_16x16x32_f16 with A = 16 rows of W_g x 32 features (16
//     contiguous bytes per lane, straight from memory) and B column 2t + e =
//     part e of an fp16 hi/lo split of z[t] (hi + lo = z to about 2^-22);
//     the two parts' sums are added by a neighbour-lane exchange.  Wave w
//     owns output tiles w, w + 8, ... (TPW of them); W moves in batches of
//     8 / TPW chunks of each tile, double-buffered in registers, and the
//     first batch is requested before step 1, so W is in flight during the
//     merge.
constexpr int kGenMT = 8;          // rows per merge work group, at most (one per wave)
constexpr int kGenMergeThreads = 512;  // eight waves
template <int TPW>
__global__ __launch_bounds__(kGenMergeThreads) void generic_merge_kernel(GenArgs a, int tb) {
  static_assert(TPW == 1 || TPW == 2, "output tiles per wave");
  constexpr int KB = 8 / TPW;  // chunks per batch
  extern __shared__ __attribute__((aligned(16))) float gsm[];
  const int S = a.num_splits;
  float* sZ = gsm;                  // [tb][RV]
  float* sw = sZ + tb * a.RV;       // [tb][S]
  float* sInv = sw + tb * S;        // [tb]
  int* sNs = (int*)(sInv + tb);     // [tb]
  const int r0 = blockIdx.x * tb, h = blockIdx.y;
  const int nt = min(tb, a.rows - r0);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, quad = lane >> 4;
  const int ntiles = a.D / 16, nck = (a.RV + 31) / 32, nb = (nck + KB - 1) / KB;
  const half_t* Wg = a.W + (size_t)(h / a.QG) * a.D * a.RV;
  // W batch b: chunks KB*b .. of this wave's tiles (rows and features
  // clamped into W_g; the products ignore what lies past them)
  auto load_batch = [&](half8 (&dst)[TPW][KB], int b) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int orow = min((w + 8 * i) * 16 + col, a.D - 1);
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int f = min(32 * (KB * b + k) + 8 * quad, a.RV - 8);
        dst[i][k] = *(const half8*)(Wg + (size_t)orow * a.RV + f);
      }
    }
  };
  half8 wa0[TPW][KB], wa1[TPW][KB];
  load_batch(wa0, 0);
  // 1. weights
  if (w < nt) {  // uniform per wave
    const int row = r0 + w;
    int tbx, L;
    gen_row(a, row, tbx, L);
    const int n_pages = min((L + kGenBS - 1) / kGenBS, a.max_blocks);
    // a length past the call's bound must not reach past the row's splits
    const int ns = min((n_pages + a.pages_per_split - 1) / a.pages_per_split, S);
    const float* mp = a.ml + ((size_t)row * a.H + h) * 2 * S;
    float mx = -INFINITY;
    for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, mp[s]);
    mx = gen_wave_max(mx);
    float den = 0.f;
    for (int s = lane; s < ns; s += 64) {
      const float m = mp[s];
      const float ws = m == -INFINITY ? 0.f : exp2f(m - mx);
      sw[w * S + s] = ws;
      den += ws * mp[S + s];
    }
    den = gen_wave_sum(den);
    if (lane == 0) {
      sInv[w] = den > 0.f ? 1.f / den : 0.f;
      sNs[w] = ns;
    }
  }
  __syncthreads();
  // 2. z of the rows
  int ns_max = 0;
  for (int t = 0; t < nt; ++t) ns_max = max(ns_max, sNs[t]);
  const int pairs = nt * a.RV;
  for (int p0 = tid; p0 < pairs; p0 += 4 * kGenMergeThreads) {  // uniform trip count
    float x[4][kGenSB], z[4];
    int t4[4], f4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pp = min(p0 + u * kGenMergeThreads, pairs - 1);
      t4[u] = pp / a.RV;
      f4[u] = pp % a.RV;
      z[u] = 0.f;
    }
    for (int s0 = 0; s0 < ns_max; s0 += kGenSB) {  // uniform
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int ns = sNs[t4[u]];
        const float* zp = a.zpart + ((size_t)(r0 + t4[u]) * a.H + h) * S * a.RV + f4[u];
#pragma unroll
        for (int i = 0; i < kGenSB; ++i)
          x[u][i] = zp[(size_t)max(min(s0 + i, ns - 1), 0) * a.RV];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int ns = sNs[t4[u]];
#pragma unroll
        for (int i = 0; i < kGenSB; ++i) {
          const float ws = s0 + i < ns ? sw[t4[u] * S + s0 + i] : 0.f;
          if (ws != 0.f) z[u] = __builtin_fmaf(ws, x[u][i], z[u]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (p0 + u * kGenMergeThreads < pairs) sZ[t4[u] * a.RV + f4[u]] = z[u] * sInv[t4[u]];
  }
  __syncthreads();
  // 3. up-projection
  const int tcol = col >> 1, part = col & 1;
  float4v acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = zero4();
  auto compute_batch = [&](const half8 (&src)[TPW][KB], int b) {
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int c = KB * b + k;
      const int f = 32 * c + 8 * quad;
      half8 bz = {};
      if (tcol < nt && f < a.RV) {
        const float4v z0 = *(const float4v*)&sZ[tcol * a.RV + f];
        const float4v z1 = *(const float4v*)&sZ[tcol * a.RV + f + 4];
        half8 hi, lo;
        split_f16x8(z0, z1, hi, lo);
        bz = part ? lo : hi;
      }
#pragma unroll
      for (int i = 0; i < TPW; ++i)  // features past RV: B is zero there
        if (w + 8 * i < ntiles && c < nck) acc[i] = mfma16x16x32(src[i][k], bz, acc[i]);
    }
  };
  for (int b = 0; b < nb; b += 2) {  // uniform
    if (b + 1 < nb) load_batch(wa1, b + 1);
    compute_batch(wa0, b);
    if (b + 1 < nb) {
      if (b + 2 < nb) load_batch(wa0, b + 2);
      compute_batch(wa1, b + 1);
    }
  }
  // lanes 2t and 2t+1 hold the hi and lo sums of row t
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tile = w + 8 * i;
    if (tile >= ntiles) break;  // uniform
    float4v o;
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = acc[i][r] + xor_lane_small<1>(acc[i][r]);
    if (part == 0 && tcol < nt) {
      half4 hv;
#pragma unroll
      for (int r = 0; r < 4; ++r) hv[r] = (half_t)(o[r] * a.v_scale);
      *(half4*)(a.out + ((size_t)(r0 + tcol) * a.H + h) * a.D + tile * 16 + 4 * quad) = hv;
    }
  }
}

// Chunked prefill for the shapes without a tuned instance, r_k <= 128 and
// r_v <= 1024: a work group takes 64 chunk queries of one request and one
// head, so every page it streams serves 64 query rows (the split kernel's
// prefill rows each walk their own prefix).  Eight waves:
//   * waves 0 to 3 form the scores of query block w (16 queries) on the
//     matrix cores, v_mfma_f32_16x16x32_f16 with the key page as A (token x
//     32 ranks, 16 contiguous bytes per lane) and q~ as B, split into an fp16
//     hi/lo pair (two products per rank chunk), then the online softmax per
//     query (log2 domain, the quad-lane reductions); q~ waits in LDS as hi/lo
//     fragments; the weights go to LDS in fp16 and are summed as rounded, the
//     rescale factors beside them; a row's reference max moves only when a
//     page's max passes it by more than 2^8 (P <= 256 in fp16), so the
//     accumulators are rescaled on few pages, by a branch the whole wave
//     takes or skips;
//   * every wave then runs P.c_v for the four query blocks over its feature
//     tiles w, w + 8, ... (v_mfma_f32_16x16x16_f16, value operands as in the split
//     kernel), so each value operand feeds four products;
//   * page p+1's value operands and key chunks are requested at the top of
//     page p, into the other of two operand slots (no copies), with no branch
//     around any request, so every use waits only for its own page;
//   * weights and factors alternate between two LDS buffers: one LDS-only
//     barrier per page.
// The causal limit (query j sees keys up to P0 + j), the sequence end and
// invalid block ids mask scores (-inf); value operands past the sequence end
// or on an invalid page are zeroed by select, so NaN sentinels never enter a
// product.  The epilogue applies W_g to the 64 rows' normalised z (below).
constexpr int kGPThreads = 512;  // eight waves
constexpr int kGPQB = 4;         // 16-query blocks per work group
constexpr int kGPQ = 16 * kGPQB; // chunk queries per work group
constexpr int kGPKC = 4;         // 32-rank chunks of a key row: r_k <= 128
constexpr int kGPIds = 8192;     // pages of a request's table: 131072 tokens

template <bool FP8>
__global__ __launch_bounds__(kGPThreads) void generic_prefill_kernel(GenArgs a, int n_qb) {
  constexpr int NFT = kGenFT / 2;  // feature tiles per wave: r_v <= 1024
  __shared__ __attribute__((aligned(16))) half_t sPh[2][kGPQB][16][16];  // [buf][block][query][token]
  __shared__ float sAl[2][kGPQB][16];                                     // [buf][block][query]
  // q~ of the work group's queries as fp16 hi/lo B fragments:
  // [block][chunk][hi, lo][quad][query] 16-byte pieces
  __shared__ __attribute__((aligned(16))) half8 sQ[kGPQB][kGPKC][2][4][16];
  __shared__ float sL[kGPQB][16];                                   // final sums
  __shared__ __attribute__((aligned(16))) float4v sRed[kGPQB][8][64];  // epilogue partials
  __shared__ int sBlk[kGPIds];
  const int h = blockIdx.y;
  const int b = blockIdx.x / n_qb, qbk = blockIdx.x % n_qb;
  const int q_begin = a.qsl[b];
  const int Cn = a.qsl[b + 1] - q_begin;
  const int j0 = qbk * kGPQ;
  if (j0 >= Cn) return;  // whole work group, before any barrier
  const int L = a.seq_lens[b];
  const int P0 = L - Cn;
  const int nq = min(kGPQ, Cn - j0);
  const int last_key = min(L - 1, P0 + j0 + nq - 1);
  const int n_pages = last_key < 0 ? 0 : min(last_key / kGenBS + 1, a.max_blocks);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, quad = lane >> 4;
  const int g = h / a.QG;
  const int ntv = (a.RV + 15) / 16;
  const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks;
  // the pages' block ids, staged once (the host keeps the table's row length
  // within kGPIds)
  for (int i = tid; i < n_pages; i += kGPThreads) sBlk[i] = bt[i];

  // score waves: query block w (w < kGPQB), lane column = query
  const bool scorer = w < kGPQB;  // uniform per wave
  const int jq = j0 + 16 * (w % kGPQB) + col;
  const int jqc = min(jq, Cn - 1);         // rows past the chunk mirror its last query
  const int lim = min(L - 1, P0 + jqc);    // the last key this query sees
  const int nkc = (a.RK + 31) / 32;
  if (scorer) {
    const float* qp = a.qt + ((size_t)(q_begin + jqc) * a.H + h) * a.RK;
#pragma unroll
    for (int c = 0; c < kGPKC; ++c) {
      const int r0 = 32 * c + 8 * quad;
      half8 hi = {}, lo = {};
      if (c < nkc && r0 < a.RK) {
        const float4v x0 = *(const float4v*)(qp + r0);
        const float4v x1 = *(const float4v*)(qp + r0 + 4);
        split_f16x8(x0, x1, hi, lo);
      }
      sQ[w][c][0][quad][col] = hi;
      sQ[w][c][1][quad][col] = lo;
    }
  }
  float m_run = -INFINITY, l_run = 0.f;
  float4v acc[NFT][kGPQB];
#pragma unroll
  for (int i = 0; i < NFT; ++i)
#pragma unroll
    for (int k = 0; k < kGPQB; ++k) acc[i][k] = zero4();
  __syncthreads();

  typedef std::conditional_t<FP8, uint32_t, half4> VRaw;
  auto load_val = [&](int blk, int ft) {
    const int f = min(16 * ft + col, a.RV - 1);
    const size_t idx = ((size_t)blk * a.RV + f) * kGenBS + 4 * quad;
    if constexpr (FP8)
      return *(const uint32_t*)((const uint8_t*)a.v_cache + idx);
    else
      return *(const half4*)((const half_t*)a.v_cache + idx);
  };
  auto to_half4 = [&](VRaw v) {
    if constexpr (FP8) {
      typedef _Float16 half2v __attribute__((ext_vector_type(2)));
      const half2v lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, false);
      const half2v hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, true);
      return half4{lo[0], lo[1], hi[0], hi[1]};
    } else {
      return v;
    }
  };
  auto to_half8 = [&](const Raw8<FP8>& k) {
    if constexpr (FP8) {
      typedef _Float16 half2v __attribute__((ext_vector_type(2)));
      half8 o;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const half2v lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k.r[e], 1.0f, false);
        const half2v hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k.r[e], 1.0f, true);
        o[4 * e + 0] = lo[0];
        o[4 * e + 1] = lo[1];
        o[4 * e + 2] = hi[0];
        o[4 * e + 3] = hi[1];
      }
      return o;
    } else {
      return k.r;
    }
  };

  auto block_at = [&](int p) { return __builtin_amdgcn_readfirstlane(sBlk[p]); };
  auto loadable = [&](int blk) { return (unsigned)blk < (unsigned)a.num_blocks ? blk : 0; };
  // page operands: value operands (every wave) and key chunks of token col,
  // ranks 32 c + 8 quad .. +7 (score waves); kc/vc this page's, kn/vn the
  // next page's
  // page operands in two slots, page p in slot p % 2 (the loop is unrolled
  // by two, so no operand is copied).  Every wave issues the same loads on
  // every page, with addresses clamped into the page (tiles past r_v re-read
  // the last feature, the waves that form no scores read the page's first
  // key bytes, the last page requests itself again): with no branch around
  // a load, each use waits only for its own page's requests.
  VRaw vr[2][NFT];
  Raw8<FP8> kr[2][kGPKC];
  auto load_page = [&](VRaw (&v)[NFT], Raw8<FP8> (&k)[kGPKC], int blk) {
#pragma unroll
    for (int i = 0; i < NFT; ++i) v[i] = load_val(blk, w + 8 * i);
    const size_t kb = ((size_t)blk * a.Hkv + g) * kGenBS * a.RK;
#pragma unroll
    for (int c = 0; c < kGPKC; ++c)
      k[c].load(a.k_cache,
                kb + (scorer ? (size_t)col * a.RK + min(32 * c + 8 * quad, a.RK - 8) : 0));
  };
  if (n_pages > 0) load_page(vr[0], kr[0], loadable(block_at(0)));
  auto page = [&](auto phase, int p) {
    constexpr int PH = decltype(phase)::value;
    VRaw (&vc)[NFT] = vr[PH];
    Raw8<FP8> (&kc)[kGPKC] = kr[PH];
    load_page(vr[PH ^ 1], kr[PH ^ 1], loadable(block_at(min(p + 1, n_pages - 1))));
    const int blk_c = block_at(p);
    const int buf = p & 1;
    const bool valid = (unsigned)blk_c < (unsigned)a.num_blocks;  // uniform
    const int nv = valid ? min(kGenBS, L - p * kGenBS) : 0;  // tokens of the page that exist
    if (scorer) {
      // q~ from LDS at every page (the block index passes through an empty
      // asm, so the compiler does not keep the fragments in registers)
      int qw = w;
      asm volatile("" : "+v"(qw));
      float4v sc = zero4();
#pragma unroll
      for (int c = 0; c < kGPKC; ++c) {
        if (c < nkc) {  // uniform; ranks past r_k have zero q~
          const half8 ka = to_half8(kc[c]);
          sc = mfma16x16x32(ka, sQ[qw][c][0][quad][col], sc);
          sc = mfma16x16x32(ka, sQ[qw][c][1][quad][col], sc);
        }
      }
      // sc[i]: token 16 p + 4 quad + i, query col
      float sv[4];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * quad + i;
        const bool ok = t < nv && p * kGenBS + t <= lim;
        sv[i] = ok ? sc[i] : -INFINITY;
        mx = fmax_nn(mx, sv[i]);
      }
      mx = quad_max(mx);
      // lazy reference: a row's reference max moves only when the page's
      // max passes it by more than 2^kGPRaise, so P <= 2^kGPRaise stays
      // well inside fp16 and the accumulators are rescaled on few pages
      // (the softmax is invariant to the reference)
      const float m_new = mx > m_run + kGPRaise ? mx : m_run;
      const float alpha = m_new == m_run ? 1.f : exp2f(m_run - m_new);  // 0 on the first page
      half4 ph;
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ph[i] = (half_t)(sv[i] == -INFINITY ? 0.f : exp2f(sv[i] - m_new));
        ps += (float)ph[i];
      }
      ps = quad_sum(ps);
      l_run = l_run * alpha + ps;
      m_run = m_new;
      *(half4*)&sPh[buf][w][col][4 * quad] = ph;
      if (quad == 0) sAl[buf][w][col] = alpha;
    }
    block_sync_lds();
    half4 pb[kGPQB];
    float al[kGPQB];
    bool moved = false;
#pragma unroll
    for (int k = 0; k < kGPQB; ++k) {
      pb[k] = *(const half4*)&sPh[buf][k][col][4 * quad];
      al[k] = sAl[buf][k][col];
      moved |= al[k] != 1.f;
    }
    if (__builtin_amdgcn_ballot_w64(moved) != 0) {  // uniform; no request inside
#pragma unroll
      for (int i = 0; i < NFT; ++i)
#pragma unroll
        for (int k = 0; k < kGPQB; ++k) acc[i][k] = acc[i][k] * al[k];
    }
    const bool part = nv < kGenBS;  // uniform: tokens past the end may hold NaN
#pragma unroll
    for (int i = 0; i < NFT; ++i) {
      if (w + 8 * i < ntv) {  // uniform
        half4 av = to_half4(vc[i]);
        if (part) {
#pragma unroll
          for (int e = 0; e < 4; ++e) av[e] = 4 * quad + e < nv ? av[e] : (half_t)0.f;
        }
#pragma unroll
        for (int k = 0; k < kGPQB; ++k) acc[i][k] = mfma16x16x16(av, pb[k], acc[i][k]);
      }
    }
  };
  int p = 0;
  for (; p + 2 <= n_pages; p += 2) {
    page(std::integral_constant<int, 0>{}, p);
    page(std::integral_constant<int, 1>{}, p + 1);
  }
  if (p < n_pages) page(std::integral_constant<int, 0>{}, p);

  // Epilogue: out = v_scale * W_g z for the 64 rows, z = acc / l rounded to
  // fp16.  A lane's accumulator tile is the B operand of a 16x16x16 product
  // as it stands (feature 16 ft + 4 quad + e of query col), so wave w forms
  // the partial outputs over its own feature tiles, output tile by output
  // tile (A = 16 rows of W_g x 16 features, 8 contiguous bytes per lane), and
  // the eight waves' partials are summed through LDS.  W_g is read once per
  // work group; the next output tile's rows are requested before the sums.
  __syncthreads();  // the loop's LDS buffers are free
  if (scorer && quad == 0) sL[w][col] = l_run;
  __syncthreads();
  half4 z16[NFT][kGPQB];
#pragma unroll
  for (int k = 0; k < kGPQB; ++k) {
    const float l = sL[k][col];
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int i = 0; i < NFT; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) z16[i][k][e] = (half_t)(acc[i][k][e] * inv);
    }
  }
  const half_t* Wg = a.W + (size_t)g * a.D * a.RV;
  const int n_ot = a.D / 16;
  auto load_w = [&](half4 (&wa)[NFT], int ot) {
#pragma unroll
    for (int i = 0; i < NFT; ++i) {
      const int f0 = 16 * (w + 8 * i) + 4 * quad;
      // features past RV (the last tile's upper half) have no W column
      wa[i] = (w + 8 * i < ntv && f0 < a.RV)
                  ? *(const half4*)(Wg + (size_t)(16 * ot + col) * a.RV + f0)
                  : half4{};
    }
  };
  half4 wc[NFT], wn[NFT];
  load_w(wc, 0);
  for (int ot = 0; ot < n_ot; ++ot) {  // uniform
    float4v part[kGPQB];
#pragma unroll
    for (int k = 0; k < kGPQB; ++k) part[k] = zero4();
#pragma unroll
    for (int i = 0; i < NFT; ++i) {
      if (w + 8 * i < ntv) {  // uniform
#pragma unroll
        for (int k = 0; k < kGPQB; ++k) part[k] = mfma16x16x16(wc[i], z16[i][k], part[k]);
      }
    }
    if (ot + 1 < n_ot) load_w(wn, ot + 1);
#pragma unroll
    for (int k = 0; k < kGPQB; ++k) sRed[k][w][lane] = part[k];
    block_sync_lds();
    // thread t sums outputs 16 ot + 4 (l / 16) + 2 hf .. +1 of query l % 16
    // of block k over the eight waves (t = 128 k + 2 l + hf)
    {
      const int k = tid >> 7, l = (tid >> 1) & 63, hf = tid & 1;
      float o0 = 0.f, o1 = 0.f;
#pragma unroll
      for (int wv = 0; wv < 8; ++wv) {
        const float4v v = sRed[k][wv][l];
        o0 += v[2 * hf];
        o1 += v[2 * hf + 1];
      }
      const int j = j0 + 16 * k + (l & 15);
      if (j < Cn) {
        typedef _Float16 half2v __attribute__((ext_vector_type(2)));
        const int d = 16 * ot + 4 * (l >> 4) + 2 * hf;
        *(half2v*)(a.out + ((size_t)(q_begin + j) * a.H + h) * a.D + d) =
            half2v{(half_t)(o0 * a.v_scale), (half_t)(o1 * a.v_scale)};
      }
    }
    block_sync_lds();  // sRed is rewritten by the next output tile
#pragma unroll
    for (int i = 0; i < NFT; ++i) wc[i] = wn[i];
  }
}

// ds_read_b64_tr_b16: within each 16-lane group, lane q addresses row
// r0 + q/4, columns c0 + 4*(q%4); lane i then receives rows r0 .. r0+3 of
// column c0 + i.
typedef short gen_short4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ half4 gen_tr16(const half_t* p) {
  typedef __attribute__((address_space(3))) gen_short4v lds_short4v;
  const gen_short4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)p);
  return __builtin_bit_cast(half4, r);
}

// q~[n, h, :] = qscale * U_g^T q[n, h, :] (fp32) on the matrix cores:
// v_mfma_f32_16x16x32_f16 with A = U_g^T (16 ranks x 32 of d, read from LDS
// through the transposing read) and B = q^T (32 of d x 16 tokens, 16
// contiguous bytes of a q row per lane); the fp16 products are exact and the
// sums fp32.  Work group (TW*16 tokens, head h), four waves: wave w takes
// token group w % TW and the rank tiles w / TW, w / TW + 4/TW, ...  U_g
// passes through LDS in 32-row chunks (ranks padded to a multiple of 16 with
// zeros), the next chunk in flight while the current one is used.
constexpr int kGenQK = 32;                   // rows of U_g per chunk
constexpr int kGenQLd = 256 + 8;             // LDS row stride (halves)
template <int TW>
__global__ __launch_bounds__(kGenThreads) void generic_qproj_kernel(
    const half_t* __restrict__ q, const half_t* __restrict__ U, int n_tokens, int H, int QG,
    int D, int RK, float qscale, float* __restrict__ qt) {
  static_assert(TW == 1 || TW == 4, "one or four 16-token groups per work group");
  constexpr int RP = 4 / TW;        // waves per token group
  constexpr int SLOTS = 16 / RP;    // rank tiles per wave: r_k <= 256
  __shared__ __attribute__((aligned(16))) half_t sU[2][kGenQK][kGenQLd];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, quad = lane >> 4;
  const int h = blockIdx.y, g = h / QG;
  const int tg = w % TW, rp = w / TW;
  const int n = blockIdx.x * TW * 16 + tg * 16 + col;  // this lane's token (B column)
  const int ntile = (RK + 15) / 16, nc = D / kGenQK;
  // the q rows of this wave's tokens, all chunks (rows past the end mirror
  // the last token and are not stored)
  half8 bq[256 / kGenQK];
  const half_t* qrow = q + ((size_t)min(n, n_tokens - 1) * H + h) * D + quad * 8;
#pragma unroll
  for (int c = 0; c < 256 / kGenQK; ++c)
    if (c < nc) bq[c] = *(const half8*)(qrow + c * kGenQK);
  // U_g chunk staging: 16-byte pieces of RK/8 per row; ranks RK .. 16*ntile
  // are zero
  const half_t* Ug = U + (size_t)g * D * RK;
  const int ppr = 2 * ntile;              // pieces per staged row
  const int pieces = kGenQK * ppr;        // <= 1024: four per thread
  half8 pre[4];
  auto fetch = [&](int c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = tid + j * kGenThreads;
      const int r = idx / ppr, pc = idx % ppr;
      const half8 z = {};
      pre[j] = (idx < pieces && 8 * pc < RK) ? *(const half8*)(Ug + (size_t)(c * kGenQK + r) * RK + 8 * pc) : z;
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = tid + j * kGenThreads;
      if (idx < pieces) *(half8*)&sU[buf][idx / ppr][8 * (idx % ppr)] = pre[j];
    }
  };
  float4v acc[SLOTS];
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) acc[i] = zero4();
  fetch(0);
  stage(0);
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 256 / kGenQK; ++c) {
    if (c >= nc) break;  // uniform
    if (c + 1 < nc) fetch(c + 1);
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      const int rt = rp + RP * i;
      if (rt < ntile) {  // uniform
        const half_t* ap = &sU[c & 1][quad * 8 + (col >> 2)][rt * 16 + 4 * (col & 3)];
        const half4 a0 = gen_tr16(ap), a1 = gen_tr16(ap + 4 * kGenQLd);
        const half8 au = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        acc[i] = mfma16x16x32(au, bq[c], acc[i]);
      }
    }
    if (c + 1 < nc) stage((c + 1) & 1);
    __syncthreads();
  }
  // D[4*quad + e][col] = rank 16 rt + 4 quad + e of token col
  if (n < n_tokens) {
    float* dst = qt + ((size_t)n * H + h) * RK;
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      const int r0 = 16 * (rp + RP * i) + 4 * quad;
      if (r0 < RK) *(float4v*)(dst + r0) = acc[i] * qscale;
    }
  }
}

bool generic_shape_ok(const ShapeKey& s) {
  return s.d % 32 == 0 && s.d <= 256 && s.rk % 8 == 0 && s.rk <= s.d && s.rk <= 256 &&
         s.rv % 8 == 0 && s.rv <= 2048 && (long)s.rv <= (long)s.Hkv * s.d && s.Hkv >= 1 &&
         s.H % s.Hkv == 0 && s.H <= 4096;
}

int generic_head_groups(const ShapeKey& s) { return (s.H + kGenSHG - 1) / kGenSHG; }

hipError_t launch_generic_qproj(const ShapeKey& s, const void* q, const void* U, int n_tokens,
                                float scale, void* qt, int precedes, hipStream_t st) {
  if (n_tokens <= 0) return hipSuccess;
  // few tokens (a decode step): a work group per 16 tokens and head, its
  // waves sharing the rank tiles; many: 64 tokens per work group
  if (n_tokens < 256)
    launch_hooked(TIME_NONE, precedes, generic_qproj_kernel<1>, dim3((n_tokens + 15) / 16, s.H),
                  dim3(kGenThreads), st, (const half_t*)q, (const half_t*)U, n_tokens, s.H,
                  s.H / s.Hkv, s.d, s.rk, scale * kLog2e, (float*)qt);
  else
    launch_hooked(TIME_NONE, precedes, generic_qproj_kernel<4>, dim3((n_tokens + 63) / 64, s.H),
                  dim3(kGenThreads), st, (const half_t*)q, (const half_t*)U, n_tokens, s.H,
                  s.H / s.Hkv, s.d, s.rk, scale * kLog2e, (float*)qt);
  return hipGetLastError();
}

// LDS of the split kernel: q~, two buffers of scores, factors and fp16
// weights, the split's block ids, and one head's z when fused (at most
// 28.3 KiB within the limits).
static size_t split_lds(const ShapeKey& s, bool fused) {
  return sizeof(float) * ((size_t)kGenSHG * s.rk + 2 * kGenSHG * kGenBS + 2 * kGenSHG +
                          kGenSHG * kGenBS + kGenSThreads + (fused ? (size_t)s.rv : 0));
}

static GenArgs gen_args(const ShapeKey& s, const void* qt, const int32_t* qsl, int rows,
                        const void* k_cache, const void* v_cache, const void* W,
                        const int32_t* block_tables, int max_blocks, const int32_t* seq_lens,
                        int num_blocks, int batch, int pages_per_split, int num_splits,
                        float* ml, float* zpart, void* out, const LatentFormat& fmt) {
  GenArgs a;
  a.H = s.H;
  a.Hkv = s.Hkv;
  a.D = s.d;
  a.RK = s.rk;
  a.RV = s.rv;
  a.QG = s.H / s.Hkv;
  a.qt = (const float*)qt;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.W = (const half_t*)W;
  a.block_tables = block_tables;
  a.max_blocks = max_blocks;
  a.num_blocks = num_blocks;
  a.seq_lens = seq_lens;
  a.qsl = qsl;
  a.batch = batch;
  a.rows = rows;
  a.pages_per_split = pages_per_split;
  a.num_splits = num_splits;
  a.v_scale = fmt.fp8 ? fmt.v_scale : 1.f;
  a.ml = ml;
  a.zpart = zpart;
  a.out = (half_t*)out;
  return a;
}

// The merge and up-projection over `rows` rows of num_splits splits each.
static hipError_t launch_generic_merge(const ShapeKey& s, const GenArgs& a, int rows,
                                       int num_splits, hipStream_t st) {
  // rows per merge work group: several rows share each fetch of W_g once
  // there are enough (row, head) pairs to keep the CUs busy, as long as
  // their z and weights fit 64 KiB of LDS
  const long pairs = (long)rows * s.H;
  int tb = pairs >= 4096 ? kGenMT : (pairs >= 1024 ? 4 : (pairs >= 256 ? 2 : 1));
  auto merge_lds = [&](int t) {
    return sizeof(float) * ((size_t)t * s.rv + (size_t)t * num_splits + 2 * (size_t)t);
  };
  while (tb > 1 && merge_lds(tb) > 65536) tb /= 2;
  const size_t mlds = merge_lds(tb);
  const dim3 mgrid((rows + tb - 1) / tb, s.H);
  const int tiles = s.d / 16;  // output tiles of 16 over the 8 waves: d <= 256
  if (tiles <= 8)
    hipLaunchKernelGGL(generic_merge_kernel<1>, mgrid, dim3(kGenMergeThreads), mlds, st, a, tb);
  else
    hipLaunchKernelGGL(generic_merge_kernel<2>, mgrid, dim3(kGenMergeThreads), mlds, st, a, tb);
  return hipGetLastError();
}

// the split kernel instance for a call: FP8 caches or not, 8 or 16
// feature tiles per wave, block ids staged in LDS or read from the table,
// key rows of more than 128 ranks or not
template <bool IDS, bool RKW>
static void launch_split(bool wide, bool fp8, dim3 grid, size_t lds, const GenArgs& a, int which,
                         hipStream_t st) {
  if (fp8) {
    if (wide)
      launch_hooked_lds(which, TIME_NONE, generic_split_kernel<true, kGenFT, IDS, RKW>, grid,
                        dim3(kGenSThreads), lds, st, a);
    else
      launch_hooked_lds(which, TIME_NONE, generic_split_kernel<true, kGenFT / 2, IDS, RKW>, grid,
                        dim3(kGenSThreads), lds, st, a);
  } else {
    if (wide)
      launch_hooked_lds(which, TIME_NONE, generic_split_kernel<false, kGenFT, IDS, RKW>, grid,
                        dim3(kGenSThreads), lds, st, a);
    else
      launch_hooked_lds(which, TIME_NONE, generic_split_kernel<false, kGenFT / 2, IDS, RKW>,
                        grid, dim3(kGenSThreads), lds, st, a);
  }
}

hipError_t launch_generic_attn(const ShapeKey& s, const void* qt, const int32_t* qsl, int rows,
                               const void* k_cache, const void* v_cache, const void* W,
                               const int32_t* block_tables, int max_blocks,
                               const int32_t* seq_lens, int num_blocks, int batch,
                               int pages_per_split, int num_splits, float* ml, float* zpart,
                               void* out, const LatentFormat& fmt, int which, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const GenArgs a = gen_args(s, qt, qsl, rows, k_cache, v_cache, W, block_tables, max_blocks,
                             seq_lens, num_blocks, batch, pages_per_split, num_splits, ml, zpart,
                             out, fmt);
  const bool fused = num_splits == 1;
  const dim3 grid((unsigned)((long)rows * generic_head_groups(s)), (unsigned)num_splits);
  const size_t lds = split_lds(s, fused);
  // feature tiles per wave: 8 cover r_v <= 1024, 16 the rest
  const bool wide = s.rv > 8 * 16 * (kGenFT / 2);
  const bool ids = pages_per_split <= kGenSThreads, rkw = s.rk > 16 * kGenSB;
  if (ids && !rkw)
    launch_split<true, false>(wide, fmt.fp8, grid, lds, a, which, st);
  else if (ids)
    launch_split<true, true>(wide, fmt.fp8, grid, lds, a, which, st);
  else if (!rkw)
    launch_split<false, false>(wide, fmt.fp8, grid, lds, a, which, st);
  else
    launch_split<false, true>(wide, fmt.fp8, grid, lds, a, which, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || fused) return e;
  return launch_generic_merge(s, a, rows, num_splits, st);
}

bool generic_prefill_tiled(const ShapeKey& s, int max_blocks) {
  return s.rk <= 32 * kGPKC && s.rv <= 8 * 16 * (kGenFT / 2) && max_blocks <= kGPIds;
}

hipError_t launch_generic_prefill(const ShapeKey& s, const void* qt, const int32_t* qsl,
                                  int total_q, int max_query_len, const void* k_cache,
                                  const void* v_cache, const void* W,
                                  const int32_t* block_tables, int max_blocks,
                                  const int32_t* seq_lens, int num_blocks, int batch, void* out,
                                  const LatentFormat& fmt, int which, hipStream_t st) {
  if (total_q <= 0 || batch <= 0 || max_query_len <= 0) return hipSuccess;
  if (max_blocks > kGPIds) return hipErrorInvalidValue;  // the staged block ids fit in LDS
  const GenArgs a = gen_args(s, qt, qsl, total_q, k_cache, v_cache, W, block_tables, max_blocks,
                             seq_lens, num_blocks, batch, max_blocks, 1, nullptr, nullptr, out,
                             fmt);
  const int n_qb = (max_query_len + kGPQ - 1) / kGPQ;
  const dim3 grid((unsigned)((long)batch * n_qb), (unsigned)s.H);
  if (fmt.fp8)
    launch_hooked_lds(which, TIME_NONE, generic_prefill_kernel<true>, grid, dim3(kGPThreads), 0,
                      st, a, n_qb);
  else
    launch_hooked_lds(which, TIME_NONE, generic_prefill_kernel<false>, grid, dim3(kGPThreads),
                      0, st, a, n_qb);
  return hipGetLastError();
}

}  // namespace starkv
