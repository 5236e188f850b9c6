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
// compiled instance of its own.  They are written for clarity over speed:
// scores and P.c_v run on the vector ALU in fp32, each work group covers at
// most 8 heads (so a value page is read once per group of 8 heads), and a
// prefill query is a row of its own that walks its causal prefix.
//
// Limits (checked on the host): d a multiple of 32 up to 256; r_k a multiple
// of 8 up to min(d, 256); r_v a multiple of 8 up to min(2048, Hkv * d).
//
// Rows: decode row b is sequence b (seq_lens[b] tokens, block-table row b);
// prefill row n is chunk query n of request b (query_start_loc[b] <= n <
// query_start_loc[b+1]), which sees the first P0 + j + 1 tokens of request b,
// j = n - query_start_loc[b], P0 = seq_lens[b] - C_b.
//
// Work group (split s, row, head group): it streams its pages one at a time.
// Per 16-token page, thread (head hh, token t) forms one score; thread hh runs
// the online-softmax update of its head (running max, rescale factor, sum)
// and writes the page's weights to LDS; every thread then updates its own
// (head, feature) accumulators, features tid + 256 j.  With one split the
// work group also normalises z and applies W_g; otherwise it writes its
// running max and sum (fp32) and its unnormalised z (fp32) for the merge.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace starkv {

constexpr int kGenThreads = 256;
constexpr int kGenHG = 8;   // heads per work group
constexpr int kGenFJ = 8;   // feature slots per thread: r_v <= 2048
constexpr int kGenBS = 16;  // tokens per page
constexpr int kGenSB = 8;   // key-row chunks a thread requests together

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

// z of one head (LDS, fp32, RV values) -> out[row, h, :] = scale * W_g z,
// one output per thread and round.
__device__ __forceinline__ void gen_upproject(const GenArgs& a, const float* z, int row, int h,
                                              float scale) {
  const int g = h / a.QG;
  for (int i = threadIdx.x; i < a.D; i += kGenThreads) {
    const half_t* wr = a.W + ((size_t)g * a.D + i) * a.RV;
    float o = 0.f;
    for (int f = 0; f < a.RV; f += 8) {
      const half8 w8 = *(const half8*)(wr + f);
#pragma unroll
      for (int e = 0; e < 8; ++e) o = __builtin_fmaf((float)w8[e], z[f + e], o);
    }
    a.out[((size_t)row * a.H + h) * a.D + i] = (half_t)(o * scale);
  }
}

template <bool FP8>
__global__ __launch_bounds__(kGenThreads) void generic_split_kernel(GenArgs a) {
  extern __shared__ __attribute__((aligned(16))) float gsm[];
  const int n_hg = (a.H + kGenHG - 1) / kGenHG;
  const int row = blockIdx.x / n_hg, hg = blockIdx.x % n_hg;
  const int s = blockIdx.y;
  const int h0 = hg * kGenHG;
  const int nh = min(kGenHG, a.H - h0);
  const int tid = threadIdx.x;
  int tb, L;
  gen_row(a, row, tb, L);
  const int n_pages = min((L + kGenBS - 1) / kGenBS, a.max_blocks);
  const int p0 = s * a.pages_per_split;
  const int p1 = min(p0 + a.pages_per_split, n_pages);
  const bool fused = a.num_splits == 1;
  if (!fused && p0 >= n_pages) return;  // whole work group, before any barrier

  float* sq = gsm;                   // [kGenHG][RK] q~ of the group's heads
  float* sS = sq + kGenHG * a.RK;    // [kGenHG][16] scores of the page
  float* sP = sS + kGenHG * kGenBS;  // [kGenHG][16] weights of the page
  float* sA = sP + kGenHG * kGenBS;  // [kGenHG] rescale factors, then sums
  float* sZ = sA + kGenHG;           // [RV] normalised z of one head (one split only)

  for (int i = tid; i < kGenHG * a.RK; i += kGenThreads) {
    const int hh = i / a.RK, r = i % a.RK;
    sq[i] = hh < nh ? a.qt[((size_t)row * a.H + h0 + hh) * a.RK + r] : 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;  // thread hh < nh: head hh's softmax state
  float acc[kGenHG][kGenFJ];
#pragma unroll
  for (int hh = 0; hh < kGenHG; ++hh)
#pragma unroll
    for (int j = 0; j < kGenFJ; ++j) acc[hh][j] = 0.f;
  __syncthreads();

  const int32_t* bt = a.block_tables + (size_t)tb * a.max_blocks;
  for (int p = p0; p < p1; ++p) {
    const int blk = bt[p];
    const int nv = ((unsigned)blk < (unsigned)a.num_blocks) ? min(kGenBS, L - p * kGenBS) : 0;
    if (nv <= 0) continue;  // uniform: an invalid block id masks its page
    // scores of (head hh, token t): two neighbouring threads per pair, each
    // taking every other 8-rank chunk of the key row.  A batch's chunks are
    // requested together (addresses clamped into the row, so no branch
    // separates the loads) and summed afterwards, one memory round trip per
    // kGenSB chunks instead of one per chunk.
    {
      const int pair = tid >> 1, half = tid & 1;
      const int hh = min(pair / kGenBS, kGenHG - 1), t = pair % kGenBS;
      const int g = min(h0 + hh, a.H - 1) / a.QG;
      const size_t kb = (((size_t)blk * a.Hkv + g) * kGenBS + t) * a.RK;
      const float* qv = sq + hh * a.RK;
      const int nch = a.RK / 8;
      float sc = 0.f;
      for (int c0 = 0; c0 < nch; c0 += 2 * kGenSB) {  // uniform
        Raw8<FP8> x[kGenSB];
#pragma unroll
        for (int i = 0; i < kGenSB; ++i) x[i].load(a.k_cache, kb + (size_t)min(c0 + half + 2 * i, nch - 1) * 8);
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
      }
      sc += __shfl_xor(sc, 1);
      if (half == 0 && pair < nh * kGenBS) sS[hh * kGenBS + t] = t < nv ? sc : -INFINITY;
    }
    __syncthreads();
    // online softmax of each head (log2 domain)
    if (tid < nh) {
      float mx = m_run;
      for (int t = 0; t < kGenBS; ++t) mx = fmaxf(mx, sS[tid * kGenBS + t]);
      const float alpha = (mx == m_run) ? 1.f : exp2f(m_run - mx);  // 0 on the first page
      float ps = 0.f;
      for (int t = 0; t < kGenBS; ++t) {
        const float sc = sS[tid * kGenBS + t];
        const float pt = sc == -INFINITY ? 0.f : exp2f(sc - mx);
        sP[tid * kGenBS + t] = pt;
        ps += pt;
      }
      l_run = l_run * alpha + ps;
      m_run = mx;
      sA[tid] = alpha;
    }
    __syncthreads();
    // P.c_v: this thread's features of every head of the group.  The value
    // columns of all its features are requested first (feature indices
    // clamped into range, so no branch separates the loads), then used.
    {
      Raw8<FP8> xv[kGenFJ][2];
#pragma unroll
      for (int j = 0; j < kGenFJ; ++j) {
        const int f = min(tid + kGenThreads * j, a.RV - 1);
        xv[j][0].load(a.v_cache, ((size_t)blk * a.RV + f) * kGenBS);
        xv[j][1].load(a.v_cache, ((size_t)blk * a.RV + f) * kGenBS + 8);
      }
#pragma unroll
      for (int j = 0; j < kGenFJ; ++j) {
        if (tid + kGenThreads * j >= a.RV) continue;
        float cv[kGenBS], c0[8], c1[8];
        xv[j][0].widen(c0);
        xv[j][1].widen(c1);
#pragma unroll
        for (int t = 0; t < kGenBS; ++t)  // slots past the end may be NaN
          cv[t] = t < nv ? (t < 8 ? c0[t] : c1[t - 8]) : 0.f;
#pragma unroll
        for (int hh = 0; hh < kGenHG; ++hh) {
          if (hh < nh) {
            float v = acc[hh][j] * sA[hh];
#pragma unroll
            for (int t = 0; t < kGenBS; ++t) v = __builtin_fmaf(sP[hh * kGenBS + t], cv[t], v);
            acc[hh][j] = v;
          }
        }
      }
    }
    __syncthreads();  // the next page rewrites sS, sP, sA
  }

  if (!fused) {
    // partial state of this split: running max and sum per head, and the
    // unnormalised z rows
    if (tid < nh) {
      float* mp = a.ml + ((size_t)row * a.H + h0 + tid) * 2 * a.num_splits + s;
      mp[0] = m_run;
      mp[a.num_splits] = l_run;
    }
#pragma unroll
    for (int hh = 0; hh < kGenHG; ++hh) {
      if (hh >= nh) break;
      float* zp = a.zpart + (((size_t)row * a.H + h0 + hh) * a.num_splits + s) * a.RV;
#pragma unroll
      for (int j = 0; j < kGenFJ; ++j) {
        const int f = tid + kGenThreads * j;
        if (f < a.RV) zp[f] = acc[hh][j];
      }
    }
    return;
  }
  // one split: per head, z = acc / l (zero for an empty row) to LDS, then
  // out = W_g z
  if (tid < nh) sA[tid] = l_run;
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < kGenHG; ++hh) {
    if (hh >= nh) break;  // uniform
    const float l = sA[hh];
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int j = 0; j < kGenFJ; ++j) {
      const int f = tid + kGenThreads * j;
      if (f < a.RV) sZ[f] = acc[hh][j] * inv;
    }
    __syncthreads();
    gen_upproject(a, sZ, row, h0 + hh, a.v_scale);
    __syncthreads();  // the next head rewrites sZ
  }
}

// Merge of the splits and the up-projection, one work group per (row, head):
// z = sum_s w_s z_s / sum_s w_s l_s with w_s = 2^(m_s - M), M the largest
// running max of the row's splits (splits past the row's pages are never
// written and never read), then out = v_scale * W_g z.
__global__ __launch_bounds__(kGenThreads) void generic_merge_kernel(GenArgs a) {
  extern __shared__ __attribute__((aligned(16))) float gsm[];
  const int row = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x;
  int tb, L;
  gen_row(a, row, tb, L);
  const int n_pages = min((L + kGenBS - 1) / kGenBS, a.max_blocks);
  const int ns = (n_pages + a.pages_per_split - 1) / a.pages_per_split;  // splits written
  const int S = a.num_splits;
  float* sw = gsm;              // [S] weights
  float* sred = sw + S;         // [kGenThreads] reduction
  float* sZ = sred + kGenThreads;  // [RV]
  const float* mp = a.ml + ((size_t)row * a.H + h) * 2 * S;
  // M = max_s m_s
  float mx = -INFINITY;
  for (int s = tid; s < ns; s += kGenThreads) mx = fmaxf(mx, mp[s]);
  sred[tid] = mx;
  __syncthreads();
  for (int w = kGenThreads / 2; w > 0; w >>= 1) {
    if (tid < w) sred[tid] = fmaxf(sred[tid], sred[tid + w]);
    __syncthreads();
  }
  const float M = sred[0];
  __syncthreads();
  float den = 0.f;
  for (int s = tid; s < ns; s += kGenThreads) {
    const float m = mp[s];
    const float w = m == -INFINITY ? 0.f : exp2f(m - M);
    sw[s] = w;
    den += w * mp[S + s];
  }
  sred[tid] = den;
  __syncthreads();
  for (int w = kGenThreads / 2; w > 0; w >>= 1) {
    if (tid < w) sred[tid] += sred[tid + w];
    __syncthreads();
  }
  const float inv = sred[0] > 0.f ? 1.f / sred[0] : 0.f;
  const float* zp = a.zpart + ((size_t)row * a.H + h) * S * a.RV;
  for (int f = tid; f < a.RV; f += kGenThreads) {
    float z = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float w = sw[s];
      if (w != 0.f) z = __builtin_fmaf(w, zp[(size_t)s * a.RV + f], z);
    }
    sZ[f] = z * inv;
  }
  __syncthreads();
  gen_upproject(a, sZ, row, h, a.v_scale);
}

// q~[n, h, :] = qscale * U_g^T q[n, h, :] (fp32): work group (16 tokens, h);
// the tokens' q rows are staged in LDS as fp32 and U_g in chunks of 32 rows
// (16-byte loads, the next chunk in flight), thread r accumulates rank r of
// all 16 tokens over d in order.
__global__ __launch_bounds__(kGenThreads) void generic_qproj_kernel(
    const half_t* __restrict__ q, const half_t* __restrict__ U, int n_tokens, int H, int QG,
    int D, int RK, float qscale, float* __restrict__ qt) {
  constexpr int TT = 16;  // tokens per work group
  constexpr int KC = 32;  // rows of U_g per staged chunk
  __shared__ float sq[TT][256];
  __shared__ __attribute__((aligned(16))) half_t sU[2][KC][256];
  const int tid = threadIdx.x;
  const int h = blockIdx.y, n0 = blockIdx.x * TT;
  const int g = h / QG;
  for (int i = tid; i < TT * D; i += kGenThreads) {
    const int tt = i / D, k = i % D;
    const int n = n0 + tt;
    sq[tt][k] = n < n_tokens ? (float)q[((size_t)n * H + h) * D + k] : 0.f;
  }
  // U_g moves through LDS in chunks of KC rows, the next chunk's 16-byte
  // pieces in flight while the current one is used (at most 4 per thread)
  const half_t* Ug = U + (size_t)g * D * RK;
  const int pieces = KC * (RK / 8);
  half8 pre[4];
  auto fetch = [&](int c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = tid + j * kGenThreads;
      if (idx < pieces)
        pre[j] = *(const half8*)(Ug + (size_t)(c * KC + idx / (RK / 8)) * RK + (idx % (RK / 8)) * 8);
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = tid + j * kGenThreads;
      if (idx < pieces) *(half8*)&sU[buf][idx / (RK / 8)][(idx % (RK / 8)) * 8] = pre[j];
    }
  };
  fetch(0);
  stage(0);
  __syncthreads();
  const int nc = D / KC;
  float acc[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) acc[tt] = 0.f;
  for (int c = 0; c < nc; ++c) {
    if (c + 1 < nc) fetch(c + 1);
    if (tid < RK) {  // thread r = tid accumulates rank r of the 16 tokens
#pragma unroll 4
      for (int k = 0; k < KC; ++k) {
        const float u = (float)sU[c & 1][k][tid];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) acc[tt] = __builtin_fmaf(sq[tt][c * KC + k], u, acc[tt]);
      }
    }
    if (c + 1 < nc) stage((c + 1) & 1);
    __syncthreads();
  }
  if (tid < RK) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
      if (n0 + tt < n_tokens) qt[((size_t)(n0 + tt) * H + h) * RK + tid] = acc[tt] * qscale;
  }
}

bool generic_shape_ok(const ShapeKey& s) {
  return s.d % 32 == 0 && s.d <= 256 && s.rk % 8 == 0 && s.rk <= s.d && s.rk <= 256 &&
         s.rv % 8 == 0 && s.rv <= 2048 && (long)s.rv <= (long)s.Hkv * s.d && s.Hkv >= 1 &&
         s.H % s.Hkv == 0 && s.H <= 4096;
}

int generic_head_groups(const ShapeKey& s) { return (s.H + kGenHG - 1) / kGenHG; }

hipError_t launch_generic_qproj(const ShapeKey& s, const void* q, const void* U, int n_tokens,
                                float scale, void* qt, int precedes, hipStream_t st) {
  if (n_tokens <= 0) return hipSuccess;
  launch_hooked(TIME_NONE, precedes, generic_qproj_kernel, dim3((n_tokens + 15) / 16, s.H),
                dim3(kGenThreads), st, (const half_t*)q, (const half_t*)U, n_tokens, s.H,
                s.H / s.Hkv, s.d, s.rk, scale * kLog2e, (float*)qt);
  return hipGetLastError();
}

// LDS of the split kernel: q~, scores, weights, factors, and one head's z
// when fused (at most 17.4 KiB within the limits).
static size_t split_lds(const ShapeKey& s, bool fused) {
  return sizeof(float) * ((size_t)kGenHG * s.rk + 2 * kGenHG * kGenBS + kGenHG +
                          (fused ? (size_t)s.rv : 0));
}

hipError_t launch_generic_attn(const ShapeKey& s, const void* qt, const int32_t* qsl, int rows,
                               const void* k_cache, const void* v_cache, const void* W,
                               const int32_t* block_tables, int max_blocks,
                               const int32_t* seq_lens, int num_blocks, int batch,
                               int pages_per_split, int num_splits, float* ml, float* zpart,
                               void* out, const LatentFormat& fmt, int which, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
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
  const bool fused = num_splits == 1;
  const dim3 grid((unsigned)((long)rows * generic_head_groups(s)), (unsigned)num_splits);
  const size_t lds = split_lds(s, fused);
  if (fmt.fp8)
    launch_hooked_lds(which, TIME_NONE, generic_split_kernel<true>, grid,
                      dim3(kGenThreads), lds, st, a);
  else
    launch_hooked_lds(which, TIME_NONE, generic_split_kernel<false>, grid,
                      dim3(kGenThreads), lds, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || fused) return e;
  const size_t mlds = sizeof(float) * ((size_t)num_splits + kGenThreads + s.rv);
  hipLaunchKernelGGL(generic_merge_kernel, dim3(rows, s.H), dim3(kGenThreads), mlds, st, a);
  return hipGetLastError();
}

}  // namespace starkv
