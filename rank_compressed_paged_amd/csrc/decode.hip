// Decode attention over a paged, low-rank-compressed KV cache (gfx950).
//
// Method (Proxima README, introduction): keys are stored as head-wise
// latents c_k[t,h] = U_h^T k[t,h] and values as one joint latent
// c_v[t] = W^T vec(v[t]) shared by all heads.  Attention never rebuilds K or
// V: with q~_h = U_h^T q_h the scores are q~_h . c_k[t,h] / sqrt(d), the
// softmax weights p sum the value latents, z_h = sum_t p c_v[t], and the
// output is the matmul out_h = W_h z_h (the "matmul per step" of the
// README's "Per-decode-step attention" notes), W_h being rows h*d..h*d+d-1.
//
// One decode step is four launches on the caller's stream:
//   1. qproj        q~ = U_h^T q, pre-scaled by scale*log2(e), fp16
//   2. decode_split split-K pass over the pages (README, "Kernel profiling
//                   breakdown": split-K attention plus a combine); one work
//                   group owns all heads of a run of pages so the joint value
//                   latent of each token is read from HBM exactly once
//   3. combine      log-sum-exp merge of the splits -> z [B, H, r_v] fp32
//   4. upproj       out_h = W_h z_h on the matrix cores, z split into an
//                   fp16 hi/lo pair so the product keeps fp32 accuracy
//
// decode_split per page (16 tokens) in a work group of NW waves:
//   * scores: wave w owns heads [w*HPW, (w+1)*HPW).  For each head the 16x64
//     key page is the A operand of v_mfma_f32_16x16x32_f16 and q~_h sits in
//     column (h - w*HPW) of B, zeros elsewhere, so one 16x16 accumulator
//     collects the scores of all the wave's heads (tokens x heads).  The
//     lane that holds column c then runs the online-softmax update of that
//     head on its 4 tokens plus a 4-lane butterfly.
//   * P (fp16) and the rescale factors go through LDS (double-buffered, one
//     barrier per page).
//   * values: wave w owns features [w*FPW, (w+1)*FPW).  Z^T[f, h] +=
//     sum_t c_v[t, f] P[h, t] with v_mfma_f32_16x16x16_f16: the feature-major
//     value page gives each lane 8 contiguous bytes, and the accumulator
//     column is the head, so the rescale is one scalar per lane.
//   * the next page's keys and values are loaded into registers before the
//     current page is processed.
#include "common.h"
#include "kernels.h"

namespace starkv {

template <int H, int RK, int RV, int NW>
struct DecodeCfg {
  static constexpr int HPW = H / NW;        // heads per wave (scores)
  static constexpr int FPW = RV / NW;       // value features per wave
  static constexpr int RT = (H + 15) / 16;  // 16-row head tiles
  static constexpr int R16 = RT * 16;
  static constexpr int FT = FPW / 16;       // 16-feature tiles per wave
  static constexpr int KC = (RK % 32 == 0) ? 32 : 16;
  static constexpr int NKC = RK / KC;
  static_assert(H % NW == 0 && HPW >= 1 && HPW <= 16, "heads per wave must be 1..16");
  static_assert(RV % (16 * NW) == 0, "value rank must split into 16-wide tiles per wave");
  static_assert(RK % 16 == 0, "key rank must be a multiple of 16");
};

constexpr int BS = 16;  // tokens per page

// ---------------------------------------------------------------------------
// 1. q~[n, h, :] = (scale*log2e) * U_h^T q[n, h, :]  (fp32 math, fp16 out)
// grid (H, ceil(N / QT)), 256 threads
// ---------------------------------------------------------------------------
template <int H, int D, int RK>
__global__ __launch_bounds__(256) void qproj_kernel(const half_t* __restrict__ q,
                                                    const half_t* __restrict__ U, int n_tokens,
                                                    float qscale, half_t* __restrict__ qt) {
  constexpr int QT = 16;
  __shared__ float sU[D][RK + 1];
  __shared__ float sQ[QT][D];
  const int h = blockIdx.x;
  const int n0 = blockIdx.y * QT;
  const int tid = threadIdx.x;
  const half_t* Uh = U + (size_t)h * D * RK;
  for (int i = tid; i < D * RK; i += 256) sU[i / RK][i % RK] = (float)Uh[i];
  for (int i = tid; i < QT * D; i += 256) {
    const int n = n0 + i / D;
    sQ[i / D][i % D] = (n < n_tokens) ? (float)q[((size_t)n * H + h) * D + (i % D)] : 0.f;
  }
  __syncthreads();
  constexpr int STEP = 256 / RK;
  const int r = tid % RK;
  for (int qi = tid / RK; qi < QT; qi += STEP) {
    const int n = n0 + qi;
    if (n >= n_tokens) break;
    float accv = 0.f;
#pragma unroll 8
    for (int i = 0; i < D; ++i) accv = fmaf(sU[i][r], sQ[qi][i], accv);
    qt[((size_t)n * H + h) * RK + r] = (half_t)(accv * qscale);
  }
}

// ---------------------------------------------------------------------------
// 2. split-K latent attention
// ---------------------------------------------------------------------------
struct SplitArgs {
  const half_t* qt;
  const half_t* k_cache;
  const half_t* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* ml;   // [B][S][2][R16]
  float* acc;  // [B][S][NW][RT][FT][64][4]
  int max_blocks, num_blocks, pages_per_split, num_splits;
};

template <int H, int RK, int RV, int NW>
struct PageRegs {
  using C = DecodeCfg<H, RK, RV, NW>;
  typedef _Float16 kvec __attribute__((ext_vector_type(C::KC / 4)));
  kvec k[C::HPW][C::NKC];
  half4 v[C::FT];
};

template <int H, int RK, int RV, int NW>
__device__ __forceinline__ void load_page(PageRegs<H, RK, RV, NW>& pr, const half_t* __restrict__ kc,
                                          const half_t* __restrict__ vc, int blk, int w, int col,
                                          int quad) {
  using C = DecodeCfg<H, RK, RV, NW>;
  using kvec = typename PageRegs<H, RK, RV, NW>::kvec;
  // keys: head (w*HPW + hl), token row `col`, k chunk `quad`
  const half_t* kb = kc + (((size_t)blk * H + w * C::HPW) * BS + col) * RK + quad * (C::KC / 4);
#pragma unroll
  for (int hl = 0; hl < C::HPW; ++hl)
#pragma unroll
    for (int c = 0; c < C::NKC; ++c)
      pr.k[hl][c] = *(const kvec*)(kb + (size_t)hl * BS * RK + c * C::KC);
  // values: feature (w*FPW + ft*16 + col), tokens 4*quad .. 4*quad+3
  const half_t* vb = vc + ((size_t)blk * RV + w * C::FPW + col) * BS + quad * 4;
#pragma unroll
  for (int ft = 0; ft < C::FT; ++ft) pr.v[ft] = *(const half4*)(vb + (size_t)ft * 16 * BS);
}

template <int H, int RK, int RV, int NW>
__global__ __launch_bounds__(NW * 64) void decode_split_kernel(SplitArgs a) {
  using C = DecodeCfg<H, RK, RV, NW>;
  using kvec = typename PageRegs<H, RK, RV, NW>::kvec;
  __shared__ __attribute__((aligned(16))) half_t sP[2][C::R16][BS];
  __shared__ float sAlpha[2][C::R16];
  __shared__ int sFlag[2];  // page index whose softmax step moved a running max

  const int s = blockIdx.x, b = blockIdx.y;
  const int L = a.seq_lens[b];
  const int n_pages = min(min((L + BS - 1) / BS, a.max_blocks), a.num_splits * a.pages_per_split);
  const int p0 = s * a.pages_per_split;
  if (p0 >= n_pages) return;
  const int p1 = min(p0 + a.pages_per_split, n_pages);

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, quad = lane >> 4;

  // rows >= H are padding: P stays zero there, alpha one
  for (int i = tid; i < 2 * C::R16 * BS; i += NW * 64) (&sP[0][0][0])[i] = (half_t)0.f;
  for (int i = tid; i < 2 * C::R16; i += NW * 64) (&sAlpha[0][0])[i] = 1.f;
  if (tid < 2) sFlag[tid] = -1;

  // q~ of head (w*HPW + col) for this lane's k chunks; B column col
  kvec qv[C::NKC];
  {
    const int hq = w * C::HPW + (col < C::HPW ? col : 0);
    const half_t* qp = a.qt + ((size_t)b * H + hq) * RK + quad * (C::KC / 4);
#pragma unroll
    for (int c = 0; c < C::NKC; ++c) qv[c] = *(const kvec*)(qp + c * C::KC);
  }
  const kvec kzero = {};

  float m_run = -INFINITY, l_run = 0.f;
  float4v acc[C::RT][C::FT];
#pragma unroll
  for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
    for (int ft = 0; ft < C::FT; ++ft) acc[rt][ft] = zero4();

  const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks;
  auto safe_block = [&](int p) {
    const int blk = bt[p];
    return ((unsigned)blk < (unsigned)a.num_blocks) ? blk : -1;
  };

  PageRegs<H, RK, RV, NW> cur, nxt;
  int blk_cur = safe_block(p0);
  if (blk_cur >= 0) load_page<H, RK, RV, NW>(cur, a.k_cache, a.v_cache, blk_cur, w, col, quad);
  __syncthreads();  // LDS init visible

  for (int p = p0; p < p1; ++p) {
    const int buf = (p - p0) & 1;
    int blk_nxt = -1;
    if (p + 1 < p1) {
      blk_nxt = safe_block(p + 1);
      if (blk_nxt >= 0) load_page<H, RK, RV, NW>(nxt, a.k_cache, a.v_cache, blk_nxt, w, col, quad);
    }
    const int valid = (blk_cur >= 0) ? min(BS, L - p * BS) : 0;  // uniform in the group

    if (valid > 0) {
      // ---- scores: tokens (rows) x wave heads (columns)
      float4v sacc = zero4();
#pragma unroll
      for (int hl = 0; hl < C::HPW; ++hl) {
#pragma unroll
        for (int c = 0; c < C::NKC; ++c) {
          const kvec bq = (col == hl) ? qv[c] : kzero;
          if constexpr (C::KC == 32)
            sacc = mfma16x16x32(cur.k[hl][c], bq, sacc);
          else
            sacc = mfma16x16x16(cur.k[hl][c], bq, sacc);
        }
      }
      // ---- online softmax of head (w*HPW + col) over this page
      float sv[4];
      float pm = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sv[r] = (quad * 4 + r < valid) ? sacc[r] : -INFINITY;
        pm = fmaxf(pm, sv[r]);
      }
      pm = max_over_quads(pm);
      const float m_new = fmaxf(m_run, pm);
      const float alpha = exp2f(m_run - m_new);
      float ps = 0.f;
      half4 ph;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pr = exp2f(sv[r] - m_new);
        ps += pr;
        ph[r] = (half_t)pr;
      }
      ps = sum_over_quads(ps);
      l_run = l_run * alpha + ps;
      m_run = m_new;
      if (col < C::HPW) {
        const int row = w * C::HPW + col;
        *(half4*)&sP[buf][row][quad * 4] = ph;
        if (quad == 0) sAlpha[buf][row] = alpha;
        if (alpha != 1.f) sFlag[buf] = p;
      }
    }
    __syncthreads();
    if (valid > 0) {
      const bool rescale = sFlag[buf] == p;  // uniform: skip when no max moved
      // ---- values: Z^T[f, h] = alpha_h Z^T[f, h] + sum_t c_v[t, f] P[h, t]
      half4 pb[C::RT];
#pragma unroll
      for (int rt = 0; rt < C::RT; ++rt) {
        pb[rt] = *(const half4*)&sP[buf][rt * 16 + col][quad * 4];
        if (rescale) {
          const float al = sAlpha[buf][rt * 16 + col];
#pragma unroll
          for (int ft = 0; ft < C::FT; ++ft) acc[rt][ft] *= al;
        }
      }
#pragma unroll
      for (int ft = 0; ft < C::FT; ++ft) {
        half4 av = cur.v[ft];
        if (valid < BS) {  // tail page: unused slots may hold anything (NaN)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (quad * 4 + e >= valid) av[e] = (half_t)0.f;
        }
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt) acc[rt][ft] = mfma16x16x16(av, pb[rt], acc[rt][ft]);
      }
    }
    if (p + 1 < p1) {
      cur = nxt;
      blk_cur = blk_nxt;
    }
  }

  // ---- partial state of this split
  const size_t ws = (size_t)b * a.num_splits + s;
  if (col < C::HPW && quad == 0) {
    a.ml[ws * 2 * C::R16 + w * C::HPW + col] = m_run;
    a.ml[ws * 2 * C::R16 + C::R16 + w * C::HPW + col] = l_run;
  }
  float4v* pa = (float4v*)(a.acc + (ws * NW + w) * (size_t)(C::RT * C::FT * 256));
#pragma unroll
  for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
    for (int ft = 0; ft < C::FT; ++ft) pa[(rt * C::FT + ft) * 64 + lane] = acc[rt][ft];
}

// ---------------------------------------------------------------------------
// 3. combine: z[b,h,:] = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s
// grid (H, B), 256 threads
// ---------------------------------------------------------------------------
template <int H, int RK, int RV, int NW>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ ml,
                                                      const float* __restrict__ acc,
                                                      const int32_t* __restrict__ seq_lens,
                                                      int max_blocks, int pages_per_split,
                                                      int num_splits, float* __restrict__ z) {
  using C = DecodeCfg<H, RK, RV, NW>;
  __shared__ float sW[256];
  __shared__ float sInv;
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int n_pages =
      min(min((seq_lens[b] + BS - 1) / BS, max_blocks), num_splits * pages_per_split);
  const int ns = (n_pages + pages_per_split - 1) / pages_per_split;
  float* zo = z + ((size_t)b * H + h) * RV;
  if (ns == 0) {
    for (int f = tid; f < RV; f += 256) zo[f] = 0.f;
    return;
  }
  // split weights (ns <= 256 is enforced by the planner)
  const float* mlb = ml + (size_t)b * num_splits * 2 * C::R16;
  float m = -INFINITY;
  for (int s = 0; s < ns; ++s) m = fmaxf(m, mlb[(size_t)s * 2 * C::R16 + h]);
  if (tid < ns) {
    const float ms = mlb[(size_t)tid * 2 * C::R16 + h];
    sW[tid] = (ms == -INFINITY) ? 0.f : exp2f(ms - m);
  }
  __syncthreads();
  if (tid == 0) {
    float den = 0.f;
    for (int s = 0; s < ns; ++s) den += sW[s] * mlb[(size_t)s * 2 * C::R16 + C::R16 + h];
    sInv = (den > 0.f) ? 1.f / den : 0.f;
  }
  __syncthreads();
  const float inv = sInv;
  const int rt = h / 16, c = h % 16;
  for (int f = tid; f < RV; f += 256) {
    const int w = f / C::FPW, ft = (f % C::FPW) / 16, fi = f % 16;
    const size_t off = ((size_t)((w * C::RT + rt) * C::FT + ft) * 64 + c + 16 * (fi / 4)) * 4 + (fi % 4);
    float num = 0.f;
    const float* ab = acc + (size_t)b * num_splits * NW * (C::RT * C::FT * 256);
    for (int s = 0; s < ns; ++s) num += sW[s] * ab[(size_t)s * NW * (C::RT * C::FT * 256) + off];
    zo[f] = num * inv;
  }
}

// ---------------------------------------------------------------------------
// 4. up-projection out[n, h, :] = W_h z[n, h, :] on the matrix cores.
// grid (H, D/DR, ceil(N/64)); 4 waves, wave w owns tokens 16w..16w+15 of the
// chunk and all DR output rows of the work group.  A = W_h (16 rows x 32
// features, 16 contiguous bytes per lane), B = z (32 features x 16 tokens)
// split into an fp16 hi/lo pair so the product keeps fp32 accuracy.
// ---------------------------------------------------------------------------
template <int H, int D, int RV, int DR>
__global__ __launch_bounds__(256) void upproj_kernel(const half_t* __restrict__ W,
                                                     const float* __restrict__ z, int n_tokens,
                                                     half_t* __restrict__ out) {
  constexpr int IT = DR / 16;
  const int h = blockIdx.x, i0 = blockIdx.y * DR;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, quad = lane >> 4;
  const int n = blockIdx.z * 64 + w * 16 + col;
  if (blockIdx.z * 64 + w * 16 >= n_tokens) return;  // wave-uniform
  const bool nv = n < n_tokens;
  const float* zr = z + ((size_t)(nv ? n : 0) * H + h) * RV + quad * 8;
  const half_t* wrow = W + ((size_t)h * D + i0 + col) * RV + quad * 8;
  float4v accv[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) accv[it] = zero4();
#pragma unroll 2
  for (int j0 = 0; j0 < RV; j0 += 32) {
    half8 hi, lo;
    const float4v z0 = nv ? *(const float4v*)(zr + j0) : zero4();
    const float4v z1 = nv ? *(const float4v*)(zr + j0 + 4) : zero4();
    split_f16x8(z0, z1, hi, lo);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const half8 av = *(const half8*)(wrow + (size_t)it * 16 * RV + j0);
      accv[it] = mfma16x16x32(av, hi, accv[it]);
      accv[it] = mfma16x16x32(av, lo, accv[it]);
    }
  }
  if (nv) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      half4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = (half_t)accv[it][r];
      *(half4*)(out + ((size_t)n * H + h) * D + i0 + it * 16 + quad * 4) = o;
    }
  }
}

template <int H, int D, int RV, int DR>
static void launch_upproj_t(const void* W, const float* z, int n_tokens, void* out, hipStream_t st) {
  hipLaunchKernelGGL((upproj_kernel<H, D, RV, DR>), dim3(H, D / DR, (n_tokens + 63) / 64), dim3(256),
                     0, st, (const half_t*)W, z, n_tokens, (half_t*)out);
}

hipError_t launch_upproj(const ShapeKey& s, const void* W, const float* z, int n_tokens,
                         bool wide_rows, void* out, hipStream_t st) {
  if (n_tokens <= 0) return hipSuccess;
  if (s.H == 32 && s.d == 128 && s.rv == 512) {
    if (wide_rows) launch_upproj_t<32, 128, 512, 128>(W, z, n_tokens, out, st);
    else launch_upproj_t<32, 128, 512, 16>(W, z, n_tokens, out, st);
  } else if (s.H == 4 && s.d == 64 && s.rv == 64) {
    if (wide_rows) launch_upproj_t<4, 64, 64, 64>(W, z, n_tokens, out, st);
    else launch_upproj_t<4, 64, 64, 16>(W, z, n_tokens, out, st);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
template <int H, int D, int RK, int RV, int NW>
static hipError_t decode_instance(const DecodePlan& p, const void* qt, const void* k_cache,
                                  const void* v_cache, const void* W, const int32_t* block_tables,
                                  int max_blocks, const int32_t* seq_lens, int num_blocks,
                                  int batch, float* ml, float* acc, float* z, void* out,
                                  hipStream_t st) {
  SplitArgs a;
  a.qt = (const half_t*)qt;
  a.k_cache = (const half_t*)k_cache;
  a.v_cache = (const half_t*)v_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.ml = ml;
  a.acc = acc;
  a.max_blocks = max_blocks;
  a.num_blocks = num_blocks;
  a.pages_per_split = p.pages_per_split;
  a.num_splits = p.num_splits;
  if (g_timing.which == TIME_DECODE_SPLIT && g_timing.start) hipEventRecord(g_timing.start, st);
  hipLaunchKernelGGL((decode_split_kernel<H, RK, RV, NW>), dim3(p.num_splits, batch), dim3(NW * 64),
                     0, st, a);
  if (g_timing.which == TIME_DECODE_SPLIT && g_timing.stop) hipEventRecord(g_timing.stop, st);
  hipLaunchKernelGGL((combine_kernel<H, RK, RV, NW>), dim3(H, batch), dim3(256), 0, st,
                     (const float*)ml, (const float*)acc, seq_lens, max_blocks,
                     p.pages_per_split, p.num_splits, z);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_upproj(ShapeKey{H, D, RK, RV}, W, z, batch, false, out, st);
}

template <int H, int D, int RK>
static hipError_t qproj_instance(const void* q, const void* U, int n, float scale, void* qt,
                                 hipStream_t st) {
  hipLaunchKernelGGL((qproj_kernel<H, D, RK>), dim3(H, (n + 15) / 16), dim3(256), 0, st,
                     (const half_t*)q, (const half_t*)U, n, scale * kLog2e, (half_t*)qt);
  return hipGetLastError();
}

hipError_t launch_qproj(const ShapeKey& s, const void* q, const void* U, int n_tokens, float scale,
                        void* qt, hipStream_t st) {
  if (n_tokens <= 0) return hipSuccess;
  if (s.H == 32 && s.d == 128 && s.rk == 64) return qproj_instance<32, 128, 64>(q, U, n_tokens, scale, qt, st);
  if (s.H == 4 && s.d == 64 && s.rk == 16) return qproj_instance<4, 64, 16>(q, U, n_tokens, scale, qt, st);
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const ShapeKey& s, const DecodePlan& p, const void* qt, const void* k_cache,
                         const void* v_cache, const void* W, const int32_t* block_tables,
                         int max_blocks, const int32_t* seq_lens, int num_blocks, int batch,
                         float* ml, float* acc, float* z, void* out, hipStream_t st) {
  if (s.H == 32 && s.d == 128 && s.rk == 64 && s.rv == 512)
    return decode_instance<32, 128, 64, 512, 4>(p, qt, k_cache, v_cache, W, block_tables, max_blocks,
                                                seq_lens, num_blocks, batch, ml, acc, z, out, st);
  if (s.H == 4 && s.d == 64 && s.rk == 16 && s.rv == 64)
    return decode_instance<4, 64, 16, 64, 4>(p, qt, k_cache, v_cache, W, block_tables, max_blocks,
                                             seq_lens, num_blocks, batch, ml, acc, z, out, st);
  return hipErrorInvalidValue;
}

}  // namespace starkv
