// Chunked-prefill attention over a paged, low-rank-compressed KV cache
// (Proxima README, "Per-prefill-chunk attention": one chunk of N new tokens
// per request attends to the request's whole cache, causally).
//
// The chunk's keys and values are appended first (append.hip); this kernel
// then attends with the latent shortcut, never rebuilding K or V:
//   S^T[t, j] = c_k[t, h] . q~[j, h]          (q~ pre-scaled by scale*log2 e)
//   P = causal softmax over t <= P0 + j, P0 = seq_len - chunk_len
//   Z^T[f, j] = sum_t c_v[t, f] P[j, t]        (normalised at the end)
// and writes z [total_q, H, r_v] fp32; the up-projection out_h = W_h z_h
// runs afterwards on the matrix cores (decode.hip, wide tiling).
//
// Work group = (request, tile of MQ queries, group of G heads), NW waves.
// Rows of the attention tile are (head, query) pairs, R = G*MQ of them.
//   * scores: wave w owns one (head, 16-query block); per page it runs
//     v_mfma_f32_16x16x32_f16 with the 16x64 key page as A and the queries'
//     q~ as B, giving tokens x queries, then the online-softmax update of its
//     16 queries (lane = query, 4 tokens per lane, 4-lane butterfly).
//   * P and the rescale factors pass through LDS (double-buffered).
//   * values: wave w owns RV/NW features for all R rows,
//     Z^T[f, row] += c_v[t, f] P[row, t] with v_mfma_f32_16x16x16_f16; the
//     accumulator column is the row, so rescaling is per lane and is skipped
//     for pages where no running max moved.
//   * work groups of one request are placed on one XCD when the batch is a
//     multiple of 8, so the request's latents are shared through that L2.
#include "common.h"
#include "kernels.h"

namespace starkv {

template <int H, int RK, int RV, int G, int MQ, int NW>
struct PrefillCfg {
  static constexpr int R = G * MQ;
  static constexpr int RT = R / 16;
  static constexpr int QB = MQ / 16;
  static constexpr int FPW = RV / NW;
  static constexpr int FT = FPW / 16;
  static constexpr int KC = (RK % 32 == 0) ? 32 : 16;
  static constexpr int NKC = RK / KC;
  static_assert(MQ % 16 == 0 && G * QB == NW, "one (head, 16-query) score unit per wave");
  static_assert(RV % (16 * NW) == 0, "value rank must split into 16-wide tiles per wave");
  static_assert(H % G == 0, "head groups must tile the heads");
};

struct PrefillArgs {
  const half_t* qt;  // [total_q, H, RK] fp16, pre-scaled
  const int32_t* qsl;
  const half_t* k_cache;
  const half_t* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* z;  // [total_q, H, RV]
  int max_blocks, num_blocks, batch, n_qtiles, n_groups;
};

constexpr int PBS = 16;

template <int H, int RK, int RV, int G, int MQ, int NW>
__global__ __launch_bounds__(NW * 64) void prefill_attn_kernel(PrefillArgs a) {
  using C = PrefillCfg<H, RK, RV, G, MQ, NW>;
  typedef _Float16 kvec __attribute__((ext_vector_type(C::KC / 4)));
  __shared__ __attribute__((aligned(16))) half_t sP[2][C::R][PBS];
  __shared__ float sAlpha[2][C::R];
  __shared__ float sL[C::R];
  __shared__ int sFlag[2];

  // ---- work decode (XCD-aware when the batch allows it)
  const int units = a.n_qtiles * a.n_groups;
  const int lin = blockIdx.x;
  int b, u;
  if ((a.batch & 7) == 0) {
    const int x = lin & 7, k = lin >> 3;
    b = x + 8 * (k / units);
    u = k % units;
  } else {
    b = lin / units;
    u = lin % units;
  }
  const int g = u / a.n_qtiles, qtile = u % a.n_qtiles;
  const int q_begin = a.qsl[b];
  const int Cn = a.qsl[b + 1] - q_begin;
  const int j0 = qtile * MQ;
  if (j0 >= Cn) return;
  const int L = a.seq_lens[b];
  const int P0 = L - Cn;
  const int last_key = min(L - 1, P0 + min(j0 + MQ, Cn) - 1);
  const int n_pages = min(last_key / PBS + 1, a.max_blocks);

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, quad = lane >> 4;
  const int hl = w / C::QB, qb = w % C::QB;
  const int h = g * G + hl;
  const int jq = min(j0 + qb * 16 + col, Cn - 1);  // rows past the chunk mirror its last query
  const int qpos = P0 + jq;
  const int row = hl * MQ + qb * 16 + col;

  if (tid < 2) sFlag[tid] = -1;

  kvec qv[C::NKC];
  {
    const half_t* qp = a.qt + ((size_t)(q_begin + jq) * H + h) * RK + quad * (C::KC / 4);
#pragma unroll
    for (int c = 0; c < C::NKC; ++c) qv[c] = *(const kvec*)(qp + c * C::KC);
  }

  float m_run = -INFINITY, l_run = 0.f;
  float4v acc[C::RT][C::FT];
#pragma unroll
  for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
    for (int ft = 0; ft < C::FT; ++ft) acc[rt][ft] = zero4();

  const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks;
  const half_t* kbase = a.k_cache + ((size_t)h * PBS + col) * RK + quad * (C::KC / 4);
  const half_t* vbase = a.v_cache + (size_t)(w * C::FPW + col) * PBS + quad * 4;
  struct Regs {
    kvec k[C::NKC];
    half4 v[C::FT];
  };
  auto safe_block = [&](int p) {
    const int blk = bt[p];
    return ((unsigned)blk < (unsigned)a.num_blocks) ? blk : -1;
  };
  auto load = [&](Regs& r, int blk) {
    const half_t* kp = kbase + (size_t)blk * H * PBS * RK;
#pragma unroll
    for (int c = 0; c < C::NKC; ++c) r.k[c] = *(const kvec*)(kp + c * C::KC);
    const half_t* vp = vbase + (size_t)blk * RV * PBS;
#pragma unroll
    for (int ft = 0; ft < C::FT; ++ft) r.v[ft] = *(const half4*)(vp + (size_t)ft * 16 * PBS);
  };
  // one page: scores of this wave's (head, 16 queries), online softmax, P via
  // LDS, then every wave's value slice for all rows
  auto process = [&](Regs& r, int p, int buf, bool ok) {
    if (ok) {
      float4v sacc = zero4();
#pragma unroll
      for (int c = 0; c < C::NKC; ++c) {
        if constexpr (C::KC == 32)
          sacc = mfma16x16x32(r.k[c], qv[c], sacc);
        else
          sacc = mfma16x16x16(r.k[c], qv[c], sacc);
      }
      float sv[4];
      float pm = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = p * PBS + quad * 4 + e;
        sv[e] = (t < L && t <= qpos) ? sacc[e] : -INFINITY;
        pm = fmaxf(pm, sv[e]);
      }
      pm = max_over_quads(pm);
      // m_new is finite from the first page on: key 0 is visible to every query
      const float m_new = fmaxf(m_run, pm);
      const float alpha = exp2f(m_run - m_new);
      float ps = 0.f;
      half4 ph;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pr = exp2f(sv[e] - m_new);
        ps += pr;
        ph[e] = (half_t)pr;
      }
      ps = sum_over_quads(ps);
      l_run = l_run * alpha + ps;
      m_run = m_new;
      *(half4*)&sP[buf][row][quad * 4] = ph;
      if (quad == 0) sAlpha[buf][row] = alpha;
      if (alpha != 1.f) sFlag[buf] = p;
    }
    block_sync_lds();
    if (ok) {
      const bool rescale = sFlag[buf] == p;
      const int valid = min(PBS, L - p * PBS);
      if (valid < PBS) {  // slots past the sequence may hold anything (NaN)
#pragma unroll
        for (int ft = 0; ft < C::FT; ++ft)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (quad * 4 + e >= valid) r.v[ft][e] = (half_t)0.f;
      }
#pragma unroll
      for (int rt = 0; rt < C::RT; ++rt) {
        const half4 pb = *(const half4*)&sP[buf][rt * 16 + col][quad * 4];
        if (rescale) {
          const float al = sAlpha[buf][rt * 16 + col];
#pragma unroll
          for (int ft = 0; ft < C::FT; ++ft) acc[rt][ft] *= al;
        }
#pragma unroll
        for (int ft = 0; ft < C::FT; ++ft) acc[rt][ft] = mfma16x16x16(r.v[ft], pb, acc[rt][ft]);
      }
    }
  };

  Regs ra, rb;
  int blk_a = safe_block(0);
  if (blk_a >= 0) load(ra, blk_a);
  __syncthreads();
  for (int p = 0; p < n_pages; p += 2) {
    int blk_b = -1;
    if (p + 1 < n_pages) {
      blk_b = safe_block(p + 1);
      if (blk_b >= 0) load(rb, blk_b);
    }
    process(ra, p, 0, blk_a >= 0);
    if (p + 1 < n_pages) {
      if (p + 2 < n_pages) {
        blk_a = safe_block(p + 2);
        if (blk_a >= 0) load(ra, blk_a);
      }
      process(rb, p + 1, 1, blk_b >= 0);
    }
  }

  // ---- normalise and write z rows of this tile
  if (quad == 0) sL[row] = l_run;
  block_sync_lds();
#pragma unroll
  for (int rt = 0; rt < C::RT; ++rt) {
    const int r_row = rt * 16 + col;
    const int r_h = g * G + r_row / MQ;
    const int r_j = j0 + r_row % MQ;
    if (r_j >= Cn) continue;
    const float lr = sL[r_row];
    const float inv = lr > 0.f ? 1.f / lr : 0.f;
    float* zr = a.z + ((size_t)(q_begin + r_j) * H + r_h) * RV + w * C::FPW + quad * 4;
#pragma unroll
    for (int ft = 0; ft < C::FT; ++ft) *(float4v*)(zr + ft * 16) = acc[rt][ft] * inv;
  }
}

template <int H, int D, int RK, int RV, int G, int MQ, int NW>
static hipError_t prefill_instance(const void* qt, const int32_t* qsl, int max_query_len,
                                   const void* k_cache, const void* v_cache, const void* W,
                                   const int32_t* block_tables, int max_blocks,
                                   const int32_t* seq_lens, int num_blocks, int batch,
                                   int total_q, float* z, void* out, hipStream_t st) {
  PrefillArgs a;
  a.qt = (const half_t*)qt;
  a.qsl = qsl;
  a.k_cache = (const half_t*)k_cache;
  a.v_cache = (const half_t*)v_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.z = z;
  a.max_blocks = max_blocks;
  a.num_blocks = num_blocks;
  a.batch = batch;
  a.n_qtiles = (max_query_len + MQ - 1) / MQ;
  a.n_groups = H / G;
  const long wgs = (long)batch * a.n_qtiles * a.n_groups;
  launch_hooked(TIME_PREFILL_ATTN, TIME_NONE, prefill_attn_kernel<H, RK, RV, G, MQ, NW>, dim3((unsigned)wgs),
                dim3(NW * 64), st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_upproj(ShapeKey{H, D, RK, RV}, W, z, total_q, true, out, st);
}

hipError_t launch_prefill(const ShapeKey& s, const void* qt, const int32_t* qsl, int total_q,
                          int max_query_len, const void* k_cache, const void* v_cache,
                          const void* W, const int32_t* block_tables, int max_blocks,
                          const int32_t* seq_lens, int num_blocks, int batch, float* z, void* out,
                          hipStream_t st) {
  if (batch <= 0 || total_q <= 0) return hipSuccess;
  if (s.H == 32 && s.d == 128 && s.rk == 64 && s.rv == 512)
    return prefill_instance<32, 128, 64, 512, 4, 32, 8>(qt, qsl, max_query_len, k_cache, v_cache,
                                                        W, block_tables, max_blocks, seq_lens,
                                                        num_blocks, batch, total_q, z, out, st);
  if (s.H == 4 && s.d == 64 && s.rk == 16 && s.rv == 64)
    return prefill_instance<4, 64, 16, 64, 4, 16, 4>(qt, qsl, max_query_len, k_cache, v_cache, W,
                                                     block_tables, max_blocks, seq_lens,
                                                     num_blocks, batch, total_q, z, out, st);
  return hipErrorInvalidValue;
}

}  // namespace starkv
