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
// One decode step is three launches on the caller's stream:
//   1. qproj        q~ = U_h^T q, pre-scaled by scale*log2(e), fp32, on the
//                   matrix cores (U_h read through the transposing LDS read);
//                   the split kernel feeds it to the score products as an
//                   fp16 hi/lo pair in otherwise unused B columns
//   2. decode_split split-K pass over the pages (README, "Kernel profiling
//                   breakdown": split-K attention plus a combine); one work
//                   group owns all heads of a run of pages so the joint value
//                   latent of each token is read from HBM exactly once
//   3. finish       log-sum-exp merge of the splits, then out_h = W_h z_h on
//                   the matrix cores, z split into an fp16 hi/lo pair so the
//                   product keeps fp32 accuracy
//
// decode_split per page (16 tokens) in a work group of NW waves:
//   * scores: wave w owns heads [w*HPW, (w+1)*HPW).  For each head the 16xr_k
//     key page is the A operand of v_mfma_f32_16x16x32_f16 and q~_h sits in
//     column (h - w*HPW) of B, zeros elsewhere, so one 16x16 accumulator
//     collects the scores of all the wave's heads (tokens x heads).  The
//     lane that holds column c then runs the online-softmax update of that
//     head on its 4 tokens plus a 4-lane butterfly.
//   * P (fp16) and the rescale factors go through LDS (double-buffered, one
//     LDS-only barrier per page, so prefetched loads stay in flight).
//   * values: wave w owns features [w*FPW, (w+1)*FPW).  Z^T[f, h] +=
//     sum_t c_v[t, f] P[h, t] with v_mfma_f32_16x16x16_f16: the feature-major
//     value page gives each lane 8 contiguous bytes, and the accumulator
//     column is the head, so the rescale is one scalar per lane; it is
//     skipped for pages where no running max moved.
//   * two register sets ping-pong: page p+1 is loaded while page p is used.
//   * the main shape runs 16 waves (2 heads and 32 value features each, four
//     waves per SIMD), which measured 1-1.5% faster than 8 waves.
#include <type_traits>

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
  static_assert(H % NW == 0 && (HPW == 1 || HPW == 2 || HPW == 4 || HPW == 8),
                "heads per wave: a power of two up to 8 (q~ hi and lo take 2 HPW columns)");
  static_assert(RV % (16 * NW) == 0, "value rank must split into 16-wide tiles per wave");
  static_assert(RK % 16 == 0, "key rank must be a multiple of 16");
};

constexpr int BS = 16;  // tokens per page
constexpr int kMaxSplitPages = 256;  // planner bound on pages per split

// ---------------------------------------------------------------------------
// 1. q~[n, h, :] = (scale*log2e) * U_g^T q[n, h, :]  -> fp32, g = h / QG the
//    key/value head of query head h (QG = 1: multi-head attention).  q~ stays
//    fp32: the attention kernels split it into an fp16 hi/lo pair for their
//    score products, since one fp16 rounding of q~ moves a score by about
//    2^-12 of its size, which peaked softmax rows (scores tens of units
//    apart) turn into output errors above 1e-3.
// grid (H, ceil(N/(64*TPW))), 4 waves; in token tile tt the wave w owns
// tokens n0+16w .. n0+16w+15 of that tile's 64.  The product is taken as
// q~^T = U_h^T q^T, so that each lane ends with 4 consecutive outputs of one
// token (one 8-byte store): A = U_h^T (16 outputs x 32 of d), read from
// U_h staged in LDS as it is in memory ([d][r], 16-byte stores) through the
// transposing LDS read (ds_read_b64_tr_b16: within each group of 16 lanes,
// lane i receives element i%4 of the 8-byte chunk addressed by lane
// 4e + i/4, e = 0..3, so lane i gets 4 consecutive d of output r0 + i);
// B = q^T (32 of d x 16 tokens, 16 contiguous bytes per lane).  The first
// tile's q rows are requested before the staging, so the two memory round
// trips overlap; TPW tiles per work group amortise the staging.
// ---------------------------------------------------------------------------
typedef short short4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ half4 lds_read_tr16(const half_t* p) {
  typedef __attribute__((address_space(3))) short4v lds_short4v;
  const short4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)p);
  return __builtin_bit_cast(half4, r);
}

// Rows y >= token_rows of the grid prefetch the up-projection basis for the
// merge that ends the step: work group (h, token_rows + p) reads part p of
// the W block of head h's key/value head.  Work groups are dealt to the 8
// XCDs round robin, so with H a multiple of 8 it runs on XCD h % 8, where
// the merge places head h's work groups; the block then waits in that XCD's
// L2 instead of in HBM.
// The loaded words only feed a value stored through `sink`, which is null.
template <int H, int D, int RK, int TPW, int QG>
__global__ __launch_bounds__(256) void qproj_kernel(const half_t* __restrict__ q,
                                                    const half_t* __restrict__ U, int n_tokens,
                                                    float qscale, float* __restrict__ qt,
                                                    int token_rows, const char* __restrict__ wpf,
                                                    int wpf_head_bytes, int wpf_part_bytes,
                                                    uint32_t* __restrict__ sink,
                                                    uint32_t* __restrict__ zero, int n_zero) {
  constexpr int LDU = RK + 8;  // halves per LDS row: 4 rows of a read group hit distinct banks
  __shared__ __attribute__((aligned(16))) half_t sU[D][LDU];
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  // the counters the fused decode step that follows waits on start at zero
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = tid; i < n_zero; i += 256) zero[i] = 0u;
  if ((int)blockIdx.y >= token_rows) {  // whole work group, before any barrier
    const char* p = wpf + (size_t)(h / QG) * wpf_head_bytes +
                    (size_t)(blockIdx.y - token_rows) * wpf_part_bytes;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    uint32_t x = 0;
#pragma unroll 8
    for (int off = tid * 16; off < wpf_part_bytes; off += 256 * 16) {
      const u32x4 v = *(const u32x4*)(p + off);
      x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (sink) *sink = x;
    return;
  }
  const int lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, quad = lane >> 4;
  auto load_q = [&](half8 (&b)[D / 32], int nb) {
    const int n = min(nb + col, n_tokens - 1);  // rows past the end are not stored
    const half_t* qrow = q + ((size_t)n * H + h) * D + quad * 8;
#pragma unroll
    for (int k = 0; k < D / 32; ++k) b[k] = *(const half8*)(qrow + k * 32);
  };
  // all of the wave's token sets are requested up front: with two waves per
  // SIMD, loading them one set at a time left the latency of each exposed
  half8 bq[TPW][D / 32];
  const int nb0 = blockIdx.y * TPW * 64 + w * 16;
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
    if (nb0 + tt * 64 < n_tokens) load_q(bq[tt], nb0 + tt * 64);
  const half_t* Uh = U + (size_t)(h / QG) * D * RK;  // the head's key/value head
  // Ranks are permuted inside the LDS copy: column 16t + 4a + r holds rank
  // 4NT*a + 4t + r (NT = RK/16 rank tiles, a = the lane's quad).  The four
  // outputs a lane takes from each of the NT tiles are then 4NT consecutive
  // ranks of one token, stored whole (a token's row in 16- or 32-byte pieces
  // instead of 8-byte ones).  Each output keeps its own products and order.
  constexpr int NT = RK / 16;
  static_assert(RK % 16 == 0, "whole rank tiles");
  for (int c = tid; c < D * RK / 4; c += 256) {
    const int i = c / (RK / 4), g = c % (RK / 4);
    *(half4*)&sU[i][16 * (g % NT) + 4 * (g / NT)] = *(const half4*)(Uh + (size_t)i * RK + 4 * g);
  }
  __syncthreads();
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int nb = nb0 + tt * 64;
    if (nb >= n_tokens) break;  // wave-uniform; no barrier follows
    float4v acc[NT];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      acc[rt] = zero4();
#pragma unroll
      for (int k = 0; k < D / 32; ++k) {
        // A fragment: LDS columns 16*rt + col, d = 32k + 8*quad .. +7
        const half_t* ap = &sU[k * 32 + quad * 8 + (col >> 2)][rt * 16 + 4 * (col & 3)];
        const half4 a0 = lds_read_tr16(ap);
        const half4 a1 = lds_read_tr16(ap + 4 * LDU);
        const half8 au = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        acc[rt] = mfma16x16x32(au, bq[tt][k], acc[rt]);
      }
    }
    // D[LDS column 16rt + 4*quad + r][token col] = rank 4NT*quad + 4rt + r,
    // so the lane's NT tiles are 4NT consecutive ranks of its token
    const int nt = nb + col;
    if (nt < n_tokens) {
      float* dst = qt + ((size_t)nt * H + h) * RK + quad * 4 * NT;
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) *(float4v*)(dst + 4 * rt) = acc[rt] * qscale;
    }
  }
}

// ---------------------------------------------------------------------------
// 2. split-K latent attention
// ---------------------------------------------------------------------------
// Arguments are separate __restrict__ pointers (not a struct) so the
// compiler can prove the block table is never written in the kernel and
// reads it with scalar loads: a vector load of a block id would need a
// vmcnt wait that also drains the page prefetch.
//   ml    [B][R16][2][SS] fp32: running max (log2 domain) of every split,
//         then its sum
//   zpart [B][R16][SS][RV] fp16: the split's z rows, normalised by its sum
// SS (split_stride) is the split count rounded up to the merge's request
// batch; slots past a sequence's last split are never written.

// Key pages per wave under grouped-query attention (QG query heads per
// key/value head): the wave's HPW query heads span KPW key/value heads, from
// kv0 = w*HPW/QG on; each of them is loaded once and feeds the score
// products of all its query heads.
template <int H, int RK, int RV, int NW, int QG>
struct KeyCfg {
  static constexpr int HPW = DecodeCfg<H, RK, RV, NW>::HPW;
  static constexpr int KPW = HPW >= QG ? HPW / QG : 1;
  static constexpr int HKV = H / QG;
  static_assert(H % QG == 0 && (HPW % QG == 0 || QG % HPW == 0), "query groups must align with waves");
};

// FP8 E4M3 codes to fp16: v_cvt_scalef32_pk_f16_fp8 with scale 1 turns the
// low or the high two bytes of a word into two fp16 values (every E4M3 value
// is exactly an fp16 value), two instructions per four codes.
__device__ __forceinline__ half4 e4m3x4_to_half4(uint32_t w) {
  typedef _Float16 half2v __attribute__((ext_vector_type(2)));
  const half2v lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  const half2v hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  return half4{lo[0], lo[1], hi[0], hi[1]};
}

// Page operands of one wave, as loaded: fp16, or FP8 codes (half the bytes,
// turned into the same fp16 operands when used).
template <int H, int RK, int RV, int NW, int QG, bool FP8>
struct PageRegs {
  using C = DecodeCfg<H, RK, RV, NW>;
  typedef _Float16 kvec __attribute__((ext_vector_type(C::KC / 4)));
  typedef uint8_t k8 __attribute__((ext_vector_type(C::KC / 4)));
  typedef uint8_t v8 __attribute__((ext_vector_type(4)));
  using kraw = std::conditional_t<FP8, k8, kvec>;
  using vraw = std::conditional_t<FP8, v8, half4>;
  kraw k[KeyCfg<H, RK, RV, NW, QG>::KPW][C::NKC];
  vraw v[C::FT];

  __device__ __forceinline__ kvec key(int kk, int c) const {
    if constexpr (FP8) {
      if constexpr (C::KC / 4 == 8) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 w = __builtin_bit_cast(u32x2, k[kk][c]);
        const half4 a = e4m3x4_to_half4(w[0]), b = e4m3x4_to_half4(w[1]);
        return kvec{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      } else {
        return e4m3x4_to_half4(__builtin_bit_cast(uint32_t, k[kk][c]));
      }
    } else {
      return k[kk][c];
    }
  }
  __device__ __forceinline__ half4 val(int ft) const {
    if constexpr (FP8)
      return e4m3x4_to_half4(__builtin_bit_cast(uint32_t, v[ft]));
    else
      return v[ft];
  }
};

template <bool NT, typename T>
__device__ __forceinline__ T ld_page(const T* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

// Element type of the caches: fp16, or FP8 codes (same layouts, one byte).
template <bool FP8>
using latent_t = std::conditional_t<FP8, uint8_t, half_t>;

template <int H, int RK, int RV, int NW, int QG, bool NT, bool FP8>
__device__ __forceinline__ void load_page(PageRegs<H, RK, RV, NW, QG, FP8>& pr,
                                          const latent_t<FP8>* __restrict__ kc,
                                          const latent_t<FP8>* __restrict__ vc, int blk, int w,
                                          int col, int quad) {
  using C = DecodeCfg<H, RK, RV, NW>;
  using K = KeyCfg<H, RK, RV, NW, QG>;
  using R = PageRegs<H, RK, RV, NW, QG, FP8>;
  // keys: key/value head (kv0 + kk), token row `col`, k chunk `quad`
  const int kv0 = w * C::HPW / QG;
  const latent_t<FP8>* kb =
      kc + (((size_t)blk * K::HKV + kv0) * BS + col) * RK + quad * (C::KC / 4);
#pragma unroll
  for (int kk = 0; kk < K::KPW; ++kk)
#pragma unroll
    for (int c = 0; c < C::NKC; ++c)
      pr.k[kk][c] = ld_page<NT>((const typename R::kraw*)(kb + (size_t)kk * BS * RK + c * C::KC));
  // values: feature (w*FPW + ft*16 + col), tokens 4*quad .. 4*quad+3
  const latent_t<FP8>* vb = vc + ((size_t)blk * RV + w * C::FPW + col) * BS + quad * 4;
#pragma unroll
  for (int ft = 0; ft < C::FT; ++ft)
    pr.v[ft] = ld_page<NT>((const typename R::vraw*)(vb + (size_t)ft * 16 * BS));
}

template <int H, int RK, int RV, int NW>
struct SplitState {
  using C = DecodeCfg<H, RK, RV, NW>;
  float m_run, l_run;
  float4v acc[C::RT][C::FT];
};

// One page: scores, online softmax, P through LDS, P.c_v.  Branch-free in
// `valid` (tokens of the page that belong to the sequence; 0 for a page past
// the split or with an invalid block id): masked tokens get score -inf,
// weight 0 and a zeroed value operand, so a fully masked page changes
// nothing.  Keeping every page on the same path lets the compiler count the
// prefetched loads exactly instead of draining them.
template <int H, int RK, int RV, int NW, int QG, bool FP8>
__device__ __forceinline__ void process_page(
    SplitState<H, RK, RV, NW>& st, PageRegs<H, RK, RV, NW, QG, FP8>& cur,
    const typename PageRegs<H, RK, RV, NW, QG, FP8>::kvec (&qv)[DecodeCfg<H, RK, RV, NW>::NKC],
    half_t (*sP)[DecodeCfg<H, RK, RV, NW>::R16][BS], float (*sAlpha)[DecodeCfg<H, RK, RV, NW>::R16],
    int* sFlag, int p, int buf, int valid, int w, int col, int quad) {
  using C = DecodeCfg<H, RK, RV, NW>;
  using K = KeyCfg<H, RK, RV, NW, QG>;
  using kvec = typename PageRegs<H, RK, RV, NW, QG, FP8>::kvec;
  const kvec kzero = {};
  // B column col < HPW holds the fp16 hi part of q~ of query head
  // w*HPW + col, column col + HPW its lo part; that head's key/value head is
  // the wave's kk-th, and the products for key page kk take only its columns
  const int hsel = col < C::HPW ? col : col - C::HPW;
  const int my_kk = col < 2 * C::HPW ? (w * C::HPW + hsel) / QG - w * C::HPW / QG : -1;
  float4v sacc = zero4();
#pragma unroll
  for (int kk = 0; kk < K::KPW; ++kk) {
#pragma unroll
    for (int c = 0; c < C::NKC; ++c) {
      const kvec bq = (my_kk == kk) ? qv[c] : kzero;
      if constexpr (C::KC == 32)
        sacc = mfma16x16x32(cur.key(kk, c), bq, sacc);
      else
        sacc = mfma16x16x16(cur.key(kk, c), bq, sacc);
    }
  }
  // score = hi product + lo product: the lo column of head col sits HPW
  // lanes away in the same row of 16 (HPW is a power of two below 16; a DPP
  // quad permutation for HPW <= 2)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if constexpr (C::HPW <= 2)
      sacc[r] += xor_lane_small<C::HPW>(sacc[r]);
    else
      sacc[r] += __shfl_xor(sacc[r], C::HPW);
  }
  // `valid` is uniform: pages wholly inside the sequence skip every mask
  const bool full = valid >= BS;
  float sv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) sv[r] = (full || quad * 4 + r < valid) ? sacc[r] : -INFINITY;
  const float pm = quad_max(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
  const float m_new = fmaxf(st.m_run, pm);
  // weights are 2^(s - m_ref): m_ref is the new running max, or 0 while every
  // score so far is masked (all s are then -inf); v_exp_f32 gives
  // 2^-inf = 0, so masked scores need no test
  const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = (m_new == st.m_run) ? 1.f : __builtin_amdgcn_exp2f(st.m_run - m_ref);
  float ps = 0.f;
  half4 ph;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float pr = __builtin_amdgcn_exp2f(sv[r] - m_ref);
    ps += pr;
    ph[r] = (half_t)pr;
  }
  ps = quad_sum(ps);
  st.l_run = st.l_run * alpha + ps;
  st.m_run = m_new;
  if (col < C::HPW) {
    const int row = w * C::HPW + col;
    *(half4*)&sP[buf][row][quad * 4] = ph;
    if (quad == 0) sAlpha[buf][row] = alpha;
    if (alpha != 1.f) sFlag[buf] = p;
  }
  block_sync_lds();
  const bool rescale = sFlag[buf] == p;  // uniform: skip when no max moved
  half4 pb[C::RT];
#pragma unroll
  for (int rt = 0; rt < C::RT; ++rt) {
    pb[rt] = *(const half4*)&sP[buf][rt * 16 + col][quad * 4];
    if (rescale) {
      const float al = sAlpha[buf][rt * 16 + col];
#pragma unroll
      for (int ft = 0; ft < C::FT; ++ft) st.acc[rt][ft] *= al;
    }
  }
  if (full) {
#pragma unroll
    for (int ft = 0; ft < C::FT; ++ft) {
      const half4 av = cur.val(ft);
#pragma unroll
      for (int rt = 0; rt < C::RT; ++rt) st.acc[rt][ft] = mfma16x16x16(av, pb[rt], st.acc[rt][ft]);
    }
    return;
  }
  // value slots past the sequence may hold anything (NaN): zero them
  const int t0 = quad * 4;
  const uint32_t m01 = (t0 < valid ? 0x0000FFFFu : 0u) | (t0 + 1 < valid ? 0xFFFF0000u : 0u);
  const uint32_t m23 = (t0 + 2 < valid ? 0x0000FFFFu : 0u) | (t0 + 3 < valid ? 0xFFFF0000u : 0u);
#pragma unroll
  for (int ft = 0; ft < C::FT; ++ft) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    u32x2 bits = __builtin_bit_cast(u32x2, cur.val(ft));
    bits[0] &= m01;
    bits[1] &= m23;
    const half4 av = __builtin_bit_cast(half4, bits);
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt) st.acc[rt][ft] = mfma16x16x16(av, pb[rt], st.acc[rt][ft]);
  }
}

// LDS of one split work item.
template <int H, int RK, int RV, int NW>
struct SplitLds {
  using C = DecodeCfg<H, RK, RV, NW>;
  __attribute__((aligned(16))) half_t sP[2][C::R16][BS];
  float sAlpha[2][C::R16];
  int sFlag[2];              // page index whose softmax step moved a running max
  int sBlk[kMaxSplitPages];  // block ids of this split, loadable
  float sL[C::R16];          // final softmax sums, by head
};

// One split work item: pages [s * pages_per_split, ...) of sequence b.
// FUSED: the partials are written with device-coherent stores and, once all
// of the work group's stores have completed, seq_done[b] is incremented with
// release semantics (the merge waits for it).
template <int H, int RK, int RV, int NW, int DEPTH, bool NT, int QG, bool FP8, bool FUSED>
__device__ __forceinline__ void split_body(
    SplitLds<H, RK, RV, NW>& lds, const int s, const int b, const float* __restrict__ qt,
    const latent_t<FP8>* __restrict__ k_cache, const latent_t<FP8>* __restrict__ v_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ seq_lens,
    float* __restrict__ ml, half_t* __restrict__ zpart, int max_blocks, int num_blocks,
    int pages_per_split, int num_splits, int split_stride, float v_scale,
    uint32_t* __restrict__ seq_done) {
  using C = DecodeCfg<H, RK, RV, NW>;
  using kvec = typename PageRegs<H, RK, RV, NW, QG, FP8>::kvec;
  auto& sP = lds.sP;
  auto& sAlpha = lds.sAlpha;
  auto& sFlag = lds.sFlag;
  auto& sBlk = lds.sBlk;
  auto& sL = lds.sL;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, quad = lane >> 4;
  const int p0 = s * pages_per_split;

  // Block ids of the split's pages are staged in LDS once: a per-page
  // scalar load from the block table would stall the next page's load issue
  // for a full memory latency under load.  They are requested together with
  // the sequence length (clamped to the table row: a split past the
  // sequence exits below), and the empty asm keeps the compiler from moving
  // them after the exit test, so the first page's request follows after one
  // memory round trip instead of two.  Invalid ids become -1 (masked page).
  static_assert(kMaxSplitPages <= NW * 64, "one block id per thread");
  const int32_t* bt = block_tables + (size_t)b * max_blocks;
  const int blk0 = bt[min(p0, max_blocks - 1)];
  const int bid = (tid < pages_per_split && p0 + tid < max_blocks) ? bt[p0 + tid] : 0;
  const int L = seq_lens[b];
  asm volatile("" ::"s"(L), "s"(blk0), "v"(bid));
  const int n_pages = min(min((L + BS - 1) / BS, max_blocks), num_splits * pages_per_split);
  if (p0 >= n_pages) return;
  const int p1 = min(p0 + pages_per_split, n_pages);

  PageRegs<H, RK, RV, NW, QG, FP8> ring[DEPTH];
  load_page<H, RK, RV, NW, QG, NT, FP8>(ring[0], k_cache, v_cache,
                               ((unsigned)blk0 < (unsigned)num_blocks) ? blk0 : 0, w, col, quad);

  // rows >= H are padding: P stays zero there, alpha one
  for (int i = tid; i < 2 * C::R16 * BS; i += NW * 64) (&sP[0][0][0])[i] = (half_t)0.f;
  for (int i = tid; i < 2 * C::R16; i += NW * 64) (&sAlpha[0][0])[i] = 1.f;
  if (tid < 2) sFlag[tid] = -1;
  if (tid < p1 - p0) sBlk[tid] = ((unsigned)bid < (unsigned)num_blocks) ? bid : -1;

  // B column col: the fp16 hi part of q~ of head w*HPW + col (col < HPW) or
  // the lo part of head w*HPW + col - HPW (HPW <= col < 2 HPW), for this
  // lane's k chunks; hi + lo carries q~ to about 2^-22 of its size
  kvec qv[C::NKC];
  {
    const int hsel = col < C::HPW ? col : (col < 2 * C::HPW ? col - C::HPW : 0);
    const bool lo_part = col >= C::HPW;
    const float* qp = qt + ((size_t)b * H + w * C::HPW + hsel) * RK + quad * (C::KC / 4);
#pragma unroll
    for (int c = 0; c < C::NKC; ++c) {
#pragma unroll
      for (int e4 = 0; e4 < C::KC / 16; ++e4) {
        const float4v x = *(const float4v*)(qp + c * C::KC + 4 * e4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const half_t hi = (half_t)x[e];
          qv[c][4 * e4 + e] = lo_part ? (half_t)(x[e] - (float)hi) : hi;
        }
      }
    }
  }

  SplitState<H, RK, RV, NW> st;
  st.m_run = -INFINITY;
  st.l_run = 0.f;
#pragma unroll
  for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
    for (int ft = 0; ft < C::FT; ++ft) st.acc[rt][ft] = zero4();

  block_sync_lds();  // block ids and LDS initialisation visible

  // page p of this split: its block id (clamped to a loadable one past the
  // split or when invalid) and how many of its tokens count
  auto page_block = [&](int p) {
    const int blk = __builtin_amdgcn_readfirstlane(sBlk[min(p, p1 - 1) - p0]);
    return blk >= 0 ? blk : 0;
  };
  auto page_valid = [&](int p) {
    if (p >= p1) return 0;
    return __builtin_amdgcn_readfirstlane(sBlk[p - p0]) >= 0 ? min(BS, L - p * BS) : 0;
  };

  // DEPTH register sets form a ring: page p+DEPTH-1 is requested while page
  // p is processed.  sched_barrier(0) keeps the scheduler from hoisting the
  // current page's matrix ops (and the waits they need) above that request.
#pragma unroll
  for (int j = 1; j < DEPTH - 1; ++j)
    load_page<H, RK, RV, NW, QG, NT, FP8>(ring[j], k_cache, v_cache, page_block(p0 + j), w, col,
                                          quad);

  for (int p = p0; p < p1; p += DEPTH) {
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
      load_page<H, RK, RV, NW, QG, NT, FP8>(ring[(j + DEPTH - 1) % DEPTH], k_cache, v_cache,
                                            page_block(p + j + DEPTH - 1), w, col, quad);
      __builtin_amdgcn_sched_barrier(0);
      process_page<H, RK, RV, NW, QG, FP8>(st, ring[j], qv, sP, sAlpha, sFlag, p + j,
                                           (p + j - p0) & 1, page_valid(p + j), w, col, quad);
    }
  }

  // ---- partial state of this split: running max and sum (fp32) per head,
  // and the split's normalised z = acc / l (fp16, a convex combination of
  // value latents, so it stays within their range), rows are heads with
  // contiguous features.  The sums move to the value layout through LDS.
  if (col < C::HPW && quad == 0) {
    float* mp = ml + ((size_t)b * C::R16 + w * C::HPW + col) * 2 * split_stride + s;
    if constexpr (FUSED) {
      st_dev(mp, st.m_run);
      st_dev(mp + split_stride, st.l_run);
    } else {
      mp[0] = st.m_run;
      mp[split_stride] = st.l_run;
    }
    sL[w * C::HPW + col] = st.l_run;
  }
  block_sync_lds();
  half_t* pz = zpart + ((size_t)b * C::R16 * split_stride + s) * RV + w * C::FPW + quad * 4;
#pragma unroll
  for (int rt = 0; rt < C::RT; ++rt) {
    const int hr = rt * 16 + col;
    if (hr < H) {  // rows past H are padding
      const float lh = sL[hr];
      const float inv = lh > 0.f ? v_scale / lh : 0.f;  // v_scale: FP8 value scale, else 1
#pragma unroll
      for (int ft = 0; ft < C::FT; ++ft) {
        half4 zh;
#pragma unroll
        for (int r = 0; r < 4; ++r) zh[r] = (half_t)(st.acc[rt][ft][r] * inv);
        if constexpr (FUSED)
          st_dev(pz + (size_t)hr * split_stride * RV + ft * 16, zh);
        else
          *(half4*)(pz + (size_t)hr * split_stride * RV + ft * 16) = zh;
      }
    }
  }
  if constexpr (FUSED) {
    // Every store of the work group has completed at the device-coherent
    // level (sc1 stores, vmcnt(0)) before the barrier, so a relaxed increment
    // publishes the partials.  A release increment would add an L2
    // write-back (buffer_wbl2) per work group: 3 us more per decode_b16 step.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (tid == 0) __hip_atomic_fetch_add(seq_done + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int H, int RK, int RV, int NW, int DEPTH, bool NT, int QG, bool FP8>
__global__ __launch_bounds__(NW * 64) void decode_split_kernel(
    const float* __restrict__ qt, const latent_t<FP8>* __restrict__ k_cache,
    const latent_t<FP8>* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ seq_lens, float* __restrict__ ml, half_t* __restrict__ zpart,
    int max_blocks, int num_blocks, int pages_per_split, int num_splits, int split_stride,
    float v_scale) {
  __shared__ SplitLds<H, RK, RV, NW> lds;
  split_body<H, RK, RV, NW, DEPTH, NT, QG, FP8, false>(
      lds, blockIdx.x, blockIdx.y, qt, k_cache, v_cache, block_tables, seq_lens, ml, zpart,
      max_blocks, num_blocks, pages_per_split, num_splits, split_stride, v_scale, nullptr);
}

// ---------------------------------------------------------------------------
// 3. finish: the log-sum-exp merge of the splits and the up-projection,
//    z[b,h,:] = sum_s w_s z_s / sum_s w_s with w_s = l_s 2^(m_s - M),
//    M = max_s m_s, then out[b,h,:] = W_h z[b,h,:], in one launch.
// One work group of 4 waves per head h and TB consecutive sequences.
//   * W_h (D x RV fp16) is requested right after the partials' first round
//     and stays in flight through the merge, which waits for the partials
//     only; it reaches the A operands of v_mfma_f32_16x16x32_f16 through LDS
//     (256-thread tiles: whole rows per load instruction) or straight from
//     memory (512-thread tiles), a product wave owning D/MW output rows;
//   * partials: thread u of the TB*RV/4 four-feature units merges its
//     features of one sequence over the splits, CB splits per round of
//     requests (weight 0 past the sequence's last split); the rounds run
//     over the padded split count, so the first requests do not wait for
//     the sequence length and their addresses are affine in the split.  z
//     is split into an fp16 hi/lo pair as it goes to LDS;
//   * B = z^T with column 2t+e holding part e of sequence t's z, read with
//     one 16-byte LDS read per product (columns past TB read a zero row);
//     the two parts share one product and are summed by a neighbour-lane add;
//   * work groups are dealt to the 8 XCDs round robin (blockIdx % 8), so the
//     ids are arranged to put every sequence group of one head on one XCD:
//     W_h then reaches that XCD's L2 once instead of once per group.
// An instruction cache that starts cold at every launch makes each
// straight-line instruction of a short kernel cost a fetch, so the merge and
// the products avoid per-element conversions in their unrolled bodies.
// ---------------------------------------------------------------------------
template <int H, int D, int RV, int TB, int CB, int NT, int QG>
struct FinishCfg {
  static constexpr int R16 = ((H + 15) / 16) * 16;
  static constexpr int F4 = RV / 4;
  static constexpr int UG = TB * F4;                  // four-feature units of the work group
  static constexpr int SG = finish_split_groups(NT, TB, RV);  // split groups (1: one)
  static constexpr int LDZ = RV + 8;                  // halves per LDS row
  // 256-thread tiles stage W_h in LDS by whole rows (each load instruction
  // covers one contiguous 1 KiB row), which moves it faster than loading the
  // product operands directly (16 rows x 64 bytes per instruction); the
  // wider tiles have no LDS left for it.
  static constexpr bool WL = NT == 256;
};

// LDS of one merge unit.
template <int H, int D, int RV, int TB, int CB, int NT, int QG>
struct FinishLds {
  using F = FinishCfg<H, D, RV, TB, CB, NT, QG>;
  // hi and lo parts of z by sequence; row TB stays zero
  __attribute__((aligned(16))) half_t sZ[2][TB + 1][F::LDZ];
  __attribute__((aligned(16))) half_t sW[F::WL ? D : 1][F::WL ? RV + 8 : 8];
  // per split group: running max, sum and four weighted features of a unit
  float sMerge[F::SG > 1 ? F::SG : 1][F::SG > 1 ? F::UG : 1][6];
};

// Bounded wait for *p >= target (device-coherent loads); after about a
// second of polling it records the failure in *err and returns, so the
// kernel always ends.
constexpr int kSpinLimit = 1 << 20;
__device__ __forceinline__ void wait_count(const uint32_t* p, uint32_t target, uint32_t* err) {
  for (int it = 0; it < kSpinLimit; ++it) {
    if (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) return;
    __builtin_amdgcn_s_sleep(1);
  }
  __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One merge unit (head h, sequence group g), placed by `unit` as the
// launch's block index.  FUSED: the unit first waits until every non-empty
// split of its sequences has signalled seq_done, then reads their partials
// with device-coherent loads.
template <int H, int D, int RV, int TB, int CB, int NT, int QG, bool FUSED>
__device__ __forceinline__ void finish_body(FinishLds<H, D, RV, TB, CB, NT, QG>& lds,
                                            const int unit, const float* __restrict__ ml,
                                            const half_t* __restrict__ zpart,
                                            const int32_t* __restrict__ seq_lens,
                                            const half_t* __restrict__ W, int batch,
                                            int max_blocks, int pages_per_split, int num_splits,
                                            int split_stride, half_t* __restrict__ out,
                                            const uint32_t* __restrict__ seq_done,
                                            uint32_t* __restrict__ err) {
  using F = FinishCfg<H, D, RV, TB, CB, NT, QG>;
  constexpr int R16 = F::R16;
  constexpr int F4 = F::F4;
  constexpr int UG = F::UG;
  constexpr int SG = F::SG;
  constexpr int NU = SG > 1 ? 1 : (UG + NT - 1) / NT;  // units per thread
  constexpr int NWV = NT / 64;
  constexpr int MW = NWV < D / 16 ? NWV : D / 16;  // waves on the products
  constexpr int RTW = D / (16 * MW);           // 16-row tiles of W_h per product wave
  constexpr int KS = RV / 32;                  // 32-feature steps
  constexpr bool UNIFORM_SEQ = F4 % 64 == 0;   // a wave's units share one sequence
  static_assert(D % (16 * MW) == 0 && RV % 32 == 0 && TB >= 1 && TB <= 8, "finish tile shape");
  static_assert(SG == 1 || SG * UG <= NT, "split groups must fit the work group");
  constexpr bool WL = F::WL;
  constexpr int WCH = WL ? D * RV / 8 / NT : 1;  // 16-byte chunks per thread
  auto& sZ = lds.sZ;
  auto& sW = lds.sW;
  auto& sMerge = lds.sMerge;
  half8 wst[WCH];

  const int groups = (batch + TB - 1) / TB;
  int h, g;
  if constexpr (H % 8 == 0) {
    const int x = unit % 8, y = unit / 8;
    h = x + 8 * (y / groups);
    g = y % groups;
  } else {
    h = unit / groups;
    g = unit % groups;
  }
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, quad = lane >> 4;
  // split group of this thread: splits sg, sg + SG, sg + 2 SG, ...
  const int sg = SG > 1 ? tid / UG : 0;
  const bool merger = SG == 1 || tid < SG * UG;

  // W_h operands (product waves): rows w*D/MW + 16*rt + col, features
  // 32*k + 8*quad .. +7, requested after the partials' first round (below)
  half8 wa[RTW][KS];
  auto load_w = [&]() {
    if constexpr (WL) {
#pragma unroll
      for (int j = 0; j < WCH; ++j) {
        const int c = tid + j * NT;  // chunk c: row c / (RV/8), 8 features
        wst[j] = *(const half8*)(W + ((size_t)(h / QG) * D + c / (RV / 8)) * RV + (c % (RV / 8)) * 8);
      }
      return;
    }
    const half_t* wrow = W + ((size_t)(h / QG) * D + w * (D / MW) + col) * RV + quad * 8;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int k = 0; k < KS; ++k) wa[rt][k] = *(const half8*)(wrow + (size_t)rt * 16 * RV + k * 32);
  };
  for (int i = tid; i < 2 * RV / 4; i += NT) {  // the zero row
    const half4 hz = {};
    *(half4*)&sZ[i / (RV / 4)][TB][(i % (RV / 4)) * 4] = hz;
  }
  if constexpr (FUSED) {
    // W_h in flight first; then every non-empty split of the group's
    // sequences must have signalled before any partial is read
    if (WL || w < MW) load_w();
    if (tid == 0) {
      for (int t = 0; t < TB; ++t) {
        const int bb = g * TB + t;
        if (bb >= batch) break;
        const int np = min(min((seq_lens[bb] + BS - 1) / BS, max_blocks), num_splits * pages_per_split);
        wait_count(seq_done + bb, (uint32_t)((np + pages_per_split - 1) / pages_per_split), err);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < NU; ++j) {
    const int u = SG > 1 ? tid % UG : tid + j * NT;
    int t = min(u / F4, TB - 1);
    if constexpr (UNIFORM_SEQ) t = __builtin_amdgcn_readfirstlane(t);
    const int f4 = u % F4;
    const int b = min(g * TB + t, batch - 1);
    const bool live_u = u < UG && g * TB + t < batch;
    // m of every split, then l; this group's first split
    const float* mp = ml + ((size_t)b * R16 + h) * 2 * split_stride + sg;
    const half_t* zp = zpart + (((size_t)b * R16 + h) * split_stride + sg) * RV + f4 * 4;
    float M = -INFINITY, den = 0.f;
    float4v num = zero4();
    float m[CB], l[CB];
    half4 a[CB];
    auto request = [&](int q0) {
#pragma unroll
      for (int i = 0; i < CB; ++i) {
        if constexpr (FUSED) {
          m[i] = ld_dev(mp + (q0 + i) * SG);
          l[i] = ld_dev(mp + split_stride + (q0 + i) * SG);
          a[i] = ld_dev(zp + (size_t)(q0 + i) * SG * RV);
        } else {
          m[i] = mp[(q0 + i) * SG];
          l[i] = mp[split_stride + (q0 + i) * SG];
          a[i] = *(const half4*)(zp + (size_t)(q0 + i) * SG * RV);
        }
      }
    };
    if (merger) request(0);
    if (!FUSED && j == 0 && (WL || w < MW)) load_w();
    __builtin_amdgcn_sched_barrier(0);  // the sequence length is read after these requests
    const int n_pages =
        min(min((seq_lens[b] + BS - 1) / BS, max_blocks), num_splits * pages_per_split);
    const int ns = (n_pages + pages_per_split - 1) / pages_per_split;
    if (merger) {
      // do-while: no guard between the first requests and their use, which
      // would let the compiler sink them below a test of the split count
      int q0 = 0;
      do {
        if (q0 > 0) request(q0);
        float mx = M;
#pragma unroll
        for (int i = 0; i < CB; ++i) mx = ((q0 + i) * SG + sg < ns) ? fmaxf(mx, m[i]) : mx;
        const float sc = (mx == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(M - mx);
        num *= sc;
        den *= sc;
        M = mx;
#pragma unroll
        for (int i = 0; i < CB; ++i) {
          const bool live = (q0 + i) * SG + sg < ns && m[i] != -INFINITY;
          const float wgt = live ? l[i] * __builtin_amdgcn_exp2f(m[i] - M) : 0.f;
          const half4 hz = {};
          const half4 av = live ? a[i] : hz;  // slots never written may hold NaN
#pragma unroll
          for (int e = 0; e < 4; ++e) num[e] = __builtin_fmaf((float)av[e], wgt, num[e]);
          den += wgt;
        }
        q0 += CB;
      } while (q0 * SG < split_stride);
    }
    if constexpr (SG > 1) {  // merge the groups' states of each unit
      if (merger) {
        float* sm = sMerge[sg][u];
        sm[0] = M;
        sm[1] = den;
#pragma unroll
        for (int e = 0; e < 4; ++e) sm[2 + e] = num[e];
      }
      block_sync_lds();
      if (sg == 0 && merger) {
        float mx = M;
#pragma unroll
        for (int k = 1; k < SG; ++k) mx = fmaxf(mx, sMerge[k][u][0]);
        const float sc = (mx == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(M - mx);
        num *= sc;
        den *= sc;
#pragma unroll
        for (int k = 1; k < SG; ++k) {
          const float mk = sMerge[k][u][0];
          const float sk = (mk == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mk - mx);
          den += sMerge[k][u][1] * sk;
#pragma unroll
          for (int e = 0; e < 4; ++e) num[e] += sMerge[k][u][2 + e] * sk;
        }
      }
    }
    if (u < UG && sg == 0 && merger) {
      const float inv = (live_u && den > 0.f) ? 1.f / den : 0.f;
      half4 zh, zl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float zv = num[e] * inv;
        zh[e] = (half_t)zv;
        zl[e] = (half_t)(zv - (float)zh[e]);
      }
      *(half4*)&sZ[0][u / F4][f4 * 4] = zh;
      *(half4*)&sZ[1][u / F4][f4 * 4] = zl;
    }
  }
  if constexpr (WL) {
#pragma unroll
    for (int j = 0; j < WCH; ++j) {
      const int c = tid + j * NT;
      *(half8*)&sW[c / (RV / 8)][(c % (RV / 8)) * 8] = wst[j];
    }
  }
  block_sync_lds();  // LDS only: (without staging) the W_h loads stay in flight
  if (w >= MW) return;  // no barrier follows
  if constexpr (WL) {
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int k = 0; k < KS; ++k)
        wa[rt][k] = *(const half8*)&sW[w * (D / MW) + rt * 16 + col][k * 32 + quad * 8];
  }

  // B column col: sequence col/2, part col%2
  const int tc = col >> 1;
  const half_t* zr = &sZ[col & 1][tc < TB ? tc : TB][quad * 8];
  float4v o[RTW];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) o[rt] = zero4();
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const half8 bop = *(const half8*)(zr + k * 32);
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) o[rt] = mfma16x16x32(wa[rt][k], bop, o[rt]);
  }
  // D[row 4*quad + r][column col]; the even column of each pair adds its
  // neighbour (the lo part) and stores four consecutive outputs
  const int b = g * TB + tc;
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    half4 ov;
#pragma unroll
    for (int r = 0; r < 4; ++r) ov[r] = (half_t)(o[rt][r] + __shfl_xor(o[rt][r], 1));
    if (tc < TB && (col & 1) == 0 && b < batch)
      *(half4*)(out + ((size_t)b * H + h) * D + w * (D / MW) + rt * 16 + quad * 4) = ov;
  }
}

template <int H, int D, int RV, int TB, int CB, int NT, int QG>
__global__ __launch_bounds__(NT) void finish_kernel(const float* __restrict__ ml,
                                                    const half_t* __restrict__ zpart,
                                                    const int32_t* __restrict__ seq_lens,
                                                    const half_t* __restrict__ W, int batch,
                                                    int max_blocks, int pages_per_split,
                                                    int num_splits, int split_stride,
                                                    half_t* __restrict__ out) {
  __shared__ FinishLds<H, D, RV, TB, CB, NT, QG> lds;
  finish_body<H, D, RV, TB, CB, NT, QG, false>(lds, blockIdx.x, ml, zpart, seq_lens, W, batch,
                                               max_blocks, pages_per_split, num_splits,
                                               split_stride, out, nullptr, nullptr);
}

// ---------------------------------------------------------------------------
// 3'. the split pass and the merge in one launch.  Work group w runs split
// items w, w + G, ... (item = sequence * num_splits + split, as the split
// kernel's grid), then merge units w, w + G, ... (unit as the merge kernel's
// block index, so a head's units keep their XCD).  A merge unit waits for its
// sequences' non-empty splits through seq_done (zeroed by the q projection
// launch before this one).  Split items never wait, and the host caps G at
// the number of work groups that can be resident at once, so every split
// item is run by a work group that is or will be resident and every wait
// ends; the wait is bounded all the same.
// ---------------------------------------------------------------------------
template <int H, int D, int RK, int RV, int NW, int DEPTH, int QG, bool FP8, int TB, int CB>
__global__ __launch_bounds__(NW * 64) void decode_fused_kernel(
    const float* __restrict__ qt, const latent_t<FP8>* __restrict__ k_cache,
    const latent_t<FP8>* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ seq_lens, float* __restrict__ ml, half_t* __restrict__ zpart,
    const half_t* __restrict__ W, half_t* __restrict__ out, uint32_t* __restrict__ sync,
    int batch, int max_blocks, int num_blocks, int pages_per_split, int num_splits,
    int split_stride, float v_scale, int n_items, int n_units) {
  __shared__ SplitLds<H, RK, RV, NW> ls;
  __shared__ FinishLds<H, D, RV, TB, CB, NW * 64, QG> lf;
  uint32_t* seq_done = sync;
  uint32_t* err = sync + batch;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    split_body<H, RK, RV, NW, DEPTH, false, QG, FP8, true>(
        ls, item % num_splits, item / num_splits, qt, k_cache, v_cache, block_tables, seq_lens,
        ml, zpart, max_blocks, num_blocks, pages_per_split, num_splits, split_stride, v_scale,
        seq_done);
    __syncthreads();
  }
  for (int unit = blockIdx.x; unit < n_units; unit += gridDim.x) {
    finish_body<H, D, RV, TB, CB, NW * 64, QG, true>(lf, unit, ml, zpart, seq_lens, W, batch,
                                                     max_blocks, pages_per_split, num_splits,
                                                     split_stride, out, seq_done, err);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// 4. up-projection of many tokens (prefill), out[n, h, :] = W_h z[n, h, :]:
// grid (H, ceil(N / (32*NW))).  W_h (D x RV
// fp16) is staged once per work group in LDS, padded so that each 16-lane
// group of a 16-byte read hits distinct banks; then every wave streams 32
// tokens of z through v_mfma_f32_32x32x16_f16 with no further barrier:
// A = z (32 tokens x 16 features, fp16; z arrives tiled in exactly this
// operand order, so each lane's 16 bytes and each wave's KiB are
// contiguous), B = W_h^T (16 features x 32 outputs, from LDS),
// D[token][output].  The z loads run up to 16 chunks ahead of their
// products: z comes from HBM, and the LDS footprint already limits the
// kernel to two waves per SIMD, which leaves the registers for the ring.
template <int H, int D, int RV, int NW, int QG>
__global__ __launch_bounds__(NW * 64) void upproj_tiled_kernel(const half_t* __restrict__ W,
                                                               const half_t* __restrict__ z,
                                                               int n_tokens,
                                                               half_t* __restrict__ out) {
  constexpr int LDW = RV + 8;  // halves per LDS row
  constexpr int DT = D / 32;   // 32-wide output tiles
  constexpr int KC = RV / 16;  // 16-feature chunks
  constexpr int ZP = KC < 16 ? KC : 16;  // z chunks in flight
  static_assert(D % 32 == 0 && RV % 16 == 0 && KC >= ZP, "tile shape");
  typedef float float16v __attribute__((ext_vector_type(16)));
  __shared__ __attribute__((aligned(16))) half_t sW[D][LDW];
  const int h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c32 = lane & 31, hf = lane >> 5;
  const half_t* Wh = W + (size_t)(h / QG) * D * RV;  // the head's key/value head
  for (int c = tid; c < D * RV / 8; c += NW * 64) {
    const int r = c / (RV / 8), k = (c % (RV / 8)) * 8;
    *(half8*)&sW[r][k] = *(const half8*)(Wh + (size_t)r * RV + k);
  }
  __syncthreads();
  const int t0 = blockIdx.y * (NW * 32) + w * 32;
  if (t0 >= n_tokens) return;  // no barrier follows
  // tiled z: block t0/32 of head h, chunk kc at +kc*512, this lane's 8
  // halves at +lane*8 (rows past n_tokens in the last block hold stale
  // values and are never stored)
  const half_t* zr = z + ((size_t)h * ((n_tokens + 31) / 32) + t0 / 32) * KC * 512 + lane * 8;
  float16v acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[dt][e] = 0.f;
  half8 zq[ZP];
#pragma unroll
  for (int j = 0; j < ZP; ++j) zq[j] = *(const half8*)(zr + j * 512);
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    const half8 av = zq[kc % ZP];
    if (kc + ZP < KC) zq[kc % ZP] = *(const half8*)(zr + (kc + ZP) * 512);
    // keep the refill issued here, ZP chunks ahead of its use, instead of
    // letting the scheduler sink it next to the products that consume it
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const half8 b = *(const half8*)&sW[dt * 32 + c32][kc * 16 + 8 * hf];
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, b, acc[dt], 0, 0, 0);
    }
  }
  // register i of tile dt holds token 8*(i/4) + 4*hf + i%4, output dt*32 + c32
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int n = t0 + 8 * (i / 4) + 4 * hf + (i % 4);
    if (n < n_tokens) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        out[((size_t)n * H + h) * D + dt * 32 + c32] = (half_t)acc[dt][i];
    }
  }
}

template <int H, int D, int RV, int NW, int QG>
static void launch_upproj_tiled_t(const void* W, const void* z, int n_tokens, void* out,
                                  hipStream_t st) {
  hipLaunchKernelGGL((upproj_tiled_kernel<H, D, RV, NW, QG>),
                     dim3(H, (n_tokens + NW * 32 - 1) / (NW * 32)), dim3(NW * 64), 0, st,
                     (const half_t*)W, (const half_t*)z, n_tokens, (half_t*)out);
}

hipError_t launch_upproj_tiled(const ShapeKey& s, const void* W, const void* z_tiled,
                               int n_tokens, void* out, hipStream_t st) {
  if (n_tokens <= 0) return hipSuccess;
  if (s.H == 32 && s.Hkv == 32 && s.d == 128 && s.rv == 512)
    launch_upproj_tiled_t<32, 128, 512, 8, 1>(W, z_tiled, n_tokens, out, st);
  else if (s.H == 32 && s.Hkv == 8 && s.d == 128 && s.rv == 512)
    launch_upproj_tiled_t<32, 128, 512, 8, 4>(W, z_tiled, n_tokens, out, st);
  else if (s.H == 32 && s.Hkv == 32 && s.d == 128 && s.rv == 256)
    launch_upproj_tiled_t<32, 128, 256, 8, 1>(W, z_tiled, n_tokens, out, st);
  else if (s.H == 4 && s.Hkv == 4 && s.d == 64 && s.rv == 64)
    launch_upproj_tiled_t<4, 64, 64, 4, 1>(W, z_tiled, n_tokens, out, st);
  else if (s.H == 4 && s.Hkv == 2 && s.d == 64 && s.rv == 64)
    launch_upproj_tiled_t<4, 64, 64, 4, 2>(W, z_tiled, n_tokens, out, st);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
// Compute units the stream's kernels may use: those set in its CU mask (the
// device's count when the mask cannot be read).
static int stream_cus(hipStream_t st) {
  uint32_t mask[16] = {};
  if (hipExtStreamGetCUMask(st, 16, mask) == hipSuccess) {
    int n = 0;
    for (uint32_t m : mask) n += __builtin_popcount(m);
    if (n > 0) return n;
  }
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
    return n;
  return 0;
}

template <int H, int D, int RK, int RV, int NW, int DEPTH, bool NT, int QG = 1, bool FP8 = false>
static hipError_t decode_instance(const DecodePlan& p, const void* qt, const void* k_cache,
                                  const void* v_cache, const void* W, const int32_t* block_tables,
                                  int max_blocks, const int32_t* seq_lens, int num_blocks,
                                  int batch, float* ml, void* zpart, void* out, float v_scale,
                                  uint32_t* sync, hipStream_t st) {
  if (p.fused) {
    // the split pass and the merge in one launch, grid capped at the work
    // groups that can be resident at once
    const int n_items = batch * p.num_splits;
    const int n_units = H * ((batch + p.finish_tb - 1) / p.finish_tb);
    const int want = n_items > n_units ? n_items : n_units;
#define STARKV_FUSED(TB_)                                                                          \
  {                                                                                                \
    auto kern = decode_fused_kernel<H, D, RK, RV, NW, DEPTH, QG, FP8, TB_, 4>;                     \
    static const int occ = [&] {                                                                   \
      int n = 0;                                                                                   \
      return hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, NW * 64, 0) == hipSuccess ? n  \
                                                                                              : 0; \
    }();                                                                                           \
    const int slots = occ * stream_cus(st);                                                        \
    if (slots <= 0) return hipErrorInvalidConfiguration;                                           \
    launch_hooked(TIME_DECODE_SPLIT, TIME_NONE, kern, dim3(want < slots ? want : slots),           \
                  dim3(NW * 64), st, (const float*)qt, (const latent_t<FP8>*)k_cache,              \
                  (const latent_t<FP8>*)v_cache, block_tables, seq_lens, ml, (half_t*)zpart,       \
                  (const half_t*)W, (half_t*)out, sync, batch, max_blocks, num_blocks,             \
                  p.pages_per_split, p.num_splits, p.split_stride, v_scale, n_items, n_units);     \
  }
    switch (p.finish_tb) {
      case 1: STARKV_FUSED(1) break;
      case 2: STARKV_FUSED(2) break;
      case 4: STARKV_FUSED(4) break;
      case 8: STARKV_FUSED(8) break;
      default: return hipErrorInvalidValue;
    }
#undef STARKV_FUSED
    return hipGetLastError();
  }
  launch_hooked(TIME_DECODE_SPLIT, TIME_NONE,
                decode_split_kernel<H, RK, RV, NW, DEPTH, NT, QG, FP8>,
                dim3(p.num_splits, batch), dim3(NW * 64), st, (const float*)qt,
                (const latent_t<FP8>*)k_cache, (const latent_t<FP8>*)v_cache, block_tables,
                seq_lens, ml, (half_t*)zpart, max_blocks, num_blocks, p.pages_per_split,
                p.num_splits, p.split_stride, v_scale);
  // merge + up-projection: TB sequences and NT threads per work group, CB
  // splits per request round (the planner picks all three; the split stride
  // is a multiple of CB times the split groups)
  const unsigned wgs = (unsigned)(H * ((batch + p.finish_tb - 1) / p.finish_tb));
#define STARKV_FINISH(TB_, CB_, NT_)                                                           \
  hipLaunchKernelGGL((finish_kernel<H, D, RV, TB_, CB_, NT_, QG>), dim3(wgs), dim3(NT_), 0, st, \
                     (const float*)ml, (const half_t*)zpart, seq_lens, (const half_t*)W, batch, \
                     max_blocks, p.pages_per_split, p.num_splits, p.split_stride, (half_t*)out)
  switch (p.finish_tb * 1000000 + p.finish_cb * 10000 + p.finish_nt) {
    case 1040256: STARKV_FINISH(1, 4, 256); break;
    case 1080256: STARKV_FINISH(1, 8, 256); break;
    case 1160256: STARKV_FINISH(1, 16, 256); break;
    case 1160512: STARKV_FINISH(1, 16, 512); break;
    case 2040256: STARKV_FINISH(2, 4, 256); break;
    case 2080256: STARKV_FINISH(2, 8, 256); break;
    case 2160256: STARKV_FINISH(2, 16, 256); break;
    case 2160512: STARKV_FINISH(2, 16, 512); break;
    case 4040256: STARKV_FINISH(4, 4, 256); break;
    case 4080256: STARKV_FINISH(4, 8, 256); break;
    case 8040256: STARKV_FINISH(8, 4, 256); break;
    default: return hipErrorInvalidValue;
  }
#undef STARKV_FINISH
  return hipGetLastError();
}

// W prefetch rows: each reads kPrefetchPart bytes of one head's W block
constexpr int kPrefetchPart = 64 * 1024;

template <int H, int D, int RK, int QG>
static hipError_t qproj_instance(const void* q, const void* U, int n, float scale, void* qt,
                                 int precedes, const void* wpf, int rv, uint32_t* zero,
                                 int n_zero, hipStream_t st) {
  const int head_bytes = D * rv * (int)sizeof(half_t);
  const bool pf = wpf != nullptr && H % 8 == 0 && head_bytes % kPrefetchPart == 0;
  const int pf_rows = pf ? head_bytes / kPrefetchPart : 0;
  if (n >= 1024) {  // many tokens: four 64-token tiles per work group
    const int rows = (n + 255) / 256;
    launch_hooked(TIME_NONE, precedes, qproj_kernel<H, D, RK, 4, QG>, dim3(H, rows + pf_rows),
                  dim3(256), st, (const half_t*)q, (const half_t*)U, n, scale * kLog2e,
                  (float*)qt, rows, (const char*)wpf, head_bytes, kPrefetchPart, (uint32_t*)nullptr,
                  zero, n_zero);
  } else {
    const int rows = (n + 63) / 64;
    launch_hooked(TIME_NONE, precedes, qproj_kernel<H, D, RK, 1, QG>, dim3(H, rows + pf_rows),
                  dim3(256), st, (const half_t*)q, (const half_t*)U, n, scale * kLog2e,
                  (float*)qt, rows, (const char*)wpf, head_bytes, kPrefetchPart, (uint32_t*)nullptr,
                  zero, n_zero);
  }
  return hipGetLastError();
}

hipError_t launch_qproj(const ShapeKey& s, const void* q, const void* U, int n_tokens, float scale,
                        void* qt, int precedes, hipStream_t st, const void* w_prefetch,
                        uint32_t* zero, int n_zero) {
  if (n_tokens <= 0) return hipSuccess;
#define STARKV_QPROJ(H_, D_, RK_, QG_) \
  return qproj_instance<H_, D_, RK_, QG_>(q, U, n_tokens, scale, qt, precedes, w_prefetch, s.rv, \
                                          zero, n_zero, st)
  if (s.H == 32 && s.d == 128 && s.rk == 64) {
    if (s.Hkv == 32) STARKV_QPROJ(32, 128, 64, 1);
    if (s.Hkv == 8) STARKV_QPROJ(32, 128, 64, 4);
  }
  if (s.H == 32 && s.d == 128 && s.rk == 32 && s.Hkv == 32) STARKV_QPROJ(32, 128, 32, 1);
  if (s.H == 4 && s.d == 64 && s.rk == 16) {
    if (s.Hkv == 4) STARKV_QPROJ(4, 64, 16, 1);
    if (s.Hkv == 2) STARKV_QPROJ(4, 64, 16, 2);
  }
#undef STARKV_QPROJ
  return hipErrorInvalidValue;
}

int decode_threads(const ShapeKey& s) { return s.H == 4 ? 4 * 64 : 16 * 64; }

hipError_t launch_decode(const ShapeKey& s, const DecodePlan& p, const void* qt, const void* k_cache,
                         const void* v_cache, const void* W, const int32_t* block_tables,
                         int max_blocks, const int32_t* seq_lens, int num_blocks, int batch,
                         float* ml, void* zpart, void* out, const LatentFormat& fmt,
                         uint32_t* sync, hipStream_t st) {
#define STARKV_DECODE_ARGS                                                                    \
  p, qt, k_cache, v_cache, W, block_tables, max_blocks, seq_lens, num_blocks, batch, ml, zpart, \
      out, fmt.fp8 ? fmt.v_scale : 1.f, sync, st
  if (fmt.fp8) {  // FP8 latents: the main shape (either head layout) and the tiny one
    if (s.H == 32 && s.Hkv == 32 && s.d == 128 && s.rk == 64 && s.rv == 512)
      return decode_instance<32, 128, 64, 512, 16, 2, false, 1, true>(STARKV_DECODE_ARGS);
    if (s.H == 32 && s.Hkv == 8 && s.d == 128 && s.rk == 64 && s.rv == 512)
      return decode_instance<32, 128, 64, 512, 16, 2, false, 4, true>(STARKV_DECODE_ARGS);
    if (s.H == 4 && s.Hkv == 4 && s.d == 64 && s.rk == 16 && s.rv == 64)
      return decode_instance<4, 64, 16, 64, 4, 2, false, 1, true>(STARKV_DECODE_ARGS);
    return hipErrorInvalidValue;
  }
  if (s.H == 32 && s.Hkv == 8 && s.d == 128 && s.rk == 64 && s.rv == 512)
    return decode_instance<32, 128, 64, 512, 16, 2, false, 4>(STARKV_DECODE_ARGS);
  if (s.H == 4 && s.Hkv == 2 && s.d == 64 && s.rk == 16 && s.rv == 64)
    return decode_instance<4, 64, 16, 64, 4, 2, false, 2>(STARKV_DECODE_ARGS);
  if (s.H == 32 && s.Hkv == 32 && s.d == 128 && s.rk == 32 && s.rv == 256)
    return decode_instance<32, 128, 32, 256, 16, 2, false>(STARKV_DECODE_ARGS);
  if (s.H == 32 && s.Hkv == 32 && s.d == 128 && s.rk == 64 && s.rv == 512)
    return decode_instance<32, 128, 64, 512, 16, 2, false>(STARKV_DECODE_ARGS);
  if (s.H == 4 && s.Hkv == 4 && s.d == 64 && s.rk == 16 && s.rv == 64)
    return decode_instance<4, 64, 16, 64, 4, 2, false>(STARKV_DECODE_ARGS);
#undef STARKV_DECODE_ARGS
  return hipErrorInvalidValue;
}

}  // namespace starkv
