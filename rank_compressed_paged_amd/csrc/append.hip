// Append: project new full-precision K/V into latents and scatter them into
// their paged slots (the README's write kernel, "Kernel profiling
// breakdown": low-rank projection plus the paged write).
//
//   c_k[n, h, :] = U_h^T k[n, h, :]       (a [N x d] x [d x r_k] product per head)
//   c_v[n, :]    = W^T vec(v[n])           (one [N x H*d] x [H*d x r_v] product)
//
// Both products are C = A B with A row-major (contraction contiguous) and B
// row-major (outputs contiguous).  Three forms, all on the matrix cores:
//   * few tokens (a decode step): append_few_kernel, one launch of about 256
//     work groups that split the value contraction and finish it with a
//     last-arriver sum (below);
//   * many tokens at the tuned shapes: append_tiled_kernel, 128 x 64 tiles
//     with both operand tiles staged through LDS, optionally with the value
//     contraction split over work groups and summed by append_reduce_kernel;
//   * any other shape: append_kernel, 64 x 64 tiles, A straight from memory.
// The epilogues round to fp16 (nearest even), or to FP8 E4M3 codes of
// latent / scale for FP8 caches, and write slot_mapping[n]; negative or
// out-of-range slots are skipped.
// Layouts: k_cache [NB, H, 16, r_k], v_cache [NB, r_v, 16].

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace starkv {

struct AppendArgs {
  const half_t* k;  // [N, H, d]
  const half_t* v;  // [N, H, d]
  const half_t* U;  // [H, d, r_k]
  const half_t* W;  // [H*d, r_v]
  const int64_t* slots;
  void* k_cache;    // fp16, or FP8 E4M3 codes when fp8
  void* v_cache;
  int N, H, D, RK, RV, num_blocks;
  int tiles_m, v_tiles_n, k_tiles_n;
  int fp8;               // store FP8 E4M3 codes of latent / scale
  float k_scale, v_scale;
  uint32_t* counters;    // few-token path: arrival counter per value column block
  float* part;           // value partials [slice][N][RV] fp32 (few-token path, split tiled path)
};

// One latent of the epilogue: fp16 rounded to nearest even, or the E4M3
// code of acc / scale, clamped to +-448 first (saturation) and rounded to
// nearest even by v_cvt_pk_fp8_f32.
__device__ __forceinline__ void store_latent(const AppendArgs& a, bool is_v, size_t idx,
                                             float acc) {
  void* base = is_v ? a.v_cache : a.k_cache;
  if (a.fp8) {
    const float x = fminf(fmaxf(acc / (is_v ? a.v_scale : a.k_scale), -448.f), 448.f);
    ((uint8_t*)base)[idx] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.f, 0, false) & 0xff);
  } else {
    ((half_t*)base)[idx] = (half_t)acc;
  }
}

constexpr int AT_M = 64, AT_N = 64, AT_K = 32, AT_LDS = AT_K + 8;

// Generic form: a 256-thread work group computes a 64 (tokens) x 64 (outputs)
// tile with v_mfma_f32_16x16x32_f16; A operands come straight from memory (8
// contiguous fp16 per lane), B is staged through LDS transposed so that each
// lane again reads 8 contiguous values.  The next K step's loads are issued
// before the current step's LDS barrier.
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  __shared__ __attribute__((aligned(16))) half_t sB[2][AT_N][AT_LDS];
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int col = lane & 15, quad = lane >> 4;

  // ---- job decode: value tiles first, then key tiles (one head each)
  int job = blockIdx.x;
  const int n_vjobs = a.tiles_m * a.v_tiles_n;
  bool is_v;
  int mt_idx, nt_idx, h = 0;
  if (job < n_vjobs) {
    is_v = true;
    mt_idx = job / a.v_tiles_n;
    nt_idx = job % a.v_tiles_n;
  } else {
    is_v = false;
    job -= n_vjobs;
    mt_idx = job / (a.H * a.k_tiles_n);
    const int rem = job % (a.H * a.k_tiles_n);
    h = rem / a.k_tiles_n;
    nt_idx = rem % a.k_tiles_n;
  }
  const int HD = a.H * a.D;
  const half_t* A = is_v ? a.v : a.k + (size_t)h * a.D;
  const int lda = HD;
  const half_t* Bm = is_v ? a.W : a.U + (size_t)h * a.D * a.RK;
  const int ldb = is_v ? a.RV : a.RK;
  const int Kdim = is_v ? HD : a.D;
  const int Ndim = is_v ? a.RV : a.RK;
  const int m_base = mt_idx * AT_M, n_base = nt_idx * AT_N;

  float4v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = zero4();

  // staging role: k row kk, outputs n0 .. n0+7
  const int kk = tid >> 3, n0 = (tid & 7) * 8;
  const bool b_ok = (n_base + n0 + 8 <= Ndim);
  const half8 hz = {};

  int arow[2];
  bool arow_ok[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int m = m_base + wm * 32 + mt * 16 + col;
    arow_ok[mt] = m < a.N;
    arow[mt] = arow_ok[mt] ? m : 0;
  }

  auto load_b = [&](int k0) {
    return b_ok ? *(const half8*)(Bm + (size_t)(k0 + kk) * ldb + n_base + n0) : hz;
  };
  auto load_a = [&](int k0, int mt) {
    return arow_ok[mt] ? *(const half8*)(A + (size_t)arow[mt] * lda + k0 + quad * 8) : hz;
  };
  // software pipeline: the next K step's global loads are in flight while
  // the current step goes through LDS and the matrix cores; LDS is
  // double-buffered so one LDS-only barrier per step suffices
  half8 bv = load_b(0);
  half8 av0 = load_a(0, 0), av1 = load_a(0, 1);
  int buf = 0;
  for (int k0 = 0; k0 < Kdim; k0 += AT_K) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sB[buf][n0 + e][kk] = bv[e];
    const half8 a0 = av0, a1 = av1;
    if (k0 + AT_K < Kdim) {
      bv = load_b(k0 + AT_K);
      av0 = load_a(k0 + AT_K, 0);
      av1 = load_a(k0 + AT_K, 1);
    }
    block_sync_lds();
    half8 bq[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) bq[nt] = *(const half8*)&sB[buf][wn * 32 + nt * 16 + col][quad * 8];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      acc[0][nt] = mfma16x16x32(a0, bq[nt], acc[0][nt]);
      acc[1][nt] = mfma16x16x32(a1, bq[nt], acc[1][nt]);
    }
    buf ^= 1;
  }

  // ---- epilogue: D[token][output], lane holds rows 4*quad + r, column col;
  // the lane's 8 slots are requested together (indices clamped into range)
  int64_t slot_of[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      slot_of[mt][r] = a.slots[min(m_base + wm * 32 + mt * 16 + quad * 4 + r, a.N - 1)];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m_base + wm * 32 + mt * 16 + quad * 4 + r;
      if (m >= a.N) continue;
      const int64_t slot = slot_of[mt][r];
      if (slot < 0) continue;
      const int64_t blk = slot / 16;
      const int off = (int)(slot % 16);
      if (blk >= a.num_blocks) continue;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int n = n_base + wn * 32 + nt * 16 + col;
        if (n >= Ndim) continue;
        if (is_v)
          store_latent(a, true, ((size_t)blk * a.RV + n) * 16 + off, acc[mt][nt][r]);
        else
          store_latent(a, false, (((size_t)blk * a.H + h) * 16 + off) * a.RK + n, acc[mt][nt][r]);
      }
    }
  }
}


// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, lane i
// receives element i%4 of the 4-element (8-byte) chunk addressed by lane
// 4e + i/4, for e = 0..3.  So if lane q of a group addresses row k0 + q/4,
// columns o0 + 4*(q%4) .. +3 of a row-major [k][output] tile, lane i gets
// the 4 consecutive k of output o0 + i: an MFMA B-operand fragment read from
// a tile stored untransposed.
typedef short short4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ half4 lds_read_tr16(const half_t* p) {
  typedef __attribute__((address_space(3))) short4v lds_short4v;
  const short4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)p);
  return __builtin_bit_cast(half4, r);
}

// ---------------------------------------------------------------------------
// Few tokens (a decode step's append), one launch.  The work is reading the
// bases (W is 4 MiB at the main shape), so it is spread over about 256 work
// groups of four waves:
//   value job (slice s, column block cb): rows R*s .. R*s+R-1 of W and its
//     CB outputs cb*CB ..; the fp32 partial products of the slice's rows,
//     [N][CB], go to the workspace with device-coherent stores, then the
//     block's arrival counter is incremented.  The work group that arrives
//     last sums the S slices' partials in slice order (so the result does
//     not depend on arrival order), rounds, writes the tokens' slots and
//     sets the counter back to zero: nothing waits, and every call leaves
//     the counters zero;
//   key job (head h): U_h staged in LDS, one 16-output tile of c_k per
//     wave over the whole contraction d, rounded and written directly.
// The B operand of v_mfma_f32_16x16x32_f16 (8 consecutive k of one output
// per lane) comes from the basis staged [k][output] through the transposing
// LDS read; A is 8 consecutive features of one token straight from memory.
// ---------------------------------------------------------------------------
constexpr int kSmallN = 64;  // tokens handled by the few-token kernel

// Rows of W per value slice: about 256 value jobs over (slices x column
// blocks of 32 outputs), at least 64 rows each.
constexpr int few_slice_rows(int K, int RV) {
  return K * (RV / 32) / 256 < 64 ? 64 : K * (RV / 32) / 256;
}

template <int H, int D, int RK, int RV>
struct FewCfg {
  static constexpr int K = H * D;           // value contraction
  static constexpr int CB = 32;             // outputs per column block
  static constexpr int NCB = RV / CB;       // column blocks (one counter each)
  static constexpr int R = few_slice_rows(K, RV);
  static constexpr int S = K / R;           // slices
  static constexpr int VJ = S * NCB;        // value jobs
  static constexpr int KCW = R / 64;        // 32-row chunks per wave (two waves per tile)
  static constexpr int LDW = CB + 16;       // halves per staged row of a W slice
  static constexpr int LDU = RK + 16;       // halves per staged row of U_h
  static constexpr int LDS_HALVES = (R * LDW > D * LDU) ? R * LDW : D * LDU;
  static_assert(RV % CB == 0 && K % R == 0 && R % 64 == 0, "few-token value tiling");
  static_assert(RK % 16 == 0 && RK <= 64 && D % 32 == 0, "few-token key tiling");
  static_assert(NCB * 4 <= (int)kWorkspaceHeaderBytes, "arrival counters");
};

template <int H, int D, int RK, int RV>
__global__ __launch_bounds__(256) void append_few_kernel(AppendArgs a) {
  using F = FewCfg<H, D, RK, RV>;
  __shared__ __attribute__((aligned(16))) half_t sT[F::LDS_HALVES];
  __shared__ float4v sRed[2][kSmallN / 16][64];  // upper k half of each (tile, token tile)
  __shared__ int sLast;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, quad = lane >> 4;
  const int n_tiles = (a.N + 15) / 16;  // <= kSmallN / 16
  uint32_t* const counters = a.counters;
  float* const part = a.part;

  if ((int)blockIdx.x >= F::VJ) {
    // ---- key job: head h, c_k = U_h^T k over d, one output tile per wave
    const int h = blockIdx.x - F::VJ;
    const half_t* Uh = a.U + (size_t)h * D * RK;
    constexpr int KC = D / 32;
    const bool active = w < RK / 16;
    auto load_k = [&](half8 (&av)[KC], int t) {
      const int m = min(t * 16 + col, a.N - 1);
#pragma unroll
      for (int c = 0; c < KC; ++c)
        av[c] = *(const half8*)(a.k + ((size_t)m * H + h) * D + c * 32 + quad * 8);
    };
    half8 av[KC];
    if (active) load_k(av, 0);
    for (int c = tid; c < D * (RK / 8); c += 256) {
      const int k = c / (RK / 8), o = (c % (RK / 8)) * 8;
      *(half8*)&sT[k * F::LDU + o] = *(const half8*)(Uh + (size_t)k * RK + o);
    }
    __syncthreads();
    if (!active) return;  // no barrier follows
    for (int t = 0; t < n_tiles; ++t) {  // uniform
      if (t > 0) load_k(av, t);
      float4v acc = zero4();
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        // B fragment: k c*32 + 8*quad .. +7 of output 16w + col (lane col
        // addresses row col/4, outputs 4*(col%4) .. +3)
        const half_t* bp = &sT[(c * 32 + quad * 8 + (col >> 2)) * F::LDU + w * 16 + 4 * (col & 3)];
        const half4 b0 = lds_read_tr16(bp);
        const half4 b1 = lds_read_tr16(bp + 4 * F::LDU);
        const half8 bq = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        acc = mfma16x16x32(av[c], bq, acc);
      }
      // D[token 4*quad + r][output 16w + col]
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = t * 16 + quad * 4 + r;
        if (n >= a.N) continue;
        const int64_t slot = a.slots[n];
        if (slot < 0 || slot / 16 >= a.num_blocks) continue;
        store_latent(a, false, (((size_t)(slot / 16) * H + h) * 16 + slot % 16) * RK + w * 16 + col,
                     acc[r]);
      }
    }
    return;
  }

  // ---- value job.  Work groups are dealt to the XCDs round robin; ids b and
  // b + 8 share an XCD, so they take the two column blocks of one 128-byte
  // line of W rows, which that XCD's L2 then fetches once.
  int cb, s;
  const int b = blockIdx.x;
  if constexpr (F::VJ % 16 == 0 && F::NCB % 2 == 0) {
    const int t = (b / 16) * 8 + b % 8;
    cb = 2 * (t % (F::NCB / 2)) + (b / 8) % 2;
    s = t / (F::NCB / 2);
  } else {
    cb = b % F::NCB;
    s = b / F::NCB;
  }
  const int k0 = s * F::R, o0 = cb * F::CB;
  const int ot = w & 1, kh = w >> 1;  // output tile, k half of the slice
  auto load_v = [&](half8 (&av)[F::KCW], int t) {
    const int m = min(t * 16 + col, a.N - 1);
#pragma unroll
    for (int c = 0; c < F::KCW; ++c)
      av[c] = *(const half8*)(a.v + (size_t)m * F::K + k0 + (kh * F::KCW + c) * 32 + quad * 8);
  };
  half8 av[F::KCW];
  load_v(av, 0);
  for (int c = tid; c < F::R * (F::CB / 8); c += 256) {
    const int k = c / (F::CB / 8), o = (c % (F::CB / 8)) * 8;
    *(half8*)&sT[k * F::LDW + o] = *(const half8*)(a.W + (size_t)(k0 + k) * RV + o0 + o);
  }
  __syncthreads();
  float4v acc[kSmallN / 16];
#pragma unroll
  for (int t = 0; t < kSmallN / 16; ++t) acc[t] = zero4();
  for (int t = 0; t < n_tiles; ++t) {  // uniform
    if (t > 0) load_v(av, t);
    float4v acc_t = zero4();
#pragma unroll
    for (int c = 0; c < F::KCW; ++c) {
      const int kr = (kh * F::KCW + c) * 32 + quad * 8;
      const half_t* bp = &sT[(kr + (col >> 2)) * F::LDW + ot * 16 + 4 * (col & 3)];
      const half4 b0 = lds_read_tr16(bp);
      const half4 b1 = lds_read_tr16(bp + 4 * F::LDW);
      const half8 bq = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
      acc_t = mfma16x16x32(av[c], bq, acc_t);
    }
#pragma unroll
    for (int t2 = 0; t2 < kSmallN / 16; ++t2)
      if (t2 == t) acc[t2] = acc_t;
  }
  // the upper k half's sums join the lower half's through LDS
  if (kh == 1)
#pragma unroll
    for (int t = 0; t < kSmallN / 16; ++t)
      if (t < n_tiles) sRed[ot][t][lane] = acc[t];
  block_sync_lds();
  if (kh == 0) {
#pragma unroll
    for (int t = 0; t < kSmallN / 16; ++t) {
      if (t >= n_tiles) break;
      const float4v sum = acc[t] + sRed[ot][t][lane];
      // D[token 4*quad + r][output 16*ot + col]
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = t * 16 + quad * 4 + r;
        if (n < a.N) st_dev(part + ((size_t)s * a.N + n) * RV + o0 + ot * 16 + col, sum[r]);
      }
    }
  }
  // every partial store of the work group has completed at the device-coherent
  // level before the arrival is counted
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  if (tid == 0) {
    const uint32_t before =
        __hip_atomic_fetch_add(counters + cb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sLast = before == (uint32_t)(F::S - 1);
  }
  __syncthreads();
  if (!sLast) return;
  // ---- the last slice of column block cb: sums, rounding, slots
  for (int u = tid; u < a.N * (F::CB / 2); u += 256) {
    const int n = u / (F::CB / 2), o = o0 + 2 * (u % (F::CB / 2));
    float2 p[F::S];
#pragma unroll
    for (int j = 0; j < F::S; ++j) p[j] = ld_dev2(part + ((size_t)j * a.N + n) * RV + o);
    float x = 0.f, y = 0.f;
#pragma unroll
    for (int j = 0; j < F::S; ++j) {
      x += p[j].x;
      y += p[j].y;
    }
    const int64_t slot = a.slots[n];
    if (slot < 0 || slot / 16 >= a.num_blocks) continue;
    const size_t base = ((size_t)(slot / 16) * RV + o) * 16 + slot % 16;
    store_latent(a, true, base, x);
    store_latent(a, true, base + 16, y);
  }
  if (tid == 0) __hip_atomic_store(counters + cb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Few-token values, second half: the slices' partials summed, rounded and
// written to the tokens' slots.  A work group takes 64 groups of four
// adjacent outputs (16-byte reads, coalesced across threads) and splits the
// NS slices into four runs of NS/4, one per thread group; the runs' sums
// are added through LDS in run order, so the result is deterministic.  All
// of a thread's reads are issued before its sum: one memory round trip.
template <int RV, int NS>
__global__ __launch_bounds__(256) void append_reduce_kernel(AppendArgs a) {
  constexpr int SR = NS < 4 ? NS : 4;  // slice runs (one per 64-thread group in use)
  constexpr int RUN = NS / SR;
  static_assert(NS % SR == 0 && RV % 4 == 0, "slice runs, output quads");
  __shared__ float4v sSum[SR][64];
  const int tid = threadIdx.x, sr = tid / 64, oq = tid % 64;
  const int e4 = blockIdx.x * 64 + oq;  // output quad: token e4 / (RV/4), outputs 4*(e4 % (RV/4)) ..
  const bool live = sr < SR && e4 < a.N * (RV / 4);
  if (live) {
    const float4v* src = (const float4v*)a.part + (size_t)sr * RUN * a.N * (RV / 4) + e4;
    float4v p[RUN];
#pragma unroll
    for (int j = 0; j < RUN; ++j) p[j] = src[(size_t)j * a.N * (RV / 4)];
    float4v sum = zero4();
#pragma unroll
    for (int j = 0; j < RUN; ++j) sum += p[j];
    sSum[sr][oq] = sum;
  }
  __syncthreads();
  if (!live || sr != 0) return;
  float4v sum = sSum[0][oq];
#pragma unroll
  for (int r = 1; r < SR; ++r) sum += sSum[r][oq];
  const int n = e4 / (RV / 4), f = 4 * (e4 % (RV / 4));
  const int64_t slot = a.slots[n];
  if (slot < 0) return;
  const int64_t blk = slot / 16;
  if (blk >= a.num_blocks) return;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    store_latent(a, true, ((size_t)blk * RV + f + i) * 16 + (int)(slot % 16), sum[i]);
}

// ---------------------------------------------------------------------------
// Many tokens (a prefill chunk's append): C = A B with A the token rows (v, or
// one head of k) and B the bases (W, or U_h), as tiles of 128 tokens x 64
// outputs.  Both operand tiles of a TK-wide K step pass through
// double-buffered LDS as they are in memory (16-byte stores, no bank
// conflicts); a wave reads its v_mfma_f32_32x32x16_f16 A operand as 16-byte
// rows and its B operand through the transposing LDS read, and each token
// row and basis row is fetched from memory once per work group.  The global
// loads run RING steps ahead through a ring of registers, since one step's
// products take far less time than a load's round trip.  Eight waves: wave
// w owns tokens 32*(w%4).. and outputs 32*(w/4).. of the tile.
// ---------------------------------------------------------------------------
constexpr int TT_M = 128, TT_N = 64;


template <int H, int D, int RK, int RV, int TK, int RING, int VS = 1>
__global__ __launch_bounds__(512) void append_tiled_kernel(AppendArgs a) {
  static_assert(RV % TT_N == 0 && RK == TT_N && D % TK == 0, "tile shape");
  static_assert(RING >= 1 && RING <= 4, "register ring of 1 to 4 steps");
  typedef float float16v __attribute__((ext_vector_type(16)));
  constexpr int LD = TK + 8;              // halves per LDS row of A
  constexpr int LDB = TT_N + 8;           // halves per LDS row of B ([k][output])
  constexpr int AC = TT_M * TK / 8 / 512;  // 16-byte A chunks per thread per step
  constexpr int BC = TK * TT_N / 8 / 512;  // 16-byte B chunks per thread per step
  static_assert(AC >= 1 && BC >= 1, "at least one chunk per thread");
  __shared__ __attribute__((aligned(16))) half_t sA[2][TT_M][LD];
  __shared__ __attribute__((aligned(16))) half_t sB[2][TK][LDB];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c32 = lane & 31, hf = lane >> 5;
  const int wm = w & 3, wn = w >> 2;

  // job decode: value tiles first, then key tiles (one head each).  Work
  // groups are dealt to the XCDs round-robin, so consecutive value jobs take
  // consecutive token tiles: the VT output tiles of one token tile then sit
  // on one XCD (when the tile count is a multiple of 8) and share its L2
  // copy of those token rows instead of fetching them once per XCD.
  constexpr int VT = RV / TT_N;
  const int tiles_m = (a.N + TT_M - 1) / TT_M;
  // With VS > 1 the value contraction (K = H*d) is split into VS equal parts,
  // one per job (split js after all output tiles of split js-1); each writes
  // fp32 partial products to a.part[js][token][output] and
  // append_reduce_kernel sums the VS parts in split order.  A value job's
  // time is set by its serial K steps (one 128-token tile alone takes about
  // as long as the whole chunk), so splitting K shortens the critical path.
  int job = blockIdx.x;
  bool is_v;
  int mt, nt = 0, h = 0, js = 0;
  if (job < tiles_m * VT * VS) {
    is_v = true;
    mt = job % tiles_m;
    nt = (job / tiles_m) % VT;
    js = job / (tiles_m * VT);
  } else {
    is_v = false;
    job -= tiles_m * VT * VS;
    mt = job / H;
    h = job % H;
  }
  constexpr int HD = H * D;
  constexpr int KS = HD / VS;  // value contraction per split
  static_assert(KS % TK == 0, "whole K steps per split");
  const half_t* A = is_v ? a.v + (size_t)js * KS : a.k + (size_t)h * D;
  const half_t* B = is_v ? a.W + (size_t)js * KS * RV + nt * TT_N : a.U + (size_t)h * D * RK;
  const int ldb = is_v ? RV : RK;
  const int n_steps = (is_v ? KS : D) / TK;
  const int m_base = mt * TT_M;

  // staging roles: A chunk i is row a_row[i], k offset a_k[i]; B chunk j is
  // k row b_k[j], outputs b_o[j] .. +7
  int a_row[AC], a_k[AC], b_k[BC], b_o[BC];
  const half_t* a_src[AC];
  const half_t* b_src[BC];
#pragma unroll
  for (int i = 0; i < AC; ++i) {
    const int c = tid + i * 512;
    a_row[i] = c / (TK / 8);
    a_k[i] = (c % (TK / 8)) * 8;
    a_src[i] = A + (size_t)min(m_base + a_row[i], a.N - 1) * HD + a_k[i];
  }
#pragma unroll
  for (int j = 0; j < BC; ++j) {
    const int c = tid + j * 512;
    b_k[j] = c / (TT_N / 8);
    b_o[j] = (c % (TT_N / 8)) * 8;
    b_src[j] = B + (size_t)b_k[j] * ldb + b_o[j];
  }

  half8 ra[RING][AC], rb[RING][BC];
  auto fetch = [&](auto slot, int step) {
    constexpr int S = decltype(slot)::value;
    const int k0 = step * TK;
#pragma unroll
    for (int i = 0; i < AC; ++i) ra[S][i] = *(const half8*)(a_src[i] + k0);
#pragma unroll
    for (int j = 0; j < BC; ++j) rb[S][j] = *(const half8*)(b_src[j] + (size_t)k0 * ldb);
  };
  auto stage = [&](auto slot, int buf) {
    constexpr int S = decltype(slot)::value;
#pragma unroll
    for (int i = 0; i < AC; ++i) *(half8*)&sA[buf][a_row[i]][a_k[i]] = ra[S][i];
#pragma unroll
    for (int j = 0; j < BC; ++j) *(half8*)&sB[buf][b_k[j]][b_o[j]] = rb[S][j];
  };
  // B fragment of chunk c: lane group g = lane/16 covers outputs
  // 16*(g%2) .. +15 of the wave's 32 and k 8*(g/2) .. +7 of the chunk
  const int grp = lane >> 4, q = lane & 15;
  const int b_row = 8 * (grp >> 1) + (q >> 2);
  const int b_col = wn * 32 + 16 * (grp & 1) + 4 * (q & 3);
  auto compute = [&](float16v& acc, int buf) {
#pragma unroll
    for (int c = 0; c < TK / 16; ++c) {
      const half8 av = *(const half8*)&sA[buf][wm * 32 + c32][c * 16 + 8 * hf];
      const half4 b0 = lds_read_tr16(&sB[buf][c * 16 + b_row][b_col]);
      const half4 b1 = lds_read_tr16(&sB[buf][c * 16 + b_row + 4][b_col]);
      const half8 bv = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, acc, 0, 0, 0);
    }
  };

  float16v acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  // prologue: step 0 staged, steps 1..RING in the ring (slot = step % RING)
  fetch(std::integral_constant<int, 0>{}, 0);
  stage(std::integral_constant<int, 0>{}, 0);
  fetch(std::integral_constant<int, 1 % RING>{}, min(1, n_steps - 1));
  if constexpr (RING > 1) fetch(std::integral_constant<int, 2 % RING>{}, min(2, n_steps - 1));
  if constexpr (RING > 2) fetch(std::integral_constant<int, 3 % RING>{}, min(3, n_steps - 1));
  if constexpr (RING > 3) fetch(std::integral_constant<int, 4 % RING>{}, min(4, n_steps - 1));
  __syncthreads();
  // step s: products of step s from LDS buffer s&1, step s+1 from the ring
  // into the other buffer, step s+1+RING into the freed ring slot.  The last
  // step stages and requests too (a repeat of the last step, into a buffer
  // nothing reads again): with no branch around the requests, each stage
  // waits only for its own step's
  auto iter = [&](auto phase, int s) {
    constexpr int P = decltype(phase)::value;  // (s + 1) % RING
    compute(acc, s & 1);
    stage(std::integral_constant<int, P>{}, (s + 1) & 1);
    fetch(std::integral_constant<int, P>{}, min(s + 1 + RING, n_steps - 1));
    __syncthreads();
  };
  int s = 0;
  for (; s + RING <= n_steps; s += RING) {
    iter(std::integral_constant<int, 1 % RING>{}, s);
    if constexpr (RING > 1) iter(std::integral_constant<int, 2 % RING>{}, s + 1);
    if constexpr (RING > 2) iter(std::integral_constant<int, 3 % RING>{}, s + 2);
    if constexpr (RING > 3) iter(std::integral_constant<int, 4 % RING>{}, s + 3);
  }
  if (s < n_steps) iter(std::integral_constant<int, 1 % RING>{}, s);
  if constexpr (RING > 1)
    if (s + 1 < n_steps) iter(std::integral_constant<int, 2 % RING>{}, s + 1);
  if constexpr (RING > 2)
    if (s + 2 < n_steps) iter(std::integral_constant<int, 3 % RING>{}, s + 2);

  // epilogue: register i holds token 8*(i/4) + 4*hf + i%4, output c32.  The
  // 16 slots are requested together (indices clamped into range): loaded
  // inside the checks below, each would wait for the one before it, 16
  // memory round trips at the end of every work group.
  const int n = wn * 32 + c32;
  if constexpr (VS > 1) {
    if (is_v) {  // partial products: 32 consecutive outputs of a token per store
      float* dst = a.part + (size_t)js * a.N * RV + nt * TT_N + n;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = m_base + wm * 32 + 8 * (i / 4) + 4 * hf + (i % 4);
        if (m < a.N) dst[(size_t)m * RV] = acc[i];
      }
      return;
    }
  }
  int64_t slot_of[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    slot_of[i] = a.slots[min(m_base + wm * 32 + 8 * (i / 4) + 4 * hf + (i % 4), a.N - 1)];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = m_base + wm * 32 + 8 * (i / 4) + 4 * hf + (i % 4);
    if (m >= a.N) continue;
    const int64_t slot = slot_of[i];
    if (slot < 0) continue;
    const int64_t blk = slot / 16;
    const int off = (int)(slot % 16);
    if (blk >= a.num_blocks) continue;
    if (is_v)
      store_latent(a, true, ((size_t)blk * RV + nt * TT_N + n) * 16 + off, acc[i]);
    else
      store_latent(a, false, (((size_t)blk * H + h) * 16 + off) * RK + n, acc[i]);
  }
}

// Splits of the value contraction in the many-token path at the main shape
// (32 key/value heads, d 128, r_k 64, r_v 512).  Alone, a value job's 64
// serial K steps take about 42 us whatever the chunk size, so small chunks
// gain from shorter jobs; from about 3k tokens the chip is busy without the
// split and the partials' round trip costs more than it saves.  Measured:
// 512 tokens 41 -> 17 us (four ways), 2048 tokens 44 -> 35 us (two ways),
// 4096 tokens 49 us unsplit against 60 (two ways).
constexpr int kSplit4MaxTokens = 1792;
constexpr int kSplit2MaxTokens = 2816;
static int tiled_splits(const ShapeKey& s, int n_tokens) {
  if (!(s.H == 32 && s.d == 128 && s.rk == 64 && s.rv == 512) || n_tokens <= kSmallN) return 1;
  return n_tokens <= kSplit4MaxTokens ? 4 : n_tokens <= kSplit2MaxTokens ? 2 : 1;
}

// Key/value views with a few-token instance (launch_few below); other shapes
// take the tiled kernel for any token count and need no workspace.
static bool few_token_instance(const ShapeKey& s) {
  return (s.H == 32 && s.d == 128 && s.rk == 64 && s.rv == 512) ||
         (s.H == 4 && s.d == 64 && s.rk == 16 && s.rv == 64) ||
         (s.H == 8 && s.d == 128 && s.rk == 64 && s.rv == 512) ||
         (s.H == 32 && s.d == 128 && s.rk == 32 && s.rv == 256);
}

// Workspace of an append: none, or the arrival counters (kWorkspaceHeaderBytes,
// zero between calls) followed by the value partials of the few-token path
// or of the split tiled path.
size_t append_workspace_bytes(const ShapeKey& s, int n_tokens) {
  if (n_tokens <= 0) return 0;
  if (n_tokens <= kSmallN) {
    if (!few_token_instance(s)) return 0;
    const int K = s.H * s.d;
    return kWorkspaceHeaderBytes + (size_t)(K / few_slice_rows(K, s.rv)) * n_tokens * s.rv * sizeof(float);
  }
  const int vs = tiled_splits(s, n_tokens);
  return vs > 1 ? kWorkspaceHeaderBytes + (size_t)vs * n_tokens * s.rv * sizeof(float) : 0;
}

template <int H, int D, int RK, int RV>
static void launch_few(const AppendArgs& a, hipStream_t st) {
  using F = FewCfg<H, D, RK, RV>;
  launch_hooked(TIME_APPEND, TIME_NONE, append_few_kernel<H, D, RK, RV>, dim3(F::VJ + H),
                dim3(256), st, a);
}

hipError_t launch_append(const ShapeKey& s, const void* k, const void* v, const void* U,
                         const void* W, const int64_t* slots, int n_tokens, int num_blocks,
                         void* k_cache, void* v_cache, const LatentFormat& fmt, void* workspace,
                         hipStream_t st) {
  if (n_tokens <= 0) return hipSuccess;
  AppendArgs a;
  a.fp8 = fmt.fp8 ? 1 : 0;
  a.k_scale = fmt.k_scale;
  a.v_scale = fmt.v_scale;
  a.k = (const half_t*)k;
  a.v = (const half_t*)v;
  a.U = (const half_t*)U;
  a.W = (const half_t*)W;
  a.slots = slots;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.N = n_tokens;
  a.H = s.H;
  a.D = s.d;
  a.RK = s.rk;
  a.RV = s.rv;
  a.num_blocks = num_blocks;
  a.counters = (uint32_t*)workspace;
  a.part = workspace ? (float*)((char*)workspace + kWorkspaceHeaderBytes) : nullptr;
  a.tiles_m = (n_tokens + AT_M - 1) / AT_M;
  a.v_tiles_n = (s.rv + AT_N - 1) / AT_N;
  a.k_tiles_n = (s.rk + AT_N - 1) / AT_N;
  const long jobs = (long)a.tiles_m * (a.v_tiles_n + (long)s.H * a.k_tiles_n);
  // a single launch: the start event is recorded on the stream just before it
  if (g_timing.which == TIME_APPEND && g_timing.start) hipEventRecord(g_timing.start, st);
  if (n_tokens <= kSmallN && workspace != nullptr) {
    if (s.H == 32 && s.d == 128 && s.rk == 64 && s.rv == 512) {
      launch_few<32, 128, 64, 512>(a, st);
      return hipGetLastError();
    }
    if (s.H == 4 && s.d == 64 && s.rk == 16 && s.rv == 64) {
      launch_few<4, 64, 16, 64>(a, st);
      return hipGetLastError();
    }
    if (s.H == 8 && s.d == 128 && s.rk == 64 && s.rv == 512) {
      launch_few<8, 128, 64, 512>(a, st);
      return hipGetLastError();
    }
    if (s.H == 32 && s.d == 128 && s.rk == 32 && s.rv == 256) {
      launch_few<32, 128, 32, 256>(a, st);
      return hipGetLastError();
    }
  }
  if (s.H == 8 && s.d == 128 && s.rk == 64 && s.rv == 512) {
    const long tiles_m = (n_tokens + TT_M - 1) / TT_M;
    launch_hooked(TIME_APPEND, TIME_NONE, append_tiled_kernel<8, 128, 64, 512, 64, 1>,
                  dim3((unsigned)(tiles_m * (512 / TT_N + 8))), dim3(512), st, a);
    return hipGetLastError();
  }
  if (s.H == 32 && s.d == 128 && s.rk == 64 && s.rv == 512) {
    const long tiles_m = (n_tokens + TT_M - 1) / TT_M;
    const dim3 grid((unsigned)(tiles_m * (512 / TT_N + 32)));
    // value contraction split VS ways, the partials summed by the reduction
    // (the workspace holds exactly the chosen split's partials)
    const int vs = workspace == nullptr ? 1 : tiled_splits(s, n_tokens);
    const dim3 gridv((unsigned)(tiles_m * (vs * 512 / TT_N + 32)));
    const dim3 gridr((unsigned)((a.N * (512 / 4) + 63) / 64));
    if (vs == 4) {
      launch_hooked(TIME_NONE, TIME_NONE, append_tiled_kernel<32, 128, 64, 512, 64, 1, 4>, gridv,
                    dim3(512), st, a);
      launch_hooked(TIME_APPEND, TIME_NONE, append_reduce_kernel<512, 4>, gridr, dim3(256), st, a);
    } else if (vs == 2) {
      launch_hooked(TIME_NONE, TIME_NONE, append_tiled_kernel<32, 128, 64, 512, 64, 1, 2>, gridv,
                    dim3(512), st, a);
      launch_hooked(TIME_APPEND, TIME_NONE, append_reduce_kernel<512, 2>, gridr, dim3(256), st, a);
    } else {
      launch_hooked(TIME_APPEND, TIME_NONE, append_tiled_kernel<32, 128, 64, 512, 64, 1>, grid,
                    dim3(512), st, a);
    }
    return hipGetLastError();
  }
  launch_hooked(TIME_APPEND, TIME_NONE, append_kernel, dim3((unsigned)jobs), dim3(256), st, a);
  return hipGetLastError();
}

}  // namespace starkv
