// Chunked-prefill attention over a paged, low-rank-compressed KV cache
// (Proxima README, "Per-prefill-chunk attention": one chunk of N new tokens
// per request attends to the request's whole cache, causally).
//
// The chunk's keys and values are appended first (append.hip); this kernel
// then attends with the latent shortcut, never rebuilding K or V:
//   S^T[t, j] = c_k[t, h] . q~[j, h]          (q~ pre-scaled by scale*log2 e)
//   P = causal softmax over t <= P0 + j, P0 = seq_len - chunk_len
//   Z^T[f, j] = sum_t c_v[t, f] P[j, t]        (normalised at the end)
// then applies the up-projection out_h = W_h z_h: in the kernel's epilogue
// for the main-shape instances (z staged in LDS, W_h rows through a register
// ring), or, for the other instances, by writing z as fp16 tiled by 32-token
// blocks in the operand order of the many-token up-projection kernel
// (decode.hip), which runs afterwards.  q~ arrives in fp32 and enters the
// score products as an fp16 hi/lo pair (two products per key chunk).
//
// Work group = (request, tile of MQ queries, group of G heads), NW waves;
// the main shape runs G = 2 heads x MQ = 64 queries = 128 (head, query) rows
// with 8 waves, two 16-token pages per step.
//   * scores: a score unit is one (head, 16-query block); per page it is
//     v_mfma_f32_16x16x32_f16 with the 16 x r_k key page as A and the
//     queries' q~ as B (tokens x queries), then the online-softmax update of
//     its 16 queries (lane = query, 4 tokens per page per lane; the max and
//     sum across the four lanes of a query use the cross-row lane swaps).
//     The key pages go through LDS (a three-step ring, each thread copying
//     one 16-byte chunk per step), so each is fetched once per work group
//     rather than once per query block: the per-CU load path, not the
//     matrix cores, is the scarcest resource of this kernel.
//   * values: wave w owns RV/NW features for all rows.  Per page,
//     Z^T[f, row] += c_v[t, f] P[row, t] is v_mfma_f32_32x32x16_f16 with the
//     feature-major value page as A (16 contiguous bytes per lane) and P as B
//     (read from LDS, where it is stored in exactly that operand order); the
//     accumulator column is the row, so rescaling is per lane.
//   * lazy rescaling: a row's reference max only moves when a step's max
//     exceeds it by more than 2^kRaise (log2 domain), so P <= 2^kRaise stays
//     well inside fp16 and the accumulators are rescaled on few steps.  The
//     softmax is invariant to the reference, so this is exact math.
//   * software pipeline: step s runs the scores and softmax of step s+1
//     beside the P.c_v products of step s, with the softmax's vector
//     instructions and the step's loads (keys of step s+3 for the LDS ring,
//     values of step s+2 into a three-step register ring) interleaved
//     between the products; one LDS-only barrier per step.
//   * masks (causal limit, sequence end, invalid block ids) only on the
//     steps that need them.
//   * block ids stream through a 2*kChunk-entry LDS ring, a few new entries
//     per step, so no block-table load sits on the critical path.
//   * work groups of one request are placed on one XCD when the batch is a
//     multiple of 8, so the request's latents are shared through that L2.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace starkv {

// v_mfma_f32_32x32x16_f16: lane l holds A[l%32][8*(l/32) + 0..7] and
// B[8*(l/32) + 0..7][l%32]; the 32x32 fp32 result has
// D[8*(i/4) + 4*(l/32) + i%4][l%32] in register i (i = 0..15).
typedef float float16v __attribute__((ext_vector_type(16)));
__device__ __forceinline__ float16v mfma32x32x16(half8 a, half8 b, float16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

template <int H, int RK, int RV, int G, int MQ, int NW>
struct PrefillCfg {
  static constexpr int R = G * MQ;           // (head, query) rows
  static constexpr int RT = R / 32;          // 32-row tiles
  static constexpr int QB = MQ / 16;         // 16-query blocks per head
  static constexpr int SU = G * QB;          // score units
  static constexpr int SUW = SU / NW;        // score units per wave
  static constexpr int FTW = RV / 32 / NW;   // 32-feature tiles per wave
  static constexpr int KC = (RK % 32 == 0) ? 32 : 16;
  static constexpr int NKC = RK / KC;
  static_assert(R % 32 == 0 && MQ % 16 == 0, "rows must tile by 32, queries by 16");
  static_assert(SU % NW == 0 && SUW >= 1, "score units must spread evenly over the waves");
  static_assert(RV % (32 * NW) == 0 && FTW >= 1, "value rank must split into 32-wide tiles");
  static_assert(H % G == 0, "head groups must tile the heads");
};

struct PrefillArgs {
  const float* qt;  // [total_q, H, RK] fp32, pre-scaled
  const int32_t* qsl;
  const void* k_cache;  // fp16, or FP8 E4M3 codes (same layouts)
  const void* v_cache;
  float v_scale;        // FP8: the value scale, folded into z; else 1
  const int32_t* block_tables;
  const int32_t* seq_lens;
  half_t* z;  // fp16, tiled [H][n_tb][RV/16][64][8], see launch_upproj_tiled
  const half_t* W;  // fused up-projection: the value basis [Hkv*D][RV]
  half_t* out;      // fused up-projection: out [total_q][H][D]
  int max_blocks, num_blocks, batch, n_qtiles, n_groups, n_tb;
};

// Instances whose epilogue applies W_h itself (out = W_h z without z ever
// leaving the chip): two heads of 64 queries, 8 waves, r_v 512, d 128.
template <int G, int MQ, int NW, int RV, int D>
constexpr bool prefill_fused() {
  return G == 2 && MQ == 64 && NW == 8 && RV == 512 && D == 128;
}

constexpr int PBS = 16;                 // tokens per page
constexpr int kChunk = 64;              // block-id ring: 2 * kChunk entries
constexpr float kRaise = 8.f;           // lazy-rescale threshold (log2 units)

// Template parameters chosen per instance:
//   PPS    pages per step: one LDS barrier, one block-id read and one
//          rescale check per PPS pages
//   DEPTH  steps of page operands held in the register ring (2 or 3)
//   SCHED  instruction order inside a step: 1 score products, then the P.c_v
//          products, then the softmax (the tiny shape); 2 as 1 with the
//          softmax's vector instructions interleaved between the products
//          (the lower rank profile); 4 as 2 with the step's loads interleaved
//          between the products too (the main shape)
// FP8 E4M3 codes to fp16 (exact), two codes per instruction.
__device__ __forceinline__ half8 e4m3x8_to_half8(uint32_t w0, uint32_t w1) {
  typedef _Float16 half2v __attribute__((ext_vector_type(2)));
  const half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  const half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  const half2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  const half2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  return half8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <int H, int RK, int RV, int G, int MQ, int NW, int PPS, int DEPTH, int SCHED, bool KLDS,
          int QG, bool FP8, int DH>
__global__ __launch_bounds__(NW * 64) void prefill_attn_kernel(PrefillArgs a) {
  static_assert(DEPTH >= 2 && DEPTH <= 3, "register ring of 2 or 3 steps");
  static_assert(PPS == 1 || PPS == 2, "one or two pages per step");
  static_assert(H % QG == 0, "query heads per key/value head");
  static_assert(!FP8 || KLDS, "FP8 keys go through the LDS key ring");
  // cache elements: fp16, or FP8 codes turned into fp16 where they are used
  // (keys as they enter the LDS ring, values before their products)
  using LT = std::conditional_t<FP8, uint8_t, half_t>;
  const LT* k_cache = (const LT*)a.k_cache;
  const LT* v_cache = (const LT*)a.v_cache;
  using C = PrefillCfg<H, RK, RV, G, MQ, NW>;
  constexpr int HKV = H / QG;  // key/value heads of a key page (query head h reads h / QG)
  typedef _Float16 kvec __attribute__((ext_vector_type(C::KC / 4)));
  constexpr int RING = 2 * kChunk;
  constexpr int TPS = PPS * PBS;  // tokens per step
  // P in the B-operand order of the 32x32x16 product:
  // [buffer][page of the step][row tile][(row % 32) / 16][token half][row % 16][8 tokens].
  // The softmax's half-waves (token halves 0 and 1 of 16 rows) then write
  // adjacent 256-byte ranges, which the LDS takes without bank conflicts
  // (with the halves 512 bytes apart a write took 1.4x as long); a
  // fragment read stays four contiguous 256-byte ranges.
  __shared__ __attribute__((aligned(16))) half_t sP[2][PPS][C::RT][2][2][16][8];
  // rescale factor of row rt*32 + r at sAlpha[buffer][r][rt]
  __shared__ __attribute__((aligned(16))) float sAlpha[2][32][C::RT];
  __shared__ float sL[C::R];
  __shared__ __attribute__((aligned(16))) int sBlk[RING];
  // KLDS: key pages of three steps, [step % 3][head][page][token][r_k + pad],
  // each loaded once per work group and shared by the head's score waves
  // (under grouped-query attention each query head's slot holds its key/value
  // head's page).  The pad of 16 elements (a 160-byte row at r_k 64) makes
  // the score products' reads (16 rows x four 16-byte chunks per wave)
  // conflict-free on the gfx950 LDS; a 144-byte row took twice as long.
  constexpr int LDKV = RK + 16;
  __shared__ __attribute__((aligned(16))) half_t sK[KLDS ? 3 : 1][G][PPS][PBS][LDKV];

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
  if (j0 >= Cn) return;  // whole work group, before any barrier
  const int L = a.seq_lens[b];
  const int P0 = L - Cn;
  const int last_key = min(L - 1, P0 + min(j0 + MQ, Cn) - 1);
  const int n_pages = min(last_key / PBS + 1, a.max_blocks);
  const int n_steps = (n_pages + PPS - 1) / PPS;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, quad = lane >> 4;   // 16x16 layouts
  const int c32 = lane & 31, hf = lane >> 5;     // 32x32 layouts
  const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks;

  // block id of a page as stored in the table (pages past the tile's range
  // repeat its last page); the range check is made where an id is read back
  // from the ring, on the scalar unit
  auto fetch_block = [&](int page) { return bt[min(page, n_pages - 1)]; };
  if (tid < RING) sBlk[tid] = fetch_block(tid);

  // ---- this wave's score units: (head, 16 queries); lane column = query
  int su_h[C::SUW], su_row[C::SUW], su_lim[C::SUW];
  // q~ as an fp16 hi/lo pair (hi + lo = q~ to about 2^-22 of its size): the
  // score products take both, so a score keeps fp32 accuracy in q~
  kvec qv[C::SUW][C::NKC], ql[C::SUW][C::NKC];
#pragma unroll
  for (int i = 0; i < C::SUW; ++i) {
    const int unit = w * C::SUW + i;
    const int hl = unit / C::QB, qb = unit % C::QB;
    const int jq = min(j0 + qb * 16 + col, Cn - 1);  // rows past the chunk mirror its last query
    su_h[i] = g * G + hl;
    su_row[i] = hl * MQ + qb * 16 + col;
    su_lim[i] = min(L - 1, P0 + jq);                 // last visible key
    const float* qp = a.qt + ((size_t)(q_begin + jq) * H + su_h[i]) * RK + quad * (C::KC / 4);
#pragma unroll
    for (int c = 0; c < C::NKC; ++c)
#pragma unroll
      for (int e4 = 0; e4 < C::KC / 16; ++e4) {
        const float4v x = *(const float4v*)(qp + c * C::KC + 4 * e4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const half_t hi = (half_t)x[e];
          qv[i][c][4 * e4 + e] = hi;
          ql[i][c][4 * e4 + e] = (half_t)(x[e] - (float)hi);
        }
      }
  }
  float m_run[C::SUW], l_run[C::SUW];
#pragma unroll
  for (int i = 0; i < C::SUW; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.f;
  }
  const int lim_min = min(L - 1, P0 + j0);  // last key the tile's first query sees

  float16v acc[C::RT][C::FTW];
#pragma unroll
  for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
    for (int ft = 0; ft < C::FTW; ++ft)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[rt][ft][e] = 0.f;

  typedef kvec KSet[PPS][C::SUW][C::NKC];
  typedef half8 VSet[PPS][C::FTW];
  typedef uint8_t v8x8 __attribute__((ext_vector_type(8)));
  typedef std::conditional_t<FP8, v8x8, half8> VElem;  // one value operand as loaded
  typedef VElem VRaw[PPS][C::FTW];
  KSet kr[KLDS ? 1 : DEPTH];  // ring of page operands in registers
  VRaw vr[DEPTH];
  // value operands of a step as fp16
  auto to_vset = [&](VSet& dst, const VRaw& src) {
#pragma unroll
    for (int pg = 0; pg < PPS; ++pg)
#pragma unroll
      for (int ft = 0; ft < C::FTW; ++ft) {
        if constexpr (FP8) {
          typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
          const u32x2 w = __builtin_bit_cast(u32x2, src[pg][ft]);
          dst[pg][ft] = e4m3x8_to_half8(w[0], w[1]);
        } else {
          dst[pg][ft] = src[pg][ft];
        }
      }
  };
  const int f_base = w * C::FTW * 32 + c32;  // feature of this lane in tile 0
  // per-lane element offsets inside one page (the page base is uniform, so
  // the loads take a scalar base plus a 32-bit vector offset)
  int k_off[C::SUW];
#pragma unroll
  for (int i = 0; i < C::SUW; ++i) k_off[i] = ((su_h[i] / QG) * PBS + col) * RK + quad * (C::KC / 4);
  const int v_off = f_base * PBS + hf * 8;

  // block id of a page, read back from the ring; ids outside the cache read
  // as -1 (uniform, so the check runs on the scalar unit)
  auto block_of = [&](int page) {
    const int v = __builtin_amdgcn_readfirstlane(sBlk[page & (RING - 1)]);
    return ((unsigned)v < (unsigned)a.num_blocks) ? v : -1;
  };
  // block ids of the PPS pages of a step, read together (one LDS round trip)
  typedef int StepIds[PPS];
  auto ids_of = [&](StepIds& ids, int step) {
#pragma unroll
    for (int pg = 0; pg < PPS; ++pg) ids[pg] = block_of(step * PPS + pg);
  };
  auto load_k = [&](KSet& dst, const StepIds& ids) {
#pragma unroll
    for (int pg = 0; pg < PPS; ++pg) {
      const int blk = ids[pg];
      const half_t* kp = (const half_t*)a.k_cache + (size_t)(blk < 0 ? 0 : blk) * (HKV * PBS * RK);
#pragma unroll
      for (int i = 0; i < C::SUW; ++i)
#pragma unroll
        for (int c = 0; c < C::NKC; ++c) dst[pg][i][c] = *(const kvec*)(kp + k_off[i] + c * C::KC);
    }
  };
  // value pages: a uniform page base plus this lane's fixed 32-bit byte
  // offset (the scalar-base addressing form, no per-lane 64-bit arithmetic)
  const uint32_t v_off_b = (uint32_t)v_off * (uint32_t)sizeof(LT);
  auto load_v = [&](VRaw& dst, const StepIds& ids) {
#pragma unroll
    for (int pg = 0; pg < PPS; ++pg) {
      const int blk = ids[pg];
      const char* vp = (const char*)v_cache + (size_t)(blk < 0 ? 0 : blk) * (RV * PBS * sizeof(LT));
#pragma unroll
      for (int ft = 0; ft < C::FTW; ++ft)
        dst[pg][ft] = *(const VElem*)(vp + v_off_b + ft * 32 * PBS * sizeof(LT));
    }
  };

  // KLDS staging: thread t copies 16-byte chunks c = t + j*NW*64 of the
  // step's key pages, ordered [head][page][token][r_k / 8].  When the chunks
  // of one (head, page) fill whole waves, every wave's chunks share their
  // head and page: the page base is then uniform and each lane adds a fixed
  // offset.
  constexpr int KCH = G * PPS * PBS * RK / 8 / (NW * 64);  // chunks per thread
  static_assert(!KLDS || (KCH >= 1 && KCH * NW * 64 * 8 == G * PPS * PBS * RK), "key chunks");
  constexpr int CPP = PBS * RK / 8;  // chunks per (head, page)
  constexpr bool KUNI = (CPP % 64) == 0;
  const int w_u = __builtin_amdgcn_readfirstlane(w);
  typedef std::conditional_t<FP8, v8x8, half8> KElem;  // 8 key values as loaded
  KElem kst[KLDS ? KCH : 1];
  auto kst_load = [&](const StepIds& ids) {
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      if constexpr (KUNI) {
        const int cw = (w_u + j * NW) * 64;  // the wave's first chunk
        const int pg = (cw / CPP) % PPS, hl = cw / (CPP * PPS);
        const int blk = ids[pg] < 0 ? 0 : ids[pg];
        const char* kp = (const char*)k_cache +
                         (((size_t)blk * HKV + (g * G + hl) / QG) * PBS * RK) * sizeof(LT);
        kst[j] = *(const KElem*)(kp + (uint32_t)((cw % CPP + lane) * 8 * sizeof(LT)));
      } else {
        const int c = tid + j * NW * 64;
        const int rc = c % (RK / 8), tok = (c / (RK / 8)) % PBS;
        const int pg = (c / (RK / 8 * PBS)) % PPS, hl = c / (RK / 8 * PBS * PPS);
        const int blk = ids[pg] < 0 ? 0 : ids[pg];
        kst[j] = *(const KElem*)(k_cache +
                                 (((size_t)blk * HKV + (g * G + hl) / QG) * PBS + tok) * RK + rc * 8);
      }
    }
  };
  auto kst_store = [&](int kb) {
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int c = tid + j * NW * 64;
      const int rc = c % (RK / 8), tok = (c / (RK / 8)) % PBS;
      const int pg = (c / (RK / 8 * PBS)) % PPS, hl = c / (RK / 8 * PBS * PPS);
      if constexpr (FP8) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 wk = __builtin_bit_cast(u32x2, kst[j]);
        *(half8*)&sK[kb][hl][pg][tok][rc * 8] = e4m3x8_to_half8(wk[0], wk[1]);
      } else {
        *(half8*)&sK[kb][hl][pg][tok][rc * 8] = kst[j];
      }
    }
  };
  // score products of the step whose keys are in LDS buffer kb
  auto score_products_lds = [&](int kb, float4v (&sacc)[PPS][C::SUW]) {
#pragma unroll
    for (int pg = 0; pg < PPS; ++pg)
#pragma unroll
      for (int i = 0; i < C::SUW; ++i) {
        const int hl = su_h[i] - g * G;
        sacc[pg][i] = zero4();
#pragma unroll
        for (int c = 0; c < C::NKC; ++c) {
          const kvec kk = *(const kvec*)&sK[kb][hl][pg][col][c * C::KC + quad * (C::KC / 4)];
          if constexpr (C::KC == 32) {
            sacc[pg][i] = mfma16x16x32(kk, qv[i][c], sacc[pg][i]);
            sacc[pg][i] = mfma16x16x32(kk, ql[i][c], sacc[pg][i]);
          } else {
            sacc[pg][i] = mfma16x16x16(kk, qv[i][c], sacc[pg][i]);
            sacc[pg][i] = mfma16x16x16(kk, ql[i][c], sacc[pg][i]);
          }
        }
      }
  };

  auto score_products = [&](const KSet& kk, float4v (&sacc)[PPS][C::SUW]) {
#pragma unroll
    for (int pg = 0; pg < PPS; ++pg)
#pragma unroll
      for (int i = 0; i < C::SUW; ++i) {
        sacc[pg][i] = zero4();
#pragma unroll
        for (int c = 0; c < C::NKC; ++c) {
          if constexpr (C::KC == 32) {
            sacc[pg][i] = mfma16x16x32(kk[pg][i][c], qv[i][c], sacc[pg][i]);
            sacc[pg][i] = mfma16x16x32(kk[pg][i][c], ql[i][c], sacc[pg][i]);
          } else {
            sacc[pg][i] = mfma16x16x16(kk[pg][i][c], qv[i][c], sacc[pg][i]);
            sacc[pg][i] = mfma16x16x16(kk[pg][i][c], ql[i][c], sacc[pg][i]);
          }
        }
      }
  };
  // online softmax of step s's tokens; P and the rescale factors go to LDS
  // buffer `buf`.  A row's reference max moves only when the step's max
  // exceeds it by more than kRaise.  MASKED: some token of the step may be
  // invisible to some row of the tile, or a page of the step may have an
  // invalid block id (blk_ok false); the masks are then applied with
  // selects.  Each lane keeps its own part of the row sum (its tokens' P,
  // as rounded to fp16 for the products, summed in fp32 by v_dot2): the four
  // quads of a row share the reference max and the rescale factor, so their
  // parts are added once, after the last step.
  auto softmax = [&](auto masked, const bool (&blk_ok)[PPS], const float4v (&sacc)[PPS][C::SUW],
                     int s, int buf) {
    constexpr bool MASKED = decltype(masked)::value;
    typedef _Float16 half2v __attribute__((ext_vector_type(2)));
    const half2v ones = {(half_t)1.f, (half_t)1.f};
#pragma unroll
    for (int i = 0; i < C::SUW; ++i) {
      float sv[PPS][4];
#pragma unroll
      for (int pg = 0; pg < PPS; ++pg)
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[pg][e] = sacc[pg][i][e];
      if constexpr (MASKED) {
#pragma unroll
        for (int pg = 0; pg < PPS; ++pg) {
          const int page = s * PPS + pg;
          const int d = (blk_ok[pg] ? su_lim[i] : -1) - (page * PBS + quad * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[pg][e] = (e <= d) ? sv[pg][e] : -INFINITY;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int pg = 0; pg < PPS; ++pg)
        mx = fmax_nn(mx, fmax_nn(fmax_nn(sv[pg][0], sv[pg][1]), fmax_nn(sv[pg][2], sv[pg][3])));
      const float pm = quad_max(mx);
      const bool raise = pm > m_run[i] + kRaise;  // false while pm is -inf
      const float m_use = raise ? pm : m_run[i];
      const float alpha = raise ? __builtin_amdgcn_exp2f(m_run[i] - pm) : 1.f;  // 0 on the first raise
      // m_use is -inf only while no key has been visible (every sv is then
      // -inf), which a step without masks never sees
      const float m_sub = (MASKED && m_use == -INFINITY) ? 0.f : m_use;
      float ps = l_run[i] * alpha;
      const int row = su_row[i];
#pragma unroll
      for (int pg = 0; pg < PPS; ++pg) {
        half4 ph;
#pragma unroll
        for (int e = 0; e < 4; ++e) ph[e] = (half_t)__builtin_amdgcn_exp2f(sv[pg][e] - m_sub);  // exp2(-inf) = 0
        ps = __builtin_amdgcn_fdot2(half2v{ph[0], ph[1]}, ones, ps, false);
        ps = __builtin_amdgcn_fdot2(half2v{ph[2], ph[3]}, ones, ps, false);
        *(half4*)&sP[buf][pg][row >> 5][(row >> 4) & 1][quad >> 1][row & 15][(quad & 1) * 4] = ph;
      }
      l_run[i] = ps;
      m_run[i] = m_use;
      sAlpha[buf][row & 31][row >> 5] = alpha;  // the four quads agree
    }
  };
  // rescale before step s's products when any row's reference moved
  auto rescale = [&](int buf) {
    float al[C::RT];
    float amin = 1.f;
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt) {
      al[rt] = sAlpha[buf][c32][rt];
      amin = fminf(amin, al[rt]);  // factors are 1 (unchanged) or below 1
    }
    if (__builtin_amdgcn_ballot_w64(amin < 1.f) != 0) {  // uniform
#pragma unroll
      for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
        for (int ft = 0; ft < C::FTW; ++ft) acc[rt][ft] *= al[rt];
    }
  };
  // P.c_v of step s (values in vv, P in LDS buffer `buf`)
  // zero the value columns of tokens past the sequence (they may hold
  // anything, NaN included) and of pages with an invalid block id
  auto mask_values = [&](VSet& vv, const StepIds& ids, int s) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int pg = 0; pg < PPS; ++pg) {
      const int page = s * PPS + pg;
      const int nv = (ids[pg] >= 0) ? min(max(L - (page * PBS + hf * 8), 0), 8) : 0;
#pragma unroll
      for (int ft = 0; ft < C::FTW; ++ft) {
        u4 bits = __builtin_bit_cast(u4, vv[pg][ft]);
#pragma unroll
        for (int d = 0; d < 4; ++d)
          bits[d] &= (2 * d + 1 < nv) ? 0xFFFFFFFFu : ((2 * d < nv) ? 0x0000FFFFu : 0u);
        vv[pg][ft] = __builtin_bit_cast(half8, bits);
      }
    }
  };
  auto value_products = [&](bool mask, VSet& vv, const StepIds& ids, int s, int buf) {
    if (mask) mask_values(vv, ids, s);  // uniform
#pragma unroll
    for (int pg = 0; pg < PPS; ++pg) {
      // all row tiles' P fragments of the page are requested before its
      // first product, so the page waits for LDS once
      half8 pb[C::RT];
#pragma unroll
      for (int rt = 0; rt < C::RT; ++rt) pb[rt] = *(const half8*)&sP[buf][pg][rt][c32 >> 4][hf][c32 & 15][0];
      if constexpr (SCHED != 2) __builtin_amdgcn_sched_barrier(0);  // keep the reads together
#pragma unroll
      for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
        for (int ft = 0; ft < C::FTW; ++ft) acc[rt][ft] = mfma32x32x16(vv[pg][ft], pb[rt], acc[rt][ft]);
    }
  };
  // ---- prologue: block ids staged, keys of steps 0..DEPTH-1 and values of
  // steps 0..DEPTH-2 in flight, step 0 scored
  block_sync_lds();
  if constexpr (KLDS) {
    // keys of steps 0 and 1 into LDS buffers 0 and 1, step 2's in flight
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      StepIds ids;
      ids_of(ids, j);
      kst_load(ids);
      kst_store(j);
    }
    StepIds ids2;
    ids_of(ids2, 2);
    kst_load(ids2);
#pragma unroll
    for (int j = 0; j + 1 < DEPTH; ++j) {
      StepIds ids;
      ids_of(ids, j);
      load_v(vr[j], ids);
    }
    block_sync_lds();
  } else {
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
      StepIds ids;
      ids_of(ids, j);
      load_k(kr[j], ids);
      if (j + 1 < DEPTH) load_v(vr[j], ids);
    }
  }
  {
    float4v sacc[PPS][C::SUW];
    if constexpr (KLDS)
      score_products_lds(0, sacc);
    else
      score_products(kr[0], sacc);
    StepIds ids0;
    ids_of(ids0, 0);
    bool ok0[PPS];
#pragma unroll
    for (int pg = 0; pg < PPS; ++pg) ok0[pg] = ids0[pg] >= 0;
    softmax(std::true_type{}, ok0, sacc, 0, 0);
  }
  // nothing of the prologue stays in flight into the loop, so the loop's
  // wait counts depend on its own loads only
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  block_sync_lds();

  // step s (register-ring phase PH = s % DEPTH): loads for the keys of step
  // s+KA and the values of step s+DEPTH-1, scores of step s+1, products of
  // step s.  P and the rescale factors alternate between two LDS buffers.
  // win[k] holds the block ids of step s+k (k = 0..KA), carried from step to
  // step so that each step reads only one new step's ids from the ring.
  // MASKED: the step needs masks (a token of step s+1 beyond some row's
  // causal limit or past the sequence, or an invalid block id in step s or
  // s+1); most steps need none and skip the selects.
  constexpr int KA = KLDS ? 3 : DEPTH;  // furthest step whose keys a step loads
  auto step = [&](auto phase, auto masked, int s, const StepIds (&win)[KA + 1]) {
    constexpr int PH = decltype(phase)::value;
    constexpr bool MASKED = decltype(masked)::value;
    int staged[PPS];
    const StepIds& id_c = win[0];
    const StepIds& id_s = win[1];
    const StepIds& id_v = win[DEPTH - 1];
    const StepIds& id_k = win[KA];
    // loads for the keys of step s+KA and the values of step s+DEPTH-1
    // (their ring slots were consumed last step)
    auto issue_loads = [&]() {
#pragma unroll
      for (int pg = 0; pg < PPS; ++pg) staged[pg] = fetch_block((s - 1) * PPS + pg + RING);
      if constexpr (KLDS) {
        kst_store((s + 2) % 3);  // keys of step s+2 (loaded last step) into LDS
        kst_load(id_k);          // keys of step s+3
      } else {
        load_k(kr[PH], id_k);
      }
      load_v(vr[(PH + DEPTH - 1) % DEPTH], id_v);
    };
    static_assert(SCHED == 1 || SCHED == 2 || SCHED == 4, "instruction orders 1, 2 and 4");
    if constexpr (SCHED != 4) issue_loads();
    float4v sacc[PPS][C::SUW];
    // a wave in its score products gets issue priority over the CU's waves in
    // their value products or softmax, so the step's score chain is not the
    // last thing to finish before the barrier
    __builtin_amdgcn_s_setprio(1);
    if constexpr (KLDS)
      score_products_lds((s + 1) % 3, sacc);
    else
      score_products(kr[(PH + 1) % DEPTH], sacc);
    __builtin_amdgcn_s_setprio(0);
    const int buf = s & 1;
    rescale(buf);
    __builtin_amdgcn_sched_barrier(0);
    VSet vcur;
    to_vset(vcur, vr[PH]);
    if constexpr (SCHED == 4) {  // masks ahead of the interleaved region
      if constexpr (MASKED) mask_values(vcur, id_c, s);
      value_products(false, vcur, id_c, s, buf);
      issue_loads();
    } else if constexpr (SCHED == 2) {  // masks ahead of the interleaved region
      if constexpr (MASKED) mask_values(vcur, id_c, s);
      value_products(false, vcur, id_c, s, buf);
    } else {
      value_products(MASKED, vcur, id_c, s, buf);
    }
    if constexpr (SCHED == 1) __builtin_amdgcn_sched_barrier(0);
    bool ok_s[PPS];
#pragma unroll
    for (int pg = 0; pg < PPS; ++pg) ok_s[pg] = id_s[pg] >= 0;
    softmax(masked, ok_s, sacc, s + 1, buf ^ 1);
    if constexpr (SCHED == 4) {
      // one P.c_v product, a few vector instructions and, every other
      // product, one of the step's loads: the loads drain through the
      // per-CU load path while the matrix cores run instead of stalling the
      // wave at the start of the step
#pragma unroll
      for (int i = 0; i < PPS * C::RT * C::FTW; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);                   // VALU
        if (i % 2 == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (SCHED == 2) {
      // one P.c_v product, then a few vector instructions, repeated, so the
      // softmax runs in the shadow of the products
#pragma unroll
      for (int i = 0; i < PPS * C::RT * C::FTW; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // pages of step s-1 (+RING) into their slots, which no wave reads any more
    if (tid == 0) {
#pragma unroll
      for (int pg = 0; pg < PPS; ++pg) sBlk[((s - 1) * PPS + pg) & (RING - 1)] = staged[pg];
    }
    block_sync_lds();
  };
  // one step, then the id window moves on
  StepIds win[KA + 1];
#pragma unroll
  for (int k = 0; k <= KA; ++k) ids_of(win[k], k);
  auto run_step = [&](auto phase, auto masked, int s) {
    StepIds next;
    ids_of(next, s + KA + 1);
    step(phase, masked, s, win);
#pragma unroll
    for (int k = 0; k < KA; ++k)
#pragma unroll
      for (int pg = 0; pg < PPS; ++pg) win[k][pg] = win[k + 1][pg];
#pragma unroll
    for (int pg = 0; pg < PPS; ++pg) win[KA][pg] = next[pg];
  };
  // DEPTH steps per loop trip (a single path through its body, so the wait
  // counts at its head see only the previous trip's loads).  Trips whose
  // steps need no masks run first: every token up to step s+DEPTH visible to
  // every row of the tile, and the ids in the window (steps s..s+KA, which
  // cover the steps that the trip's steps read) valid.  The rest of the
  // steps, from the first that may need a mask, run with masks.
  auto trip_plain = [&](int s) {
    bool ok = (s + DEPTH + 1) * TPS - 1 <= lim_min;
#pragma unroll
    for (int k = 0; k <= KA; ++k)
#pragma unroll
      for (int pg = 0; pg < PPS; ++pg) ok = ok && win[k][pg] >= 0;
    return ok;
  };
  static_assert(KA >= DEPTH, "the window covers the scores of a trip's last step");
  int s = 0;
  for (; s + DEPTH <= n_steps && trip_plain(s); s += DEPTH) {
    run_step(std::integral_constant<int, 0>{}, std::false_type{}, s);
    run_step(std::integral_constant<int, 1>{}, std::false_type{}, s + 1);
    if constexpr (DEPTH > 2) run_step(std::integral_constant<int, 2 % DEPTH>{}, std::false_type{}, s + 2);
  }
  for (; s + DEPTH <= n_steps; s += DEPTH) {
    run_step(std::integral_constant<int, 0>{}, std::true_type{}, s);
    run_step(std::integral_constant<int, 1>{}, std::true_type{}, s + 1);
    if constexpr (DEPTH > 2) run_step(std::integral_constant<int, 2 % DEPTH>{}, std::true_type{}, s + 2);
  }
  if (s < n_steps) run_step(std::integral_constant<int, 0>{}, std::true_type{}, s);
  if constexpr (DEPTH > 2)
    if (s + 1 < n_steps) run_step(std::integral_constant<int, 1>{}, std::true_type{}, s + 1);

  // ---- normalise: every row's softmax sum
#pragma unroll
  for (int i = 0; i < C::SUW; ++i) {
    const float l = quad_sum(l_run[i]);  // the four quads' parts
    sL[su_row[i]] = l;                    // the four quads agree
  }
  block_sync_lds();
  if constexpr (prefill_fused<G, MQ, NW, RV, DH>()) {
    // ---- out = W_h z in the epilogue.  z (this tile's 128 rows x r_v,
    // normalised, fp16) is staged in LDS one half of the features at a time
    // by the waves that hold it; wave w then accumulates out rows of head
    // w / 4 (64 queries) x 32 of d (block w % 4) with v_mfma_f32_32x32x16_f16:
    // A = z rows from LDS, B = 8 consecutive features of one row of W_h
    // straight from memory (a 16-entry register ring runs over both halves,
    // so the second half's loads go out during the first half's products).
    constexpr int FH = RV / 2;             // features per half
    constexpr int LDZ = FH + 72;           // 656-byte rows: conflict-free 16-byte reads of 32 rows
    constexpr int WPH = NW / G;            // waves per head
    constexpr int KH = FH / 16;            // 16-feature chunks per half
    static_assert(DH / WPH == 32 && MQ % 32 == 0 && KH == 16, "fused up-projection tile");
    __shared__ __attribute__((aligned(16))) half_t sZ[C::R][LDZ];
    const int hl = w_u / WPH, db = w_u % WPH;
    const int r_h = g * G + hl;
    // row d = 32 db + c32 of W_h (its key/value head), features from 8 hf
    const half_t* Wd = a.W + ((size_t)(r_h / QG) * DH + db * 32 + c32) * RV + 8 * hf;
    constexpr int WRING = 8;  // W operands in flight
    half8 wr[WRING];
#pragma unroll
    for (int kc = 0; kc < WRING; ++kc) wr[kc] = *(const half8*)(Wd + kc * 16);
    float inv[C::RT];
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt) {
      const float lr = sL[rt * 32 + c32];
      inv[rt] = lr > 0.f ? a.v_scale / lr : 0.f;
    }
    float16v oacc[MQ / 32];
#pragma unroll
    for (int mt = 0; mt < MQ / 32; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[mt][e] = 0.f;
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      if ((w_u * C::FTW * 32) / FH == ps) {  // uniform: the waves holding this half
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
          for (int ft = 0; ft < C::FTW; ++ft)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              // features w*64 + 32 ft + 8 jj + 4 hf + 0..3 of row 32 rt + c32
              const int f = w_u * C::FTW * 32 + ft * 32 + 8 * jj + 4 * hf - ps * FH;
              half4 o;
#pragma unroll
              for (int r = 0; r < 4; ++r) o[r] = (half_t)(acc[rt][ft][4 * jj + r] * inv[rt]);
              *(half4*)&sZ[rt * 32 + c32][f] = o;
            }
      }
      block_sync_lds();
#pragma unroll
      for (int kc = 0; kc < KH; ++kc) {
        const int k = ps * KH + kc;  // chunk over both halves
        const half8 b = wr[k % WRING];
        if (k + WRING < 2 * KH) wr[k % WRING] = *(const half8*)(Wd + (k + WRING) * 16);
#pragma unroll
        for (int mt = 0; mt < MQ / 32; ++mt) {
          const half8 av = *(const half8*)&sZ[hl * MQ + mt * 32 + c32][kc * 16 + 8 * hf];
          oacc[mt] = mfma32x32x16(av, b, oacc[mt]);
        }
      }
      if (ps == 0) block_sync_lds();  // the second half overwrites sZ
    }
    // register i of tile mt: row 8 (i/4) + 4 hf + i%4 of the tile, column d = 32 db + c32
#pragma unroll
    for (int mt = 0; mt < MQ / 32; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r_j = j0 + mt * 32 + 8 * (i / 4) + 4 * hf + (i % 4);
        if (r_j < Cn)
          a.out[((size_t)(q_begin + r_j) * H + r_h) * DH + db * 32 + c32] = (half_t)oacc[mt][i];
      }
    return;
  }
  // ---- otherwise write z rows of this tile for the up-projection kernel
#pragma unroll
  for (int rt = 0; rt < C::RT; ++rt) {
    const int row = rt * 32 + c32;
    const int r_h = g * G + row / MQ;
    const int r_j = j0 + row % MQ;
    if (r_j >= Cn) continue;
    const float lr = sL[row];
    const float inv = lr > 0.f ? a.v_scale / lr : 0.f;
    // z tiled for the up-projection: [head][token / 32][feature / 16][lane][8]
    // with lane = token % 32 + 32 * ((feature / 8) % 2)
    const int tok = q_begin + r_j;
    half_t* zb = a.z + ((size_t)r_h * a.n_tb + tok / 32) * (RV / 16) * 512;
#pragma unroll
    for (int ft = 0; ft < C::FTW; ++ft)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        // features f_base - c32 + 32*ft + 8*jj + 4*hf + 0..3
        const int f0 = f_base - c32 + ft * 32 + 8 * jj;
        half4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = (half_t)(acc[rt][ft][4 * jj + r] * inv);
        *(half4*)(zb + (f0 / 16) * 512 + (tok % 32 + 32 * ((f0 / 8) % 2)) * 8 + 4 * hf) = o;
      }
  }
}

template <int H, int D, int RK, int RV, int G, int MQ, int NW, int PPS, int DEPTH, int SCHED,
          bool KLDS = false, int QG = 1, bool FP8 = false>
static hipError_t prefill_instance(const void* qt, const int32_t* qsl, int max_query_len,
                                   const void* k_cache, const void* v_cache, const void* W,
                                   const int32_t* block_tables, int max_blocks,
                                   const int32_t* seq_lens, int num_blocks, int batch,
                                   int total_q, void* z, void* out, float v_scale,
                                   hipStream_t st) {
  PrefillArgs a;
  a.qt = (const float*)qt;
  a.qsl = qsl;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.v_scale = v_scale;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.z = (half_t*)z;
  a.W = (const half_t*)W;
  a.out = (half_t*)out;
  a.max_blocks = max_blocks;
  a.num_blocks = num_blocks;
  a.batch = batch;
  a.n_qtiles = (max_query_len + MQ - 1) / MQ;
  a.n_groups = H / G;
  a.n_tb = (total_q + 31) / 32;
  const long wgs = (long)batch * a.n_qtiles * a.n_groups;
  launch_hooked(TIME_PREFILL_ATTN, TIME_NONE,
                prefill_attn_kernel<H, RK, RV, G, MQ, NW, PPS, DEPTH, SCHED, KLDS, QG, FP8, D>,
                dim3((unsigned)wgs), dim3(NW * 64), st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (prefill_fused<G, MQ, NW, RV, D>()) return hipSuccess;  // out written by the kernel
  return launch_upproj_tiled(ShapeKey{H, D, RK, RV, H / QG}, W, z, total_q, out, st);
}

hipError_t launch_prefill(const ShapeKey& s, const void* qt, const int32_t* qsl, int total_q,
                          int max_query_len, const void* k_cache, const void* v_cache,
                          const void* W, const int32_t* block_tables, int max_blocks,
                          const int32_t* seq_lens, int num_blocks, int batch, void* z, void* out,
                          const LatentFormat& fmt, hipStream_t st) {
  if (batch <= 0 || total_q <= 0) return hipSuccess;
#define STARKV_PREFILL_ARGS                                                                    \
  qt, qsl, max_query_len, k_cache, v_cache, W, block_tables, max_blocks, seq_lens, num_blocks, \
      batch, total_q, z, out, fmt.fp8 ? fmt.v_scale : 1.f, st
  if (fmt.fp8) {  // FP8 latents: the main shape (either head layout) and the tiny one
    if (s.H == 32 && s.Hkv == 32 && s.d == 128 && s.rk == 64 && s.rv == 512)
      return prefill_instance<32, 128, 64, 512, 2, 64, 8, 2, 3, 4, true, 1, true>(STARKV_PREFILL_ARGS);
    if (s.H == 32 && s.Hkv == 8 && s.d == 128 && s.rk == 64 && s.rv == 512)
      return prefill_instance<32, 128, 64, 512, 2, 64, 8, 2, 3, 4, true, 4, true>(STARKV_PREFILL_ARGS);
    if (s.H == 4 && s.Hkv == 4 && s.d == 64 && s.rk == 16 && s.rv == 64)
      return prefill_instance<4, 64, 16, 64, 4, 16, 2, 2, 2, 1, true, 1, true>(STARKV_PREFILL_ARGS);
    return hipErrorInvalidValue;
  }
  if (s.H == 32 && s.Hkv == 8 && s.d == 128 && s.rk == 64 && s.rv == 512)
    return prefill_instance<32, 128, 64, 512, 2, 64, 8, 2, 3, 4, true, 4>(STARKV_PREFILL_ARGS);
  if (s.H == 4 && s.Hkv == 2 && s.d == 64 && s.rk == 16 && s.rv == 64)
    return prefill_instance<4, 64, 16, 64, 4, 16, 2, 2, 2, 1, true, 2>(STARKV_PREFILL_ARGS);
  // r_k 32: a step's two key pages of two heads are too few chunks for the
  // LDS key ring, so the waves load their keys directly
  if (s.H == 32 && s.Hkv == 32 && s.d == 128 && s.rk == 32 && s.rv == 256)
    return prefill_instance<32, 128, 32, 256, 2, 64, 8, 2, 2, 2, false>(STARKV_PREFILL_ARGS);
  if (s.H == 32 && s.Hkv == 32 && s.d == 128 && s.rk == 64 && s.rv == 512)
    return prefill_instance<32, 128, 64, 512, 2, 64, 8, 2, 3, 4, true>(STARKV_PREFILL_ARGS);
  if (s.H == 4 && s.Hkv == 4 && s.d == 64 && s.rk == 16 && s.rv == 64)
    return prefill_instance<4, 64, 16, 64, 4, 16, 2, 2, 2, 1, true>(STARKV_PREFILL_ARGS);
#undef STARKV_PREFILL_ARGS
  return hipErrorInvalidValue;
}

}  // namespace starkv
