// Bases from samples: the step before the attention path.  The pages
// calibrate U_h and W offline by a short knowledge distillation (Proxima
// README, introduction and "Quick start"), which needs a trained model and
// stays out of scope.  This is the unlearned stand-in: the least-squares
// optimal rank-r linear compressions of K/V samples (Eckart-Young).  U_h
// spans the top-r_k eigenspace of G_h = K_h^T K_h (the keys of head h as
// rows, head-wise as the pages decompose keys); W spans the top-r_v
// eigenspace of G_v = V^T V (rows vec(v[n]), head-major, joint across heads as
// the pages decompose values).
//
// Method: subspace iteration from the caller's starting matrices,
//     Y = G Q,  Q = orth(Y)       (iters times)
// with orth one Cholesky QR (S = Y^T Y in fp64, S = L L^T, Q = Y L^-T) and,
// on the last iteration, a second one (Cholesky QR2), which leaves Q
// orthonormal to fp32 rounding.  Any orthonormal basis of the subspace
// serves the compression (attention only sees B B^T), so no small
// eigenproblem is solved at the end.
//
// Kernels (all batched over problems: H key problems of size d, one value
// problem of size H*d):
//   gram_kernel        lower TMxTM tiles of X^T X for fp16 samples, fp32
//                      sums, v_mfma_f32_32x32x16_f16 with operands read
//                      through the transposing LDS read
//   symm_f32_kernel    Y = G Q, G stored as its lower tiles (fp32 matrix cores)
//   syrk_f64_kernel    row slices of S = Y^T Y, lower 64x64 tiles, fp64 sums
//   sum_slices_kernel  S = sum of the slices
//   chol_panel_kernel  four waves per problem: factor the 64x64 diagonal
//                      block of the current panel in 16-column sub-blocks
//                      and invert it in 16x16 blocks (D = L11^-1)
//   chol_rows_kernel   the panel rows below, L_I = A_Ip D^T
//   chol_update_kernel the trailing update A_IJ -= L_I L_J^T over the lower
//                      tiles
//   trsm_kernel        Q = Y L^-T, a work group per 32 rows
//   to_f16_kernel      the result, rounded to fp16
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace starkv {

typedef float float16v __attribute__((ext_vector_type(16)));
typedef short short4v __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each 16-lane group, lane q addresses row
// r0 + q/4, columns c0 + 4*(q%4); lane i then receives rows r0 .. r0+3 of
// column c0 + i.
__device__ __forceinline__ half4 fit_tr16(const half_t* p) {
  typedef __attribute__((address_space(3))) short4v lds_short4v;
  const short4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)p);
  return __builtin_bit_cast(half4, r);
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Work groups are dispatched to the 8 XCDs round-robin (block b to XCD
// b % 8).  For a grid of `total` blocks (a multiple of 8), give block b the
// task (b % 8) * total / 8 + b / 8, so that tasks with neighbouring indices,
// which share operands, run on one XCD and meet in its L2.
__device__ __forceinline__ int xcd_task(int b, int total) {
  return (total & 7) ? b : (b & 7) * (total >> 3) + (b >> 3);
}

// Row I and column J <= I of lower-triangle tile t (row-major order).
__device__ __forceinline__ void tri_index(int t, int& I, int& J) {
  int i = (int)((sqrtf(8.f * (float)t + 1.f) - 1.f) * 0.5f);
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  while (i * (i + 1) / 2 > t) --i;
  I = i;
  J = t - i * (i + 1) / 2;
}

// ---------------------------------------------------------------------------
// Gram matrices.  Tasks 0 .. tiles_v-1 are the lower tiles of G_v (X = v
// samples, n = H*d); the next H * tiles_k are the lower tiles of each G_h
// (X = the d columns of head h of the k samples).  Task order is row-major
// over each triangle, so neighbouring tasks share a strip; block b runs task
// (b % 8) * ceil(T / 8) + b / 8, which keeps neighbours on one XCD (its L2).
// Work group: 4 waves, wave w owning the (TM/2)^2 quadrant (w/2, w%2) as
// (TM/64)^2 32x32 accumulators.  Per 32-sample chunk the two TM-column
// strips are staged in LDS as they lie in memory (whole rows, 16-byte
// pieces), double-buffered; samples past N load as zero.  Diagonal tiles are
// computed whole, so G[i][j] is valid whenever j/TM <= i/TM.
// ---------------------------------------------------------------------------
constexpr int kGramK = 32;

template <int TM>
__global__ __launch_bounds__(256) void gram_kernel(const half_t* __restrict__ kx,
                                                   const half_t* __restrict__ vx, int N, int H,
                                                   int d, float* __restrict__ Gk,
                                                   float* __restrict__ Gv, int tiles_v,
                                                   int tiles_k, int* __restrict__ info) {
  constexpr int LS = TM + 16;          // LDS row stride (halves): 8-bank row shift
  constexpr int CPR = TM / 8;          // 16-byte pieces per strip row
  constexpr int NCH = kGramK * CPR / 256;
  constexpr int WT = TM / 2, MB = WT / 32;
  __shared__ __attribute__((aligned(16))) half_t sI[2][kGramK][LS];
  __shared__ __attribute__((aligned(16))) half_t sJ[2][kGramK][LS];

  const int total = tiles_v + H * tiles_k;
  const int per = ceil_div(total, 8);
  const int t = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (blockIdx.x == 0 && threadIdx.x == 0 && info) info[0] = 0;
  if (t >= total) return;
  const int ld = H * d;
  const half_t* X;
  float* G;
  int n, I, J;
  if (t < tiles_v) {
    X = vx;
    G = Gv;
    n = ld;
    tri_index(t, I, J);
  } else {
    const int u = t - tiles_v, h = u / tiles_k;
    X = kx + (size_t)h * d;
    G = Gk + (size_t)h * d * d;
    n = d;
    tri_index(u - h * tiles_k, I, J);
  }
  const int ci = I * TM, cj = J * TM;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wi = w >> 1, wj = w & 1;
  const int grp = lane >> 4, q = lane & 15;
  const int f_row = 8 * (grp >> 1) + (q >> 2);
  const int f_col = 16 * (grp & 1) + 4 * (q & 3);

  half8 ra[NCH], rb[NCH];
  auto load = [&](int s0) {
#pragma unroll
    for (int e = 0; e < NCH; ++e) {
      const int pc = tid + 256 * e, row = pc / CPR, col = (pc % CPR) * 8;
      const bool ok = s0 + row < N;
      const size_t off = (size_t)(ok ? s0 + row : 0) * ld + col;
      const half8 z = {};
      ra[e] = ok ? *(const half8*)(X + off + ci) : z;
      rb[e] = ok ? *(const half8*)(X + off + cj) : z;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int e = 0; e < NCH; ++e) {
      const int pc = tid + 256 * e, row = pc / CPR, col = (pc % CPR) * 8;
      *(half8*)&sI[buf][row][col] = ra[e];
      *(half8*)&sJ[buf][row][col] = rb[e];
    }
  };

  float16v acc[MB][MB];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  load(0);
  store(0);
  __syncthreads();
  int buf = 0;
  for (int s0 = 0; s0 < N; s0 += kGramK) {
    const bool more = s0 + kGramK < N;  // uniform
    if (more) load(s0 + kGramK);
#pragma unroll
    for (int c = 0; c < kGramK / 16; ++c) {
      half8 av[MB], bv[MB];
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const half_t* ap = &sI[buf][16 * c + f_row][wi * WT + 32 * m + f_col];
        const half_t* bp = &sJ[buf][16 * c + f_row][wj * WT + 32 * m + f_col];
        const half4 a0 = fit_tr16(ap), a1 = fit_tr16(ap + 4 * LS);
        const half4 b0 = fit_tr16(bp), b1 = fit_tr16(bp + 4 * LS);
        av[m] = half8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        bv[m] = half8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
      }
#pragma unroll
      for (int a = 0; a < MB; ++a)
#pragma unroll
        for (int b = 0; b < MB; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
    if (more) store(buf ^ 1);
    block_sync_lds();
    buf ^= 1;
  }
  // register e of a 32x32 accumulator: row 8*(e/4) + 4*(lane/32) + e%4,
  // column lane%32
  const int c32 = lane & 31, hf = lane >> 5;
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = ci + wi * WT + 32 * a + 8 * (e / 4) + 4 * hf + (e % 4);
        const int col = cj + wj * WT + 32 * b + c32;
        G[(size_t)row * n + col] = acc[a][b][e];
      }
}

// ---------------------------------------------------------------------------
// Y_p = G_p Q_p: G_p n x n holding only its lower TM-tiles (element [i][k]
// is read from [k][i] when k/TM > i/TM), Q_p and Y_p n x r row-major fp32.
// grid (ceil(r/64), n/64, problems); 4 waves, wave w computing the 32x32
// block (w/2, w%2) of the 64x64 tile on the fp32 matrix cores
// (v_mfma_f32_32x32x2_f32: lane l supplies A[l%32][l/32] and B[l/32][l%32]).
// k runs in 64-deep chunks: the next chunk is loaded into registers while
// the current one is used from LDS (double-buffered), one LDS-only barrier
// per chunk (the loads stay in flight across it).  n is a multiple of 64, so
// a chunk never straddles a TM-tile.
// ---------------------------------------------------------------------------
constexpr int kSymmK = 64;

__global__ __launch_bounds__(256) void symm_f32_kernel(const float* __restrict__ G, size_t sg,
                                                       int n, int tm, const float* __restrict__ Q,
                                                       size_t sq, float* __restrict__ Y, size_t sy,
                                                       int r) {
  __shared__ __attribute__((aligned(16))) float sA[2][kSymmK][64 + 4];  // [k][row]
  __shared__ __attribute__((aligned(16))) float sB[2][kSymmK][64 + 4];  // [k][column]
  const int p = blockIdx.z;
  const float* Gp = G + (size_t)p * sg;
  const float* Qp = Q + (size_t)p * sq;
  float* Yp = Y + (size_t)p * sy;
  // the column tiles of one row block (which share its rows of G) together
  const int nx = gridDim.x;
  const int t = xcd_task(blockIdx.y * nx + blockIdx.x, nx * gridDim.y);
  const int r0 = (t / nx) * 64, c0 = (t % nx) * 64;
  const int tid = threadIdx.x;
  constexpr int NE = kSymmK * 64 / 256;  // elements of each operand per thread
  float ra[NE], rb[NE];
  // element idx = tid + 256 e of a chunk: A as (row, k) pairs laid out along
  // whichever index is contiguous in memory; B as (k, column)
  auto load = [&](int k0) {
    const bool mirror = (k0 / tm) > (r0 / tm);  // uniform
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int idx = tid + 256 * e;
      ra[e] = mirror ? Gp[(size_t)(k0 + (idx >> 6)) * n + r0 + (idx & 63)]
                     : Gp[(size_t)(r0 + idx / kSymmK) * n + k0 + idx % kSymmK];
      const int kb = idx >> 6, cb = idx & 63;
      rb[e] = (c0 + cb < r) ? Qp[(size_t)(k0 + kb) * r + c0 + cb] : 0.f;
    }
  };
  auto store = [&](int k0, int buf) {
    const bool mirror = (k0 / tm) > (r0 / tm);
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int idx = tid + 256 * e;
      if (mirror)
        sA[buf][idx >> 6][idx & 63] = ra[e];
      else
        sA[buf][idx % kSymmK][idx / kSymmK] = ra[e];
      sB[buf][idx >> 6][idx & 63] = rb[e];
    }
  };
  const int lane = tid & 63, w = tid >> 6, wi = w >> 1, wj = w & 1;
  const int l32 = lane & 31, lk = lane >> 5;
  float16v acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  load(0);
  store(0, 0);
  __syncthreads();
  int buf = 0;
  for (int k0 = 0; k0 < n; k0 += kSymmK) {
    const bool more = k0 + kSymmK < n;
    if (more) load(k0 + kSymmK);
#pragma unroll
    for (int kk = 0; kk < kSymmK; kk += 2) {
      const float av = sA[buf][kk + lk][32 * wi + l32];
      const float bv = sB[buf][kk + lk][32 * wj + l32];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
    }
    if (more) store(k0 + kSymmK, buf ^ 1);
    block_sync_lds();
    buf ^= 1;
  }
  // register e: row 8*(e/4) + 4*(lane/32) + e%4, column lane%32 of the block
  const int c = c0 + 32 * wj + l32;
  if (c < r) {
#pragma unroll
    for (int e = 0; e < 16; ++e)
      Yp[(size_t)(r0 + 32 * wi + 8 * (e / 4) + 4 * lk + (e % 4)) * r + c] = acc[e];
  }
}

// ---------------------------------------------------------------------------
// Slice s of S_p = X_p^T Y_p: sum over rows [s*rows, (s+1)*rows) of X_p and
// Y_p (n x r fp32) of the exact fp64 products; lower 64x64 tiles only
// (X = Y, a symmetric S), or every tile (full).
// grid (tiles, problems * slices); 256 threads, 4x4 outputs each; 32-row
// chunks, the next one loaded into registers while the current one is used.
// Output: S + (p * slices + s) * r * r.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void syrk_f64_kernel(const float* __restrict__ X,
                                                       const float* __restrict__ Y, size_t sy,
                                                       int n, int r, int slices, int rows,
                                                       int full, double* __restrict__ S) {
  __shared__ __attribute__((aligned(16))) float sa[2][32][64 + 4];
  __shared__ __attribute__((aligned(16))) float sb[2][32][64 + 4];
  // the tiles of one row slice (which share its rows of Y) together
  const int nt = gridDim.x;
  const int task = xcd_task(blockIdx.y * nt + blockIdx.x, nt * gridDim.y);
  const int p = (task / nt) / slices, s = (task / nt) % slices;
  int I, J;
  if (full) {
    const int nbk = (r + 63) / 64;
    I = (task % nt) / nbk;
    J = (task % nt) % nbk;
  } else {
    tri_index(task % nt, I, J);
  }
  const float* Xp = X + (size_t)p * sy;
  const float* Yp = Y + (size_t)p * sy;
  const int a0 = I * 64, b0 = J * 64;
  const int i_beg = s * rows, i_end = min(n, i_beg + rows);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float ya[8], yb[8];
  auto load = [&](int i0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int idx = tid + e * 256, ii = idx >> 6, c = idx & 63;
      const bool rok = i0 + ii < i_end;
      ya[e] = (rok && a0 + c < r) ? Xp[(size_t)(i0 + ii) * r + a0 + c] : 0.f;
      yb[e] = (rok && b0 + c < r) ? Yp[(size_t)(i0 + ii) * r + b0 + c] : 0.f;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int idx = tid + e * 256;
      sa[buf][idx >> 6][idx & 63] = ya[e];
      sb[buf][idx >> 6][idx & 63] = yb[e];
    }
  };
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  load(i_beg);
  store(0);
  __syncthreads();
  int buf = 0;
  for (int i0 = i_beg; i0 < i_end; i0 += 32) {
    const bool more = i0 + 32 < i_end;
    if (more) load(i0 + 32);
#pragma unroll 4
    for (int ii = 0; ii < 32; ++ii) {
      const float4v av = *(const float4v*)&sa[buf][ii][ty * 4];
      const float4v bv = *(const float4v*)&sb[buf][ii][tx * 4];
      double bd[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) bd[b] = (double)bv[b];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const double ad = (double)av[a];
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_fma(ad, bd[b], acc[a][b]);
      }
    }
    if (more) store(buf ^ 1);
    block_sync_lds();
    buf ^= 1;
  }
  double* Sp = S + ((size_t)p * slices + s) * r * r;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int ra = a0 + ty * 4 + a, cb = b0 + tx * 4 + b;
      if (ra < r && cb < r) Sp[(size_t)ra * r + cb] = acc[a][b];
    }
}

// A_p = sum over s of S_(p*slices + s), entries in the lower 64-tiles only
// (or all of them: full).
__global__ __launch_bounds__(256) void sum_slices_kernel(const double* __restrict__ S, int r,
                                                         int slices, int problems, int full,
                                                         double* __restrict__ A) {
  const size_t rr = (size_t)r * r;
  const size_t total = rr * problems;
  for (size_t x = (size_t)blockIdx.x * 256 + threadIdx.x; x < total; x += (size_t)gridDim.x * 256) {
    const size_t p = x / rr, e = x % rr;
    const int i = (int)(e / r), j = (int)(e % r);
    if (!full && j / 64 > i / 64) continue;
    double s = 0.0;
    for (int k = 0; k < slices; ++k) s += S[(p * slices + k) * rr + e];
    A[x] = s;
  }
}

// ---------------------------------------------------------------------------
// Blocked Cholesky, panel p (columns 64p .. 64p+nb-1, nb = min(64, r-64p)):
// factor the 64x64 diagonal block and invert it, one wave per problem.
//  1. Lane i holds row i in registers.  At step k every lane reads the
//     pivot from lane k and takes its reciprocal square root s itself; lanes
//     i >= k scale their element of column k, l_i = a_ik * s (lane k gets
//     sqrt(a_kk)), and publish it as row k of L^T in LDS (each step its own
//     row, so nothing is overwritten); then each lane updates the rest of its
//     row from that row.  A wave's LDS operations complete in order, so the
//     lanes need no barrier.  Steps run in blocks of eight with static
//     register indices; after a block the row shifts down by eight.  A pivot
//     that is not positive (rank-deficient samples) is replaced by 1 and
//     counted in *info.
//  2. D = L11^-1: lane c holds column c of the identity and sweeps it down
//     (row k times 1/L_kk = s_k, then subtract L_ik times it from the rows
//     below), in the same blocks of eight.
// Writes L11 (upper part zero) into L and D into Dinv[p].
// ---------------------------------------------------------------------------
__device__ __forceinline__ double readlane_f64(double x, int lane) {
  const long long b = __builtin_bit_cast(long long, x);
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffll), lane);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
  return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
}

// 1/sqrt(x) for x > 0: the hardware estimate and two Newton steps.
__device__ __forceinline__ double rsqrt_f64(double x) {
  double y = __builtin_amdgcn_rsq(x);
  const double hx = 0.5 * x;
  y = y * __builtin_fma(-hx * y, y, 1.5);
  y = y * __builtin_fma(-hx * y, y, 1.5);
  return y;
}

__global__ __launch_bounds__(256) void chol_panel_kernel(const double* __restrict__ A,
                                                         double* __restrict__ L,
                                                         double* __restrict__ Dinv, int r, int p,
                                                         int* __restrict__ info) {
  // Four waves, blocked by 16 columns; lane = row of the 64x64 block.
  // Factor: wave w holds columns 16w .. 16w+15 of its row in registers.  For
  // sub-block sb the owning wave factors its 16 columns for all rows alone
  // (pivot from lane k by readlane, fp64 reciprocal square root, the scaled
  // column published in LDS as row k of L^T and read back by the same wave,
  // whose LDS operations complete in order, then the update of the block's
  // later columns); after one barrier every later wave subtracts the rank-16
  // product L[:, sb] L[c, sb]^T from its own columns c.  Updates only ever
  // touch columns not yet factored, and values above the diagonal are never
  // read as pivots or results.
  // Inverse D = L^-1 in 16x16 blocks: each wave inverts one diagonal block
  // by forward substitution (lane = column), then the off-diagonal blocks
  // follow by distance from the diagonal, D_IJ = -D_II sum_{K=J}^{I-1}
  // L_IK D_KJ, one block per wave and level, a barrier between levels.
  __shared__ double sLt[64][64 + 1];  // row k = column k of L (zero above the diagonal)
  __shared__ double sD[64][64 + 1];   // D, row-major, filled block by block
  __shared__ double sT[4][16][16 + 1];  // per-wave scratch of the off-diagonal blocks
  __shared__ double sS[64];            // 1 / L_kk
  const int prob = blockIdx.x;
  const int nbk = ceil_div(r, 64);
  const double* Ap = A + (size_t)prob * r * r;
  double* Lp = L + (size_t)prob * r * r;
  double* Dp = Dinv + ((size_t)prob * nbk + p) * 64 * 64;
  const int j0 = 64 * p, nb = min(64, r - j0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  double a[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int c = 16 * w + t;
    a[t] = (lane < nb && c <= lane) ? Ap[(size_t)(j0 + lane) * r + j0 + c] : 0.0;
  }
  for (int sb = 0; sb < 4; ++sb) {
    const int c0 = 16 * sb;
    if (c0 >= nb) break;  // uniform
    if (w == sb) {        // uniform: the owner factors its 16 columns
#pragma unroll
      for (int tk = 0; tk < 16; ++tk) {
        const int k = c0 + tk;
        if (k < nb) {
          double dk = readlane_f64(a[tk], k);
          if (!(dk > 0.0)) {
            if (lane == 0 && info) atomicAdd(info, 1);
            dk = 1.0;
          }
          const double sc = rsqrt_f64(dk);
          const double l = lane == k ? dk * sc : (lane > k ? a[tk] * sc : 0.0);
          sLt[k][lane] = l;
          if (lane == 0) sS[k] = sc;
          double lr[16];
#pragma unroll
          for (int t = tk + 1; t < 16; ++t) lr[t] = sLt[k][c0 + t];  // L[c0 + t][k]
#pragma unroll
          for (int t = tk + 1; t < 16; ++t) a[t] -= l * lr[t];
        }
      }
    }
    __syncthreads();
    if (w > sb) {  // uniform: rank-16 update of this wave's columns
      double lm[16];
#pragma unroll
      for (int m = 0; m < 16; ++m) lm[m] = sLt[c0 + m][lane];  // L[lane][c0 + m]
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        double lc[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) lc[t] = sLt[c0 + m][16 * w + t];  // L[16w + t][c0 + m]
#pragma unroll
        for (int t = 0; t < 16; ++t) a[t] -= lm[m] * lc[t];
      }
    }
  }
  __syncthreads();
  // inverse, diagonal blocks: wave J inverts L_JJ, lane = column (16 lanes)
  const int nsb = ceil_div(nb, 16);
  if (w < nsb && lane < 16) {
    const int c0 = 16 * w;
    double x[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) x[t] = (t == lane && c0 + t < nb) ? 1.0 : 0.0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (c0 + k < nb) {
        x[k] *= sS[c0 + k];
#pragma unroll
        for (int t = k + 1; t < 16; ++t) x[t] -= sLt[c0 + k][c0 + t] * x[k];  // L[c0+t][c0+k]
      }
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) sD[c0 + t][c0 + lane] = x[t];
  }
  // zero the blocks above the diagonal (never written otherwise)
  for (int e = tid; e < 64 * 64; e += 256) {
    const int i = e / 64, j = e % 64;
    if (j / 16 > i / 16) sD[i][j] = 0.0;
  }
  __syncthreads();
  // off-diagonal blocks by distance dist = I - J; lane = (row r = lane / 4,
  // columns 4 (lane % 4) .. +3) of the 16x16 block
  for (int dist = 1; dist < nsb; ++dist) {
    const int J = w, I = w + dist;
    if (I < nsb) {  // uniform
      const int I0 = 16 * I, J0 = 16 * J, rr = lane >> 2, cc = 4 * (lane & 3);
      // T = sum_{K=J}^{I-1} L_IK D_KJ
      double tv[4] = {0.0, 0.0, 0.0, 0.0};
      for (int m = J0; m < I0; ++m) {
        const double lim = sLt[m][I0 + rr];  // L[I0 + rr][m]
#pragma unroll
        for (int q = 0; q < 4; ++q) tv[q] += lim * sD[m][J0 + cc + q];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) sT[w][rr][cc + q] = tv[q];
      wave_sync_lds();  // this wave's own writes, read back below
      // D_IJ = -D_II T
      double dv[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const double dim = sD[I0 + rr][I0 + m];
#pragma unroll
        for (int q = 0; q < 4; ++q) dv[q] += dim * sT[w][m][cc + q];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) sD[I0 + rr][J0 + cc + q] = -dv[q];
    }
    __syncthreads();
  }
  // D out (zero past nb and above the diagonal), then L11
  for (int e = tid; e < 64 * 64; e += 256) {
    const int i = e / 64, j = e % 64;
    Dp[(size_t)i * 64 + j] = (i < nb && j < nb && j <= i) ? sD[i][j] : 0.0;
  }
  for (int i = w; i < nb; i += 4)
    if (lane < nb) Lp[(size_t)(j0 + i) * r + j0 + lane] = lane <= i ? sLt[lane][i] : 0.0;
}

// ---------------------------------------------------------------------------
// Panel rows below the diagonal block of panel p: L_I = A[I-rows, panel] D_p^T
// for each 64-row block I > p.  grid (ceil(r/64) - p - 1, problems), 256
// threads, 4 rows x 4 columns each.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void chol_rows_kernel(const double* __restrict__ A,
                                                        double* __restrict__ L,
                                                        const double* __restrict__ Dinv, int r,
                                                        int p) {
  __shared__ double sA[64][65];
  __shared__ double sD[64][65];
  const int prob = blockIdx.y;
  const int nbk = ceil_div(r, 64);
  const int I = p + 1 + blockIdx.x;
  const double* Ap = A + (size_t)prob * r * r;
  double* Lp = L + (size_t)prob * r * r;
  const double* Dp = Dinv + ((size_t)prob * nbk + p) * 64 * 64;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int pc = 64 * p, ri = 64 * I;
  for (int e = tid; e < 64 * 64; e += 256) {
    const int row = e >> 6, col = e & 63;
    sA[row][col] = (ri + row < r) ? Ap[(size_t)(ri + row) * r + pc + col] : 0.0;
    sD[row][col] = Dp[e];
  }
  __syncthreads();
  double o[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) o[a][b] = 0.0;
#pragma unroll 8
  for (int m = 0; m < 64; ++m) {
    double dv[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) dv[b] = sD[tx * 4 + b][m];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const double av = sA[ty * 4 + a][m];
#pragma unroll
      for (int b = 0; b < 4; ++b) o[a][b] = __builtin_fma(av, dv[b], o[a][b]);
    }
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int row = ri + ty * 4 + a;
    if (row < r) {
#pragma unroll
      for (int b = 0; b < 4; ++b) Lp[(size_t)row * r + pc + tx * 4 + b] = o[a][b];
    }
  }
}

// ---------------------------------------------------------------------------
// After panel p: A[I-rows, J-cols] -= L[I-rows, panel p] L[J-rows, panel p]^T
// for every lower tile (I, J), p < J <= I < ceil(r/64).  grid (tiles,
// problems), 256 threads, each 4x4 of the 64x64 product.  Each tile of A is
// owned by one work group; L's panel is only read.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void chol_update_kernel(double* __restrict__ A,
                                                          const double* __restrict__ L, int r,
                                                          int p) {
  __shared__ double sPI[64][65];
  __shared__ double sPJ[64][65];
  const int prob = blockIdx.y;
  int It, Jt;
  tri_index(blockIdx.x, It, Jt);
  const int I = p + 1 + It, J = p + 1 + Jt;
  double* Ap = A + (size_t)prob * r * r;
  const double* Lp = L + (size_t)prob * r * r;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int pc = 64 * p, ri = 64 * I, rj = 64 * J;
  for (int e = tid; e < 64 * 64; e += 256) {
    const int row = e >> 6, col = e & 63;
    sPI[row][col] = (ri + row < r) ? Lp[(size_t)(ri + row) * r + pc + col] : 0.0;
    sPJ[row][col] = (rj + row < r) ? Lp[(size_t)(rj + row) * r + pc + col] : 0.0;
  }
  __syncthreads();
  double c[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) c[a][b] = 0.0;
#pragma unroll 8
  for (int m = 0; m < 64; ++m) {
    double bj[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) bj[b] = sPJ[tx * 4 + b][m];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const double ai = sPI[ty * 4 + a][m];
#pragma unroll
      for (int b = 0; b < 4; ++b) c[a][b] = __builtin_fma(ai, bj[b], c[a][b]);
    }
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int row = ri + ty * 4 + a, col = rj + tx * 4 + b;
      if (row < r && col < r) Ap[(size_t)row * r + col] -= c[a][b];
    }
}

// ---------------------------------------------------------------------------
// Q_p = Y_p L_p^-T (n x r, fp32), row by row: for column block J
//     R = Y[:, J] - Q[:, <J] L[J, <J]^T,   Q[:, J] = R D_J^T.
// grid (ceil(n/32), problems), 256 threads (32 rows x 8 groups of 8
// columns); the work group's rows of Q stay in LDS.  The operand blocks run
// as one sequence of steps, (J, 0) .. (J, J-1) for the blocks L[J, mc] and
// (J, J) for D_J, each staged transposed in LDS as fp32 ([m][c]), loaded
// into registers two steps ahead.  L and D are fp64 and used in fp32 (the
// second Cholesky QR round restores orthogonality to fp32 rounding).
// ---------------------------------------------------------------------------
constexpr int kTrsmRows = 32;
constexpr int kFitMaxRank = 512;

__global__ __launch_bounds__(256) void trsm_kernel(const float* __restrict__ Y, size_t sy,
                                                   const double* __restrict__ L,
                                                   const double* __restrict__ Dinv, int n, int r,
                                                   float* __restrict__ Q) {
  __shared__ __attribute__((aligned(16))) float sQ[kTrsmRows][kFitMaxRank + 4];
  __shared__ __attribute__((aligned(16))) float sT[2][64][64 + 4];
  __shared__ float sR[kTrsmRows][64 + 1];
  const int prob = blockIdx.y;
  const int nbk = ceil_div(r, 64);
  const int steps = nbk * (nbk + 1) / 2;
  const float* Yp = Y + (size_t)prob * sy;
  float* Qp = Q + (size_t)prob * sy;
  const double* Lp = L + (size_t)prob * r * r;
  const double* Dp = Dinv + (size_t)prob * nbk * 64 * 64;
  const int tid = threadIdx.x, rr = tid >> 3, cq = (tid & 7) * 8;
  const int row = blockIdx.x * kTrsmRows + rr;
  const bool rok = row < n;
  // step s = (J, mc), mc <= J, in lower-triangle order; element e = tid +
  // 256 u is (c, m) = (e / 64, e % 64) of L[64J + c][64mc + m] (mc < J) or
  // D_J[c][m] (mc == J).  Loads are kept raw (fp64) and converted at the LDS
  // store, two steps after they were issued.
  auto load = [&](int st_idx, double* dst) {
    int J, mc;
    tri_index(st_idx, J, mc);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = tid + 256 * u, c = e >> 6, m = e & 63;
      if (mc < J)
        dst[u] = (64 * J + c < r) ? Lp[(size_t)(64 * J + c) * r + 64 * mc + m] : 0.0;
      else
        dst[u] = Dp[(size_t)J * 64 * 64 + e];
    }
  };
  auto store = [&](const double* src, int buf) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = tid + 256 * u;
      sT[buf][e & 63][e >> 6] = (float)src[u];
    }
  };
  auto load_y = [&](int J, float* y) {
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int c = 64 * J + cq + b;
      y[b] = (rok && c < r) ? Yp[(size_t)row * r + c] : 0.f;
    }
  };
  float acc[8], ynext[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) ynext[b] = 0.f;
  // one step: s uses sT[buf]; the registers `nxt` receive step s + 2, and
  // `cur` (holding step s + 1) goes to the other buffer at the end
  auto step = [&](int st_idx, int buf, double* nxt, const double* cur) {
    int J, mc;
    tri_index(st_idx, J, mc);
    if (st_idx + 2 < steps) load(st_idx + 2, nxt);
    if (mc == 0 && J + 1 < nbk) load_y(J + 1, ynext);
    if (mc < J) {
#pragma unroll 8
      for (int m = 0; m < 64; ++m) {
        const float qv = sQ[rr][64 * mc + m];
        const float4v l0 = *(const float4v*)&sT[buf][m][cq];
        const float4v l1 = *(const float4v*)&sT[buf][m][cq + 4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          acc[b] = __builtin_fmaf(-qv, l0[b], acc[b]);
          acc[b + 4] = __builtin_fmaf(-qv, l1[b], acc[b + 4]);
        }
      }
    } else {
#pragma unroll
      for (int b = 0; b < 8; ++b) sR[rr][cq + b] = acc[b];
      block_sync_lds();
      float o[8];
#pragma unroll
      for (int b = 0; b < 8; ++b) o[b] = 0.f;
#pragma unroll 8
      for (int m = 0; m < 64; ++m) {
        const float rv = sR[rr][m];
        const float4v d0 = *(const float4v*)&sT[buf][m][cq];
        const float4v d1 = *(const float4v*)&sT[buf][m][cq + 4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          o[b] = __builtin_fmaf(rv, d0[b], o[b]);
          o[b + 4] = __builtin_fmaf(rv, d1[b], o[b + 4]);
        }
      }
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const int c = 64 * J + cq + b;
        if (c < r) {
          sQ[rr][c] = o[b];
          if (rok) Qp[(size_t)row * r + c] = o[b];
        }
        acc[b] = ynext[b];
      }
    }
    if (st_idx + 1 < steps) store(cur, buf ^ 1);
    block_sync_lds();
  };
  double stA[16], stB[16];
  load_y(0, acc);
  load(0, stA);
  store(stA, 0);
  if (steps > 1) load(1, stA);
  __syncthreads();
  for (int s0 = 0; s0 < steps; s0 += 2) {
    step(s0, 0, stB, stA);
    if (s0 + 1 < steps) step(s0 + 1, 1, stA, stB);
  }
}

// Convergence of the returned basis Q_p (orthonormal n x r) of each problem:
// with Y_p = G_p Q_p and T_p = Q_p^T Y_p (the Rayleigh matrix, fp64), the
// invariant-subspace residual R_p = Y_p - Q_p T_p, formed explicitly (the
// difference of squared norms ||Y||^2 - ||T||^2 would lose it below the
// square root of Q's fp32 orthonormality error).  Work group (32 rows, p):
// the rows of Q in LDS, thread j of each round accumulating column j of
// those 32 rows of Q T in fp64 (T read once per work group); the partial
// sums of |R|^2 and |Y|^2 go to part[(p * blocks + block) * 2 + {0, 1}].
constexpr int kResRows = 32;
__global__ __launch_bounds__(256) void fit_resid_rows_kernel(const float* __restrict__ Q,
                                                             const float* __restrict__ Y,
                                                             size_t sq, int n, int r,
                                                             const double* __restrict__ T,
                                                             double* __restrict__ part) {
  __shared__ float sQ[kResRows][512];
  __shared__ double red[2][256];
  const int blk = blockIdx.x, p = blockIdx.y, tid = threadIdx.x;
  const int i0 = blk * kResRows;
  const float* Qp = Q + (size_t)p * sq;
  const float* Yp = Y + (size_t)p * sq;
  const double* Tp = T + (size_t)p * r * r;
  for (int x = tid; x < kResRows * r; x += 256) {
    const int row = x / r, k = x % r;
    sQ[row][k] = i0 + row < n ? Qp[(size_t)(i0 + row) * r + k] : 0.f;
  }
  __syncthreads();
  double rr = 0.0, yy = 0.0;
  for (int j = tid; j < r; j += 256) {
    double acc[kResRows];
#pragma unroll
    for (int row = 0; row < kResRows; ++row) acc[row] = 0.0;
    for (int k = 0; k < r; ++k) {
      const double t = Tp[(size_t)k * r + j];
#pragma unroll
      for (int row = 0; row < kResRows; ++row) acc[row] = __builtin_fma((double)sQ[row][k], t, acc[row]);
    }
#pragma unroll
    for (int row = 0; row < kResRows; ++row) {
      if (i0 + row < n) {
        const double y = (double)Yp[(size_t)(i0 + row) * r + j];
        const double d = y - acc[row];
        rr = __builtin_fma(d, d, rr);
        yy = __builtin_fma(y, y, yy);
      }
    }
  }
  red[0][tid] = rr;
  red[1][tid] = yy;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) {
      red[0][tid] += red[0][tid + w];
      red[1][tid] += red[1][tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    part[((size_t)p * gridDim.x + blk) * 2] = red[0][0];
    part[((size_t)p * gridDim.x + blk) * 2 + 1] = red[1][0];
  }
}

// *out = max_p sqrt(sum |R_p|^2 / sum |Y_p|^2) (0 when Y_p is zero), summing
// the row blocks' partials in order.  One work group.
__global__ __launch_bounds__(64) void fit_resid_final_kernel(const double* __restrict__ part,
                                                             int blocks, int problems,
                                                             float* __restrict__ out) {
  if (threadIdx.x != 0) return;
  double worst = 0.0;
  for (int p = 0; p < problems; ++p) {
    double rr = 0.0, yy = 0.0;
    for (int b = 0; b < blocks; ++b) {
      rr += part[((size_t)p * blocks + b) * 2];
      yy += part[((size_t)p * blocks + b) * 2 + 1];
    }
    worst = fmax(worst, yy > 0.0 ? sqrt(rr / yy) : 0.0);
  }
  *out = (float)worst;
}

__global__ __launch_bounds__(256) void to_f16_kernel(const float* __restrict__ src, size_t n,
                                                     half_t* __restrict__ dst) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    dst[i] = (half_t)src[i];
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
static int fit_tile(int d) { return d % 128 == 0 ? 128 : 64; }
static int syrk_slices(int n) { return (n + 511) / 512; }
static size_t align256_(size_t x) { return (x + 255) & ~(size_t)255; }

FitWorkspace fit_workspace_layout(const ShapeKey& s) {
  const size_t nv = (size_t)s.H * s.d, nk = s.d;
  const size_t rk = s.rk, rv = s.rv;
  const size_t nbk_k = (rk + 63) / 64, nbk_v = (rv + 63) / 64;
  FitWorkspace w;
  size_t off = 0;
  w.gv_off = off;
  off = align256_(off + nv * nv * 4);
  w.gk_off = off;
  off = align256_(off + (size_t)s.H * nk * nk * 4);
  w.qv_off[0] = off;
  off = align256_(off + nv * rv * 4);
  w.qv_off[1] = off;
  off = align256_(off + nv * rv * 4);
  w.qk_off[0] = off;
  off = align256_(off + (size_t)s.H * nk * rk * 4);
  w.qk_off[1] = off;
  off = align256_(off + (size_t)s.H * nk * rk * 4);
  // slices of S_v (unused when one slice), and the residual's row-block sums
  w.sv_off = off;
  off = align256_(off + std::max<size_t>((size_t)syrk_slices((int)nv) * rv * rv,
                                         2 * (size_t)ceil_div((int)nv, kResRows)) * 8);
  w.sk_off = off;
  off = align256_(off + (size_t)s.H * std::max<size_t>((size_t)syrk_slices((int)nk) * rk * rk,
                                                       2 * (size_t)ceil_div((int)nk, kResRows)) * 8);
  w.av_off = off;
  off = align256_(off + rv * rv * 8);
  w.ak_off = off;
  off = align256_(off + (size_t)s.H * rk * rk * 8);
  w.lv_off = off;
  off = align256_(off + rv * rv * 8);
  w.lk_off = off;
  off = align256_(off + (size_t)s.H * rk * rk * 8);
  w.dv_off = off;
  off = align256_(off + nbk_v * 64 * 64 * 8);
  w.dk_off = off;
  off = align256_(off + (size_t)s.H * nbk_k * 64 * 64 * 8);
  w.total = off;
  return w;
}

namespace {

struct OrthProblem {
  int P, n, r;
  double *S, *A, *L, *D;
};

// Q = Y L^-T with S = Y^T Y = L L^T, for P problems of n x r (Y, Q at stride n*r).
hipError_t orth(const OrthProblem& o, const float* Y, float* Q, int* info, hipStream_t st) {
  const int slices = syrk_slices(o.n), rows = ceil_div(o.n, slices);
  const int nbk = ceil_div(o.r, 64);
  const int tiles = nbk * (nbk + 1) / 2;
  const size_t sy = (size_t)o.n * o.r;
  double* dst = slices > 1 ? o.S : o.A;
  hipLaunchKernelGGL(syrk_f64_kernel, dim3(tiles, o.P * slices), dim3(256), 0, st, Y, Y, sy, o.n,
                     o.r, slices, rows, 0, dst);
  if (slices > 1) {
    const size_t total = (size_t)o.P * o.r * o.r;
    const int blocks = (int)std::min<size_t>((total + 255) / 256, 2048);
    hipLaunchKernelGGL(sum_slices_kernel, dim3(blocks), dim3(256), 0, st, o.S, o.r, slices, o.P,
                       0, o.A);
  }
  for (int p = 0; p < nbk; ++p) {
    hipLaunchKernelGGL(chol_panel_kernel, dim3(o.P), dim3(256), 0, st, o.A, o.L, o.D, o.r, p,
                       info);
    const int m = nbk - p - 1;
    if (m > 0) {
      hipLaunchKernelGGL(chol_rows_kernel, dim3(m, o.P), dim3(256), 0, st, o.A, o.L, o.D, o.r, p);
      hipLaunchKernelGGL(chol_update_kernel, dim3(m * (m + 1) / 2, o.P), dim3(256), 0, st, o.A,
                         o.L, o.r, p);
    }
  }
  hipLaunchKernelGGL(trsm_kernel, dim3(ceil_div(o.n, kTrsmRows), o.P), dim3(256), 0, st, Y, sy,
                     o.L, o.D, o.n, o.r, Q);
  return hipGetLastError();
}

// The residual of the returned basis Q (see fit_resid_rows_kernel): Y = G Q
// into Yw, T = Q^T Y (every tile, fp64) into o.A, then the reduction.
hipError_t residual(const OrthProblem& o, const float* G, int tm, const float* Q, float* Yw,
                    float* out, hipStream_t st) {
  const size_t sg = (size_t)o.n * o.n, sq = (size_t)o.n * o.r;
  hipLaunchKernelGGL(symm_f32_kernel, dim3(ceil_div(o.r, 64), o.n / 64, o.P), dim3(256), 0, st, G,
                     sg, o.n, tm, Q, sq, Yw, sq, o.r);
  const int slices = syrk_slices(o.n), rows = ceil_div(o.n, slices);
  const int nbk = ceil_div(o.r, 64);
  double* dst = slices > 1 ? o.S : o.A;
  hipLaunchKernelGGL(syrk_f64_kernel, dim3(nbk * nbk, o.P * slices), dim3(256), 0, st, Q, Yw, sq,
                     o.n, o.r, slices, rows, 1, dst);
  if (slices > 1) {
    const size_t total = (size_t)o.P * o.r * o.r;
    const int blocks = (int)std::min<size_t>((total + 255) / 256, 2048);
    hipLaunchKernelGGL(sum_slices_kernel, dim3(blocks), dim3(256), 0, st, o.S, o.r, slices, o.P,
                       1, o.A);
  }
  // the slices of S are free again: they take the row blocks' partial sums
  const int blocks = ceil_div(o.n, kResRows);
  hipLaunchKernelGGL(fit_resid_rows_kernel, dim3(blocks, o.P), dim3(256), 0, st, Q, Yw, sq, o.n,
                     o.r, o.A, o.S);
  hipLaunchKernelGGL(fit_resid_final_kernel, dim3(1), dim3(64), 0, st, o.S, blocks, o.P, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fit(const ShapeKey& s, const void* k, const void* v, int n_samples,
                      const float* u0, const float* w0, int iters, void* U, void* W,
                      void* workspace, int* info, float* residual_out, hipStream_t st) {
  const FitWorkspace ws = fit_workspace_layout(s);
  char* wb = (char*)workspace;
  float* Gv = (float*)(wb + ws.gv_off);
  float* Gk = (float*)(wb + ws.gk_off);
  const int tm = fit_tile(s.d);
  const int nbv = s.H * s.d / tm, nbk = s.d / tm;
  const int tiles_v = nbv * (nbv + 1) / 2, tiles_k = nbk * (nbk + 1) / 2;
  const int total = tiles_v + s.H * tiles_k;
  const dim3 ggrid(8 * ceil_div(total, 8));
  if (g_timing.which == TIME_FIT_GRAM && g_timing.start) (void)hipEventRecord(g_timing.start, st);
  if (tm == 128)
    launch_hooked(TIME_FIT_GRAM, TIME_NONE, gram_kernel<128>, ggrid, dim3(256), st,
                  (const half_t*)k, (const half_t*)v, n_samples, s.H, s.d, Gk, Gv, tiles_v,
                  tiles_k, info);
  else
    launch_hooked(TIME_FIT_GRAM, TIME_NONE, gram_kernel<64>, ggrid, dim3(256), st,
                  (const half_t*)k, (const half_t*)v, n_samples, s.H, s.d, Gk, Gv, tiles_v,
                  tiles_k, info);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  struct Side {
    int P, n, r;
    const float* G;
    const float* q0;
    float* buf[2];
    OrthProblem o;
    half_t* out;
  };
  Side sides[2] = {
      {1, s.H * s.d, s.rv, Gv, w0, {(float*)(wb + ws.qv_off[0]), (float*)(wb + ws.qv_off[1])},
       {1, s.H * s.d, s.rv, (double*)(wb + ws.sv_off), (double*)(wb + ws.av_off),
        (double*)(wb + ws.lv_off), (double*)(wb + ws.dv_off)},
       (half_t*)W},
      {s.H, s.d, s.rk, Gk, u0, {(float*)(wb + ws.qk_off[0]), (float*)(wb + ws.qk_off[1])},
       {s.H, s.d, s.rk, (double*)(wb + ws.sk_off), (double*)(wb + ws.ak_off),
        (double*)(wb + ws.lk_off), (double*)(wb + ws.dk_off)},
       (half_t*)U}};
  for (Side& sd : sides) {
    const size_t sg = (size_t)sd.n * sd.n, sq = (size_t)sd.n * sd.r;
    const dim3 mgrid(ceil_div(sd.r, 64), sd.n / 64, sd.P);
    const float* q = sd.q0;
    // buf[1] takes Y = G Q, buf[0] the orthonormalised Q
    for (int it = 0; it < iters; ++it) {
      hipLaunchKernelGGL(symm_f32_kernel, mgrid, dim3(256), 0, st, sd.G, sg, sd.n, tm, q, sq,
                         sd.buf[1], sq, sd.r);
      e = orth(sd.o, sd.buf[1], sd.buf[0], info, st);
      if (e != hipSuccess) return e;
      q = sd.buf[0];
    }
    e = orth(sd.o, sd.buf[0], sd.buf[1], info, st);  // second round of the last QR
    if (e != hipSuccess) return e;
    if (residual_out) {  // keys into [0], values into [1]
      e = residual(sd.o, sd.G, tm, sd.buf[1], sd.buf[0], residual_out + (&sd == &sides[0] ? 1 : 0),
                   st);
      if (e != hipSuccess) return e;
    }
    const size_t cnt = (size_t)sd.P * sq;
    const int blocks = (int)std::min<size_t>((cnt + 255) / 256, 4096);
    hipLaunchKernelGGL(to_f16_kernel, dim3(blocks), dim3(256), 0, st, sd.buf[1], cnt, sd.out);
  }
  return hipGetLastError();
}

}  // namespace starkv
