// Shared device helpers for the gfx950 (CDNA4) kernels of the paged
// low-rank-compressed attention library.
//
// Matrix-core conventions used throughout (wave64):
//  * v_mfma_f32_16x16x16_f16: lane l holds A[l%16][4*(l/16) + 0..3] and
//    B[4*(l/16) + 0..3][l%16]; the 16x16 fp32 result has D[4*(l/16)+r][l%16]
//    in register r (r = 0..3).
//  * v_mfma_f32_16x16x32_f16: as above with 8 consecutive k per lane:
//    A[l%16][8*(l/16) + 0..7], B[8*(l/16) + 0..7][l%16]; same D layout.
// Because a contraction index may be permuted freely as long as A and B use
// the same permutation, kernels map k to whatever memory order makes each
// lane's 8 or 16 bytes contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace starkv {

typedef _Float16 half_t;
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float4v mfma16x16x16(half4 a, half4 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4v mfma16x16x32(half8 a, half8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float4v zero4() { return float4v{0.f, 0.f, 0.f, 0.f}; }

// fp32 -> (hi, lo) fp16 pairs with hi + lo == x to about 2^-22 relative.
__device__ __forceinline__ void split_f16x8(float4v a, float4v b, half8& hi, half8& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const half_t ha = (half_t)a[e];
    const half_t hb = (half_t)b[e];
    hi[e] = ha;
    hi[e + 4] = hb;
    lo[e] = (half_t)(a[e] - (float)ha);
    lo[e + 4] = (half_t)(b[e] - (float)hb);
  }
}
__device__ __forceinline__ void split_f16x4(float4v a, half4& hi, half4& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const half_t ha = (half_t)a[e];
    hi[e] = ha;
    lo[e] = (half_t)(a[e] - (float)ha);
  }
}

// Reductions over the four lanes l, l^16, l^32, l^48 (the four 4-row
// slices of one column of a 16x16 product) with the cross-row lane swaps,
// which stay in the vector ALU instead of going through the LDS pipe as
// __shfl_xor does.  With both operands equal,
// permlane16_swap leaves lane l of one result and lane l^16 of the other
// holding x[l] and x[l^16]; permlane32_swap does the same for l^32.
// Maxima use the NaN-propagating maximum (v_maximum3_f32), which needs no
// quieting of its inputs, unlike fmaxf: the scores it sees are finite or
// -inf (masked), never NaN.
__device__ __forceinline__ float fmax_nn(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float quad_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmax_nn(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmax_nn(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// x of lane l ^ X for X = 1 or 2 (within each group of four lanes), through
// a DPP quad permutation: one vector instruction, no LDS.
template <int X>
__device__ __forceinline__ float xor_lane_small(float x) {
  static_assert(X == 1 || X == 2, "quad permutations only");
  constexpr int ctrl = X == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, 0xF, 0xF, false));
}

// Work-group barrier that orders LDS only: waits for this wave's LDS (and
// scalar) operations, then s_barrier.  Unlike __syncthreads() it does not
// wait for outstanding global loads, so register prefetches issued before
// it stay in flight across the barrier.  Use only where the barrier guards
// LDS data.
__device__ __forceinline__ void block_sync_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Wait for this wave's own LDS operations (no barrier): enough when a wave
// reads back what it wrote itself.
__device__ __forceinline__ void wave_sync_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Stores and loads of data that work groups of one launch pass to each
// other (split partials): device-scope relaxed atomics, which gfx950 issues
// as ordinary global stores / loads with the sc1 bit, so they write through to
// and read from the device-coherent level instead of an XCD's own L2.  The
// writer waits for its stores (vmcnt(0)) before it publishes them with an
// atomic counter; the reader loads them after it has seen the count.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(half_t* p, half4 v) {
  __hip_atomic_store((uint64_t*)p, __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ half4 ld_dev(const half_t* p) {
  return __builtin_bit_cast(half4, __hip_atomic_load((const uint64_t*)p, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT));
}

__device__ __forceinline__ float2 ld_dev2(const float* p) {
  return __builtin_bit_cast(float2, __hip_atomic_load((const uint64_t*)p, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT));
}

}  // namespace starkv
