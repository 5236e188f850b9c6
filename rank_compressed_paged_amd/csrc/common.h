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

// Butterfly over the four lanes that share l%16 (l, l^16, l^32, l^48).
__device__ __forceinline__ float max_over_quads(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float sum_over_quads(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

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
