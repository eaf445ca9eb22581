// dsa_common.h -- shared device helpers for the libdsa gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa.h"

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

#define DSA_WAVE 64

// Order-preserving map of an fp32 score to an unsigned key: a > b as floats
// (with -0 taken equal to +0 by the caller) iff key(a) > key(b).
__device__ __forceinline__ uint32_t score_key(float v) {
  uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Canonical zero: -0 + +0 = +0 under round-to-nearest.
__device__ __forceinline__ float canon_zero(float v) { return v + 0.0f; }

// FP8 MFMA, 32x32 output tile, K = 64 bytes per lane-half (E4M3 x E4M3).
// Lane l holds A[row l%32][k (l/32)*32 .. +32) and B[k ..][col l%32];
// result register r of lane l is D[(r/4)*8 + (l/32)*4 + r%4][l%32].
__device__ __forceinline__ f32x16 mfma_fp8_32x32x64(const i32x8 &a, const i32x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// bf16 MFMA 16x16x32: lane l holds A[row l%16][k (l/16)*8 .. +8], B likewise
// by column; result register r of lane l is D[(l/16)*4 + r][l%16].
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint32_t t = __shfl_xor(v, o);
    v = t > v ? t : v;
  }
  return v;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint32_t t = __shfl_xor(v, o);
    v = t < v ? t : v;
  }
  return v;
}
__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// s_waitcnt immediate: at most n vector-memory operations outstanding
// (expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Workgroup barrier for LDS traffic only: this wave's LDS operations complete,
// then the hardware barrier (a compiler barrier for memory too).  Unlike
// __syncthreads() it carries no release fence on global memory, which would
// also wait for every load and store in flight; a kernel that shares
// direct-to-LDS loads across waves waits for its own explicitly before it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Lane index within the wave and the number of lanes below it in `mask`.
__device__ __forceinline__ int lane_id() { return __lane_id(); }
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

