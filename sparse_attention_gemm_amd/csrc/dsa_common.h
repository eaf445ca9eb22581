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

// Lane index within the wave and the number of lanes below it in `mask`.
__device__ __forceinline__ int lane_id() { return __lane_id(); }
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// Host side -----------------------------------------------------------------
namespace dsa {
dsa_status fail(dsa_status st, const char *fmt, ...);
dsa_status hip_check(hipError_t e, const char *what);
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Launchers (each validates nothing: the C ABI layer does).
hipError_t launch_quantize(const float *x, int64_t rows, int32_t cols, uint8_t *x8, float *scale,
                           hipStream_t s);
hipError_t launch_indexer_scores_fp8(const uint8_t *q, const float *qs, const uint8_t *k,
                                     const float *ks, const float *w, const int32_t *q_pos,
                                     int32_t T, int32_t S, int32_t H_I, float *scores, int64_t ld,
                                     hipStream_t s);
hipError_t launch_indexer_scores_f32(const float *q, const float *k, const float *w,
                                     const int32_t *q_pos, int32_t T, int32_t S, int32_t H_I,
                                     int32_t D_I, float *scores, int64_t ld, hipStream_t s);
// Rows take min(n_valid[t], n_cap) candidates (n_cap guards the row length).
hipError_t launch_topk(const float *scores, int64_t ld, const int32_t *n_valid, int32_t n_cap, int32_t T,
                       int32_t k, int32_t *idx, hipStream_t s);
// Fused prefill selection; cand: prefill_candidate_bytes(L) of scratch.
size_t prefill_candidate_bytes(int32_t L);
hipError_t launch_prefill_indexer_topk(const uint8_t *q8, const float *qs, const uint8_t *k8,
                                       const float *ks, const float *w, int32_t L, int32_t k,
                                       int32_t *idx, uint32_t *cand, hipStream_t s);
// Sparse MLA.  block_table != NULL: idx holds logical positions of sequence
// t (page size 64); otherwise idx holds rows of kv.  Entries that do not map
// to a row in [0, N) are skipped like -1.  splits > 1 needs the
// partial buffers (part_o [T,splits,H,512] f32, part_ml [T,splits,H,2] f32).
hipError_t launch_sparse_mla_bf16(const void *q, const void *kv, const int32_t *idx,
                                  const int32_t *block_table, int32_t max_blocks, int64_t N, int32_t T,
                                  int32_t H, int32_t k, float sm_scale, void *out, float *lse,
                                  int32_t splits, void *part_o, float *part_ml, hipStream_t s);
hipError_t launch_sparse_mla_f32(const float *q, const float *kv, const int32_t *idx, int64_t N, int32_t T,
                                 int32_t H, int32_t k, float sm_scale, float *out, float *lse,
                                 hipStream_t s);
hipError_t launch_decode_indexer(const uint8_t *q8, const float *qs, const float *w,
                                 const uint8_t *k8_pool, const float *ks_pool,
                                 const int32_t *block_table, int32_t max_blocks,
                                 const int32_t *ctx_len, int32_t B, int32_t max_ctx, int64_t n_pool_rows,
                                 float *scores, int64_t ld, hipStream_t s);
// Masked MHA in MLA's multi-head form (BF16; per head 128 + 64 logit dims,
// 128 value dims, latent 512 + 64).  workspace: masked_mha_workspace_bytes(L, H).
size_t masked_mha_workspace_bytes(int32_t L, int32_t H);
hipError_t launch_masked_mha(const void *q, const void *kv, const void *w_uk, const void *w_uv,
                             const int32_t *idx, int32_t L, int32_t H, int32_t k, float sm_scale, void *out,
                             float *lse, void *workspace, hipStream_t s);
// Index scores at listed positions (E4M3, D_I = 128, H_I 32 or 64) and the
// indexer KL-alignment loss (H / 16 in {1, 2, 4, 8}, k <= 2048).
hipError_t launch_indexer_scores_at(const uint8_t *q8, const float *qs, const uint8_t *k8, const float *ks,
                                    const float *w, const int32_t *idx, int32_t T, int32_t S, int32_t H_I, int32_t k,
                                    float *out, hipStream_t s);
hipError_t launch_indexer_kl(const void *q, const void *kv, const int32_t *idx, const float *scores, const float *lse,
                             int64_t N, int32_t T, int32_t H, int32_t k, float sm_scale, float *kl, hipStream_t s);
hipError_t launch_positions(int32_t *q_pos, int32_t *n_valid, int32_t L, hipStream_t s);
hipError_t launch_cache_append(const void *latent, const uint8_t *k8, const float *ks,
                               const int32_t *pos, int32_t B, int32_t D_I,
                               const int32_t *block_table, int32_t max_blocks, int64_t n_pool_rows,
                               void *kv_pool, uint8_t *k8_pool, float *ks_pool, hipStream_t s);
}  // namespace dsa
