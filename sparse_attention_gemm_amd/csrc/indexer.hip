// Unfused lightning-indexer scores: the full [T, S] score matrix.
//
// Used for decode-sized problems, for the tiny fp32 workload and to check the
// fused prefill kernel stage by stage.  Scores of keys the query may not see
// (s > q_pos[t]) are written as -inf.
#include "dsa_common.h"
#include "dsa_launch.h"
#include "indexer_core.h"

namespace {

constexpr int kTilesPerWave = 8;  // 512 keys per wave: amortises the query load

// grid: (ceil(S / (64*kTilesPerWave)), ceil(T/4)); 4 waves, one token each.
// NHALF head halves of 32 (H_I = 32 * NHALF).
template <int NHALF>
__global__ __launch_bounds__(256) void indexer_scores_fp8_kernel(
    const uint8_t *__restrict__ q8, const float *__restrict__ qs, const uint8_t *__restrict__ k8,
    const float *__restrict__ ks, const float *__restrict__ w, const int32_t *__restrict__ q_pos,
    int32_t T, int32_t S, float *__restrict__ scores, int64_t ld) {
  constexpr int H_I = 32 * NHALF;
  __shared__ uint8_t qscratch[4][kQueryScratch];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = blockIdx.y * 4 + wave;
  if (t >= T) return;
  const int p = q_pos[t];
  float *orow = scores + (int64_t)t * ld;
  const int sbeg = blockIdx.x * 64 * kTilesPerWave;
  const int send = min(S, sbeg + 64 * kTilesPerWave);
  if (sbeg > p) {
    for (int s = sbeg + lane; s < send; s += 64) orow[s] = -INFINITY;
    return;
  }
  IdxQuery<2 * NHALF> Q;
  idx_load_query<2 * NHALF>(Q, q8 + (int64_t)t * H_I * 128, w + (int64_t)t * H_I, qs[t], lane, qscratch[wave]);
  const int g = lane >> 4, c = lane & 15;
  for (int s0 = sbeg; s0 < send; s0 += 64) {
    const int s = s0 + lane;
    if (s0 > p) {
      if (s < send) orow[s] = -INFINITY;
      continue;
    }
    i32x8 b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int key = min(s0 + 16 * u + c, S - 1);
      b[u] = *reinterpret_cast<const i32x8 *>(k8 + (int64_t)key * 128 + 32 * g);
    }
    const float tot = idx_score64<2 * NHALF>(Q, b);
    if (s < send) orow[s] = (s <= p) ? canon_zero(tot * ks[s]) : -INFINITY;
  }
}

// Any other E4M3 shape (H_I <= 64 heads, D_I <= 128): the products of the
// E4M3 payloads are exact in fp32 and are summed with IEEE fp32 fused
// multiply-adds in dimension order, then the heads in order, then the two
// scales.  (The FP8 MFMA of the full-size kernel sums its 128 products with a
// coarser internal alignment; these small shapes are off the hot path and
// keep plain fp32 sums.)  grid: (ceil(S/64), ceil(T/4)); each thread owns one
// (t, s); keys are staged in LDS as floats with a padded row.
constexpr int kF32MaxD = 128;
__global__ __launch_bounds__(256) void indexer_scores_fp8_fma_kernel(
    const uint8_t *__restrict__ q8, const float *__restrict__ qs, const uint8_t *__restrict__ k8,
    const float *__restrict__ ks, const float *__restrict__ w, const int32_t *__restrict__ q_pos, int32_t T,
    int32_t S, int32_t H_I, int32_t D_I, float *__restrict__ scores, int64_t ld) {
  __shared__ float kt[64][kF32MaxD + 1];
  const int s0 = blockIdx.x * 64;
  for (int i = threadIdx.x; i < 64 * D_I; i += 256) {
    const int r = i / D_I, d = i - r * D_I;
    const int s = s0 + r;
    kt[r][d] = s < S ? __builtin_amdgcn_cvt_f32_fp8(k8[(int64_t)s * D_I + d], 0) : 0.0f;
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.y * 4 + wave;
  const int s = s0 + lane;
  if (t >= T || s >= S) return;
  const int p = q_pos[t];
  if (s > p) {
    scores[(int64_t)t * ld + s] = -INFINITY;
    return;
  }
  const uint8_t *qt = q8 + (int64_t)t * H_I * D_I;
  float acc = 0.0f;
  for (int j = 0; j < H_I; ++j) {
    float dot = 0.0f;
    for (int d = 0; d < D_I; ++d) dot = fmaf(__builtin_amdgcn_cvt_f32_fp8(qt[j * D_I + d], 0), kt[lane][d], dot);
    acc = fmaf(w[(int64_t)t * H_I + j], fmaxf(dot, 0.0f), acc);
  }
  scores[(int64_t)t * ld + s] = canon_zero(acc * (qs[t] * ks[s]));
}

// fp32 operands (no quantisation).  Same grid and staging.
__global__ __launch_bounds__(256) void indexer_scores_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ w,
    const int32_t *__restrict__ q_pos, int32_t T, int32_t S, int32_t H_I, int32_t D_I,
    float *__restrict__ scores, int64_t ld) {
  __shared__ float kt[64][kF32MaxD + 1];
  const int s0 = blockIdx.x * 64;
  for (int i = threadIdx.x; i < 64 * D_I; i += 256) {
    const int r = i / D_I, d = i - r * D_I;
    const int s = s0 + r;
    kt[r][d] = s < S ? k[(int64_t)s * D_I + d] : 0.0f;
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.y * 4 + wave;
  const int s = s0 + lane;
  if (t >= T || s >= S) return;
  const int p = q_pos[t];
  if (s > p) {
    scores[(int64_t)t * ld + s] = -INFINITY;
    return;
  }
  const float *qt = q + (int64_t)t * H_I * D_I;
  float acc = 0.0f;
  for (int j = 0; j < H_I; ++j) {
    float dot = 0.0f;
    for (int d = 0; d < D_I; ++d) dot = fmaf(qt[j * D_I + d], kt[lane][d], dot);
    acc = fmaf(w[(int64_t)t * H_I + j], fmaxf(dot, 0.0f), acc);
  }
  scores[(int64_t)t * ld + s] = canon_zero(acc);
}

}  // namespace

namespace dsa {
hipError_t launch_indexer_scores_fp8(const uint8_t *q, const float *qs, const uint8_t *k,
                                     const float *ks, const float *w, const int32_t *q_pos,
                                     int32_t T, int32_t S, int32_t H_I, int32_t D_I, float *scores, int64_t ld,
                                     hipStream_t s) {
  if (T == 0 || S == 0) return hipSuccess;
  dim3 grid((S + 64 * kTilesPerWave - 1) / (64 * kTilesPerWave), (T + 3) / 4);
  if (D_I != 128 || (H_I != 32 && H_I != 64)) {
    hipLaunchKernelGGL(indexer_scores_fp8_fma_kernel, dim3((S + 63) / 64, (T + 3) / 4), dim3(256), 0, s, q, qs, k, ks,
                       w, q_pos, T, S, H_I, D_I, scores, ld);
    return hipGetLastError();
  }
  if (H_I == 64)
    hipLaunchKernelGGL(indexer_scores_fp8_kernel<2>, grid, dim3(256), 0, s, q, qs, k, ks, w, q_pos, T, S,
                       scores, ld);
  else
    hipLaunchKernelGGL(indexer_scores_fp8_kernel<1>, grid, dim3(256), 0, s, q, qs, k, ks, w, q_pos, T, S,
                       scores, ld);
  return hipGetLastError();
}

hipError_t launch_indexer_scores_f32(const float *q, const float *k, const float *w,
                                     const int32_t *q_pos, int32_t T, int32_t S, int32_t H_I,
                                     int32_t D_I, float *scores, int64_t ld, hipStream_t s) {
  if (T == 0 || S == 0) return hipSuccess;
  dim3 grid((S + 63) / 64, (T + 3) / 4);
  hipLaunchKernelGGL(indexer_scores_f32_kernel, grid, dim3(256), 0, s, q, k, w, q_pos, T, S, H_I, D_I,
                     scores, ld);
  return hipGetLastError();
}
}  // namespace dsa
