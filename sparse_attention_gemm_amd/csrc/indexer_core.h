// indexer_core.h -- the FP8 lightning-indexer score of one query token against
// a 64-key tile, on gfx950 MFMA.
//
// Score (index score of mizuki-eaf.pages.dev, "How it works"; ReLU and FP8
// there, the head-weighted form is the workload's definition):
//     I[t,s] = sum_j w[t,j] * ReLU(qs[t] ks[s] <q8[t,j], k8[s]>)
//            = ks[s] * sum_j (w[t,j] qs[t]) * ReLU(<q8[t,j], k8[s]>)    (qs, ks > 0)
// The dot products are E4M3 x E4M3 MFMAs (32x32x64, exact products, fp32
// sums); D_I = 128 is two K steps.  Heads run along the MFMA rows (32 per
// tile), keys along the columns.  Each lane then holds 16 heads of one key
// per head tile and applies ReLU and its head weights in registers; the two
// lane halves hold complementary heads and are combined with one
// permlane32 swap, which also scatters the 64 keys of the tile one per lane.
//
// Every kernel that produces index scores goes through idx_score64(), so the
// unfused score matrix and the fused streaming top-k see identical values.
#pragma once
#include "dsa_common.h"

template <int NHT>  // head tiles of 32: H_I = 32 * NHT
struct IdxQuery {
  i32x8 a[NHT][2];     // A operand: q8 rows (heads) x 64-byte K steps
  float w[NHT][16];    // head weight (times q scale) of this lane's 16 rows per tile
};

// q8_t: the token's [H_I][128] payload; w_t: its [H_I] weights.
template <int NHT>
__device__ __forceinline__ void idx_load_query(IdxQuery<NHT> &Q, const uint8_t *__restrict__ q8_t,
                                               const float *__restrict__ w_t, float qs, int lane) {
  const int row = lane & 31, half = lane >> 5;
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      Q.a[ht][ks] = *reinterpret_cast<const i32x8 *>(q8_t + (ht * 32 + row) * 128 + ks * 64 + half * 32);
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int head = ht * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
      Q.w[ht][r] = w_t[head] * qs;
    }
}

// b[u][ks]: B operand of sub-tile u (keys u*32 + lane%32), bytes ks*64 + (lane/32)*32.
// Returns, in lane l, sum_j w'_j ReLU(<q8_j, k8[key l of the tile]>) (without ks).
template <int NHT>
__device__ __forceinline__ float idx_score64(const IdxQuery<NHT> &Q, const i32x8 (&b)[2][2]) {
  float part[2];
  f32x16 c[2][NHT];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      f32x16 z = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      z = mfma_fp8_32x32x64(Q.a[ht][0], b[u][0], z);
      c[u][ht] = mfma_fp8_32x32x64(Q.a[ht][1], b[u][1], z);
    }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    float p = 0.0f;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
      for (int r = 0; r < 16; ++r) p = fmaf(Q.w[ht][r], fmaxf(c[u][ht][r], 0.0f), p);
    part[u] = p;
  }
  // lanes 0-31: sub-tile 0 summed over both halves; lanes 32-63: sub-tile 1.
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[1]), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}
