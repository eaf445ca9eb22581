// indexer_core.h -- the FP8 lightning-indexer score of one query token against
// a 64-key tile, on gfx950 MFMA.
//
// Score (index score of mizuki-eaf.pages.dev, "How it works"; ReLU and FP8
// there, the head-weighted form is the workload's definition):
//     I[t,s] = sum_j w[t,j] * ReLU(qs[t] ks[s] <q8[t,j], k8[s]>)
//            = ks[s] * sum_j (w[t,j] qs[t]) * ReLU(<q8[t,j], k8[s]>)    (qs, ks > 0)
// The dot products are E4M3 x E4M3 MFMAs (16x16x128: the whole D_I = 128 in
// one instruction; products exact, fp32 sums).  Heads run along the MFMA
// rows, keys along the columns: lane (g = l/16, c = l%16) receives 4 heads
// (4g..4g+3 of a 16-head tile) of key c and applies ReLU and its head
// weights in registers.  A 64-key tile is 4 key blocks of 16; the four lane
// groups' partial sums are then reduce-scattered with two permlane swaps so
// that lane l ends up with key l of the tile.
//
// Heads are processed in halves of 32 (two 16-head tiles).  The score of a
// key is   half(heads 0..31) + half(heads 32..63),   each half with a fixed
// accumulation order, so a kernel that splits the halves across two
// wavefronts produces exactly the same fp32 value as one that computes both.
#pragma once
#include "dsa_common.h"

// FP8 MFMA 16x16x128 (E4M3 x E4M3): lane l holds A[row l%16][k 32(l/16) .. +32]
// and B[k ..][col l%16]; register r of the result is D[4(l/16) + r][l%16].
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(const i32x8 &a, const i32x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// x + (the same register of lane l^32), for two registers at once: returns
// lanes 0-31: x[l] + x[l+32];  lanes 32-63: y[l-32] + y[l].
__device__ __forceinline__ float swap32_sum(float x, float y) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Same across 16-lane rows: rows 0,2 get x summed with the next row, rows 1,3
// get y summed with the previous row.
__device__ __forceinline__ float swap16_sum(float x, float y) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ReLU of an MFMA dot product.  fmaxf would first quiet a possible signalling
// NaN (one extra v_max per element); the products of finite E4M3 payloads are
// finite and far below FLT_MAX, so a clamp to [0, FLT_MAX] is the same
// function in a single v_med3.
__device__ __forceinline__ float relu_dot(float d) { return __builtin_amdgcn_fmed3f(d, 0.0f, 3.402823466e38f); }

// One half (32 heads) of a query's indexer heads.
struct IdxHalf {
  i32x8 a[2];      // A operand: 16-head tiles x 128 bytes
  float w[2][4];   // head weight (times q scale) of this lane's 4 rows per tile
};

// q8_t: the token's [H_I][128] payload; w_t its [H_I] weights; head0: first head of the half.
__device__ __forceinline__ void idx_load_half(IdxHalf &Q, const uint8_t *__restrict__ q8_t,
                                              const float *__restrict__ w_t, float qs, int head0, int lane) {
  const int g = lane >> 4, c = lane & 15;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    Q.a[i] = *reinterpret_cast<const i32x8 *>(q8_t + (head0 + 16 * i + c) * 128 + 32 * g);
#pragma unroll
    for (int r = 0; r < 4; ++r) Q.w[i][r] = w_t[head0 + 16 * i + 4 * g + r] * qs;
  }
}

// b[u]: B operand of key block u (keys 16u + lane%16), bytes 32*(lane/16) .. +32.
// Returns, in lane l, sum over the half's heads of w' ReLU(<q8_j, k8[key l]>) (without ks).
__device__ __forceinline__ float idx_half_score64(const IdxHalf &Q, const i32x8 (&b)[4]) {
  f32x4 d[4][2];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int i = 0; i < 2; ++i) d[u][i] = mfma_fp8_16x16x128(Q.a[i], b[u], f32x4{0.f, 0.f, 0.f, 0.f});
  float v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float p = 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) p = fmaf(Q.w[i][r], relu_dot(d[u][i][r]), p);
    v[u] = p;
  }
  // lane groups g = 0..3 hold 4 heads each of the same keys: sum them, and
  // scatter the four key blocks so that lane l holds key l
  const float s02 = swap32_sum(v[0], v[2]);  // rows 0,1: block 0 (g, g+2); rows 2,3: block 2
  const float s13 = swap32_sum(v[1], v[3]);  // rows 0,1: block 1;          rows 2,3: block 3
  return swap16_sum(s02, s13);               // row 0: block 0, row 1: block 1, row 2: block 2, row 3: block 3
}

// Both halves of a 64-head query against a 64-key tile: returns, in lane l,
// half(0..31) + half(32..63) of key l (without ks) -- the same operations in
// the same order as two idx_half_score64 calls.  The issue order is fixed
// (scheduling fences, and an empty asm that pins each partial sum): each MFMA
// of key block u is followed by the ReLU/weight epilogue of one MFMA result of block u-1, so the matrix core
// and the VALU overlap within the wave and no result is waited for.
__device__ __forceinline__ float idx_full_score64(const IdxHalf &Q0, const IdxHalf &Q1, const i32x8 (&b)[4]) {
  const IdxHalf *Q[2] = {&Q0, &Q1};
  f32x4 d[2][2][2];  // [block parity][half][head tile]
  float p[2] = {0.0f, 0.0f};
  float v[2][4];
#pragma unroll
  for (int u = 0; u <= 4; ++u) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int h = m >> 1, i = m & 1;
      if (u < 4) d[u & 1][h][i] = mfma_fp8_16x16x128(Q[h]->a[i], b[u], f32x4{0.f, 0.f, 0.f, 0.f});
      __builtin_amdgcn_sched_barrier(0);
      if (u > 0) {
        const f32x4 &dd = d[(u - 1) & 1][h][i];
#pragma unroll
        for (int r = 0; r < 4; ++r) p[h] = fmaf(Q[h]->w[i][r], relu_dot(dd[r]), p[h]);
        asm volatile("" : "+v"(p[h]));  // computed here, not sunk below later MFMAs
        if (i == 1) {
          v[h][u - 1] = p[h];
          p[h] = 0.0f;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float hs[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float s02 = swap32_sum(v[h][0], v[h][2]);
    const float s13 = swap32_sum(v[h][1], v[h][3]);
    hs[h] = swap16_sum(s02, s13);
  }
  return hs[0] + hs[1];
}

// B operands of a 64-key tile whose rows are `stride` bytes apart.
__device__ __forceinline__ void idx_load_keys(i32x8 (&b)[4], const uint8_t *__restrict__ rows, int stride, int lane) {
  const int g = lane >> 4, c = lane & 15;
#pragma unroll
  for (int u = 0; u < 4; ++u) b[u] = *reinterpret_cast<const i32x8 *>(rows + (16 * u + c) * stride + 32 * g);
}
