// indexer_core.h -- the FP8 lightning-indexer score of one query token against
// a 64-key tile, on gfx950 MFMA.
//
// Score (index score of mizuki-eaf.pages.dev, "How it works"; ReLU and FP8
// there, the head-weighted form is the workload's definition):
//     I[t,s] = sum_j w[t,j] * ReLU(qs[t] ks[s] <q8[t,j], k8[s]>)
//            = ks[s] * sum_j w'_j ReLU(D_j),   w'_j = w[t,j] qs[t],  D_j = <q8[t,j], k8[s]>
// (qs, ks > 0).  With ReLU(x) = (x + |x|) / 2 the head sum splits into
//     sum_j (w'_j / 2) |D_j|   +   (1/2) <qbar, k8[s]>,   qbar = sum_j w'_j q8[t,j]
// The first part costs one fused multiply-add per (head, key) with an
// absolute-value source modifier (instead of a ReLU and a multiply-add); the
// linear part is one more E4M3 MFMA per 16 keys, whose A tile holds qbar
// (computed once per query in fp32) as six E4M3 pieces with power-of-two
// scales: qbar = sum_m 2^e_m P_m up to a residual below 2^-24 of max|qbar|.
// The dot products are E4M3 x E4M3 MFMAs (16x16x128: the whole D_I = 128 in
// one instruction; products exact, summed by the matrix core to an fp32
// result within 2^-12 of the sum of their magnitudes, not as a chain of IEEE
// fp32 additions).  Heads (or pieces) run along
// the MFMA rows, keys along the columns: lane (g = l/16, c = l%16) receives
// rows 4g..4g+3 of key c.  The four lane groups' partial sums of a 64-key
// tile are reduce-scattered with two permlane swaps so that lane l ends up
// with key l.  Every kernel scores through idx_score64 with the same query
// state, so fused and unfused paths give bit-identical scores.
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

constexpr int kLinPieces = 6;                    // E4M3 pieces of qbar
constexpr int kQueryScratch = kLinPieces * 128;  // LDS bytes per wave for idx_load_query

// One query token's indexer state for 16*NT heads (NT = 4: 64 heads).
template <int NT>
struct IdxQuery {
  i32x8 a[NT];      // A operand: 16-head tiles x 128 bytes
  float wh[NT][4];  // w' / 2 of this lane's 4 rows per tile
  i32x8 lin;        // A operand: rows 0..5 the pieces of qbar, other rows zero
  float sh[4];      // piece scale / 2 of this lane's rows of `lin` (0 for zero rows)
};

// q8_t: the token's [16*NT][128] payload; w_t its weights; scratch: this
// wave's kQueryScratch bytes of LDS (free again on return).
template <int NT>
__device__ __forceinline__ void idx_load_query(IdxQuery<NT> &Q, const uint8_t *__restrict__ q8_t,
                                               const float *__restrict__ w_t, float qs, int lane,
                                               uint8_t *scratch) {
  const int g = lane >> 4, c = lane & 15;
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    Q.a[i] = *reinterpret_cast<const i32x8 *>(q8_t + (16 * i + c) * 128 + 32 * g);
#pragma unroll
    for (int r = 0; r < 4; ++r) Q.wh[i][r] = (w_t[16 * i + 4 * g + r] * qs) * 0.5f;
  }
  // qbar over dims 2*lane, 2*lane+1, heads in order
  float q0 = 0.0f, q1 = 0.0f;
  for (int j = 0; j < 16 * NT; ++j) {
    const float wq = w_t[j] * qs;
    const int two = *reinterpret_cast<const uint16_t *>(q8_t + j * 128 + 2 * lane);
    q0 = fmaf(wq, __builtin_amdgcn_cvt_f32_fp8(two, 0), q0);
    q1 = fmaf(wq, __builtin_amdgcn_cvt_f32_fp8(two, 1), q1);
  }
  // pieces: scale 2^e with max|r| <= 448 * 2^e; P = RNE(r / 2^e); r -= 2^e P
  float shs[kLinPieces];
#pragma unroll
  for (int m = 0; m < kLinPieces; ++m) {
    const float amax = wave_max(fmaxf(fabsf(q0), fabsf(q1)));  // uniform
    int packed = 0;
    float s = 0.0f;
    if (amax > 0.0f) {
      int ex;
      const float f = frexpf(amax, &ex);            // amax = f 2^ex, f in [0.5, 1)
      const int e = ex - 9 + (f > 0.875f ? 1 : 0);  // 448 = 0.875 2^9
      s = ldexpf(1.0f, e);
      packed = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(q0, -e), ldexpf(q1, -e), 0, false);
      q0 = fmaf(-s, __builtin_amdgcn_cvt_f32_fp8(packed, 0), q0);
      q1 = fmaf(-s, __builtin_amdgcn_cvt_f32_fp8(packed, 1), q1);
    }
    shs[m] = 0.5f * s;
    *reinterpret_cast<uint16_t *>(scratch + m * 128 + 2 * lane) = (uint16_t)packed;
  }
  __builtin_amdgcn_wave_barrier();
  if (c < kLinPieces) {
    Q.lin = *reinterpret_cast<const i32x8 *>(scratch + c * 128 + 32 * g);
  } else {
    Q.lin = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int r = 0; r < 4; ++r) Q.sh[r] = g == 0 ? shs[r] : (g == 1 && r < kLinPieces - 4) ? shs[4 + r] : 0.0f;
}

// Score of a 64-key tile: returns, in lane l, sum_j w'_j ReLU(D_j) of key l
// (without ks).  get_b(u) yields the B operand of key block u (keys 16u +
// lane%16, bytes 32*(lane/16) .. +32); it is called in order u = 0..3, one
// block ahead of its MFMAs, and after_loads() right after the last call.  The
// MFMAs (per key block: the NT head tiles, then the pieces of qbar) issue in
// a fixed order; each result is consumed after the next MFMA has been
// issued, so the matrix core and the VALU overlap with two results live.
template <int NT, typename GetB, typename After>
__device__ __forceinline__ float idx_score64(const IdxQuery<NT> &Q, GetB &&get_b, After &&after_loads) {
  constexpr int NM = NT + 1;
  constexpr int NTOT = 4 * NM;
  f32x4 d[2];
  float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  i32x8 b[2];
  b[0] = get_b(0);
#pragma unroll
  for (int k = 0; k < NTOT + 1; ++k) {
    if (k < NTOT) {
      const int u = k / NM, m = k % NM;
      if (m == 0 && u + 1 < 4) {
        b[(u + 1) & 1] = get_b(u + 1);
        if (u + 1 == 3) after_loads();
      }
      d[k & 1] = mfma_fp8_16x16x128(m < NT ? Q.a[m < NT ? m : 0] : Q.lin, b[u & 1], f32x4{0.f, 0.f, 0.f, 0.f});
    }
    __builtin_amdgcn_sched_barrier(0);
    if (k >= 1) {
      const int kk = k - 1, u = kk / NM, m = kk % NM;
      const f32x4 dd = d[kk & 1];
      if (m < NT) {
#pragma unroll
        for (int r = 0; r < 4; ++r) p[u] = fmaf(Q.wh[m < NT ? m : 0][r], fabsf(dd[r]), p[u]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) p[u] = fmaf(Q.sh[r], dd[r], p[u]);
      }
      asm volatile("" : "+v"(p[u]));  // computed here, not sunk below later MFMAs
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // lane groups g = 0..3 hold rows 4g..4g+3 of the same keys: sum them, and
  // scatter the four key blocks so that lane l holds key l
  const float s02 = swap32_sum(p[0], p[2]);  // rows 0,1: block 0 (g, g+2); rows 2,3: block 2
  const float s13 = swap32_sum(p[1], p[3]);  // rows 0,1: block 1;          rows 2,3: block 3
  return swap16_sum(s02, s13);               // row 0: block 0, row 1: block 1, row 2: block 2, row 3: block 3
}

// The same with the four B operands already in registers.
template <int NT>
__device__ __forceinline__ float idx_score64(const IdxQuery<NT> &Q, const i32x8 (&b)[4]) {
  return idx_score64<NT>(Q, [&](int u) { return b[u]; }, [] {});
}

// B operands of a 64-key tile whose rows are `stride` bytes apart.
__device__ __forceinline__ void idx_load_keys(i32x8 (&b)[4], const uint8_t *__restrict__ rows, int stride, int lane) {
  const int g = lane >> 4, c = lane & 15;
#pragma unroll
  for (int u = 0; u < 4; ++u) b[u] = *reinterpret_cast<const i32x8 *>(rows + (16 * u + c) * stride + 32 * g);
}
