// Backward of the lightning indexer for its KL-alignment loss.
//
// In sparse training the indexer's input is detached and the indexer is
// trained by the KL loss alone (mizuki-eaf.pages.dev, two-stage continued
// pre-training / sparse training; m.36881.com.cn, sparse training).  Given
// the gradient g[t, a] of the loss with respect to the index score of entry a
// of query t (dsa_indexer_kl_bwd), the score
//     I[t, a] = sum_j w[t,j] ReLU(x_ja),   x_ja = (qs q8[t,j]) . (ks k8[r_a])
// gives, with respect to the head weights and the dequantised query and key
// (the FP8 encoding is passed straight through):
//     dw[t, j]   = sum_a g_a ReLU(x_ja)
//     dq[t, j]   = sum_a g_a w_j [x_ja > 0] ks_a k8_a
//     u[t, a]    = g_a qs sum_j w_j [x_ja > 0] q8_j      (the pair's share of dk[r_a])
// dk[r] is then the sum of u over the pairs that selected r, taken by the
// deterministic inverted-selection reduce (scatter.hip).
//
// indexer_bwd_kernel: one workgroup of four waves per query, 64 entries per
// tile; wave w owns heads 16 w .. 16 w + 15.  Per tile:
//  * x^T (keys x the wave's heads) = K8 Q8^T on the FP8 MFMA, exactly as in
//    the forward (E4M3 x E4M3 products, the matrix core's fp32 sum); the lane holding x for
//    head c and keys 4 g + r (+16 n) forms the coefficients
//    mc = g ks w [x > 0] and nc = w [x > 0] and its dw partial;
//  * dq (the wave's heads x 128 dims) += MC KF on the bf16 MFMA: the E4M3
//    payload KF is exact in bf16, and mc is split into two bf16 terms
//    (hi + lo, relative residue below 2^-17), so each product carries far less
//    error than the fp32 sums; KF comes from LDS through the transposing
//    read, MC straight from the x^T lanes (the MFMA output layout is the A
//    operand layout, up to a fixed key permutation both operands share);
//  * u^T (128 dims x the wave's 16 keys) = QF^T NC^T: QF^T (the query's
//    payload, exact in bf16) is held in registers for the whole query and NC
//    (hi + lo) passes through LDS, from the wave that owns a head to the
//    wave that owns a key; each lane stores 4 dims of one key's u row.
// The query's selection and score gradient sit in LDS; each tile's key rows
// are fetched one tile ahead and written to LDS after the tile's last read
// of them.
#include "dsa_common.h"
#include "dsa_launch.h"
#include "indexer_core.h"

namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kHI = 64, kDI = 128, kTile = 64;
constexpr int kK8Row = kDI + 16;      // LDS bytes per E4M3 key row (36 dwords: conflict-free 32-byte reads)
constexpr int kBfRow = 2 * kDI + 32;  // LDS bytes per bf16 row of 128 (8 dwords apart mod 64 for the
                                      // transposing read)
constexpr int kNcRow = 2 * kHI + 16;  // LDS bytes per key of nc (bf16 x 64 heads)
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format
constexpr int kCpolNT = 2;                    // cache policy: streaming (non-temporal)

struct IdxBwdSmem {
  uint8_t k8t[kTile * kK8Row];   // the tile's E4M3 key rows
  uint8_t kf[kTile * kBfRow];    // their payload as bf16 (also the query's payload during set-up)
  uint8_t nch[kTile * kNcRow];   // nc = w [x > 0], bf16 hi part, [key][head]
  uint8_t ncl[kTile * kNcRow];   // ... and lo part
  int32_t sidx[DSA_MAX_K];       // the query's selection
  float sg[DSA_MAX_K];           // and score gradient
  float gk[kTile];               // g_a ks_a of the tile's entries (0 where invalid)
  float ga[kTile];               // g_a (0 where invalid)
};

// The four E4M3 bytes of `four`, in memory order, as bf16 bit patterns packed
// in two words (exact: an E4M3 value has at most 4 significant bits, so its
// fp32 form has zero low halves).
__device__ __forceinline__ i32x2 e4m3x4_to_bf16x4(int four) {
  const uint32_t a = __float_as_uint(__builtin_amdgcn_cvt_f32_fp8(four, 0));
  const uint32_t b = __float_as_uint(__builtin_amdgcn_cvt_f32_fp8(four, 1));
  const uint32_t c = __float_as_uint(__builtin_amdgcn_cvt_f32_fp8(four, 2));
  const uint32_t d = __float_as_uint(__builtin_amdgcn_cvt_f32_fp8(four, 3));
  return i32x2{(int)((a >> 16) | (b & 0xFFFF0000u)), (int)((c >> 16) | (d & 0xFFFF0000u))};
}

// bf16 of v rounded to nearest even, and the bf16 of what remains.
__device__ __forceinline__ void split_bf16(float v, __bf16 &hi, __bf16 &lo) {
  hi = (__bf16)v;
  lo = (__bf16)(v - (float)hi);
}

// A operand of a 16x16x32 MFMA from a row-major [K rows][M cols] bf16 matrix
// in LDS: lane (g, c) gets column m0 + c, rows k0 + 8 g .. + 8.
__device__ __forceinline__ bf16x8 tr_rows8(const uint8_t *base, int row_bytes, int k0, int m0, int g, int c) {
  const uint8_t *p = base + (k0 + 8 * g + (c >> 2)) * row_bytes + (m0 + 4 * (c & 3)) * 2;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 4 * row_bytes));
  const i16x4 lohi[2] = {lo, hi};
  return *reinterpret_cast<const bf16x8 *>(lohi);
}

// B operand from the same kind of matrix with the K order of an x^T lane:
// lane (g, c) gets column m0 + c, rows k0 + 4 g .. + 4 and k0 + 16 + 4 g .. + 4.
__device__ __forceinline__ bf16x8 tr_rows4x2(const uint8_t *base, int row_bytes, int k0, int m0, int g, int c) {
  const uint8_t *p = base + (k0 + 4 * g + (c >> 2)) * row_bytes + (m0 + 4 * (c & 3)) * 2;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 16 * row_bytes));
  const i16x4 lohi[2] = {lo, hi};
  return *reinterpret_cast<const bf16x8 *>(lohi);
}

__global__ __launch_bounds__(256, 2) void indexer_bwd_kernel(const uint8_t *__restrict__ q8, const float *__restrict__ qs,
                                                             const uint8_t *__restrict__ k8, const float *__restrict__ ks,
                                                             const float *__restrict__ w, const int32_t *__restrict__ idx,
                                                             const float *__restrict__ grad, int64_t t0, int S, int k,
                                                             float *__restrict__ dw, float *__restrict__ dq,
                                                             float *__restrict__ u) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  IdxBwdSmem &sm = *reinterpret_cast<IdxBwdSmem *>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tc = blockIdx.x;  // query within the chunk
  const int64_t t = t0 + tc;
  const uint8_t *qrow = q8 + t * kHI * kDI;
  const float qsv = qs[t];
  const int head = 16 * wave + c;  // this lane's head in x^T and in the dq product
  const float wv = w[t * kHI + head];
  // set-up: the query payload as bf16, row-major [head][dim]; the selection and score gradient
  for (int e = tid; e < kHI * kDI / 4; e += 256) {
    const int four = *reinterpret_cast<const int *>(qrow + 4 * e);
    const int j = (4 * e) / kDI, d = (4 * e) % kDI;
    *reinterpret_cast<i32x2 *>(sm.kf + j * kBfRow + 2 * d) = e4m3x4_to_bf16x4(four);
  }
  for (int a = tid; a < k; a += 256) {
    sm.sidx[a] = idx[t * k + a];
    sm.sg[a] = grad[t * k + a];
  }
  const i32x8 qb = *reinterpret_cast<const i32x8 *>(qrow + head * kDI + 32 * g);  // B of x^T: head c, dims 32 g ..
  __syncthreads();
  // QF^T, the A operand of u^T: dims 16 i + c, heads 32 s + 8 g .. +8
  bf16x8 qfT[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int s = 0; s < 2; ++s) qfT[i][s] = tr_rows8(sm.kf, kBfRow, 32 * s, 16 * i, g, c);
  __syncthreads();  // kf is free

  // one tile ahead: this thread's two 16-byte pieces of the tile's key rows, and (tid < 64) one entry's ks
  i32x4 pk[2];
  float pks = 0.0f;
  auto fetch = [&](int a0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid + 256 * i, a = a0 + (e >> 3);
      const int32_t r = a < k ? sm.sidx[a] : -1;
      const int64_t rr = (r >= 0 && r < S) ? r : 0;
      pk[i] = *reinterpret_cast<const i32x4 *>(k8 + rr * kDI + (e & 7) * 16);
    }
    if (tid < kTile) {
      const int a = a0 + tid;
      const int32_t r = a < k ? sm.sidx[a] : -1;
      pks = ks[(r >= 0 && r < S) ? r : 0];
    }
  };
  auto put = [&](int a0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid + 256 * i, key = e >> 3, part = e & 7;
      *reinterpret_cast<i32x4 *>(sm.k8t + key * kK8Row + part * 16) = pk[i];
      i32x4 lo, hi;
      const i32x2 b0 = e4m3x4_to_bf16x4(pk[i][0]), b1 = e4m3x4_to_bf16x4(pk[i][1]);
      const i32x2 b2 = e4m3x4_to_bf16x4(pk[i][2]), b3 = e4m3x4_to_bf16x4(pk[i][3]);
      lo = i32x4{b0[0], b0[1], b1[0], b1[1]};
      hi = i32x4{b2[0], b2[1], b3[0], b3[1]};
      *reinterpret_cast<i32x4 *>(sm.kf + key * kBfRow + part * 32) = lo;
      *reinterpret_cast<i32x4 *>(sm.kf + key * kBfRow + part * 32 + 16) = hi;
    }
    if (tid < kTile) {
      const int a = a0 + tid;
      const int32_t r = a < k ? sm.sidx[a] : -1;
      const float gv = (r >= 0 && r < S) ? sm.sg[a] : 0.0f;
      sm.gk[tid] = gv * pks;
      sm.ga[tid] = gv;
    }
  };

  const int ntile = (k + kTile - 1) / kTile;
  // u rows of this query as a bounded buffer: stores of entries >= k are dropped
  f32x4 dqa[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) dqa[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dwp = 0.0f;  // sum over this lane's keys of g ks max(x, 0), for head c
  fetch(0);
  put(0);
  if (ntile > 1) fetch(kTile);
  __syncthreads();
  for (int j = 0; j < ntile; ++j) {
    const int a0 = j * kTile;
    // x^T for the wave's heads: lane (g, c) gets keys 16 n + 4 g + r of head c
    f32x4 xo[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const i32x8 ka = *reinterpret_cast<const i32x8 *>(sm.k8t + (16 * n + c) * kK8Row + 32 * g);
      xo[n] = mfma_fp8_16x16x128(ka, qb, f32x4{0.f, 0.f, 0.f, 0.f});
    }
    // coefficients; mc as the A operand of the dq product (K-step s: keys 32 s + 4 g + r, 32 s + 16 + 4 g + r)
    bf16x8 mh[2], ml[2];
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = 16 * n + 4 * g + r;
        const float x = xo[n][r], gkv = sm.gk[key];
        const bool pos = x > 0.0f;  // qs, ks > 0: the sign of the payload dot
        dwp = fmaf(gkv, pos ? x : 0.0f, dwp);
        __bf16 h, l;
        split_bf16(pos ? gkv * wv : 0.0f, h, l);
        mh[n >> 1][4 * (n & 1) + r] = h;
        ml[n >> 1][4 * (n & 1) + r] = l;
        split_bf16(pos ? wv : 0.0f, h, l);
        *reinterpret_cast<__bf16 *>(sm.nch + key * kNcRow + 2 * head) = h;
        *reinterpret_cast<__bf16 *>(sm.ncl + key * kNcRow + 2 * head) = l;
      }
    // dq (heads 16 wave + 4 g + r, dims 16 i + c) += MC KF
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16x8 b = tr_rows4x2(sm.kf, kBfRow, 32 * s, 16 * i, g, c);
        dqa[i] = mfma_bf16_16x16x32(mh[s], b, dqa[i]);
        dqa[i] = mfma_bf16_16x16x32(ml[s], b, dqa[i]);
      }
    const float usc = sm.ga[16 * wave + c] * qsv;  // scale of this lane's u column (key 16 wave + c)
    // nc is complete; the tile's key rows and coefficients are no longer read.
    // LDS only: the previous tile's u stores and the prefetched rows stay in
    // flight (put() waits for its own registers).
    lds_barrier();
    if (j + 1 < ntile) {
      put(a0 + kTile);
      if (j + 2 < ntile) fetch(a0 + 2 * kTile);
    }
    // u^T (dims 16 i + 4 g + r, key 16 wave + c) = QF^T NC^T
    const uint8_t *nh = sm.nch + (16 * wave + c) * kNcRow + 16 * g;
    const uint8_t *nl = sm.ncl + (16 * wave + c) * kNcRow + 16 * g;
    f32x4 ua[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ua[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8 bh = *reinterpret_cast<const bf16x8 *>(nh + 64 * s);
      const bf16x8 bl = *reinterpret_cast<const bf16x8 *>(nl + 64 * s);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ua[i] = mfma_bf16_16x16x32(qfT[i][s], bh, ua[i]);
        ua[i] = mfma_bf16_16x16x32(qfT[i][s], bl, ua[i]);
      }
    }
    const int off = ((a0 + 16 * wave + c) * kDI + 4 * g) * 4;
    // built here from scalar values, so the descriptor stays in SGPRs (one
    // held across the loop was kept in VGPRs and each store became a loop)
    const __amdgpu_buffer_rsrc_t ur =
        __builtin_amdgcn_make_buffer_rsrc((void *)(u + tc * k * kDI), 0, k * kDI * 4, (int)kRsrcWord3);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, ua[i] * usc), ur, off + 64 * i, 0, kCpolNT);
    lds_barrier();  // nc is no longer read; the next tile's rows are in LDS (the u stores stay in flight)
  }
  // dq of heads 16 wave + 4 g + r
  float *dqrow = dq + (t * kHI + 16 * wave + 4 * g) * kDI + c;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) dqrow[r * kDI + 16 * i] = dqa[i][r];
  // dw of head c: the lane's partials over its keys, summed over the four key groups
  float v = dwp;
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  if (g == 0) dw[t * kHI + head] = v * qsv;
}

}  // namespace

namespace dsa {
size_t indexer_bwd_smem_bytes() { return sizeof(IdxBwdSmem); }

hipError_t launch_indexer_bwd_chunk(const uint8_t *q8, const float *qs, const uint8_t *k8, const float *ks,
                                    const float *w, const int32_t *idx, const float *grad, int64_t t0, int32_t Tc,
                                    int32_t S, int32_t k, float *dw, float *dq, float *u, hipStream_t s) {
  if (Tc <= 0) return hipSuccess;
  static bool attr_done = false;  // per process: the attribute holds for every device
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void *)indexer_bwd_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)sizeof(IdxBwdSmem));
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  hipLaunchKernelGGL(indexer_bwd_kernel, dim3(Tc), dim3(256), sizeof(IdxBwdSmem), s, q8, qs, k8, ks, w, idx, grad, t0,
                     S, k, dw, dq, u);
  return hipGetLastError();
}
}  // namespace dsa
