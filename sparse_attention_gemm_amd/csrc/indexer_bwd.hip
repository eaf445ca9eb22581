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
// tile.  The products x come from the FP8 MFMA exactly as in the forward
// (E4M3 x E4M3 products, fp32 sums): wave w computes the 64 heads against
// the tile's key block w.  The coefficients g ks w [x > 0] and w [x > 0] go
// to LDS; then each thread accumulates, in fp32, 32 dims of dq for one head
// (over the tile's keys) and 32 dims of u for one key (over the heads).
#include "dsa_common.h"
#include "dsa_launch.h"
#include "indexer_core.h"

namespace {

constexpr int kHI = 64, kDI = 128, kTile = 64, kCoefPad = kTile + 1;

// the four E4M3 bytes of `four`, in memory order, as fp32 (exact)
__device__ __forceinline__ f32x4 e4m3x4_to_f32(int four) {
  return f32x4{__builtin_amdgcn_cvt_f32_fp8(four, 0), __builtin_amdgcn_cvt_f32_fp8(four, 1),
               __builtin_amdgcn_cvt_f32_fp8(four, 2), __builtin_amdgcn_cvt_f32_fp8(four, 3)};
}

struct IdxBwdSmem {
  float qf[kHI][kDI];           // E4M3 payload of the query, as fp32
  float kf[kTile][kDI];         // E4M3 payload of the tile's keys, as fp32
  float mc[kHI][kCoefPad];      // g_a ks_a w_j [x_ja > 0]        (head-major)
  float nc[kTile][kCoefPad];    // w_j [x_ja > 0]                 (key-major)
  float ga[kTile];              // g of the tile's entries (0 where invalid)
  float dwred[4][kHI];          // per-wave dw partials
};

__global__ __launch_bounds__(256) void indexer_bwd_kernel(const uint8_t *__restrict__ q8, const float *__restrict__ qs,
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
  // the query payload as fp32 (LDS), and the four head tiles as MFMA A operands
  for (int e = tid; e < kHI * kDI / 4; e += 256) {
    const int four = *reinterpret_cast<const int *>(qrow + 4 * e);
    const int j = (4 * e) / kDI, d = (4 * e) % kDI;
    *reinterpret_cast<f32x4 *>(&sm.qf[j][d]) = e4m3x4_to_f32(four);
  }
  i32x8 qa[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) qa[m] = *reinterpret_cast<const i32x8 *>(qrow + (16 * m + c) * kDI + 32 * g);
  float wj[4][4];  // w of this lane's result rows: head 16 m + 4 g + r
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) wj[m][r] = w[t * kHI + 16 * m + 4 * g + r];
  float dwp[4][4] = {};  // dw partials of the same rows, over this lane's keys
  // thread roles of the FMA phases: (head or key) = tid / 4, dims 32 (tid % 4) .. +32
  const int hr = tid >> 2, d0 = 32 * (tid & 3);
  float dqa[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) dqa[i] = 0.0f;
  const int32_t *irow = idx + t * k;
  const float *grow = grad + t * k;
  for (int a0 = 0; a0 < k; a0 += kTile) {
    __syncthreads();  // the previous tile's LDS is no longer read
    // this wave's key block: entry a0 + 16 wave + c
    const int a = a0 + 16 * wave + c;
    const int32_t r_raw = a < k ? irow[a] : -1;
    const bool valid = r_raw >= 0 && r_raw < S;
    const int32_t r = valid ? r_raw : 0;
    const float gv = valid ? grow[a] : 0.0f, ksv = ks[r];
    const uint8_t *krow = k8 + (int64_t)r * kDI;
    const i32x8 kb = *reinterpret_cast<const i32x8 *>(krow + 32 * g);
    // payload of the key as fp32: lane (g, c) converts bytes 32 g .. +32 of key c
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<f32x4 *>(&sm.kf[16 * wave + c][32 * g + 4 * i]) = e4m3x4_to_f32(kb[i]);
    if (g == 0) sm.ga[16 * wave + c] = gv;
    // x for the 64 heads against key 16 wave + c: lane (g, c) gets heads 16 m + 4 g + r
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const f32x4 x = mfma_fp8_16x16x128(qa[m], kb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int j = 16 * m + 4 * g + rr;
        const bool pos = valid && x[rr] > 0.0f;  // qs, ks > 0: the sign of the payload dot
        dwp[m][rr] = fmaf(gv, pos ? x[rr] * (qsv * ksv) : 0.0f, dwp[m][rr]);
        sm.mc[j][16 * wave + c] = pos ? gv * ksv * wj[m][rr] : 0.0f;
        sm.nc[16 * wave + c][j] = pos ? wj[m][rr] : 0.0f;
      }
    }
    __syncthreads();
    // dq[hr][d0 .. +32] += sum over the tile's keys of mc[hr][key] kf[key][d0 ..]
    for (int kk = 0; kk < kTile; ++kk) {
      const float mcv = sm.mc[hr][kk];
      const f32x4 *kv4 = reinterpret_cast<const f32x4 *>(&sm.kf[kk][d0]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const f32x4 v = kv4[i];
#pragma unroll
        for (int h = 0; h < 4; ++h) dqa[4 * i + h] = fmaf(mcv, v[h], dqa[4 * i + h]);
      }
    }
    // u of key hr: g qs sum over heads of nc[hr][j] qf[j][d0 ..]
    float ua[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) ua[i] = 0.0f;
    for (int j = 0; j < kHI; ++j) {
      const float ncv = sm.nc[hr][j];
      const f32x4 *q4 = reinterpret_cast<const f32x4 *>(&sm.qf[j][d0]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const f32x4 v = q4[i];
#pragma unroll
        for (int h = 0; h < 4; ++h) ua[4 * i + h] = fmaf(ncv, v[h], ua[4 * i + h]);
      }
    }
    const int ae = a0 + hr;
    if (ae < k) {
      const float sc = sm.ga[hr] * qsv;
      f32x4 *dst = reinterpret_cast<f32x4 *>(u + (tc * k + ae) * kDI + d0);
#pragma unroll
      for (int i = 0; i < 8; ++i) dst[i] = f32x4{ua[4 * i] * sc, ua[4 * i + 1] * sc, ua[4 * i + 2] * sc, ua[4 * i + 3] * sc};
    }
  }
  // dq of head hr
  f32x4 *dqd = reinterpret_cast<f32x4 *>(dq + (t * kHI + hr) * kDI + d0);
#pragma unroll
  for (int i = 0; i < 8; ++i) dqd[i] = f32x4{dqa[4 * i], dqa[4 * i + 1], dqa[4 * i + 2], dqa[4 * i + 3]};
  // dw: sum the lane's partials over the 16 keys of its lane group, then over the waves
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      float v = dwp[m][rr];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o);
      if (c == 0) sm.dwred[wave][16 * m + 4 * g + rr] = v;
    }
  __syncthreads();
  if (tid < kHI) dw[t * kHI + tid] = (sm.dwred[0][tid] + sm.dwred[1][tid]) + (sm.dwred[2][tid] + sm.dwred[3][tid]);
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
