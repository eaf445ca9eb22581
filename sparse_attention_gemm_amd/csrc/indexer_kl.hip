// The indexer's KL-alignment loss (forward) and the index scores it needs.
//
// In both continued-pre-training stages the indexer is trained by a KL loss
// that aligns its output distribution with the main attention's
// (mizuki-eaf.pages.dev, two-stage continued pre-training; m.36881.com.cn,
// dense warm-up and sparse training; m.digipub.cc, section 2).  Per query
// token t, over a set S_t of positions (the top-k selection in sparse
// training, every causal position in the dense warm-up):
//   p(s)  = (1/H) sum_h softmax_s(sm_scale q_h . c_s)     main attention, heads averaged
//   pi(s) = softmax_s(I[t, s])                             the indexer's distribution
//   KL_t  = sum_s p(s) (log p(s) - log pi(s))
//
//  * indexer_scores_at_kernel: I[t, s] for the listed positions, through the
//    same FP8 core (and the same expression) as the fused selection, so the
//    values are bit-identical to the scores the selection ranked;
//  * indexer_kl_kernel: one workgroup per query token (the loss, or its
//    gradient with respect to the index scores).  Each head's softmax
//    is taken against the head's log-sum-exp from the sparse-MLA forward
//    (the same set of entries), the heads are summed, and the aggregate is
//    normalised by its own sum, so p sums to one exactly:
//      P(s) = sum_h exp(z_hs - lse_h),  Z = sum_s P(s)
//      KL_t = (1/Z) sum_s P(s) (log P(s) - I_s) - log Z + logsumexp_s I_s
//    Latent rows are gathered 32 per tile into LDS with direct-to-LDS loads
//    (double-buffered); the logits S = Q C^T (bf16 MFMA, fp32 sums) put the
//    heads along rows, so the head sum is in-lane adds plus permlane swaps.
#include <type_traits>

#include "dsa_common.h"
#include "dsa_launch.h"
#include "indexer_core.h"

namespace {

typedef __attribute__((address_space(3))) void lds_void;

// ---------------------------------------------------------- scores at positions
// One wave per query row (4 per workgroup), 64 entries per step: lane l holds
// entry 64 j + l; the B operand of key block u in lane (g, c) is bytes
// 32 g .. +32 of the E4M3 row of entry 16 u + c.
template <int NT>
__global__ __launch_bounds__(256) void indexer_scores_at_kernel(const uint8_t *__restrict__ q8,
                                                                const float *__restrict__ qs,
                                                                const uint8_t *__restrict__ k8,
                                                                const float *__restrict__ ks,
                                                                const float *__restrict__ w,
                                                                const int32_t *__restrict__ idx, int T, int S,
                                                                int k, float *__restrict__ out) {
  __shared__ __align__(16) uint8_t qscratch[4][kQueryScratch];
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;  // uniform per wave; no barrier below
  constexpr int HI = 16 * NT;
  IdxQuery<NT> Q;
  idx_load_query<NT>(Q, q8 + (int64_t)t * HI * 128, w + (int64_t)t * HI, qs[t], lane, qscratch[wave]);
  const int32_t *irow = idx + (int64_t)t * k;
  float *orow = out + (int64_t)t * k;
  for (int j0 = 0; j0 < k; j0 += 64) {
    const int a = j0 + lane;
    const int pos_raw = a < k ? irow[a] : -1;
    const bool valid = pos_raw >= 0 && pos_raw < S;
    const int pos = valid ? pos_raw : 0;
    const float ksv = ks[pos];
    auto get_b = [&](int u) {
      const int pu = __shfl(pos, 16 * u + c);
      return *reinterpret_cast<const i32x8 *>(k8 + (int64_t)pu * 128 + 32 * g);
    };
    const float tot = idx_score64<NT>(Q, get_b, [] {});
    if (a < k) orow[a] = valid ? canon_zero(tot * ksv) : -INFINITY;
  }
}

// ------------------------------------------------------------------- KL loss
constexpr int kBN = 32;                               // entries per tile
constexpr int kRowSlots = 74;                         // latent row: 72 x 16 B of data + 2 pad (1184 B)
constexpr int kRowBytes = kRowSlots * 16;
constexpr int kTileBytes = kBN * kRowBytes;
constexpr int kGatherInsts = kBN * kRowSlots / 64;    // 37 wave-wide 1 KB loads
static_assert(kBN * kRowSlots % 64 == 0, "whole gather instructions");
constexpr int kSteps = 576 / 32;                      // 18 K steps of the logits MFMA

// LDS of one workgroup: two tile buffers (static arrays, so that the compiler
// can tell a gather into one from the LDS reads of the other), then, dynamic,
// the resolved rows and scores of the query's entries (kpad = k rounded up to
// the tile), per-wave key partials, and (gradient only) each entry's head sum P.
__shared__ __align__(16) uint8_t g_kl_t0[kTileBytes];
__shared__ __align__(16) uint8_t g_kl_t1[kTileBytes];
template <int B>
__device__ __forceinline__ uint8_t *kl_tile() {
  return B == 0 ? g_kl_t0 : g_kl_t1;
}
__host__ __device__ constexpr int kl_smem_bytes(int kpad, int nw, bool grad) {
  return kpad * 4 * 2 + 2 * nw * kBN * 4 + (grad ? kpad * 4 : 0);
}

// x of this lane plus x of lane l ^ 32 (resp. l ^ 16).
__device__ __forceinline__ float pair_sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_sum16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Direct-to-LDS gather of tile rows [r0, r0+32): slot q of the tile holds row
// q / 74, 16-byte chunk q % 74 (chunks 72, 73 repeat chunk 71); entries with
// no row load row 0 (they are masked).  rec: buffer loads indexed by row (a
// 1152-byte record each), which the compiler counts in the vector-memory
// counter only, so it keeps exact counts of the LDS reads issued after them;
// usable while every row lies within 4 GiB of kv (32-bit offsets).  Else the
// flat form.
template <int NW, bool rec>
__device__ __forceinline__ void kl_gather(uint8_t *__restrict__ dst, const int *__restrict__ rows, int r0,
                                          const __bf16 *__restrict__ kv, int64_t N, int wave, int lane) {
  int l = lane;
  asm volatile("" : "+v"(l));
#pragma unroll
  for (int n = 0; n < (kGatherInsts + NW - 1) / NW; ++n) {
    const int i = wave + n * NW;  // uniform
    if (i >= kGatherInsts) break;
    const int slot = i * 64 + l;
    const int r = slot / kRowSlots;
    const int j = min(slot - r * kRowSlots, 71);
    const int pr = rows[r0 + r];
    if constexpr (rec) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void *)kv, (short)(576 * 2), (int)(N < 0xFFFFFFFFll ? N : 0xFFFFFFFFll), (int)0x00020000u);
      __builtin_amdgcn_struct_ptr_buffer_load_lds(rs, (lds_void *)(dst + i * 1024), 16, pr >= 0 ? pr : 0, j * 16,
                                                  0, 0, 0);
    } else {
      __builtin_amdgcn_global_load_lds(kv + ((int64_t)(pr >= 0 ? pr : 0) * 576 + j * 8),
                                       (lds_void *)(dst + i * 1024), 16, 0, 0);
    }
  }
}

// One workgroup of NW waves per query token; wave w owns heads 16 w .. +16.
// GRAD = false: the loss kl[t].  GRAD = true: the gradient of dkl[t] * KL_t
// with respect to the index scores of the entries (the target p carries no
// gradient): since pi = softmax(I) and p sums to one,
//   d KL_t / d I_a = pi_a - p_a,   out[t, a] = dkl[t] (pi_a - P_a / Z)
// (0 where the entry has no row); P_a is kept in LDS until Z is known.
template <int NW, bool GRAD, bool rec>
__global__ __launch_bounds__(NW * 64) void indexer_kl_kernel(const __bf16 *__restrict__ q,
                                                             const __bf16 *__restrict__ kv,
                                                             const int32_t *__restrict__ idx,
                                                             const float *__restrict__ scores,
                                                             const float *__restrict__ lse, const float *__restrict__ dkl,
                                                             int64_t N, int H, int k, float scale_log2,
                                                             float *__restrict__ out) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t t = blockIdx.x;
  const int ntiles = (k + kBN - 1) / kBN, kpad = ntiles * kBN;
  int *rows = reinterpret_cast<int *>(smem);
  float *sc = reinterpret_cast<float *>(rows + kpad);
  float *part = sc + kpad;  // [2][NW][32]
  float *pP = part + 2 * NW * kBN;  // GRAD: each entry's head sum

  // entries: rows of kv (or -1) and their index scores (-inf where no row)
  for (int a = tid; a < kpad; a += NW * 64) {
    const int r = a < k ? idx[t * k + a] : -1;
    const bool v = r >= 0 && r < N;
    rows[a] = v ? r : -1;
    sc[a] = v ? scores[t * k + a] : -INFINITY;
  }
  // Q of the wave's heads (A operand: lane (g, c) holds head 16 w + c, dims
  // 32 s + 8 g .. +8) and the base-2 log-sum-exp of the heads in its result
  // rows 4 g + r
  const int h0 = 16 * wave;
  bf16x8 qa[kSteps];
#pragma unroll
  for (int s = 0; s < kSteps; ++s)
    qa[s] = *reinterpret_cast<const bf16x8 *>(q + ((t * H + h0 + c) * 576) + 32 * s + 8 * g);
  float lse2[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) lse2[r] = lse[t * H + h0 + 4 * g + r] * 1.4426950408889634f;
  __syncthreads();  // rows and scores visible

  float accA = 0.0f, accZ = 0.0f;  // wave 0, lanes 0..31: this lane's key of every tile
  auto consume = [&](int j) {      // wave 0: fold tile j's per-wave partials
    if (lane < kBN) {
      float P = 0.0f;
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) P += part[((j & 1) * NW + w2) * kBN + lane];
      const int a = j * kBN + lane;
      if (rows[a] >= 0 && P > 0.0f) {
        if (!GRAD) accA += P * (logf(P) - sc[a]);
        accZ += P;
      }
      if (GRAD) pP[a] = rows[a] >= 0 ? P : 0.0f;
    }
  };
  kl_gather<NW, rec>(g_kl_t0, rows, 0, kv, N, wave, lane);
  // tile it in buffer it & 1; unrolled by two so that each buffer is a fixed object
  auto step = [&](auto bc, int it) {
    constexpr int B = decltype(bc)::value;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's gathers of tile it have landed
    __syncthreads();                // every wave's; part[(it-1)&1] is complete; tile it-1 is free
    if (it + 1 < ntiles) kl_gather<NW, rec>(kl_tile<B ^ 1>(), rows, (it + 1) * kBN, kv, N, wave, lane);
    if (wave == 0 && it > 0) consume(it - 1);
    const uint8_t *tb = kl_tile<B>();
    // S[head 4g + r][key c] (keys 0..15) and [key 16 + c] (keys 16..31)
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const bf16x8 b0 = *reinterpret_cast<const bf16x8 *>(tb + c * kRowBytes + st * 64 + g * 16);
      const bf16x8 b1 = *reinterpret_cast<const bf16x8 *>(tb + (16 + c) * kRowBytes + st * 64 + g * 16);
      s0 = mfma_bf16_16x16x32(qa[st], b0, s0);
      s1 = mfma_bf16_16x16x32(qa[st], b1, s1);
    }
    // this lane's four heads, summed: exp(z - lse) in base 2
    float e0 = 0.0f, e1 = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      e0 += __builtin_amdgcn_exp2f(fmaf(s0[r], scale_log2, -lse2[r]));
      e1 += __builtin_amdgcn_exp2f(fmaf(s1[r], scale_log2, -lse2[r]));
    }
    // sum over the four lane groups (heads 4g..4g+3, g = 0..3; lanes c, c+16,
    // c+32, c+48): with both operands equal, a permlane swap returns the
    // lane's and its partner's values
    const float y0 = pair_sum16(pair_sum32(e0)), y1 = pair_sum16(pair_sum32(e1));
    if (g == 0) {
      part[(B * NW + wave) * kBN + c] = y0;
      part[(B * NW + wave) * kBN + 16 + c] = y1;
    }
  };
  for (int it = 0; it < ntiles; it += 2) {
    step(std::integral_constant<int, 0>(), it);
    if (it + 1 < ntiles) step(std::integral_constant<int, 1>(), it + 1);
  }
  __syncthreads();  // the last tile's partials
  if (wave != 0) return;
  consume(ntiles - 1);
  // lanes 0..31 hold their keys' sums; reduce, and log-sum-exp of the scores
  accA = wave_sum(accA);
  accZ = wave_sum(accZ);
  float smax = -INFINITY;
  for (int a = lane; a < kpad; a += 64) smax = fmaxf(smax, sc[a]);
  smax = wave_max(smax);
  float ssum = 0.0f;
  if (smax != -INFINITY)
    for (int a = lane; a < kpad; a += 64) ssum += rows[a] >= 0 ? expf(sc[a] - smax) : 0.0f;
  ssum = wave_sum(ssum);
  if (!GRAD) {
    if (lane == 0) out[t] = accZ > 0.0f ? accA / accZ - logf(accZ) + (smax + logf(ssum)) : 0.0f;
    return;
  }
  // pi_a - P_a / Z, scaled by the token's upstream gradient; wave 0 wrote pP
  const float lse_i = smax + logf(ssum), invZ = accZ > 0.0f ? 1.0f / accZ : 0.0f, dk = dkl[t];
  for (int a = lane; a < k; a += 64)
    out[t * k + a] = (rows[a] >= 0 && accZ > 0.0f) ? dk * (expf(sc[a] - lse_i) - pP[a] * invZ) : 0.0f;
}

// The KL score gradient from head sums of P formed elsewhere (the sparse-MLA
// backward forms every P of the selection with the forward's lse, and sums
// them over each group of heads): one workgroup per query token, each thread
// holding 8 entries (a = tid + 256 i) with all their loads in flight,
//   P_a = sum over the groups of psum[tc, group, a],  Z = sum of P_a over the
//   valid entries with P_a > 0,  out[t, a] = dkl[t] (pi_a - P_a / Z)
// with pi = softmax of the index scores over the valid entries, and 0 where
// the entry has no row (or no valid entry has P > 0), as in indexer_kl_kernel.
constexpr int kKlThreads = 256;
constexpr int kKlPer = 2048 / kKlThreads;  // entries per thread (k <= 2048)
static_assert(kKlPer * kKlThreads >= DSA_MAX_K, "every entry of a row has a thread");

// Sum (or max) over the workgroup in a fixed order: waves, then the 4 wave results.
template <bool MAX>
__device__ __forceinline__ float kl_block_reduce(float v, float *red) {
  v = MAX ? wave_max(v) : wave_sum(v);
  const int wave = threadIdx.x >> 6;
  __syncthreads();  // earlier readers of red are done
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kKlThreads / 64; ++w) r = MAX ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

__global__ __launch_bounds__(kKlThreads) void kl_grad_from_head_sums_kernel(const int32_t *__restrict__ idx,
                                                                            const float *__restrict__ scores,
                                                                            const float *__restrict__ dkl,
                                                                            const float *__restrict__ psum,
                                                                            int64_t N, int k, int nhg, int64_t t0,
                                                                            float *__restrict__ out) {
  __shared__ float red[kKlThreads / 64];
  const int tid = threadIdx.x;
  const int64_t tc = blockIdx.x, t = t0 + tc;
  const int32_t *irow = idx + t * k;
  const float *srow = scores + t * k;
  const float *ps = psum + tc * nhg * k;
  float P[kKlPer], sc[kKlPer];
  bool v[kKlPer];
#pragma unroll
  for (int i = 0; i < kKlPer; ++i) {
    const int a = tid + kKlThreads * i;
    const bool in = a < k;
    const int32_t r = in ? irow[a] : -1;
    v[i] = r >= 0 && r < N;
    sc[i] = in ? srow[a] : -INFINITY;
    float s = 0.0f;
    for (int n = 0; n < nhg; ++n) s += in ? ps[n * k + a] : 0.0f;
    P[i] = s;
  }
  float z = 0.0f, m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kKlPer; ++i) {
    if (v[i] && P[i] > 0.0f) z += P[i];
    if (v[i]) m = fmaxf(m, sc[i]);
  }
  const float accZ = kl_block_reduce<false>(z, red);
  const float smax = kl_block_reduce<true>(m, red);
  float e = 0.0f;
  if (smax != -INFINITY)
#pragma unroll
    for (int i = 0; i < kKlPer; ++i) e += v[i] ? expf(sc[i] - smax) : 0.0f;
  const float ssum = kl_block_reduce<false>(e, red);
  const float lse_i = smax + logf(ssum), invZ = accZ > 0.0f ? 1.0f / accZ : 0.0f, dk = dkl[t];
#pragma unroll
  for (int i = 0; i < kKlPer; ++i) {
    const int a = tid + kKlThreads * i;
    if (a < k) out[t * k + a] = (v[i] && accZ > 0.0f) ? dk * (expf(sc[i] - lse_i) - P[i] * invZ) : 0.0f;
  }
}

}  // namespace

namespace dsa {
hipError_t launch_indexer_scores_at(const uint8_t *q8, const float *qs, const uint8_t *k8, const float *ks,
                                    const float *w, const int32_t *idx, int32_t T, int32_t S, int32_t H_I, int32_t k,
                                    float *out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + 3) / 4);
  if (H_I == 64)
    hipLaunchKernelGGL(indexer_scores_at_kernel<4>, grid, dim3(256), 0, s, q8, qs, k8, ks, w, idx, T, S, k, out);
  else
    hipLaunchKernelGGL(indexer_scores_at_kernel<2>, grid, dim3(256), 0, s, q8, qs, k8, ks, w, idx, T, S, k, out);
  return hipGetLastError();
}

template <bool GRAD>
static hipError_t launch_kl(const void *q, const void *kv, const int32_t *idx, const float *scores, const float *lse,
                            const float *dkl, int64_t N, int32_t T, int32_t H, int32_t k, float sm_scale, float *out,
                            hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int kpad = (k + kBN - 1) / kBN * kBN;
  const float sl2 = sm_scale * 1.4426950408889634f;
  const bool rec = N * (576 * 2) <= (int64_t(1) << 32);  // every row within 4 GiB: record-indexed gathers
#define DSA_KL_CASE(NW)                                                                                          \
  case NW: {                                                                                                     \
    const int bytes = kl_smem_bytes(kpad, NW, GRAD);                                                             \
    static bool attr_done = false; /* per process: the attribute holds for every device */                       \
    if (!attr_done) {                                                                                            \
      for (const void *f : {(const void *)indexer_kl_kernel<NW, GRAD, true>,                                      \
                            (const void *)indexer_kl_kernel<NW, GRAD, false>}) {                                  \
        hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,                         \
                                           kl_smem_bytes(2048, NW, GRAD));                                        \
        if (e != hipSuccess) return e;                                                                           \
      }                                                                                                          \
      attr_done = true;                                                                                          \
    }                                                                                                            \
    if (rec)                                                                                                     \
      hipLaunchKernelGGL((indexer_kl_kernel<NW, GRAD, true>), dim3(T), dim3(NW * 64), bytes, s,                  \
                         (const __bf16 *)q, (const __bf16 *)kv, idx, scores, lse, dkl, N, H, k, sl2, out);       \
    else                                                                                                         \
      hipLaunchKernelGGL((indexer_kl_kernel<NW, GRAD, false>), dim3(T), dim3(NW * 64), bytes, s,                 \
                         (const __bf16 *)q, (const __bf16 *)kv, idx, scores, lse, dkl, N, H, k, sl2, out);       \
    break;                                                                                                       \
  }
  switch (H / 16) {
    DSA_KL_CASE(1)
    DSA_KL_CASE(2)
    DSA_KL_CASE(4)
    DSA_KL_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef DSA_KL_CASE
  return hipGetLastError();
}

hipError_t launch_indexer_kl(const void *q, const void *kv, const int32_t *idx, const float *scores, const float *lse,
                             int64_t N, int32_t T, int32_t H, int32_t k, float sm_scale, float *kl, hipStream_t s) {
  return launch_kl<false>(q, kv, idx, scores, lse, nullptr, N, T, H, k, sm_scale, kl, s);
}

hipError_t launch_indexer_kl_grad(const void *q, const void *kv, const int32_t *idx, const float *scores,
                                  const float *lse, const float *dkl, int64_t N, int32_t T, int32_t H, int32_t k,
                                  float sm_scale, float *grad, hipStream_t s) {
  return launch_kl<true>(q, kv, idx, scores, lse, dkl, N, T, H, k, sm_scale, grad, s);
}

hipError_t launch_kl_grad_from_head_sums(const int32_t *idx, const float *scores, const float *dkl, const float *psum,
                                         int64_t N, int32_t k, int32_t nhg, int64_t t0, int32_t Tc, float *grad,
                                         hipStream_t s) {
  if (Tc <= 0) return hipSuccess;
  hipLaunchKernelGGL(kl_grad_from_head_sums_kernel, dim3((uint32_t)Tc), dim3(kKlThreads), 0, s, idx, scores, dkl,
                     psum, N, k, nhg, t0, grad);
  return hipGetLastError();
}
}  // namespace dsa
