// Masked multi-head attention for short prefill.
//
// For short sequences the pages run the selection through a masked MHA mode
// that simulates DSA (mizuki-eaf.pages.dev, "parity evaluation"; m.digipub.cc,
// section 2): MLA in its multi-head form, where every head has its own key and
// value up-projected from the shared latent, attending densely over its causal
// positions with everything outside the query's top-k selection masked out.
// It computes the same attention as the MQA-mode sparse kernel (with the
// up-projections absorbed into the query there), with per-head widths of 192
// (128 + 64 rope) for the logits and 128 for the value instead of 576 and 512,
// and dense tiles instead of gathered rows: the cheaper form while the causal
// window is short.
//
// Three kernels:
//  * mha_upproj_kernel: K_h = W_uk[h] c and V_h = W_uv[h] c for every token
//    (bf16 MFMA GEMM, 128 output dims x 128 tokens per workgroup, K staged
//    through LDS in chunks of 64);
//  * mha_mask_kernel: one bit per (query, position), built in LDS from the
//    query's selected positions;
//  * masked_mha_kernel: flash-attention forward per (64 queries, head), keys
//    in tiles of 32 loaded straight into LDS, logits computed transposed
//    (S^T = K Q^T) so that each lane holds 8 keys of one query -- the B
//    operand layout of the PV MFMA -- and the value operand read with the
//    transposing LDS load; online softmax in fp32 per query.
#include <algorithm>

#include "dsa_common.h"

namespace {

constexpr int kDc = 512;   // compressed latent dims
constexpr int kDr = 64;    // rope dims (shared by every head)
constexpr int kDn = 128;   // per-head key dims from the up-projection
constexpr int kDvh = 128;  // per-head value dims
constexpr int kDq = kDn + kDr;
constexpr int kDl = kDc + kDr;

typedef __attribute__((address_space(3))) void lds_void;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ------------------------------------------------------------- up-projection
constexpr int kUpE = 128;    // output dims per workgroup (one head)
constexpr int kUpT = 128;    // tokens per workgroup
constexpr int kUpK = 64;     // latent dims per LDS chunk
constexpr int kUpRow = 144;  // LDS bytes per row of a chunk: 128 + 16 pad (36 dwords: conflict-free reads)
constexpr int kUpBuf = (kUpE + kUpT) * kUpRow;
constexpr int kUpLoads = (kUpE + kUpT) * (kUpK * 2 / 16) / 256;  // 16-byte loads per thread per chunk
static_assert(kUpLoads == 8, "chunk loads per thread");

// out[s, h, e] = sum_c w[h, e, c] kv[s, c] for one head h (blockIdx.y) and
// 128 tokens (blockIdx.x); blockIdx.z picks W_uk -> K or W_uv -> V.  The MFMA
// computes the transpose, D[e][s] = W[e][:] . kv[s][:], so that a lane ends
// with four consecutive output dims of one token (one 8-byte store).  Wave w
// owns output dims 64 (w & 1) .. +64 and tokens 64 (w >> 1) .. +64.
__global__ __launch_bounds__(256) void mha_upproj_kernel(const __bf16 *__restrict__ kv,
                                                         const __bf16 *__restrict__ w_uk,
                                                         const __bf16 *__restrict__ w_uv, int L, int H,
                                                         __bf16 *__restrict__ kout, __bf16 *__restrict__ vout) {
  extern __shared__ __align__(16) uint8_t up_smem[];  // two chunk buffers of kUpBuf bytes
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.y;
  const int s0 = blockIdx.x * kUpT;
  const __bf16 *w = (blockIdx.z == 0 ? w_uk : w_uv) + (int64_t)h * kUpE * kDc;
  __bf16 *out = blockIdx.z == 0 ? kout : vout;
  // thread loads: rows 0..127 are W rows (e), 128..255 are token rows; 8
  // chunks of 16 bytes per row and chunk
  auto load_chunk = [&](int kc, i32x4 (&r)[kUpLoads]) {
#pragma unroll
    for (int i = 0; i < kUpLoads; ++i) {
      const int slot = i * 256 + tid;
      const int row = slot >> 3, part = slot & 7;
      const __bf16 *src = row < kUpE ? w + (int64_t)row * kDc + kc * kUpK + part * 8
                                     : kv + (int64_t)min(s0 + row - kUpE, L - 1) * kDl + kc * kUpK + part * 8;
      r[i] = *reinterpret_cast<const i32x4 *>(src);
    }
  };
  auto store_chunk = [&](uint8_t *dst, const i32x4 (&r)[kUpLoads]) {
#pragma unroll
    for (int i = 0; i < kUpLoads; ++i) {
      const int slot = i * 256 + tid;
      *reinterpret_cast<i32x4 *>(dst + (slot >> 3) * kUpRow + (slot & 7) * 16) = r[i];
    }
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int e0 = 64 * (wave & 1), t0 = 64 * (wave >> 1);
  i32x4 r[kUpLoads];
  load_chunk(0, r);
  store_chunk(up_smem, r);
  __syncthreads();
  constexpr int nchunks = kDc / kUpK;
  for (int kc = 0; kc < nchunks; ++kc) {
    const uint8_t *cur = up_smem + (kc & 1) * kUpBuf;
    if (kc + 1 < nchunks) load_chunk(kc + 1, r);  // in flight during this chunk's MFMAs
#pragma unroll
    for (int ks = 0; ks < kUpK / 32; ++ks) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        a[m] = *reinterpret_cast<const bf16x8 *>(cur + (e0 + 16 * m + c) * kUpRow + ks * 64 + g * 16);
#pragma unroll
      for (int n = 0; n < 4; ++n)
        b[n] = *reinterpret_cast<const bf16x8 *>(cur + (kUpE + t0 + 16 * n + c) * kUpRow + ks * 64 + g * 16);
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[m][n] = mfma_bf16_16x16x32(a[m], b[n], acc[m][n]);
    }
    if (kc + 1 < nchunks) store_chunk(up_smem + ((kc + 1) & 1) * kUpBuf, r);
    __syncthreads();
  }
  // lane (g, c) of tile (m, n): output dims e0 + 16m + 4g .. +4 of token t0 + 16n + c
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int s = s0 + t0 + 16 * n + c;
    if (s >= L) continue;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      bf16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (__bf16)acc[m][n][i];
      *reinterpret_cast<bf16x4 *>(out + ((int64_t)s * H + h) * kDn + e0 + 16 * m + 4 * g) = v;
    }
  }
}

// ---------------------------------------------------------------------- mask
// mask[t, j] bit b = 1 iff position 32 j + b is among idx[t, :] and causal
// (entries outside [0, t] are ignored).  One workgroup per query row; the
// row's words are built in LDS (L <= 65536: at most 2048 words).
constexpr int kMaskMaxWords = 2048;
__global__ __launch_bounds__(256) void mha_mask_kernel(const int32_t *__restrict__ idx, int L, int k,
                                                       uint32_t *__restrict__ mask) {
  __shared__ uint32_t words[kMaskMaxWords];
  const int nw = (L + 31) >> 5;
  const int64_t t = blockIdx.x;
  for (int i = threadIdx.x; i < nw; i += 256) words[i] = 0;
  __syncthreads();
  for (int a = threadIdx.x; a < k; a += 256) {
    const int s = idx[t * k + a];
    if (s >= 0 && s <= t) atomicOr(&words[s >> 5], 1u << (s & 31));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nw; i += 256) mask[t * nw + i] = words[i];
}

// ------------------------------------------------------------ attention
constexpr int kQB = 64;                 // queries per workgroup (16 per wave)
constexpr int kKT = 32;                 // keys per tile
constexpr int kKRowSlots = 25;          // K row: 24 x 16 B of data (192 dims) + 1 pad (100 dwords)
constexpr int kVRowSlots = 18;          // V row: 16 x 16 B of data (128 dims) + 2 pad (72 dwords)
constexpr int kKRow = kKRowSlots * 16;
constexpr int kVRow = kVRowSlots * 16;
constexpr int kKInsts = (kKT * kKRowSlots + 63) / 64;  // 13 wave-wide 1 KB loads (the last one partly padding)
constexpr int kVInsts = kKT * kVRowSlots / 64;         // 9
static_assert(kKT * kVRowSlots % 64 == 0, "whole V instructions");
constexpr int kKTile = kKInsts * 1024;
constexpr int kVTile = kVInsts * 1024;
constexpr int kAttnSmem = 2 * (kKTile + kVTile);
constexpr int kSteps = kDq / 32;  // 6 K steps of the logits MFMA
constexpr int kVT = kDvh / 16;    // 8 value tiles of the PV MFMA

// Direct-to-LDS loads of key tile `tile` of head h into (dk, dv).  K slot
// q = 25 r + j holds, for key r, bytes 16 j of (K_h[s] no-rope 256 B, then the
// rope 128 B of the latent row) for j < 24 (j = 24 repeats chunk 23); V slot
// 18 r + j holds 16 bytes j of V_h[s] (j >= 16 repeat chunk 15).  Keys past
// L - 1 read key L - 1 (masked: they are after every query).
__device__ __forceinline__ void mha_load_tile(uint8_t *dk, uint8_t *dv, const __bf16 *__restrict__ kbuf,
                                              const __bf16 *__restrict__ vbuf, const __bf16 *__restrict__ kv,
                                              int L, int H, int h, int tile, int wave, int lane) {
  int l = lane;
  asm volatile("" : "+v"(l));
#pragma unroll
  for (int n = 0; n < (kKInsts + 3) / 4; ++n) {
    const int i = wave + 4 * n;  // uniform
    if (i >= kKInsts) break;
    const int slot = i * 64 + l;
    const int r = min(slot / kKRowSlots, kKT - 1);
    const int j = min(slot - (slot / kKRowSlots) * kKRowSlots, 23);
    const int64_t s = min(tile * kKT + r, L - 1);
    const __bf16 *src = j < 16 ? kbuf + (s * H + h) * kDn + j * 8 : kv + s * kDl + kDc + (j - 16) * 8;
    __builtin_amdgcn_global_load_lds(src, (lds_void *)(dk + i * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int n = 0; n < (kVInsts + 3) / 4; ++n) {
    const int i = wave + 4 * n;
    if (i >= kVInsts) break;
    const int slot = i * 64 + l;
    const int r = slot / kVRowSlots;
    const int j = min(slot - r * kVRowSlots, 15);
    const int64_t s = min(tile * kKT + r, L - 1);
    __builtin_amdgcn_global_load_lds(vbuf + (s * H + h) * kDvh + j * 8, (lds_void *)(dv + i * 1024), 16, 0, 0);
  }
}

// One workgroup per (64 queries, head); queries are issued longest-first.
// Wave w owns queries q0 + 16 w .. +16; lane (g, c) holds query q0 + 16 w + c
// for the softmax and the output (its own four value dims per tile).
__global__ __launch_bounds__(256) void masked_mha_kernel(const __bf16 *__restrict__ q,
                                                         const __bf16 *__restrict__ kv,
                                                         const __bf16 *__restrict__ kbuf,
                                                         const __bf16 *__restrict__ vbuf,
                                                         const uint32_t *__restrict__ mask, int L, int H,
                                                         float scale_log2, __bf16 *__restrict__ out,
                                                         float *__restrict__ lse) {
  extern __shared__ __align__(16) uint8_t smem_raw[];  // K tiles [2][kKTile], then V tiles [2][kVTile]
  auto ktile = [&](int b) { return smem_raw + b * kKTile; };
  auto vtile = [&](int b) { return smem_raw + 2 * kKTile + b * kVTile; };
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nqb = (L + kQB - 1) / kQB;
  const int qb = nqb - 1 - (int)(blockIdx.x / H);  // longest rows first
  const int h = (int)(blockIdx.x % H);
  const int q0 = qb * kQB;
  const int t = q0 + 16 * wave + c;  // this lane's query
  const int tq = min(t, L - 1);
  const int nw = (L + 31) >> 5;
  const int ntiles = (min(q0 + kQB, L) + kKT - 1) / kKT;  // causal bound of the workgroup

  // Q^T of the lane's query: dims 32 s + 8 g .. +8
  bf16x8 qr[kSteps];
#pragma unroll
  for (int s = 0; s < kSteps; ++s)
    qr[s] = *reinterpret_cast<const bf16x8 *>(q + ((int64_t)tq * H + h) * kDq + 32 * s + 8 * g);
  f32x4 o[kVT];
#pragma unroll
  for (int v = 0; v < kVT; ++v) o[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;
  const uint32_t *mrow = mask + (int64_t)tq * nw;
  uint32_t mword = mrow[0];

  mha_load_tile(ktile(0), vtile(0), kbuf, vbuf, kv, L, H, h, 0, wave, lane);
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of tile `it` (and its mask word) have landed
    __syncthreads();                // ... and every wave's; the other buffer is free
    const uint32_t mw = t < L ? mword : 0u;
    if (it + 1 < ntiles) {
      mword = mrow[it + 1];
      mha_load_tile(ktile(buf ^ 1), vtile(buf ^ 1), kbuf, vbuf, kv, L, H, h, it + 1, wave, lane);
    }
    const uint8_t *kt = ktile(buf), *vt = vtile(buf);
    // logits S^T[key, query]: x[r] = key 4g + r, x[4 + r] = key 16 + 4g + r
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(kt + c * kKRow + s * 64 + g * 16);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(kt + (16 + c) * kKRow + s * 64 + g * 16);
      s0 = mfma_bf16_16x16x32(a0, qr[s], s0);
      s1 = mfma_bf16_16x16x32(a1, qr[s], s1);
    }
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = (mw >> (4 * g + r)) & 1u ? s0[r] * scale_log2 : -INFINITY;
      x[4 + r] = (mw >> (16 + 4 * g + r)) & 1u ? s1[r] * scale_log2 : -INFINITY;
    }
    // online softmax over the query's keys (lanes c, c+16, c+32, c+48)
    float mx = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
    {
      const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
      const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
    }
    const float m_new = fmaxf(m_run, mx);
    const float msub = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - msub);  // 0 while nothing was seen
    m_run = m_new;
    bf16x8 pb;
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = __builtin_amdgcn_exp2f(x[i] - msub);
      psum += p;
      pb[i] = (__bf16)p;
    }
    l_run = l_run * alpha + psum;
    // PV: O^T[dv, query] += V^T[dv, keys] P^T[keys, query]
    const uint8_t *vb = vt + (4 * g + (c >> 2)) * kVRow + (c & 3) * 8;
#pragma unroll
    for (int v = 0; v < kVT; ++v) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vb + v * 32));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vb + v * 32 + 16 * kVRow));
      const i16x4 lohi[2] = {lo, hi};
      const bf16x8 va = *reinterpret_cast<const bf16x8 *>(lohi);
#pragma unroll
      for (int r = 0; r < 4; ++r) o[v][r] *= alpha;
      o[v] = mfma_bf16_16x16x32(va, pb, o[v]);
    }
  }
  // the four lane groups hold different keys of the same query
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (t >= L) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  // lane (g, c): value dims 16 v + 4 g .. +4 of query t
#pragma unroll
  for (int v = 0; v < kVT; ++v) {
    bf16x4 o4;
#pragma unroll
    for (int r = 0; r < 4; ++r) o4[r] = (__bf16)(o[v][r] * inv);
    *reinterpret_cast<bf16x4 *>(out + ((int64_t)t * H + h) * kDvh + 16 * v + 4 * g) = o4;
  }
  if (lse && g == 0)
    lse[(int64_t)t * H + h] = l_tot > 0.0f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

namespace dsa {
size_t masked_mha_workspace_bytes(int32_t L, int32_t H) {
  const size_t kvb = (size_t)L * H * kDn * 2;
  return 2 * align_up(kvb, 256) + align_up((size_t)L * ((L + 31) / 32) * 4, 256);
}

hipError_t launch_masked_mha(const void *q, const void *kv, const void *w_uk, const void *w_uv,
                             const int32_t *idx, int32_t L, int32_t H, int32_t k, float sm_scale, void *out,
                             float *lse, void *workspace, hipStream_t s) {
  if (L == 0) return hipSuccess;
  const size_t kvb = align_up((size_t)L * H * kDn * 2, 256);
  __bf16 *kbuf = (__bf16 *)workspace;
  __bf16 *vbuf = (__bf16 *)((char *)workspace + kvb);
  uint32_t *mask = (uint32_t *)((char *)workspace + 2 * kvb);
  static bool attr_done = false;  // per process: the attribute holds for every device
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void *)mha_upproj_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kUpBuf);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  hipLaunchKernelGGL(mha_upproj_kernel, dim3((L + kUpT - 1) / kUpT, H, 2), dim3(256), 2 * kUpBuf, s, (const __bf16 *)kv,
                     (const __bf16 *)w_uk, (const __bf16 *)w_uv, L, H, kbuf, vbuf);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mha_mask_kernel, dim3(L), dim3(256), 0, s, idx, L, k, mask);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nqb = (L + kQB - 1) / kQB;
  hipLaunchKernelGGL(masked_mha_kernel, dim3((uint32_t)nqb * H), dim3(256), kAttnSmem, s, (const __bf16 *)q,
                     (const __bf16 *)kv, kbuf, vbuf, mask, L, H, sm_scale * 1.4426950408889634f, (__bf16 *)out,
                     lse);
  return hipGetLastError();
}
}  // namespace dsa
