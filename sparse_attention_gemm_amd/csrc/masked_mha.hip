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
//    (bf16 MFMA GEMM with fp32 accumulation, 128 output dims x 128 tokens per
//    workgroup, operands staged through LDS in chunks of 64), stored in fp16:
//    the same MFMA rate as bf16 with a quarter of its rounding error;
//  * mha_mask_kernel: one bit per (query, position), built in LDS from the
//    query's selected positions;
//  * masked_mha_kernel: flash-attention forward per (128 queries, head), keys
//    in tiles of 32 loaded straight into LDS, logits computed transposed
//    (S^T = K Q^T) so that each lane holds 8 keys of one query -- the B
//    operand layout of the PV MFMA -- and the value operand read with the
//    transposing LDS load; online softmax in fp32 per query, probabilities
//    and values in fp16.
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
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// fp16 MFMA 16x16x32, same lane layout as the bf16 one.
__device__ __forceinline__ f32x4 mfma_f16_16x16x32(const f16x8 &a, const f16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// fp32 -> fp16, round to nearest even, saturating at the largest finite value.
__device__ __forceinline__ _Float16 to_f16_sat(float x) { return (_Float16)fminf(fmaxf(x, -65504.0f), 65504.0f); }
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ------------------------------------------------------------- up-projection
constexpr int kUpE = 128;    // output dims per workgroup (one head)
constexpr int kUpT = 128;    // tokens per workgroup
constexpr int kUpK = 64;     // latent dims per LDS chunk
constexpr int kUpRow = 144;  // LDS bytes per row of a chunk: 128 + 16 pad (36 dwords: conflict-free reads)
constexpr int kUpBuf = (kUpE + kUpT) * kUpRow;
constexpr int kUpLoads = (kUpE + kUpT) * (kUpK * 2 / 16) / 256;  // 16-byte loads per thread per chunk
static_assert(kUpLoads == 8, "chunk loads per thread");

// out[s, h, e] = fp16(sum_c w[h, e, c] kv[s, c]) for one head h (blockIdx.y) and
// 128 tokens (blockIdx.x); blockIdx.z picks W_uk -> K or W_uv -> V.  The MFMA
// computes the transpose, D[e][s] = W[e][:] . kv[s][:], so that a lane ends
// with four consecutive output dims of one token (one 8-byte store).  Wave w
// owns output dims 64 (w & 1) .. +64 and tokens 64 (w >> 1) .. +64.
__global__ __launch_bounds__(256) void mha_upproj_kernel(const __bf16 *__restrict__ kv,
                                                         const __bf16 *__restrict__ w_uk,
                                                         const __bf16 *__restrict__ w_uv, int L, int H,
                                                         _Float16 *__restrict__ kout, _Float16 *__restrict__ vout) {
  extern __shared__ __align__(16) uint8_t up_smem[];  // two chunk buffers of kUpBuf bytes
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.y;
  const int s0 = blockIdx.x * kUpT;
  const __bf16 *w = (blockIdx.z == 0 ? w_uk : w_uv) + (int64_t)h * kUpE * kDc;
  _Float16 *out = blockIdx.z == 0 ? kout : vout;
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
      f16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = to_f16_sat(acc[m][n][i]);
      *reinterpret_cast<f16x4 *>(out + ((int64_t)s * H + h) * kDn + e0 + 16 * m + 4 * g) = v;
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
constexpr int kQW = 32;                 // queries per wave (two groups of 16)
constexpr int kQB = 4 * kQW;            // queries per workgroup
constexpr int kKT = 32;                 // keys per tile
constexpr int kKRowSlots = 25;          // K row: 24 x 16 B of data (192 dims) + 1 pad (100 dwords)
constexpr int kVRowSlots = 18;          // V row: 16 x 16 B of data (128 dims) + 2 pad (72 dwords)
constexpr int kKRow = kKRowSlots * 16;
constexpr int kVRow = kVRowSlots * 16;
constexpr int kKInsts = (kKT * kKRowSlots + 63) / 64;  // 13 wave-wide 1 KB loads (the last one partly padding)
constexpr int kVInsts = kKT * kVRowSlots / 64;         // 9
constexpr int kMInsts = kQB * 4 / 256;                 // 2 wave-wide 256 B loads: one mask word per query
static_assert(kKT * kVRowSlots % 64 == 0, "whole V instructions");
constexpr int kTileInsts = kKInsts + kVInsts + kMInsts;
static_assert(kTileInsts % 4 == 0, "every wave issues the same number of loads per tile");
constexpr int kInstsPerWave = kTileInsts / 4;
constexpr int kVOff = kKInsts * 1024;            // V rows follow the K rows in a tile buffer
constexpr int kMOff = kVOff + kVInsts * 1024;    // then the mask words of the workgroup's queries
constexpr int kTileBytes = kMOff + kMInsts * 256;
constexpr int kNBuf = 3;                         // tile j+2 loads while tile j is computed
constexpr int kAttnSmem = kNBuf * kTileBytes;
constexpr int kSteps = kDq / 32;  // 6 K steps of the logits MFMA
constexpr int kNopeSteps = kDn / 32;  // the first 4 cover the up-projected (fp16) dims
constexpr int kVT = kDvh / 16;    // 8 value tiles of the PV MFMA
// A query's exponent reference moves only when its running max exceeds it by
// more than this (base-2 units): probabilities stay below 2^8, and the output
// is rescaled only on the rare tiles that raise the max that far.
constexpr float kRefSlack = 8.0f;

// s_waitcnt immediate: at most n vector-memory operations outstanding
// (expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Direct-to-LDS loads of key tile `tile` of head h into buffer dst; each wave
// issues kInstsPerWave of the tile's kTileInsts instructions.
//  * K: slot q = 25 r + j holds, for key r, 16 bytes j of (K_h no-rope 256 B,
//    then the 128 B rope part of the latent row) for j < 24 (j = 24 and the
//    tail slots repeat data);
//  * V: slot 18 r + j holds 16 bytes j of V_h (j >= 16 repeat chunk 15);
//  * mask: word q of the workgroup's query q0 + q for this tile.
// Keys past L - 1 read key L - 1, queries past L - 1 the row of query L - 1
// (both are excluded by the mask or never stored).
__device__ __forceinline__ void mha_load_tile(uint8_t *dst, const _Float16 *__restrict__ kbuf,
                                              const _Float16 *__restrict__ vbuf, const __bf16 *__restrict__ kv,
                                              const uint32_t *__restrict__ mask, int L, int H, int h, int q0,
                                              int nw, int tile, int wave, int lane) {
  int l = lane;
  asm volatile("" : "+v"(l));
#pragma unroll
  for (int n = 0; n < kInstsPerWave; ++n) {
    const int i = wave + 4 * n;  // uniform
    if (i < kKInsts) {
      const int slot = i * 64 + l;
      const int r = min(slot / kKRowSlots, kKT - 1);
      const int j = min(slot - (slot / kKRowSlots) * kKRowSlots, 23);
      const int64_t s = min(tile * kKT + r, L - 1);
      const void *src = j < 16 ? (const void *)(kbuf + (s * H + h) * kDn + j * 8)
                               : (const void *)(kv + s * kDl + kDc + (j - 16) * 8);
      __builtin_amdgcn_global_load_lds(src, (lds_void *)(dst + i * 1024), 16, 0, 0);
    } else if (i < kKInsts + kVInsts) {
      const int slot = (i - kKInsts) * 64 + l;
      const int r = slot / kVRowSlots;
      const int j = min(slot - r * kVRowSlots, 15);
      const int64_t s = min(tile * kKT + r, L - 1);
      __builtin_amdgcn_global_load_lds(vbuf + (s * H + h) * kDvh + j * 8, (lds_void *)(dst + i * 1024), 16, 0,
                                       0);
    } else {
      const int m = i - kKInsts - kVInsts;
      const int64_t t = min(q0 + m * 64 + l, L - 1);
      __builtin_amdgcn_global_load_lds(mask + t * nw + tile, (lds_void *)(dst + kMOff + m * 256), 4, 0, 0);
    }
  }
}

// Max of the query's 8 keys in this lane and its 3 partner lanes (c, c+16,
// c+32, c+48 hold the same query).  With both operands equal, a permlane swap
// returns the row pair's two halves.
__device__ __forceinline__ float query_max(const float (&x)[8]) {
  float mx = x[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  mx = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// One workgroup per (128 queries, head).  Wave w owns queries q0 + 32 w ..
// +32 in two groups of 16; lane (g, c) holds query q0 + 32 w + 16 u + c of
// group u for the softmax and the output (its four value dims per value
// tile).  Each K and V fragment read from LDS feeds both groups' MFMAs.
// Workgroups are numbered head-major with each head's longest query blocks
// first, and consecutive numbers go to the same XCD (workgroup i runs on XCD
// i mod 8), so that one head's keys and values stay in one L2.
__global__ __launch_bounds__(256) void masked_mha_kernel(const __bf16 *__restrict__ q,
                                                         const __bf16 *__restrict__ kv,
                                                         const _Float16 *__restrict__ kbuf,
                                                         const _Float16 *__restrict__ vbuf,
                                                         const uint32_t *__restrict__ mask, int L, int H,
                                                         float scale_log2, __bf16 *__restrict__ out,
                                                         float *__restrict__ lse) {
  extern __shared__ __align__(16) uint8_t smem_raw[];  // kNBuf tile buffers of kTileBytes
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nqb = (L + kQB - 1) / kQB;
  int lin;
  {
    const int n = gridDim.x, i = blockIdx.x, x = i & 7, per = n >> 3, rem = n & 7;
    lin = x * per + min(x, rem) + (i >> 3);
  }
  const int h = lin / nqb;
  const int q0 = (nqb - 1 - lin % nqb) * kQB;
  const int nw = (L + 31) >> 5;
  const int ntiles = (min(q0 + kQB, L) + kKT - 1) / kKT;  // causal bound of the workgroup
  const int wave_last = min(q0 + kQW * wave + kQW - 1, L - 1);  // this wave's last query

  // Q^T of the lane's two queries, dims 32 s + 8 g .. +8: the no-rope steps
  // in fp16 (exact for |q| within fp16's normal range) against the fp16 K_h,
  // the rope steps in bf16 against the latent's rope dims
  f16x8 qn[2][kNopeSteps];
  bf16x8 qr[2][kSteps - kNopeSteps];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int64_t tq = min(q0 + kQW * wave + 16 * u + c, L - 1);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const bf16x8 v = *reinterpret_cast<const bf16x8 *>(q + (tq * H + h) * kDq + 32 * s + 8 * g);
      if (s < kNopeSteps) {
#pragma unroll
        for (int i = 0; i < 8; ++i) qn[u][s][i] = to_f16_sat((float)v[i]);
      } else {
        qr[u][s - kNopeSteps] = v;
      }
    }
  }
  f32x4 o[2][kVT];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < kVT; ++v) o[u][v] = f32x4{0.f, 0.f, 0.f, 0.f};
  // exponent reference (base 2, scaled) and the lane's share of the softmax sum;
  // the finite start keeps exp2 of masked (-inf) logits at 0 before any key
  float m_ref[2] = {-1e30f, -1e30f}, l_run[2] = {0.0f, 0.0f};
  // transposing-load lane roles: row 4g + (c>>2) of each 4-row group, value chunk (c&3)
  const int tr_off = kVOff + (4 * g + (c >> 2)) * kVRow + (c & 3) * 8;
  const uint32_t lane_bits = 0x000F000Fu << (4 * g);  // the lane's 8 keys of a tile

  auto buf = [&](int j) { return smem_raw + (j % kNBuf) * kTileBytes; };
  mha_load_tile(buf(0), kbuf, vbuf, kv, mask, L, H, h, q0, nw, 0, wave, lane);
  if (ntiles > 1) mha_load_tile(buf(1), kbuf, vbuf, kv, mask, L, H, h, q0, nw, 1, wave, lane);
  for (int it = 0; it < ntiles; ++it) {
    if (it + 1 < ntiles)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kInstsPerWave));  // tile it landed (tile it+1 may be in flight)
    else
      __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // every wave's loads of tile it landed; nobody reads tile it-1 any more
    if (it + 2 < ntiles) mha_load_tile(buf(it + 2), kbuf, vbuf, kv, mask, L, H, h, q0, nw, it + 2, wave, lane);
    if (it * kKT > wave_last) continue;  // past every query of this wave
    const uint8_t *tb = buf(it);
    const uint32_t mw0 = *reinterpret_cast<const uint32_t *>(tb + kMOff + (kQW * wave + c) * 4);
    const uint32_t mw1 = *reinterpret_cast<const uint32_t *>(tb + kMOff + (kQW * wave + 16 + c) * 4);
    if (__builtin_amdgcn_ballot_w64((mw0 | mw1) != 0u) == 0) continue;  // nothing selected in this tile
    // logits S^T[key, query]: x[r] = key 4g + r, x[4 + r] = key 16 + 4g + r
    f32x4 s[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) s[u][0] = s[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      if (st < kNopeSteps) {
        const f16x8 a0 = *reinterpret_cast<const f16x8 *>(tb + c * kKRow + st * 64 + g * 16);
        const f16x8 a1 = *reinterpret_cast<const f16x8 *>(tb + (16 + c) * kKRow + st * 64 + g * 16);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          s[u][0] = mfma_f16_16x16x32(a0, qn[u][st], s[u][0]);
          s[u][1] = mfma_f16_16x16x32(a1, qn[u][st], s[u][1]);
        }
      } else {
        const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(tb + c * kKRow + st * 64 + g * 16);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(tb + (16 + c) * kKRow + st * 64 + g * 16);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          s[u][0] = mfma_bf16_16x16x32(a0, qr[u][st - kNopeSteps], s[u][0]);
          s[u][1] = mfma_bf16_16x16x32(a1, qr[u][st - kNopeSteps], s[u][1]);
        }
      }
    }
    float x[2][8];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[u][r] = s[u][0][r];
        x[u][4 + r] = s[u][1][r];
      }
    // mask the unselected keys, unless every lane's keys are all selected
    const bool partial = (mw0 & lane_bits) != lane_bits || (mw1 & lane_bits) != lane_bits;
    if (__builtin_amdgcn_ballot_w64(partial) != 0) {
      const uint32_t mw[2] = {mw0, mw1};
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int bit = (r < 4 ? 0 : 12) + 4 * g + r;
          x[u][r] = (mw[u] >> bit) & 1u ? x[u][r] : -INFINITY;
        }
    }
    float mx[2];
    bool raise = false;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      mx[u] = query_max(x[u]) * scale_log2;
      raise |= mx[u] > m_ref[u] + kRefSlack;
    }
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // rare: move the references, rescale what was summed
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bool up = mx[u] > m_ref[u] + kRefSlack;
        const float alpha = up ? __builtin_amdgcn_exp2f(m_ref[u] - mx[u]) : 1.0f;
        m_ref[u] = up ? mx[u] : m_ref[u];
        l_run[u] *= alpha;
#pragma unroll
        for (int v = 0; v < kVT; ++v)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[u][v][r] *= alpha;
      }
    }
    // probabilities in fp16 (at most 2^8 against the reference)
    f16x8 pb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float psum = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(x[u][i], scale_log2, -m_ref[u]));
        psum += p;
        pb[u][i] = (_Float16)p;
      }
      l_run[u] += psum;
    }
    // PV: O^T[dv, query] += V^T[dv, keys] P^T[keys, query]
#pragma unroll
    for (int v = 0; v < kVT; ++v) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(tb + tr_off + v * 32));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(tb + tr_off + v * 32 + 16 * kVRow));
      const i16x4 lohi[2] = {lo, hi};
      const f16x8 va = *reinterpret_cast<const f16x8 *>(lohi);
#pragma unroll
      for (int u = 0; u < 2; ++u) o[u][v] = mfma_f16_16x16x32(va, pb[u], o[u][v]);
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    // the four lane groups hold different keys of the same query
    float l_tot = l_run[u] + __shfl_xor(l_run[u], 16);
    l_tot += __shfl_xor(l_tot, 32);
    const int t = q0 + kQW * wave + 16 * u + c;
    if (t >= L) continue;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    // lane (g, c): value dims 16 v + 4 g .. +4 of query t
#pragma unroll
    for (int v = 0; v < kVT; ++v) {
      bf16x4 o4;
#pragma unroll
      for (int r = 0; r < 4; ++r) o4[r] = (__bf16)(o[u][v][r] * inv);
      *reinterpret_cast<bf16x4 *>(out + ((int64_t)t * H + h) * kDvh + 16 * v + 4 * g) = o4;
    }
    if (lse && g == 0)
      lse[(int64_t)t * H + h] = l_tot > 0.0f ? (m_ref[u] + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  }
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
  _Float16 *kbuf = (_Float16 *)workspace;
  _Float16 *vbuf = (_Float16 *)((char *)workspace + kvb);
  uint32_t *mask = (uint32_t *)((char *)workspace + 2 * kvb);
  static bool attr_done = false;  // per process: the attribute holds for every device
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void *)mha_upproj_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kUpBuf);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void *)masked_mha_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            kAttnSmem);
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
