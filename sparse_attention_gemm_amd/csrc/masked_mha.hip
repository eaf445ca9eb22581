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

#include <type_traits>

#include "dsa_common.h"
#include "dsa_launch.h"
#include "dsa_sizes.h"

namespace {

constexpr int kDc = 512;   // compressed latent dims
constexpr int kDr = 64;    // rope dims (shared by every head)
constexpr int kDn = dsa::kMhaDn;  // per-head key dims from the up-projection
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

// s_waitcnt immediate: at most n vector-memory operations outstanding
// (expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// ------------------------------------------------------------- up-projection
constexpr int kUpE = 2 * kDn;  // output rows per workgroup: K_h (W_uk[h] rows), then V_h (W_uv[h] rows)
constexpr int kUpT = dsa::kMhaUpT;  // tokens per workgroup (K_h and V_h rows are padded to a multiple of this)
constexpr int kUpK = 32;       // latent dims per LDS chunk
constexpr int kUpSlots = 4;    // LDS row: 4 x 16 B, unpadded; chunk j of row r sits at chunk up_chunk(r, j)
constexpr int kUpRow = kUpSlots * 16;
// Swizzle of the 16-byte chunks of a 64-byte row: with the operand reads
// (lane 16g + c: row c, chunk g) it spreads a read over distinct banks
// (measured on gfx950: half the LDS cycles of a 16-byte row padding).
__host__ __device__ constexpr int up_chunk(int r, int j) { return j ^ ((r >> 1) & 3); }
constexpr int kUpRows = kUpE + kUpT;                       // W rows, then token rows
constexpr int kUpInsts = kUpRows * kUpSlots / 64;          // 32 wave-wide 1 KB loads per chunk
static_assert(kUpRows * kUpSlots % 64 == 0 && kUpInsts % 8 == 0, "whole loads, the same count per wave");
constexpr int kUpStage = kUpInsts * 1024;                  // 32 KB
constexpr int kUpNBuf = 3;                                 // chunk kc+2 loads while chunk kc is computed
constexpr int kUpSmem = kUpNBuf * kUpStage;
constexpr int kUpChunks = kDc / kUpK;                      // 16

// K_h[s, e] = fp16(sum_c w_uk[h, e, c] kv[s, c]) and V_h[s, e] likewise, for
// one head h (blockIdx.y) and 256 tokens (blockIdx.x): a 256 x 256 x 512 GEMM
// per workgroup, which reads 512 KB for 67 MFLOP.  The MFMA computes the
// transpose D[e][s] = W[e][:] . kv[s][:], so a lane ends with four
// consecutive output dims of one token (one 8-byte store).  Eight waves: wave
// w owns rows 64 (w & 3) .. +64 (K_h for w & 3 < 2, V_h otherwise) and tokens
// 128 (w >> 2) .. +128.  Operands reach LDS by direct-to-LDS loads in chunks of
// 32 latent dims (64-byte rows, chunk-swizzled), three chunks deep; token rows
// past L read row L - 1 and their outputs land in the padding rows.
__global__ __launch_bounds__(512) void mha_upproj_kernel(const __bf16 *__restrict__ kv,
                                                         const __bf16 *__restrict__ w_uk,
                                                         const __bf16 *__restrict__ w_uv, int L, int H,
                                                         _Float16 *__restrict__ kout, _Float16 *__restrict__ vout) {
  extern __shared__ __align__(16) uint8_t up_smem[];  // kUpNBuf chunk buffers of kUpStage bytes
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.y;
  const int s0 = blockIdx.x * kUpT;
  // this wave's loads: instruction i = wave + 8 n, slot i*64 + lane -> LDS row slot/4, chunk slot%4,
  // which holds the source row's chunk up_chunk(row, slot%4)
  const char *src[kUpInsts / 8];
  {
    int l = lane;
    asm volatile("" : "+v"(l));
#pragma unroll
    for (int n = 0; n < kUpInsts / 8; ++n) {
      const int slot = (wave + 8 * n) * 64 + l;
      const int row = slot / kUpSlots, j = up_chunk(row, slot % kUpSlots);
      const __bf16 *p;
      if (row < kDn)
        p = w_uk + ((int64_t)h * kDn + row) * kDc;
      else if (row < kUpE)
        p = w_uv + ((int64_t)h * kDvh + row - kDn) * kDc;
      else
        p = kv + (int64_t)min(s0 + row - kUpE, L - 1) * kDl;
      src[n] = (const char *)p + j * 16;
    }
  }
  auto load_chunk = [&](int kc, uint8_t *dst) {
#pragma unroll
    for (int n = 0; n < kUpInsts / 8; ++n)
      __builtin_amdgcn_global_load_lds(src[n] + kc * kUpK * 2, (lds_void *)(dst + (wave + 8 * n) * 1024), 16, 0, 0);
  };
  f32x4 acc[4][8];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int e0 = 64 * (wave & 3), t0 = kUpE + 128 * (wave >> 2);  // LDS row of the wave's first W / token row
  load_chunk(0, up_smem);
  load_chunk(1, up_smem + kUpStage);
  int cur = 0, nxt2 = 2 * kUpStage;
  auto step = [](int b) { return b == (kUpNBuf - 1) * kUpStage ? 0 : b + kUpStage; };
  for (int kc = 0; kc < kUpChunks; ++kc, cur = step(cur), nxt2 = step(nxt2)) {
    if (kc + 1 < kUpChunks)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kUpInsts / 8));  // chunk kc landed; chunk kc+1 may be in flight
    else
      __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // every wave's loads of chunk kc landed; chunk kc-1's buffer is free
    if (kc + 2 < kUpChunks) load_chunk(kc + 2, up_smem + nxt2);
    const uint8_t *b = up_smem + cur + c * kUpRow + up_chunk(c, g) * 16;  // rows 16i + c share the swizzle of c
    bf16x8 a[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) a[m] = *reinterpret_cast<const bf16x8 *>(b + (e0 + 16 * m) * kUpRow);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const bf16x8 bb = *reinterpret_cast<const bf16x8 *>(b + (t0 + 16 * n) * kUpRow);
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[m][n] = mfma_bf16_16x16x32(a[m], bb, acc[m][n]);
    }
  }
  // lane (g, c) of tile (m, n): output dims e0 + 16m + 4g .. +4 of token s0 + 128 (w >> 2) + 16n + c
  _Float16 *out = (wave & 3) < 2 ? kout : vout;
  const int eo = 64 * (wave & 1);  // first dim of the wave within K_h or V_h
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int64_t s = s0 + 128 * (wave >> 2) + 16 * n + c;  // rows past L (up to the block's end) are written too
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      f16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = to_f16_sat(acc[m][n][i]);
      *reinterpret_cast<f16x4 *>(out + (s * H + h) * kDn + eo + 16 * m + 4 * g) = v;
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
constexpr int kQW = 32;        // queries per wave (two groups of 16)
constexpr int kQB = 4 * kQW;   // queries per workgroup
static_assert(kQB == dsa::kMhaQB, "queries per workgroup");
constexpr int kKT = 32;        // keys per tile
// A tile buffer holds four regions, each filled by whole direct-to-LDS
// instructions (1 KB, or 256 B for the mask words); instruction i writes
// 16 (or 4) bytes per lane in lane order.  Row strides are padded so that the
// operand reads below hit distinct banks.
constexpr int kKnSlots = 18;  // K no-rope row: 16 x 16 B (128 fp16 dims) + 2 pad (72 dwords)
constexpr int kKrSlots = 8;   // K rope row: 8 x 16 B (64 bf16 dims), unpadded; chunk j of row r at kr_chunk(r, j)
constexpr int kVSlots = 18;   // V row: 16 x 16 B (128 fp16 dims) + 2 pad (72 dwords)
constexpr int kKnRow = kKnSlots * 16, kKrRow = kKrSlots * 16, kVRow = kVSlots * 16;
// Row strides (72-dword rows) and the rope swizzle keep the operand reads
// (lane 16g + c: row c, 16-byte chunk g of a K step) on distinct banks
// (measured on gfx950: half the LDS cycles of 68- or 36-dword rows).
__host__ __device__ constexpr int kr_chunk(int r, int j) { return j ^ (r & 7); }
constexpr int kKnInsts = (kKT * kKnSlots + 63) / 64;  // 9
constexpr int kKrInsts = (kKT * kKrSlots + 63) / 64;  // 4
constexpr int kVInsts = (kKT * kVSlots + 63) / 64;    // 9
constexpr int kMInsts = kQB * 4 / 256;                // 2: one mask word per query
constexpr int kKrOff = kKnInsts * 1024;
constexpr int kVOff = kKrOff + kKrInsts * 1024;
constexpr int kMOff = kVOff + kVInsts * 1024;
constexpr int kTileBytes = kMOff + kMInsts * 256;
constexpr int kTileInsts = kKnInsts + kKrInsts + kVInsts + kMInsts;  // 24
constexpr int kInstsW = kTileInsts / 4;                              // 6 per wave
static_assert(kTileInsts % 4 == 0, "every wave issues the same number of loads per tile");
constexpr int kNBuf = 3;                  // tile j+2 loads while tile j is computed
// LDS of the attention kernel, as separate static arrays: the kNBuf tile
// buffers and the mask table (entry n keeps fp16 element e of a group's 8
// probabilities iff bit e of n is set).  Distinct objects let the compiler
// tell an LDS read of one buffer from the loads in flight into another; in
// one block it waited for the next tile's loads before reading the current
// tile.
__shared__ __align__(16) uint8_t g_mha_r0[kTileBytes];
__shared__ __align__(16) uint8_t g_mha_r1[kTileBytes];
__shared__ __align__(16) uint8_t g_mha_r2[kTileBytes];
__shared__ __align__(16) uint4 g_mha_lut[256];
static_assert(kNBuf == 3, "three ring buffers");
template <int B>
__device__ __forceinline__ uint8_t *mha_ring() {
  return B == 0 ? g_mha_r0 : (B == 1 ? g_mha_r1 : g_mha_r2);
}
constexpr int kSteps = kDq / 32;       // 6 K steps of the logits MFMA
constexpr int kNopeSteps = kDn / 32;   // the first 4 cover the up-projected (fp16) dims
constexpr int kVT = kDvh / 16;         // 8 value tiles of the PV MFMA (a ninth sums the probabilities)
constexpr float kUnset = -1e30f;       // no reference yet
constexpr uint32_t kRaiseBits = 0x5C00u;  // fp16 bits of 2^8
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format

// Per-half unsigned max of two packed 16-bit pairs.
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const u16x2 m = __builtin_elementwise_max(*reinterpret_cast<const u16x2 *>(&a), *reinterpret_cast<const u16x2 *>(&b));
  return *reinterpret_cast<const uint32_t *>(&m);
}


// Per-workgroup state shared by the walks.
struct MhaCtx {
  const char *kn, *kr, *vb, *mk;     // tile-0 bases: K_h no-rope, latent rope, V_h, mask column 0
  int kr_len, mk_len;                // bytes readable from the rope and mask bases
  int64_t kv_tile;                   // bytes between tiles in K_h / V_h (32 keys x H heads x 256 B)
  uint32_t loff[kInstsW];           // the lane's byte offset within its instructions' tiles
  int wave, lane, g, c;
  int L, H, h, q0, ntiles, wave_last;
};

// Raw buffer descriptor of [base + skip, base + len): loads past the end read
// 0.  Uniform 32-bit arithmetic (scalar unit).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char *base, int len, int skip) {
  return __builtin_amdgcn_make_buffer_rsrc((void *)(base + skip), 0, max(len - skip, 0), (int)kRsrcWord3);
}
// Descriptor of base + skip with no bound (the K_h / V_h rows of every tile exist).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char *base, int64_t skip) {
  return __builtin_amdgcn_make_buffer_rsrc((void *)(base + skip), 0, 0x7fffffff, (int)kRsrcWord3);
}

// Issue this wave's direct-to-LDS loads of tile `tile` into buffer dst.
// Instruction i = wave + 4n covers its region's slots in lane order; a slot
// past a region's data loads a duplicate of valid data.  Each region is read
// through a descriptor rebased on the tile and bounded by its buffer, so the
// rope rows past L (the caller's latent has L rows) read 0; K_h and V_h rows
// past L exist (padded to whole up-projection blocks).  All of them are
// masked.
__device__ __forceinline__ void mha_load_tile(const MhaCtx &cx, uint8_t *dst, int tile) {
  const __amdgpu_buffer_rsrc_t rkn = tile_rsrc(cx.kn, tile * cx.kv_tile);
  const __amdgpu_buffer_rsrc_t rkr = tile_rsrc(cx.kr, cx.kr_len, tile * kKT * kDl * 2);
  const __amdgpu_buffer_rsrc_t rvb = tile_rsrc(cx.vb, tile * cx.kv_tile);
  const __amdgpu_buffer_rsrc_t rmk = tile_rsrc(cx.mk, cx.mk_len, tile * 4);
#pragma unroll
  for (int n = 0; n < kInstsW; ++n) {
    const int i = cx.wave + 4 * n;  // uniform
    if (i >= kTileInsts) break;
    if (i < kKnInsts)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rkn, (lds_void *)(dst + i * 1024), 16, cx.loff[n], 0, 0, 0);
    else if (i < kKnInsts + kKrInsts)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rkr, (lds_void *)(dst + kKrOff + (i - kKnInsts) * 1024), 16,
                                               cx.loff[n], 0, 0, 0);
    else if (i < kKnInsts + kKrInsts + kVInsts)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rvb, (lds_void *)(dst + kVOff + (i - kKnInsts - kKrInsts) * 1024),
                                               16, cx.loff[n], 0, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rmk, (lds_void *)(dst + kMOff + (i - kKnInsts - kKrInsts - kVInsts) * 256), 4, cx.loff[n], 0, 0, 0);
  }
}

// Max of the query's 8 keys in this lane and its 3 partner lanes (c, c+16,
// c+32, c+48 hold the same query).  With both operands equal, a permlane swap
// returns the row pair's two halves.
__device__ __forceinline__ float query_max(const float (&x)[8]) {
  float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  mx = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// Q^T of the lane's two queries, dims 32 s + 8 g .. +8: the no-rope steps in
// fp16 (exact for |q| within fp16's normal range) against the fp16 K_h, the
// rope steps in bf16 against the latent's rope dims.
__device__ __forceinline__ void mha_load_q(const MhaCtx &cx, const __bf16 *__restrict__ q, f16x8 (&qn)[2][kNopeSteps],
                                           bf16x8 (&qr)[2][kSteps - kNopeSteps]) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int64_t tq = min(cx.q0 + kQW * cx.wave + 16 * u + cx.c, cx.L - 1);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const bf16x8 v = *reinterpret_cast<const bf16x8 *>(q + (tq * cx.H + cx.h) * kDq + 32 * s + 8 * cx.g);
      if (s < kNopeSteps) {
#pragma unroll
        for (int i = 0; i < 8; ++i) qn[u][s][i] = to_f16_sat((float)v[i]);
      } else {
        qr[u][s - kNopeSteps] = v;
      }
    }
  }
}

// The walk over the workgroup's key tiles (loads pipelined kNBuf - 1 tiles
// ahead, one barrier per tile).  Per group u: logits S^T[key, query] with
// x[r] = key 4g + r, x[4 + r] = key 16 + 4g + r of the tile; probabilities
// p = 2^(x * scale_log2 - m_ref) in fp16, the unselected ones zeroed by an
// AND with the mask table's lane masks; the PV MFMA takes V^T through the
// transposing LDS load, and a ninth tile of constant ones rows sums the
// probabilities: o[u][kVT] row 0 is the query's softmax sum.
// A query's reference m_ref only moves up: when some probability of the
// wave reaches 2^8 (or the query has no reference yet, which makes its
// selected probabilities infinite), the wave takes the re-reference branch:
// the exact max of each query's selected logits in the tile becomes its
// reference where it lies above the old one, the query's accumulators are
// scaled down to it, and the probabilities are formed again.  So every
// probability that reaches the sums is below 2^8.
__device__ __forceinline__ void mha_walk(const MhaCtx &cx, const f16x8 (&qn)[2][kNopeSteps],
                                         const bf16x8 (&qr)[2][kSteps - kNopeSteps], float scale_log2,
                                         float (&m_ref)[2], f32x4 (&o)[2][kVT + 1]) {
  const int g = cx.g, c = cx.c, wave = cx.wave;
  const int tr_off = kVOff + (4 * g + (c >> 2)) * kVRow + (c & 3) * 8;
  const uint4 *lut = g_mha_lut;
  f16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = c == 0 ? (_Float16)1.0f : (_Float16)0.0f;
  // tile it sits in ring buffer it % 3; the walk is unrolled by three so that
  // every buffer is a fixed object
  mha_load_tile(cx, mha_ring<0>(), 0);
  if (cx.ntiles > 1) mha_load_tile(cx, mha_ring<1>(), 1);
  auto tile_step = [&](auto bc, int it) {
    constexpr int B = decltype(bc)::value;
    if (it + 1 < cx.ntiles) {  // tile it landed; tile it+1 may still be in flight
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kInstsW));
    } else {
      __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();  // every wave's loads of tile it landed; nobody reads tile it-1 any more
    if (it + 2 < cx.ntiles) mha_load_tile(cx, mha_ring<(B + 2) % 3>(), it + 2);
    if (it * kKT > cx.wave_last) return;  // past every query of this wave
    const uint8_t *tb = mha_ring<B>();
    uint32_t mw[2];
    mw[0] = *reinterpret_cast<const uint32_t *>(tb + kMOff + (kQW * wave + c) * 4);
    mw[1] = *reinterpret_cast<const uint32_t *>(tb + kMOff + (kQW * wave + 16 + c) * 4);
    if (__builtin_amdgcn_ballot_w64((mw[0] | mw[1]) != 0u) == 0) return;  // nothing selected in this tile
    f32x4 s[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) s[u][0] = s[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < kNopeSteps; ++st) {
      const f16x8 a0 = *reinterpret_cast<const f16x8 *>(tb + c * kKnRow + st * 64 + g * 16);
      const f16x8 a1 = *reinterpret_cast<const f16x8 *>(tb + (16 + c) * kKnRow + st * 64 + g * 16);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        s[u][0] = mfma_f16_16x16x32(a0, qn[u][st], s[u][0]);
        s[u][1] = mfma_f16_16x16x32(a1, qn[u][st], s[u][1]);
      }
    }
#pragma unroll
    for (int st = 0; st < kSteps - kNopeSteps; ++st) {
      // rows c and 16 + c share the swizzle of c
      const int kro = kKrOff + c * kKrRow + kr_chunk(c, 4 * st + g) * 16;
      const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(tb + kro);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(tb + kro + 16 * kKrRow);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        s[u][0] = mfma_bf16_16x16x32(a0, qr[u][st], s[u][0]);
        s[u][1] = mfma_bf16_16x16x32(a1, qr[u][st], s[u][1]);
      }
    }
    float x[2][8];
    uint4 keep[2];  // fp16 lane masks of the selected keys, in x order
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[u][r] = s[u][0][r];
        x[u][4 + r] = s[u][1][r];
      }
      keep[u] = lut[((mw[u] >> (4 * g)) & 0xFu) | ((mw[u] >> (12 + 4 * g)) & 0xF0u)];
    }
    uint4 pbits[2];
    auto probabilities = [&]() {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        f16x8 p;
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = (_Float16)__builtin_amdgcn_exp2f(fmaf(x[u][i], scale_log2, -m_ref[u]));
        const uint4 b = *reinterpret_cast<const uint4 *>(&p);
        pbits[u] = uint4{b.x & keep[u].x, b.y & keep[u].y, b.z & keep[u].z, b.w & keep[u].w};
      }
    };
    probabilities();
    // largest kept probability of the lane (non-negative fp16 orders like its bits)
    uint32_t top = pk_max_u16(pk_max_u16(pk_max_u16(pbits[0].x, pbits[0].y), pk_max_u16(pbits[0].z, pbits[0].w)),
                              pk_max_u16(pk_max_u16(pbits[1].x, pbits[1].y), pk_max_u16(pbits[1].z, pbits[1].w)));
    top = pk_max_u16(top, top >> 16) & 0xFFFFu;
    if (__builtin_amdgcn_ballot_w64(top >= kRaiseBits) != 0) {  // rare: move references up
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t sel = ((mw[u] >> (4 * g)) & 0xFu) | ((mw[u] >> (12 + 4 * g)) & 0xF0u);
        float xm[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) xm[r] = (sel >> r) & 1u ? x[u][r] : -INFINITY;
        const float mx = query_max(xm) * scale_log2;
        const float ref = mx > m_ref[u] ? mx : m_ref[u];
        const float alpha = __builtin_amdgcn_exp2f(m_ref[u] - ref);  // 0 from the unset reference
        m_ref[u] = ref;
#pragma unroll
        for (int v = 0; v <= kVT; ++v)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[u][v][r] *= alpha;
      }
      probabilities();
    }
    f16x8 pb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) pb[u] = *reinterpret_cast<const f16x8 *>(&pbits[u]);
    // PV: O^T[dv, query] += V^T[dv, keys] P^T[keys, query]
    lds_i16x4 *vrow = (lds_i16x4 *)(tb + tr_off);  // LDS-space pointer: the reads below take immediate offsets
#pragma unroll
    for (int v = 0; v < kVT; ++v) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(vrow + v * 4);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(vrow + v * 4 + 16 * kVRow / 8);
      const i16x4 lohi[2] = {lo, hi};
      const f16x8 va = *reinterpret_cast<const f16x8 *>(lohi);
#pragma unroll
      for (int u = 0; u < 2; ++u) o[u][v] = mfma_f16_16x16x32(va, pb[u], o[u][v]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) o[u][kVT] = mfma_f16_16x16x32(ones, pb[u], o[u][kVT]);
  };
  for (int it = 0; it < cx.ntiles; it += 3) {
    tile_step(std::integral_constant<int, 0>(), it);
    if (it + 1 < cx.ntiles) tile_step(std::integral_constant<int, 1>(), it + 1);
    if (it + 2 < cx.ntiles) tile_step(std::integral_constant<int, 2>(), it + 2);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // the tile buffers are free
}

// The query's softmax sum, from row 0 of the sums tile (lane (0, c)).
__device__ __forceinline__ float query_sum(const f32x4 &sums, int c) { return __shfl(sums[0], c); }

// Normalise and store the lane's outputs (value dims 16 v + 4 g .. +4) and lse.
__device__ __forceinline__ void mha_epilogue(const MhaCtx &cx, const float (&m_ref)[2], const float (&l)[2],
                                             const f32x4 (&o)[2][kVT + 1], __bf16 *__restrict__ out,
                                             float *__restrict__ lse) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int t = cx.q0 + kQW * cx.wave + 16 * u + cx.c;
    if (t >= cx.L) continue;
    const float inv = l[u] > 0.0f ? 1.0f / l[u] : 0.0f;
#pragma unroll
    for (int v = 0; v < kVT; ++v) {
      bf16x4 o4;
#pragma unroll
      for (int r = 0; r < 4; ++r) o4[r] = (__bf16)(o[u][v][r] * inv);
      *reinterpret_cast<bf16x4 *>(out + ((int64_t)t * cx.H + cx.h) * kDvh + 16 * v + 4 * cx.g) = o4;
    }
    if (lse && cx.g == 0)
      lse[(int64_t)t * cx.H + cx.h] = l[u] > 0.0f ? (m_ref[u] + log2f(l[u])) * 0.69314718055994531f : -INFINITY;
  }
}

// One workgroup per (128 queries, head).  Wave w owns queries q0 + 32 w ..
// +32 in two groups of 16; lane (g, c) holds query q0 + 32 w + 16 u + c of
// group u for the softmax and the output.  Each K and V fragment read from
// LDS feeds both groups' MFMAs.  Workgroups are numbered head-major with each
// head's longest query blocks first, and consecutive numbers go to the same
// XCD (workgroup i runs on XCD i mod 8), so that one head's keys and values
// stay in one L2.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void masked_mha_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ kv, const _Float16 *__restrict__ kbuf,
    const _Float16 *__restrict__ vbuf, const uint32_t *__restrict__ mask, int L, int H, float scale_log2,
    __bf16 *__restrict__ out, float *__restrict__ lse) {
  MhaCtx cx;
  const int tid = threadIdx.x;
  cx.lane = tid & 63;
  cx.g = cx.lane >> 4;
  cx.c = cx.lane & 15;
  cx.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  cx.L = L;
  cx.H = H;
  const int nqb = (L + kQB - 1) / kQB;
  int lin;
  {
    const int n = gridDim.x, i = blockIdx.x, x = i & 7, per = n >> 3, rem = n & 7;
    lin = x * per + min(x, rem) + (i >> 3);
  }
  cx.h = lin / nqb;
  cx.q0 = (nqb - 1 - lin % nqb) * kQB;
  cx.ntiles = (min(cx.q0 + kQB, L) + kKT - 1) / kKT;           // causal bound of the workgroup
  cx.wave_last = min(cx.q0 + kQW * cx.wave + kQW - 1, L - 1);  // this wave's last query
  const int nw = (L + 31) >> 5;
  cx.kn = (const char *)(kbuf + cx.h * kDn);
  cx.vb = (const char *)(vbuf + cx.h * kDvh);
  cx.kr = (const char *)(kv + kDc);
  cx.mk = (const char *)mask;
  cx.kr_len = L * kDl * 2 - kDc * 2;  // < 2^31 for L <= 65536
  cx.mk_len = L * nw * 4;
  cx.kv_tile = (int64_t)kKT * H * kDn * 2;
  // lane offsets of this wave's instructions (fixed for every tile)
#pragma unroll
  for (int n = 0; n < kInstsW; ++n) {
    const int i = cx.wave + 4 * n;
    uint32_t off = 0;
    if (i < kKnInsts) {
      const int slot = i * 64 + cx.lane, r = min(slot / kKnSlots, kKT - 1), j = min(slot % kKnSlots, 15);
      off = (uint32_t)r * H * kDn * 2 + j * 16;
    } else if (i < kKnInsts + kKrInsts) {
      const int slot = (i - kKnInsts) * 64 + cx.lane, r = slot / kKrSlots, j = kr_chunk(r, slot % kKrSlots);
      off = (uint32_t)r * kDl * 2 + j * 16;
    } else if (i < kKnInsts + kKrInsts + kVInsts) {
      const int slot = (i - kKnInsts - kKrInsts) * 64 + cx.lane, r = min(slot / kVSlots, kKT - 1),
                j = min(slot % kVSlots, 15);
      off = (uint32_t)r * H * kDvh * 2 + j * 16;
    } else if (i < kTileInsts) {
      const int t = min(cx.q0 + (i - kKnInsts - kKrInsts - kVInsts) * 64 + cx.lane, L - 1);
      off = (uint32_t)t * nw * 4;
    }
    cx.loff[n] = off;
  }
  // mask table: entry n keeps fp16 element e of a group's 8 probabilities iff bit e of n is set
  {
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
      w[d] = ((tid >> (2 * d)) & 1 ? 0x0000FFFFu : 0u) | ((tid >> (2 * d + 1)) & 1 ? 0xFFFF0000u : 0u);
    g_mha_lut[tid] = uint4{w[0], w[1], w[2], w[3]};
  }
  // (the table is read only after the walk's first barrier)
  f16x8 qn[2][kNopeSteps];
  bf16x8 qr[2][kSteps - kNopeSteps];
  mha_load_q(cx, q, qn, qr);
  f32x4 o[2][kVT + 1];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v <= kVT; ++v) o[u][v] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref[2] = {kUnset, kUnset}, l[2];
  mha_walk(cx, qn, qr, scale_log2, m_ref, o);
#pragma unroll
  for (int u = 0; u < 2; ++u) l[u] = query_sum(o[u][kVT], cx.c);
  mha_epilogue(cx, m_ref, l, o, out, lse);
}

}  // namespace

namespace dsa {
static size_t mha_groups(int32_t L, int32_t H) { return (size_t)(L + kQB - 1) / kQB * H; }

hipError_t launch_masked_mha(const void *q, const void *kv, const void *w_uk, const void *w_uv,
                             const int32_t *idx, int32_t L, int32_t H, int32_t k, float sm_scale, void *out,
                             float *lse, void *workspace, hipStream_t s) {
  if (L == 0) return hipSuccess;
  const size_t kvb = masked_mha_kv_bytes(L, H);
  _Float16 *kbuf = (_Float16 *)workspace;
  _Float16 *vbuf = (_Float16 *)((char *)workspace + kvb);
  uint32_t *mask = (uint32_t *)((char *)workspace + 2 * kvb);
  static bool attr_done = false;  // per process: the attribute holds for every device
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void *)mha_upproj_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kUpSmem);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  hipLaunchKernelGGL(mha_upproj_kernel, dim3((L + kUpT - 1) / kUpT, H), dim3(512), kUpSmem, s, (const __bf16 *)kv,
                     (const __bf16 *)w_uk, (const __bf16 *)w_uv, L, H, kbuf, vbuf);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mha_mask_kernel, dim3(L), dim3(256), 0, s, idx, L, k, mask);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((uint32_t)mha_groups(L, H));
  const float sl2 = sm_scale * 1.4426950408889634f;
  // the attention kernel's LDS is static (g_mha_*)
  hipLaunchKernelGGL(masked_mha_kernel, grid, dim3(256), 0, s, (const __bf16 *)q, (const __bf16 *)kv, kbuf,
                     vbuf, mask, L, H, sl2, (__bf16 *)out, lse);
  return hipGetLastError();
}
}  // namespace dsa
