// Sparse MLA forward in MQA mode over the selected latent rows.
//
// Main attention runs only over the KV entries picked by the top-k
// (mizuki-eaf.pages.dev, "How it works"; m.digipub.cc, section 2) and is MLA
// in MQA mode: one latent row per token, shared by every query head of a
// query token, which is what lets a kernel fetch each KV entry once for all
// heads (mizuki-eaf.pages.dev, "built on MLA").  Latent width 576 (512 + 64
// rope); the value is the first 512 dims.
//
// bf16 kernel (one workgroup per query token and group of 16*NW heads):
//  * the physical rows of the workgroup's selection are resolved once (index,
//    then block table when paged) into LDS;
//  * the selected latent rows are gathered 32 at a time straight from global
//    memory into LDS (direct-to-LDS loads, no register staging), row-major,
//    into three buffers; each row is fetched once for all heads;
//  * logits are computed transposed, S^T = C Q^T (keys x heads), with bf16
//    MFMA 16x16x32 and Q^T resident in registers; in that layout each lane
//    holds 8 keys of one head, which is exactly the B operand layout the PV
//    MFMA needs (up to a fixed permutation of the keys), so P never moves
//    between lanes;
//  * the value operand of PV (value dims x keys) is read from the same
//    row-major tile with the transposing LDS load, which hands each lane four
//    keys of one value column;
//  * probabilities and PV are pipelined across tiles with one barrier per
//    tile: while tile j+2 is gathered, the probabilities of tile j+1 are
//    formed and published and PV runs on tile j;
//  * online softmax in fp32 (base-2 exponent with the scale folded in),
//    output O^T (value dims x heads) accumulated in fp32 registers;
//  * optional split of the selection across workgroups with an LSE-weighted
//    combine (used when there are too few queries to fill the GPU).
#include <algorithm>

#include "dsa_common.h"
#include "dsa_launch.h"

namespace {

constexpr int kBN = 32;                  // selected rows per tile
constexpr int kRowSlots = 74;            // 16-byte slots per LDS row: 72 of data + 2 pad; a row stride
                                         // of 40 dwords mod 64 keeps both tile read patterns conflict-free
constexpr int kCRow = kRowSlots * 16;    // LDS bytes per gathered row
constexpr int kTileBytes = kBN * kCRow;  // 37376
constexpr int kTileSlots = kBN * kRowSlots;
constexpr int kGatherInsts = (kTileSlots + 63) / 64;  // wave-wide 1 KB direct-to-LDS loads per tile
constexpr int kPBytes = 8 * 64 * 16;    // P^T of up to 8 head tiles, in B-operand lane order
constexpr int kNBuf = 3;                 // gathered tiles: PV of tile j, logits of tile j+1, gather of j+2
constexpr int kSmemMla = kNBuf * kTileBytes + 2 * kPBytes + 128 * 4 + 2048 * 4 + 16;

typedef __attribute__((address_space(3))) void lds_void;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Row of kv for entry e of query t, or -1 (padding, or not a row of [0, N)).
__device__ __forceinline__ int64_t phys_row(const int32_t *__restrict__ irow, const int32_t *__restrict__ bt,
                                            int max_blocks, int64_t N, int64_t t, int e, int k) {
  if (e >= k) return -1;
  const int32_t sel = irow[e];
  if (sel < 0) return -1;
  if (!bt) return sel < N ? sel : -1;
  if ((sel >> 6) >= max_blocks) return -1;
  const int32_t blk = bt[t * max_blocks + (sel >> 6)];
  const int64_t row = (int64_t)blk * 64 + (sel & 63);
  return (blk >= 0 && row < N) ? row : -1;
}

// Issue the direct-to-LDS loads of tile rows [r0, r0+32) of this workgroup's
// selection (rows[] holds physical rows, -1 for skipped entries, which load
// row 0 instead and are masked later).  Instruction i of the tile writes LDS
// slots [64i, 64i+64); slot s holds row s/74, 16-byte chunk s%74 (chunks 72
// and 73 are padding and reload chunk 71).
template <int NW>
__device__ __forceinline__ void gather_tile_async(uint8_t *__restrict__ dst, const int *__restrict__ rows,
                                                  int r0, const __bf16 *__restrict__ kv, int wave, int lane) {
  static_assert(kTileSlots == kGatherInsts * 64, "every gather instruction is full");
  // Lane roles are recomputed per tile from a laundered lane id: hoisting
  // them would hold a 64-bit address per instruction for the whole kernel.
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
    const __bf16 *src = kv + ((int64_t)(pr >= 0 ? pr : 0) * 576 + j * 8);
    __builtin_amdgcn_global_load_lds(src, (lds_void *)(dst + i * 1024), 16, 0, 0);
  }
}

// Shared state of one sparse-MLA workgroup.
struct MlaCtx {
  const __bf16 *kv;
  uint8_t *tiles;       // kNBuf x kTileBytes of LDS
  uint8_t *pbuf;        // P^T exchange, two buffers of [head tile][lane] x 16 bytes
  float *lbuf;          // softmax sums of the workgroup's heads
  const int *rows;      // physical rows of the workgroup's entries (LDS)
  int *flag;            // LDS: set when a tile overshoots the softmax reference
  int tb, te;           // tile range of this workgroup
  int wave, lane, g, c;
};

// Logits of one tile for the wave's 16 heads: S^T[keys, heads] for key
// blocks [0,16) and [16,32), unscaled, -inf where masked; lane (g,c) gets
// x[r] = key 4g+r and x[4+r] = key 16+4g+r of head c.  The LDS operands of
// step s+1 are requested before the MFMAs of step s; the scheduling fences
// keep at most two steps of operands live.
__device__ __forceinline__ void tile_logits(const uint8_t *__restrict__ ct, const int *__restrict__ rv,
                                            const bf16x8 (&qr)[18], float scale_log2, int g, int c,
                                            float (&x)[8]) {
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
  const uint8_t *arow0 = ct + c * kCRow + g * 16;
  const uint8_t *arow1 = arow0 + 16 * kCRow;
  bf16x8 op[2][2];
  op[0][0] = *reinterpret_cast<const bf16x8 *>(arow0);
  op[0][1] = *reinterpret_cast<const bf16x8 *>(arow1);
#pragma unroll
  for (int s = 0; s < 18; ++s) {
    const int cs = s & 1;
    if (s + 1 < 18) {
      op[cs ^ 1][0] = *reinterpret_cast<const bf16x8 *>(arow0 + (s + 1) * 64);
      op[cs ^ 1][1] = *reinterpret_cast<const bf16x8 *>(arow1 + (s + 1) * 64);
    }
    s0 = mfma_bf16_16x16x32(op[cs][0], qr[s], s0);
    s1 = mfma_bf16_16x16x32(op[cs][1], qr[s], s1);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    x[r] = rv[4 * g + r] >= 0 ? s0[r] : -INFINITY;
    x[4 + r] = rv[16 + 4 * g + r] >= 0 ? s1[r] : -INFINITY;
  }
}

// Max over the tile's keys for the lane's head (lanes c, c+16, c+32, c+48),
// in base-2 units (scale > 0).  The cross-row steps are permlane swaps: with
// both operands equal, the two results hold the row pair's two halves.
__device__ __forceinline__ float tile_max(const float (&x)[8], float scale_log2) {
  float mx = x[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  mx = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  mx = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
  return mx * scale_log2;
}

// Walk the workgroup's tiles: wait for tile i, barrier, prefetch tile i+1,
// then body(ct, rv) on tile i.  The gather of tile i+1 overlaps the body.
template <int NW, typename Body>
__device__ __forceinline__ void for_each_tile(const MlaCtx &cx, Body &&body) {
  if (cx.tb < cx.te) gather_tile_async<NW>(cx.tiles, cx.rows, 0, cx.kv, cx.wave, cx.lane);
  int cur = 0;
  for (int tile = cx.tb; tile < cx.te; ++tile, cur ^= 1) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of `tile` have landed in LDS
    __syncthreads();                // ... and every wave's; the other buffer is no longer read
    if (tile + 1 < cx.te)
      gather_tile_async<NW>(cx.tiles + (cur ^ 1) * kTileBytes, cx.rows, (tile + 1 - cx.tb) * kBN, cx.kv, cx.wave,
                            cx.lane);
    body(cx.tiles + cur * kTileBytes, cx.rows + (tile - cx.tb) * kBN);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// s_waitcnt immediate: at most n vector-memory operations outstanding
// (expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Wait until only the newest tile's gathers may still be in flight (every
// tile costs a wave the same number of gather instructions).
template <int NW>
__device__ __forceinline__ void wait_all_but_newest_tile(int wave) {
  constexpr int base = kGatherInsts / NW, rem = kGatherInsts % NW;
  if (rem != 0 && wave < rem)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(base + 1));
  else
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(base));
}

// One accumulation pass over the workgroup's tiles.
//  * Logits/softmax: wave w owns head tile w (heads 16w..16w+15 of the
//    workgroup).  It turns its logits into bf16 probabilities and publishes
//    them, already in the PV B-operand lane order, in LDS.
//  * PV: wave w owns value dims [w*512/NW, (w+1)*512/NW) for ALL NW head
//    tiles: O^T[dv, head] += V^T[dv, keys] P^T[keys, head].  V^T comes from
//    the row-major tile through the transposing LDS load, P^T from LDS.
//    Splitting PV by value dims reads each tile's values once per workgroup
//    instead of once per wave.
//  * The two are pipelined across tiles with one barrier per tile: iteration
//    j computes the probabilities of tile j+1 and then PV of tile j with the
//    probabilities every wave published before the barrier.  Three tile
//    buffers (j, j+1, and j+2 being gathered) and two P buffers.
// fixed = false: each head's exponent reference is the max of its first tile
// with a valid entry; a later tile more than 64 above it sets cx.flag and the
// pass is discarded (returns false, nothing written).  fixed = true: the
// references are given (exact maxima).
template <int NW, bool fixed, bool late>
__device__ __forceinline__ bool mla_pass(const MlaCtx &cx, const bf16x8 (&qr)[18], float &m_ref, float scale_log2,
                                         int64_t t, int H, int hw0, __bf16 *__restrict__ out,
                                         float *__restrict__ lse, int splits, int sp, __bf16 *__restrict__ part_o,
                                         float *__restrict__ part_ml) {
  constexpr int MT = 32 / NW;  // value-dim tiles of 16 per wave
  const int g = cx.g, c = cx.c, wave = cx.wave;
  f32x4 o[MT][NW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int n = 0; n < NW; ++n) o[i][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float l_run = 0.0f;
  // transposing-load lane roles: row 4g + (c>>2) of each 4-row group, value chunk (c&3),
  // starting at this wave's first value tile
  const int tr_off = (4 * g + (c >> 2)) * kCRow + (c & 3) * 8 + wave * MT * 32;
  const int n = cx.te - cx.tb;
  auto tile_of = [&](int j) { return cx.tiles + (j % kNBuf) * kTileBytes; };
  auto gather = [&](int j) { gather_tile_async<NW>(tile_of(j), cx.rows, j * kBN, cx.kv, cx.wave, cx.lane); };
  // logits and probabilities of tile j, published in P buffer j&1
  auto score_tile = [&](int j) {
    float x[8];
    tile_logits(tile_of(j), cx.rows + j * kBN, qr, scale_log2, g, c, x);
    bool over = false;
    if (!fixed) {
      const float mx = tile_max(x, scale_log2);
      if (m_ref == -INFINITY) m_ref = mx;  // O and l are still zero for this head
      over = mx > m_ref + 64.0f;
    }
    const float msub = (m_ref == -INFINITY) ? 0.0f : m_ref;
    bf16x8 pb;
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // exponent <= 64 unless the pass is discarded; results below 2^-126 of
      // the reference flush to zero (v_exp_f32), which no sum can notice
      const float p = __builtin_amdgcn_exp2f(fmaf(x[i], scale_log2, -msub));
      psum += p;
      pb[i] = (__bf16)p;
    }
    l_run += psum;
    if (!fixed && __ballot(over) && cx.lane == 0) *cx.flag = 1;
    *reinterpret_cast<bf16x8 *>(cx.pbuf + (j & 1) * kPBytes + (wave * 64 + cx.lane) * 16) = pb;
  };
  // PV of tile j with the probabilities in P buffer j&1
  auto pv_tile = [&](int j) {
    const uint8_t *ct = tile_of(j);
    const uint8_t *pj = cx.pbuf + (j & 1) * kPBytes;
    // value operands of this wave's MT tiles (keys 4g..4g+3 | 16+4g..16+4g+3)
    bf16x8 va[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(ct + tr_off + i * 32));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(ct + tr_off + i * 32 + 16 * kCRow));
      const i16x4 lohi[2] = {lo, hi};
      va[i] = *reinterpret_cast<const bf16x8 *>(lohi);
    }
    bf16x8 pn[2];
    pn[0] = *reinterpret_cast<const bf16x8 *>(pj + cx.lane * 16);
#pragma unroll
    for (int nn = 0; nn < NW; ++nn) {
      if (nn + 1 < NW) pn[(nn + 1) & 1] = *reinterpret_cast<const bf16x8 *>(pj + ((nn + 1) * 64 + cx.lane) * 16);
#pragma unroll
      for (int i = 0; i < MT; ++i) o[i][nn] = mfma_bf16_16x16x32(va[i], pn[nn & 1], o[i][nn]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (n > 0) {
    gather(0);
    if (n > 1) {
      gather(1);
      wait_all_but_newest_tile<NW>(wave);  // tile 0 landed (tile 1 may be in flight)
    } else {
      __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();
    score_tile(0);
    for (int j = 0; j < n; ++j) {
      __builtin_amdgcn_s_waitcnt(0);  // this wave's gathers of tile j+1 have landed
      __syncthreads();  // P(j) from every wave; tile j+1 from every wave; nobody reads tile j-1 any more
      if (!late && j + 2 < n) gather(j + 2);
      if (j + 1 < n) score_tile(j + 1);
      if (late && j + 2 < n) gather(j + 2);
      pv_tile(j);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (!fixed) {
    // Uniform: every wave reads the flag after the final barrier, and nothing
    // writes it again until the redo's set-up clears it.  The barrier below
    // keeps that clear behind every wave's read, so no wave can miss the
    // overshoot and take the accept path alone.
    const int over = *cx.flag;
    if (over) {
      __syncthreads();
      return false;
    }
  }
  // softmax sums of the wave's head tile -> LDS, for the waves that own other value dims
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (g == 0) cx.lbuf[wave * 16 + c] = l_tot;
  const float mr = m_ref == -INFINITY ? 0.0f : m_ref;
  const int head_own = hw0 + wave * 16 + c;
  if (g == 0) {
    if (splits == 1) {
      if (lse) lse[t * H + head_own] = l_tot > 0.0f ? (mr + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    } else {
      float *pm = part_ml + ((t * splits + sp) * H + head_own) * 2;
      pm[0] = l_tot > 0.0f ? mr : -INFINITY;
      pm[1] = l_tot;
    }
  }
  __syncthreads();
#pragma unroll
  for (int n = 0; n < NW; ++n) {
    const int head = hw0 + n * 16 + c;
    const float lh = cx.lbuf[n * 16 + c];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int dv = (wave * MT + i) * 16 + 4 * g;
      // the output, or this split's partial output, normalised by its own sum
      __bf16 *dst = splits == 1 ? out + (t * H + head) * 512 : part_o + ((t * splits + sp) * H + head) * 512;
      const float inv = lh > 0.0f ? 1.0f / lh : 0.0f;
      bf16x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (__bf16)(o[i][n][r] * inv);
      *reinterpret_cast<bf16x4 *>(dst + dv) = v;
    }
  }
  return true;
}

// Work item of one workgroup: query token t, head group hg, selection split
// sp.  Resolves the item's physical rows into LDS, loads Q^T of the wave's
// head tile (lane (g, c) holds head hw0 + 16*wave + c, dims 32*s + 8*g .. +8
// for step s) and clears the overshoot flag.
struct MlaItem {
  int64_t t;
  int hg, sp, hw0;
};

template <int NW>
__device__ __forceinline__ MlaItem mla_setup(MlaCtx &cx, bf16x8 (&qr)[18], const __bf16 *__restrict__ q,
                                             uint8_t *smem_raw, int64_t wid, const int32_t *__restrict__ idx,
                                             const int32_t *__restrict__ bt, int max_blocks, int64_t N, int H, int k,
                                             int splits) {
  cx.tiles = smem_raw;
  cx.pbuf = smem_raw + kNBuf * kTileBytes;
  cx.lbuf = reinterpret_cast<float *>(cx.pbuf + 2 * kPBytes);
  int *rows = reinterpret_cast<int *>(cx.lbuf + 128);   // <= 2048 physical rows
  cx.rows = rows;
  cx.flag = rows + 2048;
  const int n_hg = H / (16 * NW);
  MlaItem it;
  it.sp = (int)(wid % splits);
  const int64_t rest = wid / splits;
  it.hg = (int)(rest % n_hg);
  it.t = rest / n_hg;
  const int tid = threadIdx.x;
  cx.wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: per-wave values stay in SGPRs
  cx.lane = tid & 63;
  cx.g = cx.lane >> 4;
  cx.c = cx.lane & 15;
  it.hw0 = it.hg * NW * 16;  // first head of the workgroup
  const int ntiles = (k + kBN - 1) / kBN;
  const int per = (ntiles + splits - 1) / splits;
  cx.tb = it.sp * per;
  cx.te = min(ntiles, cx.tb + per);
  // Q^T first: its loads are in flight while the rows are resolved
  const __bf16 *qrow = q + (it.t * H + it.hw0 + 16 * cx.wave + cx.c) * 576 + cx.g * 8;
#pragma unroll
  for (int s = 0; s < 18; ++s) qr[s] = *reinterpret_cast<const bf16x8 *>(qrow + s * 32);
  const int32_t *irow = idx + it.t * k;
  // physical rows of this workgroup's entries [tb*32, te*32)
  for (int e = tid; e < (cx.te - cx.tb) * kBN; e += NW * 64)
    rows[e] = (int)phys_row(irow, bt, max_blocks, N, it.t, cx.tb * kBN + e, k);
  if (tid == 0) *cx.flag = 0;
  __syncthreads();
  return it;
}

// Recomputes work item `wid` with exact per-head maxima: one logits-only
// pass for the maxima, then the accumulation pass with those references.
// Out of line: it only runs when the first pass was discarded (rare), and
// keeps its registers out of the main pass.
template <int NW, bool late>
__device__ __noinline__ void mla_redo_item(const __bf16 *__restrict__ q, const __bf16 *__restrict__ kv,
                                           const int32_t *__restrict__ idx, const int32_t *__restrict__ bt,
                                           int max_blocks, int64_t N, int H, int k, float scale_log2,
                                           __bf16 *__restrict__ out, float *__restrict__ lse, int splits,
                                           __bf16 *__restrict__ part_o, float *__restrict__ part_ml, int64_t wid) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  MlaCtx cx;
  cx.kv = kv;
  bf16x8 qr[18];
  const MlaItem it = mla_setup<NW>(cx, qr, q, smem_raw, wid, idx, bt, max_blocks, N, H, k, splits);
  float m_ref = -INFINITY;
  for_each_tile<NW>(cx, [&](const uint8_t *ct, const int *rv) {
    float x[8];
    tile_logits(ct, rv, qr, scale_log2, cx.g, cx.c, x);
    m_ref = fmaxf(m_ref, tile_max(x, scale_log2));
  });
  mla_pass<NW, true, late>(cx, qr, m_ref, scale_log2, it.t, H, it.hw0, out, lse, splits, it.sp, part_o, part_ml);
}

// NW waves: 16*NW heads per workgroup; for the logits wave w owns 16 heads,
// for PV it owns 512/NW value dims of all 16*NW heads.
//
// Softmax reference: each head's exponent reference m_ref (base 2, scale
// folded in) is the max of the first tile in which the head has a valid
// entry, and then stays fixed, so the accumulators are only ever written by
// MFMAs.  Probabilities are exp2(x - m_ref); while x <= m_ref + 64 they stay
// below 2^64, far inside the fp32/bf16 range, and the result is the same
// softmax.  If any tile overshoots that, the pass is discarded and the
// workgroup recomputes the item with exact maxima (mla_redo_item).
template <int NW, bool late>
__global__ __launch_bounds__(NW * 64, 1) void sparse_mla_bf16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ kv, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ bt, int max_blocks, int64_t N, int T, int H, int k, float scale_log2,
    __bf16 *__restrict__ out, float *__restrict__ lse, int splits, __bf16 *__restrict__ part_o,
    float *__restrict__ part_ml) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  MlaCtx cx;
  cx.kv = kv;
  bf16x8 qr[18];
  const MlaItem it = mla_setup<NW>(cx, qr, q, smem_raw, blockIdx.x, idx, bt, max_blocks, N, H, k, splits);
  float m_ref = -INFINITY;
  if (mla_pass<NW, false, late>(cx, qr, m_ref, scale_log2, it.t, H, it.hw0, out, lse, splits, it.sp, part_o,
                                part_ml))
    return;
  mla_redo_item<NW, late>(q, kv, idx, bt, max_blocks, N, H, k, scale_log2, out, lse, splits, part_o, part_ml, blockIdx.x);
}

// LSE-weighted combine of split partials.  grid (T*H/4), block 256: 4 heads,
// 64 threads per head, 8 value dims per thread.  Split s left its output
// normalised by its own sum l_s, with reference m_s:
//     out = sum_s w_s l_s P_s / sum_s w_s l_s,   w_s = 2^(m_s - max m).
// Lane s < splits reads the (m_s, l_s) pair; the partials of up to eight
// splits are requested together before any is used.
constexpr int kCombineBatch = 8;
__global__ __launch_bounds__(256) void mla_combine_kernel(const __bf16 *__restrict__ part_o,
                                                          const float *__restrict__ part_ml, int T, int H,
                                                          int splits, __bf16 *__restrict__ out,
                                                          float *__restrict__ lse) {
  const int64_t th = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (th >= (int64_t)T * H) return;  // uniform per wave
  const int lane = threadIdx.x & 63;
  const int64_t t = th / H;
  const int h = (int)(th % H);
  float ms = -INFINITY, ls = 0.0f;
  if (lane < splits) {
    const float *pm = part_ml + ((t * splits + lane) * H + h) * 2;
    ms = pm[0];
    ls = pm[1];
  }
  const float M = wave_max(ms);
  // weight of split `lane` times its sum (0 for empty splits)
  const float wl = ms == -INFINITY ? 0.0f : exp2f(ms - M) * ls;
  const float Lsum = wave_sum(wl);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += kCombineBatch) {
    bf16x8 pv[kCombineBatch];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u)
      if (s0 + u < splits)
        pv[u] = *reinterpret_cast<const bf16x8 *>(part_o + ((t * splits + s0 + u) * H + h) * 512 + lane * 8);
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      if (s0 + u < splits) {
        const float wgt = __shfl(wl, s0 + u);
        if (wgt != 0.0f) {  // empty splits hold no partial
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(wgt, (float)pv[u][i], acc[i]);
        }
      }
    }
  }
  const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (__bf16)(acc[i] * inv);
  *reinterpret_cast<bf16x8 *>(out + th * 512 + lane * 8) = v;
  if (lse && lane == 0) lse[th] = Lsum > 0.0f ? (M + log2f(Lsum)) * 0.69314718055994531f : -INFINITY;
}

// fp32 path (small problems): one workgroup of 256 threads per query token,
// heads in turn; logits one entry per thread, output one value dim per thread.
constexpr int kF32MaxK = 2048;
__global__ __launch_bounds__(256) void sparse_mla_f32_kernel(const float *__restrict__ q,
                                                             const float *__restrict__ kv,
                                                             const int32_t *__restrict__ idx, int64_t N, int T, int H,
                                                             int k, float sm_scale, float *__restrict__ out,
                                                             float *__restrict__ lse) {
  __shared__ float qs[576];
  __shared__ float z[kF32MaxK];
  __shared__ int sel[kF32MaxK];
  __shared__ float red[8];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < k; e += 256) {
    const int32_t v = idx[t * k + e];
    sel[e] = (v >= 0 && v < N) ? v : -1;
  }
  __syncthreads();
  for (int h = 0; h < H; ++h) {
    for (int d = tid; d < 576; d += 256) qs[d] = q[(t * H + h) * 576 + d];
    __syncthreads();
    float mx = -INFINITY;
    for (int e = tid; e < k; e += 256) {
      float v = -INFINITY;
      if (sel[e] >= 0) {
        const float *row = kv + (int64_t)sel[e] * 576;
        float dot = 0.0f;
        for (int d = 0; d < 576; ++d) dot = fmaf(qs[d], row[d], dot);
        v = dot * sm_scale;
      }
      z[e] = v;
      mx = fmaxf(mx, v);
    }
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    const float msub = mx == -INFINITY ? 0.0f : mx;
    float sum = 0.0f;
    for (int e = tid; e < k; e += 256) {
      const float p = expf(z[e] - msub);
      z[e] = p;
      sum += p;
    }
    sum = wave_sum(sum);
    if (lane == 0) red[4 + wave] = sum;
    __syncthreads();
    sum = (red[4] + red[5]) + (red[6] + red[7]);
    const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;
    for (int d = tid; d < 512; d += 256) {
      float acc = 0.0f;
      for (int e = 0; e < k; ++e)
        if (sel[e] >= 0) acc = fmaf(z[e], kv[(int64_t)sel[e] * 576 + d], acc);
      out[(t * H + h) * 512 + d] = acc * inv;
    }
    if (lse && tid == 0) lse[t * H + h] = sum > 0.0f ? msub + logf(sum) : -INFINITY;
    __syncthreads();
  }
}

template <int NW, bool late>
hipError_t launch_bf16_variant(const void *q, const void *kv, const int32_t *idx, const int32_t *bt,
                               int max_blocks, int64_t N, int T, int H, int k, float scale_log2, void *out, float *lse,
                               int splits, __bf16 *part_o, float *part_ml, hipStream_t s) {
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void *)sparse_mla_bf16_kernel<NW, late>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kSmemMla);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int64_t items = (int64_t)T * (H / (16 * NW)) * splits;
  hipLaunchKernelGGL((sparse_mla_bf16_kernel<NW, late>), dim3((uint32_t)items), dim3(NW * 64), kSmemMla, s,
                     (const __bf16 *)q, (const __bf16 *)kv, idx, bt, max_blocks, N, T, H, k, scale_log2,
                     (__bf16 *)out, lse, splits, part_o, part_ml);
  return hipGetLastError();
}

// Order of a tile's gather within an iteration.  Issued before the logits
// (early), it has a whole iteration to land, but while it is in flight the
// compiler cannot count the logits' LDS reads (the direct-to-LDS load is a
// flat instruction) and waits for all of them at every step.  Issued after
// the logits (late), those reads overlap the MFMAs and the gather has about
// half an iteration.  Measured: late is 3-4% faster over a long prefill
// selection (whose rows come largely from L2/MALL); early is faster for split
// decode items, whose rows come from HBM.
template <int NW>
hipError_t launch_bf16_nw(const void *q, const void *kv, const int32_t *idx, const int32_t *bt,
                          int max_blocks, int64_t N, int T, int H, int k, float scale_log2, void *out, float *lse,
                          int splits, __bf16 *part_o, float *part_ml, hipStream_t s) {
  if (splits == 1)
    return launch_bf16_variant<NW, true>(q, kv, idx, bt, max_blocks, N, T, H, k, scale_log2, out, lse, splits, part_o,
                                         part_ml, s);
  return launch_bf16_variant<NW, false>(q, kv, idx, bt, max_blocks, N, T, H, k, scale_log2, out, lse, splits, part_o,
                                        part_ml, s);
}

// ------------------------------------------------------------------ backward
//
// In sparse training the main model is trained by the language-modelling
// loss through the attention over the selected entries (mizuki-eaf.pages.dev,
// two-stage continued pre-training / sparse training; m.36881.com.cn, sparse
// training).  For query t, head h, entry a (latent row c_a, value v_a =
// c_a[0..512)), with P from the forward's own log-sum-exp and the upstream
// gradient dO:
//   dP_a = dO . v_a,   D = dO . o,   dS_a = P_a (dP_a - D)
//   dq   = s sum_a dS_a c_a
//   dkv[r_a] += s dS_a q + P_a dO        (value dims get the second term)
// Three kernels per chunk of queries, then the inverted-selection reduce:
//  * mla_bwd_delta_kernel: D[t,h] = dO . o (o: the forward's output);
//  * mla_bwd_ds_kernel: per (query, 16*NW heads), the forward's gather and
//    logits, dP with dO^T resident, then dq^T += C^T dS^T (the transposing
//    LDS read of the forward's PV, over all 576 dims, with the wave's own dS
//    as the B operand); s dS and P go to the workspace key-major [pair][head]
//    in bf16;
//  * mla_bwd_g_kernel: per query, the pair gradients G[pair, :] =
//    (s dS)^T q + P^T dO, a GEMM over the heads (K = heads, bf16 MFMA, fp32
//    sums) with q and dO resident per wave for its 48 dims;
//  * dkv[r] = sum of G over r's pairs in increasing pair order (scatter.hip).

// D[t, h] = sum_d dO[t,h,d] o[t,h,d]: one wave per (t, h), 8 dims per lane.
__global__ __launch_bounds__(256) void mla_bwd_delta_kernel(const __bf16 *__restrict__ out,
                                                            const __bf16 *__restrict__ dout, int64_t TH,
                                                            float *__restrict__ D) {
  const int64_t th = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (th >= TH) return;  // uniform per wave
  const int lane = threadIdx.x & 63;
  const bf16x8 o = *reinterpret_cast<const bf16x8 *>(out + th * 512 + lane * 8);
  const bf16x8 g = *reinterpret_cast<const bf16x8 *>(dout + th * 512 + lane * 8);
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc = fmaf((float)o[i], (float)g[i], acc);
  acc = wave_sum(acc);
  if (lane == 0) D[th] = acc;
}

// S^T-layout dot products of a gathered tile with NS resident 32-dim B
// operands (dims 0 .. 32 NS): lane (g, c) gets x[r] = key 4g+r and x[4+r] =
// key 16+4g+r of head c (no masking).
template <int NS>
__device__ __forceinline__ void tile_dot(const uint8_t *__restrict__ ct, const bf16x8 (&b)[NS], int g, int c,
                                         float (&x)[8]) {
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
  const uint8_t *arow0 = ct + c * kCRow + g * 16;
  const uint8_t *arow1 = arow0 + 16 * kCRow;
  bf16x8 op[2][2];
  op[0][0] = *reinterpret_cast<const bf16x8 *>(arow0);
  op[0][1] = *reinterpret_cast<const bf16x8 *>(arow1);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int cs = s & 1;
    if (s + 1 < NS) {
      op[cs ^ 1][0] = *reinterpret_cast<const bf16x8 *>(arow0 + (s + 1) * 64);
      op[cs ^ 1][1] = *reinterpret_cast<const bf16x8 *>(arow1 + (s + 1) * 64);
    }
    s0 = mfma_bf16_16x16x32(op[cs][0], b[s], s0);
    s1 = mfma_bf16_16x16x32(op[cs][1], b[s], s1);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    x[r] = s0[r];
    x[4 + r] = s1[r];
  }
}

constexpr int kBwdNBuf = 2;
// LDS of the dS kernel: two gathered tiles and the resolved rows of the query's entries
constexpr int kSmemBwd = kBwdNBuf * kTileBytes + 2048 * 4;

// One workgroup of NW waves per (query t0 + blockIdx.x, head group blockIdx.y
// of 16 NW heads); wave w owns heads 16 w .. +16 of the group.
template <int NW>
__global__ __launch_bounds__(NW * 64, 1) void mla_bwd_ds_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ kv, const int32_t *__restrict__ idx,
    const float *__restrict__ lse, const __bf16 *__restrict__ dout, const float *__restrict__ Dd, int64_t N, int H,
    int k, float sm_scale, int64_t t0, float *__restrict__ dq, __bf16 *__restrict__ dsT, __bf16 *__restrict__ pT) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  uint8_t *tiles = smem_raw;
  int *rows = reinterpret_cast<int *>(smem_raw + kBwdNBuf * kTileBytes);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tc = blockIdx.x, t = t0 + tc;
  const int head = blockIdx.y * 16 * NW + 16 * wave + c;  // this lane's head
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  const int ntiles = (k + kBN - 1) / kBN;
  // Q^T and dO^T of the wave's heads (B operands: lane (g, c) holds head c, dims 32 s + 8 g .. +8)
  bf16x8 qr[18], gr[16];
  const __bf16 *qrow = q + (t * H + head) * 576 + g * 8;
  const __bf16 *grow = dout + (t * H + head) * 512 + g * 8;
#pragma unroll
  for (int s = 0; s < 18; ++s) qr[s] = *reinterpret_cast<const bf16x8 *>(qrow + s * 32);
#pragma unroll
  for (int s = 0; s < 16; ++s) gr[s] = *reinterpret_cast<const bf16x8 *>(grow + s * 32);
  const float lse2 = lse[t * H + head] * 1.4426950408889634f;  // base-2 log-sum-exp of head c
  const float Dh = Dd[t * H + head];
  const int32_t *irow = idx + t * k;
  for (int e = tid; e < ntiles * kBN; e += NW * 64) rows[e] = (int)phys_row(irow, nullptr, 0, N, t, e, k);
  // dq^T accumulators: dims 16 i + 4 g + r of head c
  f32x4 acc[36];
#pragma unroll
  for (int i = 0; i < 36; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int tr_base = (4 * g + (c >> 2)) * kCRow + (c & 3) * 8;
  __syncthreads();
  if (ntiles > 0) gather_tile_async<NW>(tiles, rows, 0, kv, wave, lane);
  for (int j = 0; j < ntiles; ++j) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's gathers of tile j have landed
    __syncthreads();                // ... and every wave's; tile j-1 is free
    if (j + 1 < ntiles) gather_tile_async<NW>(tiles + ((j + 1) & 1) * kTileBytes, rows, (j + 1) * kBN, kv, wave, lane);
    const uint8_t *ct = tiles + (j & 1) * kTileBytes;
    const int *rv = rows + j * kBN;
    float x[8], dp[8];
    tile_dot<18>(ct, qr, g, c, x);
    tile_dot<16>(ct, gr, g, c, dp);
    bf16x8 dsb;
    float pv[8], dsv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = i < 4 ? 4 * g + i : 16 + 4 * g + (i - 4);
      const float p = rv[key] >= 0 ? __builtin_amdgcn_exp2f(fmaf(x[i], scale_log2, -lse2)) : 0.0f;
      pv[i] = p;
      dsv[i] = p * (dp[i] - Dh);
      dsb[i] = (__bf16)dsv[i];
    }
    // dq^T[dims, head] += C^T[dims, keys] dS^T[keys, head]
#pragma unroll
    for (int i = 0; i < 36; ++i) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(ct + tr_base + i * 32));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(ct + tr_base + i * 32 + 16 * kCRow));
      const i16x4 lohi[2] = {lo, hi};
      acc[i] = mfma_bf16_16x16x32(*reinterpret_cast<const bf16x8 *>(lohi), dsb, acc[i]);
    }
    // s dS and P of the tile's entries, key-major
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = j * kBN + (i < 4 ? 4 * g + i : 16 + 4 * g + (i - 4));
      if (key < k) {
        const int64_t o = (tc * k + key) * H + head;
        dsT[o] = (__bf16)(sm_scale * dsv[i]);
        pT[o] = (__bf16)pv[i];
      }
    }
  }
  float *dqrow = dq + (t * H + head) * 576 + 4 * g;
#pragma unroll
  for (int i = 0; i < 36; ++i)
    *reinterpret_cast<f32x4 *>(dqrow + 16 * i) =
        f32x4{sm_scale * acc[i][0], sm_scale * acc[i][1], sm_scale * acc[i][2], sm_scale * acc[i][3]};
}

// Pair gradients of one query: G[pair, d] = sum_h (s dS)[pair, h] q[h, d] +
// P[pair, h] dO[h, d] (the dO term for d < 512).  Workgroup (query,
// blockIdx.y) of four waves covers dim tiles 12 y .. 12 y + 11 (16 dims
// each); wave w owns three of them and holds their B operands (q and dO with
// the heads along K) for the whole key loop.  KS = H / 32 K steps.
constexpr int kGTilesPerWave = 3;
constexpr int kGTilesPerGroup = 4 * kGTilesPerWave;  // 36 tiles of 16 dims: 3 groups
template <int KS>
__global__ __launch_bounds__(256) void mla_bwd_g_kernel(const __bf16 *__restrict__ q, const __bf16 *__restrict__ dout,
                                                        const __bf16 *__restrict__ dsT, const __bf16 *__restrict__ pT,
                                                        int k, int64_t t0, float *__restrict__ G) {
  constexpr int H = 32 * KS;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tc = blockIdx.x, t = t0 + tc;
  const int ti0 = blockIdx.y * kGTilesPerGroup + kGTilesPerWave * wave;  // uniform
  // B operands: lane (g, c) holds heads 32 s + 8 g .. +8 of dim 16 (ti0 + j) + c
  bf16x8 bq[kGTilesPerWave][KS], bo[kGTilesPerWave][KS];
#pragma unroll
  for (int jt = 0; jt < kGTilesPerWave; ++jt) {
    const int d = 16 * (ti0 + jt) + c;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t h = 32 * s + 8 * g + e;
        bq[jt][s][e] = q[(t * H + h) * 576 + d];
        bo[jt][s][e] = d < 512 ? dout[(t * H + h) * 512 + d] : (__bf16)0.0f;
      }
    }
  }
  const __bf16 *dsq = dsT + tc * k * H;
  const __bf16 *pq = pT + tc * k * H;
  float *Gq = G + tc * k * 576;
  for (int kb = 0; kb < k; kb += 16) {
    // A operands: lane (g, c) holds key kb + c, heads 32 s + 8 g .. +8
    const int key = kb + c;
    bf16x8 ads[KS], ap[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (key < k) {
        ads[s] = *reinterpret_cast<const bf16x8 *>(dsq + (int64_t)key * H + 32 * s + 8 * g);
        ap[s] = *reinterpret_cast<const bf16x8 *>(pq + (int64_t)key * H + 32 * s + 8 * g);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) ads[s][e] = ap[s][e] = (__bf16)0.0f;
      }
    }
#pragma unroll
    for (int jt = 0; jt < kGTilesPerWave; ++jt) {
      const int ti = ti0 + jt;
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) o = mfma_bf16_16x16x32(ads[s], bq[jt][s], o);
      if (ti < 32) {  // value dims: uniform per wave and tile
#pragma unroll
        for (int s = 0; s < KS; ++s) o = mfma_bf16_16x16x32(ap[s], bo[jt][s], o);
      }
      // rows 4 g + r (keys), column c (dim)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kr = kb + 4 * g + r;
        if (kr < k) Gq[(int64_t)kr * 576 + 16 * ti + c] = o[r];
      }
    }
  }
}

}  // namespace

namespace dsa {
hipError_t launch_sparse_mla_bf16(const void *q, const void *kv, const int32_t *idx,
                                  const int32_t *block_table, int32_t max_blocks, int64_t N, int32_t T,
                                  int32_t H, int32_t k, float sm_scale, void *out, float *lse,
                                  int32_t splits, void *part_o_v, float *part_ml, hipStream_t s) {
  if (T == 0) return hipSuccess;
  __bf16 *part_o = (__bf16 *)part_o_v;
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  hipError_t e;
  if (H % 128 == 0)
    e = launch_bf16_nw<8>(q, kv, idx, block_table, max_blocks, N, T, H, k, scale_log2, out, lse, splits,
                          part_o, part_ml, s);
  else if (H % 64 == 0)
    e = launch_bf16_nw<4>(q, kv, idx, block_table, max_blocks, N, T, H, k, scale_log2, out, lse, splits,
                          part_o, part_ml, s);
  else if (H % 32 == 0)
    e = launch_bf16_nw<2>(q, kv, idx, block_table, max_blocks, N, T, H, k, scale_log2, out, lse, splits,
                          part_o, part_ml, s);
  else
    e = launch_bf16_nw<1>(q, kv, idx, block_table, max_blocks, N, T, H, k, scale_log2, out, lse, splits,
                          part_o, part_ml, s);
  if (e != hipSuccess || splits == 1) return e;
  const int64_t th = (int64_t)T * H;
  hipLaunchKernelGGL(mla_combine_kernel, dim3((uint32_t)((th + 3) / 4)), dim3(256), 0, s, part_o, part_ml, T,
                     H, splits, (__bf16 *)out, lse);
  return hipGetLastError();
}

hipError_t launch_mla_bwd_delta(const void *out, const void *dout, int64_t TH, float *D, hipStream_t s) {
  if (TH == 0) return hipSuccess;
  hipLaunchKernelGGL(mla_bwd_delta_kernel, dim3((uint32_t)((TH + 3) / 4)), dim3(256), 0, s, (const __bf16 *)out,
                     (const __bf16 *)dout, TH, D);
  return hipGetLastError();
}

template <int NW>
static hipError_t launch_ds_nw(const void *q, const void *kv, const int32_t *idx, const float *lse, const void *dout,
                               const float *D, int64_t N, int32_t H, int32_t k, float sm_scale, int64_t t0, int32_t Tc,
                               float *dq, void *dsT, void *pT, hipStream_t s) {
  static bool attr_done = false;  // per process: the attribute holds for every device
  if (!attr_done) {
    hipError_t e =
        hipFuncSetAttribute((const void *)mla_bwd_ds_kernel<NW>, hipFuncAttributeMaxDynamicSharedMemorySize, kSmemBwd);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  hipLaunchKernelGGL(mla_bwd_ds_kernel<NW>, dim3((uint32_t)Tc, H / (16 * NW)), dim3(NW * 64), kSmemBwd, s,
                     (const __bf16 *)q, (const __bf16 *)kv, idx, lse, (const __bf16 *)dout, D, N, H, k, sm_scale, t0,
                     dq, (__bf16 *)dsT, (__bf16 *)pT);
  return hipGetLastError();
}

// Queries [t0, t0 + Tc): dq of those queries; s dS and P [Tc, k, H] bf16; then
// the pair gradients G [Tc, k, 576] fp32.  H a multiple of 32, at most 128.
hipError_t launch_mla_bwd_chunk(const void *q, const void *kv, const int32_t *idx, const float *lse, const void *dout,
                                const float *D, int64_t N, int32_t H, int32_t k, float sm_scale, int64_t t0,
                                int32_t Tc, float *dq, void *dsT, void *pT, float *G, hipStream_t s) {
  if (Tc <= 0) return hipSuccess;
  hipError_t e = H % 64 == 0 ? launch_ds_nw<4>(q, kv, idx, lse, dout, D, N, H, k, sm_scale, t0, Tc, dq, dsT, pT, s)
                             : launch_ds_nw<2>(q, kv, idx, lse, dout, D, N, H, k, sm_scale, t0, Tc, dq, dsT, pT, s);
  if (e != hipSuccess) return e;
  switch (H / 32) {
    case 1:
      hipLaunchKernelGGL(mla_bwd_g_kernel<1>, dim3((uint32_t)Tc, 36 / kGTilesPerGroup), dim3(256), 0, s, (const __bf16 *)q,
                         (const __bf16 *)dout, (const __bf16 *)dsT, (const __bf16 *)pT, k, t0, G);
      break;
    case 2:
      hipLaunchKernelGGL(mla_bwd_g_kernel<2>, dim3((uint32_t)Tc, 36 / kGTilesPerGroup), dim3(256), 0, s, (const __bf16 *)q,
                         (const __bf16 *)dout, (const __bf16 *)dsT, (const __bf16 *)pT, k, t0, G);
      break;
    case 3:
      hipLaunchKernelGGL(mla_bwd_g_kernel<3>, dim3((uint32_t)Tc, 36 / kGTilesPerGroup), dim3(256), 0, s, (const __bf16 *)q,
                         (const __bf16 *)dout, (const __bf16 *)dsT, (const __bf16 *)pT, k, t0, G);
      break;
    case 4:
      hipLaunchKernelGGL(mla_bwd_g_kernel<4>, dim3((uint32_t)Tc, 36 / kGTilesPerGroup), dim3(256), 0, s, (const __bf16 *)q,
                         (const __bf16 *)dout, (const __bf16 *)dsT, (const __bf16 *)pT, k, t0, G);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_sparse_mla_f32(const float *q, const float *kv, const int32_t *idx, int64_t N, int32_t T,
                                 int32_t H, int32_t k, float sm_scale, float *out, float *lse,
                                 hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(sparse_mla_f32_kernel, dim3(T), dim3(256), 0, s, q, kv, idx, N, T, H, k, sm_scale,
                     out, lse);
  return hipGetLastError();
}
}  // namespace dsa
