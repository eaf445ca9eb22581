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
//    into three buffers; each row is fetched once for all heads; the buffers
//    are separate static arrays and the loop is unrolled by three, so the
//    compiler can tell a gather from the LDS reads of the other buffers;
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
#include <type_traits>

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

// LDS of the forward kernel, as separate static arrays: the three gathered
// tiles are distinct objects, so the compiler can tell an LDS read of one tile
// from the direct-to-LDS gather into another and waits for neither.
__shared__ __align__(16) uint8_t g_mla_t0[kTileBytes];
__shared__ __align__(16) uint8_t g_mla_t1[kTileBytes];
__shared__ __align__(16) uint8_t g_mla_t2[kTileBytes];
__shared__ __align__(16) uint8_t g_mla_p[2 * kPBytes];
__shared__ __align__(16) float g_mla_l[128];
__shared__ __align__(16) int g_mla_rows[2048];
__shared__ int g_mla_flag;
template <int B>
__device__ __forceinline__ uint8_t *mla_tile() {
  return B == 0 ? g_mla_t0 : (B == 1 ? g_mla_t1 : g_mla_t2);
}

// The gather of the forward kernel: the same LDS image as gather_tile_async,
// through buffer loads indexed by row (a 1152-byte record per latent row, so
// any row below 2^32 is reachable).  Unlike the flat form, the compiler counts
// these loads in the vector-memory counter only and keeps exact counts of the
// LDS reads issued after them.
template <int NW>
__device__ __forceinline__ void gather_tile_rec(uint8_t *__restrict__ dst, const int *__restrict__ rows, int r0,
                                                const __bf16 *__restrict__ kv, int64_t N, int wave, int lane) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)kv, (short)(576 * 2), (int)(N < 0xFFFFFFFFll ? N : 0xFFFFFFFFll), (int)0x00020000u);
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
    __builtin_amdgcn_struct_ptr_buffer_load_lds(rs, (lds_void *)(dst + i * 1024), 16, pr >= 0 ? pr : 0, j * 16, 0, 0,
                                                0);
  }
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

// The forward kernel's gather: record-indexed buffer loads when every byte
// of kv lies within 4 GiB of its start (32-bit buffer offsets), else the flat
// form, into the same LDS image.
template <int NW, bool rec>
__device__ __forceinline__ void gather_tile_fwd(uint8_t *__restrict__ dst, const int *__restrict__ rows, int r0,
                                                const __bf16 *__restrict__ kv, int64_t N, int wave, int lane) {
  if constexpr (rec)
    gather_tile_rec<NW>(dst, rows, r0, kv, N, wave, lane);
  else
    gather_tile_async<NW>(dst, rows, r0, kv, wave, lane);
}

// Shared state of one sparse-MLA workgroup.
struct MlaCtx {
  const __bf16 *kv;
  uint8_t *pbuf;        // P^T exchange, two buffers of [head tile][lane] x 16 bytes
  float *lbuf;          // softmax sums of the workgroup's heads
  const int *rows;      // physical rows of the workgroup's entries (LDS)
  int *flag;            // LDS: set when a tile overshoots the softmax reference
  int64_t N;            // latent rows
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
template <int NW, bool rec, typename Body>
__device__ __forceinline__ void for_each_tile(const MlaCtx &cx, Body &&body) {
  if (cx.tb < cx.te) gather_tile_fwd<NW, rec>(g_mla_t0, cx.rows, 0, cx.kv, cx.N, cx.wave, cx.lane);
  int cur = 0;
  for (int tile = cx.tb; tile < cx.te; ++tile, cur ^= 1) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of `tile` have landed in LDS
    __syncthreads();                // ... and every wave's; the other buffer is no longer read
    if (tile + 1 < cx.te)
      gather_tile_fwd<NW, rec>(cur ? g_mla_t0 : g_mla_t1, cx.rows, (tile + 1 - cx.tb) * kBN, cx.kv, cx.N, cx.wave,
                               cx.lane);
    body(cur ? g_mla_t1 : g_mla_t0, cx.rows + (tile - cx.tb) * kBN);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

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
template <int NW, bool fixed, bool late, bool rec>
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
  auto gather = [&](uint8_t *dst, int j) {
    gather_tile_fwd<NW, rec>(dst, cx.rows, j * kBN, cx.kv, cx.N, cx.wave, cx.lane);
  };
  // logits and probabilities of tile j (in ct), published in P buffer j&1
  auto score_tile = [&](const uint8_t *ct, int j) {
    float x[8];
    tile_logits(ct, cx.rows + j * kBN, qr, scale_log2, g, c, x);
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
  // PV of tile j (in ct) with the probabilities in P buffer j&1
  auto pv_tile = [&](const uint8_t *ct, int j) {
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
  // Iteration j with tile j in buffer B = j % 3 (tile j+1 in B+1, j+2 in B+2):
  // the loop is unrolled by three so that every buffer is a fixed object.
  auto step = [&](auto bc, int j) {
    constexpr int B = decltype(bc)::value;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's gathers of tile j+1 have landed
    __syncthreads();  // P(j) from every wave; tile j+1 from every wave; nobody reads tile j-1 any more
    if (!late && j + 2 < n) gather(mla_tile<(B + 2) % 3>(), j + 2);
    if (j + 1 < n) score_tile(mla_tile<(B + 1) % 3>(), j + 1);
    if (late && j + 2 < n) gather(mla_tile<(B + 2) % 3>(), j + 2);
    pv_tile(mla_tile<B>(), j);
  };
  if (n > 0) {
    gather(g_mla_t0, 0);
    if (n > 1) {
      gather(g_mla_t1, 1);
      wait_all_but_newest_tile<NW>(wave);  // tile 0 landed (tile 1 may be in flight)
    } else {
      __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();
    score_tile(g_mla_t0, 0);
    for (int j = 0; j < n; j += 3) {
      step(std::integral_constant<int, 0>(), j);
      if (j + 1 < n) step(std::integral_constant<int, 1>(), j + 1);
      if (j + 2 < n) step(std::integral_constant<int, 2>(), j + 2);
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
  if (g == 0 && head_own < H) {  // heads past H pad the last head tile
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
    if (head >= H) continue;  // padding of the last head tile
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
                                             int64_t wid, const int32_t *__restrict__ idx,
                                             const int32_t *__restrict__ bt, int max_blocks, int64_t N, int H, int k,
                                             int splits) {
  cx.pbuf = g_mla_p;
  cx.lbuf = g_mla_l;
  int *rows = g_mla_rows;  // <= 2048 physical rows
  cx.rows = rows;
  cx.flag = &g_mla_flag;
  cx.N = N;
  const int n_hg = (H + 16 * NW - 1) / (16 * NW);  // the last group is padded when 16 NW does not divide H
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
  // Q^T first: its loads are in flight while the rows are resolved.  Heads
  // past H (padding of the last head tile) get a zero query: finite logits,
  // and their outputs are never written.
  const int qh = it.hw0 + 16 * cx.wave + cx.c;
  const bool qvalid = qh < H;
  const __bf16 *qrow = q + (it.t * H + (qvalid ? qh : 0)) * 576 + cx.g * 8;
#pragma unroll
  for (int s = 0; s < 18; ++s) {
    const bf16x8 v = *reinterpret_cast<const bf16x8 *>(qrow + s * 32);
    qr[s] = qvalid ? v : bf16x8{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  }
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
template <int NW, bool late, bool rec>
__device__ __noinline__ void mla_redo_item(const __bf16 *__restrict__ q, const __bf16 *__restrict__ kv,
                                           const int32_t *__restrict__ idx, const int32_t *__restrict__ bt,
                                           int max_blocks, int64_t N, int H, int k, float scale_log2,
                                           __bf16 *__restrict__ out, float *__restrict__ lse, int splits,
                                           __bf16 *__restrict__ part_o, float *__restrict__ part_ml, int64_t wid) {
  MlaCtx cx;
  cx.kv = kv;
  bf16x8 qr[18];
  const MlaItem it = mla_setup<NW>(cx, qr, q, wid, idx, bt, max_blocks, N, H, k, splits);
  float m_ref = -INFINITY;
  for_each_tile<NW, rec>(cx, [&](const uint8_t *ct, const int *rv) {
    float x[8];
    tile_logits(ct, rv, qr, scale_log2, cx.g, cx.c, x);
    m_ref = fmaxf(m_ref, tile_max(x, scale_log2));
  });
  mla_pass<NW, true, late, rec>(cx, qr, m_ref, scale_log2, it.t, H, it.hw0, out, lse, splits, it.sp, part_o,
                                part_ml);
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
template <int NW, bool late, bool rec>
__global__ __launch_bounds__(NW * 64, 1) void sparse_mla_bf16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ kv, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ bt, int max_blocks, int64_t N, int T, int H, int k, float scale_log2,
    __bf16 *__restrict__ out, float *__restrict__ lse, int splits, __bf16 *__restrict__ part_o,
    float *__restrict__ part_ml) {
  MlaCtx cx;
  cx.kv = kv;
  bf16x8 qr[18];
  const MlaItem it = mla_setup<NW>(cx, qr, q, blockIdx.x, idx, bt, max_blocks, N, H, k, splits);
  float m_ref = -INFINITY;
  if (mla_pass<NW, false, late, rec>(cx, qr, m_ref, scale_log2, it.t, H, it.hw0, out, lse, splits, it.sp, part_o,
                                     part_ml))
    return;
  mla_redo_item<NW, late, rec>(q, kv, idx, bt, max_blocks, N, H, k, scale_log2, out, lse, splits, part_o, part_ml,
                               blockIdx.x);
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
  // LDS: the static arrays of the kernel (g_mla_*), no dynamic part
  const int64_t items = (int64_t)T * ((H + 16 * NW - 1) / (16 * NW)) * splits;
  if (N * (576 * 2) <= (int64_t(1) << 32))  // every row within 4 GiB: record-indexed gathers
    hipLaunchKernelGGL((sparse_mla_bf16_kernel<NW, late, true>), dim3((uint32_t)items), dim3(NW * 64), 0, s,
                       (const __bf16 *)q, (const __bf16 *)kv, idx, bt, max_blocks, N, T, H, k, scale_log2,
                       (__bf16 *)out, lse, splits, part_o, part_ml);
  else
    hipLaunchKernelGGL((sparse_mla_bf16_kernel<NW, late, false>), dim3((uint32_t)items), dim3(NW * 64), 0, s,
                       (const __bf16 *)q, (const __bf16 *)kv, idx, bt, max_blocks, N, T, H, k, scale_log2,
                       (__bf16 *)out, lse, splits, part_o, part_ml);
  return hipGetLastError();
}

// Order of a tile's gather within an iteration.  Issued before the logits
// (early), it has a whole iteration to land; issued after them (late), about
// half an iteration.  With record-indexed gathers the compiler counts the
// logits' LDS reads exactly either way (with the flat form it waits for all
// of them at every step while a gather is in flight).  Measured at L = 131072:
// late 69.4-70.0 ms against early 70.8-71.4; early is faster for split decode
// items, whose rows come from HBM.
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
//  * mla_bwd_ds_kernel: per (query, 16*HT heads), the forward's gather and
//    logits, and dP with dO^T resident (one LDS read of each tile fragment
//    feeds both), each wave on one head tile and half of each tile's keys;
//    s dS and P are staged in LDS, and dq^T += C^T (s dS)^T (the transposing
//    LDS read of the forward's PV) is split over the waves by latent dims;
//    s dS and P go to the workspace key-major [pair][head] in bf16;
//  * mla_bwd_g_kernel: per query, the pair gradients G[pair, :] =
//    (s dS)^T q + P^T dO, a GEMM over the heads (K = heads, bf16 MFMA, fp32
//    sums, stored rounded to bf16) with q^T and dO^T resident in registers and
//    s dS, P streamed;
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

// S^T-layout dot products of one 16-key half (keys 16 kb .. +16) of a
// gathered tile with the resident Q^T (all 576 dims) and dO^T (the 512 value
// dims) of a head tile: lane (g, c) gets x[r] / dp[r] = key 16 kb + 4 g + r of
// head c (no masking).  Each tile fragment is read from LDS once for both
// products; the operands of the next step are in flight.
__device__ __forceinline__ void half_tile_dot_pair(const uint8_t *__restrict__ ct, const bf16x8 (&bq)[18],
                                                   const bf16x8 (&bo)[16], int kb, int g, int c, f32x4 &x,
                                                   f32x4 &dp) {
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, d0 = {0.f, 0.f, 0.f, 0.f};
  const uint8_t *arow = ct + (16 * kb + c) * kCRow + g * 16;
  bf16x8 op[3];
  op[0] = *reinterpret_cast<const bf16x8 *>(arow);
  op[1] = *reinterpret_cast<const bf16x8 *>(arow + 64);
#pragma unroll
  for (int s = 0; s < 18; ++s) {
    if (s + 2 < 18) op[(s + 2) % 3] = *reinterpret_cast<const bf16x8 *>(arow + (s + 2) * 64);
    s0 = mfma_bf16_16x16x32(op[s % 3], bq[s], s0);
    if (s < 16) d0 = mfma_bf16_16x16x32(op[s % 3], bo[s], d0);
  }
  x = s0;
  dp = d0;
}

// LDS byte address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Transposing LDS reads issued as one block that also waits for them.  LLVM
// cannot tell these reads from the direct-to-LDS gathers in flight, and would
// otherwise wait for every outstanding gather (the next tiles') before each
// of them; the buffers they read were completed by an explicit wait and a
// barrier.  Reads a[n] at base + OFF[n].
#define DSA_TR_READ2(a, base, o0, o1)                                                             \
  asm volatile(                                                                                   \
      "ds_read_b64_tr_b16 %0, %2 offset:%3\n\t"                                                   \
      "ds_read_b64_tr_b16 %1, %2 offset:%4\n\t"                                                   \
      "s_waitcnt lgkmcnt(0)"                                                                      \
      : "=&v"(a[0]), "=&v"(a[1])                                                                  \
      : "v"(base), "i"(o0), "i"(o1)                                                               \
      : "memory")

#define DSA_TR_READ4(a, base, o0, o1, o2, o3)                                                     \
  asm volatile(                                                                                   \
      "ds_read_b64_tr_b16 %0, %4 offset:%5\n\t"                                                   \
      "ds_read_b64_tr_b16 %1, %4 offset:%6\n\t"                                                   \
      "ds_read_b64_tr_b16 %2, %4 offset:%7\n\t"                                                   \
      "ds_read_b64_tr_b16 %3, %4 offset:%8\n\t"                                                   \
      "s_waitcnt lgkmcnt(0)"                                                                      \
      : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])                                        \
      : "v"(base), "i"(o0), "i"(o1), "i"(o2), "i"(o3)                                             \
      : "memory")

constexpr int kStageRow = 2 * kBN + 8;  // LDS bytes per head row of staged s dS or P (32 keys + pad):
                                        // 18 dwords keeps both the 8-byte writes and the
                                        // transposing reads conflict-free
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format
// LDS of the dS kernel: three gathered tiles, the resolved rows of the query's
// entries, two buffers of staged s dS and P (16 HT heads x 32 keys each), and
// two buffers of per-head-tile sums of P (HT x 32 fp32)
template <int HT>
constexpr int smem_bwd_bytes() {
  return 2048 * 4 + 2 * 2 * 16 * HT * kStageRow + 2 * HT * kBN * 4;
}

// Sum of v over the 16 lanes of each DPP row (every lane gets its row's sum).
// DPP controls: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
__device__ __forceinline__ float row16_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  return v;
}

// One workgroup of 2 HT waves per (query t0 + blockIdx.x, head group
// blockIdx.y of 16 HT heads).  Two roles per wave, pipelined across tiles
// with one barrier per tile:
//  * logits and dP: wave w owns head tile w % HT and keys 16 (w / HT) .. +16
//    of each tile, with that head tile's Q^T and dO^T resident; it forms P and
//    dS and stages s dS and P head-major in LDS (bf16);
//  * dq^T[dims, heads] += C^T[dims, keys] (s dS)^T[keys, heads] over the
//    staged s dS of every head tile: wave w owns the value-dim tiles
//    w + 2 HT m (all HT head tiles) and two (rope-dim tile, head tile) pairs,
//    18 accumulator tiles for every HT, so each dim of the gathered tile is
//    read once per workgroup for dq.
// Iteration j: barrier; gather tile j+2; tile j's staged values leave for the
// key-major workspace rows as 16-byte runs; logits and dP of tile j+1; dq of
// tile j.  The only vector-memory operations a tile waits for are its own
// gathers (loads and stores complete in issue order).
// KL: also the sum over the group's heads of each entry's P, the indexer KL
// loss's target before normalisation: each wave sums its 16 heads across
// the lanes of a DPP row, the head tiles meet in LDS, and wave HT adds them
// in head-tile order and stores psum[tc, head group, entry] (fp32).
template <int HT, bool KL, bool rec>
__global__ __launch_bounds__(HT * 128, 1) void mla_bwd_ds_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ kv, const int32_t *__restrict__ idx,
    const float *__restrict__ lse, const __bf16 *__restrict__ dout, const float *__restrict__ Dd, int64_t N, int H,
    int k, float sm_scale, int64_t t0, float *__restrict__ dq, __bf16 *__restrict__ dsT, __bf16 *__restrict__ pT,
    float *__restrict__ psum) {
  constexpr int NW = 2 * HT;
  constexpr int kHeads = 16 * HT;
  constexpr int kStageBuf = 2 * kHeads * kStageRow;  // s dS rows, then P rows
  constexpr int DT = 32 / NW;                         // value-dim tiles per wave
  static_assert(DT <= 8 && DT * HT == 16, "16 value-dim accumulator tiles per wave");
  extern __shared__ __align__(16) uint8_t smem_raw[];
  int *rows = reinterpret_cast<int *>(smem_raw);  // the gathered tiles are the static g_mla_t*
  uint8_t *stage = smem_raw + 2048 * 4;
  float *hsum = reinterpret_cast<float *>(stage + 2 * kStageBuf);  // [2][HT][32]
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ht = wave % HT, kb = wave / HT;  // uniform
  const int64_t tc = blockIdx.x, t = t0 + tc;
  const int hbase = blockIdx.y * kHeads;
  const int head = hbase + 16 * ht + c;  // this lane's head for the logits
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  const int ntiles = (k + kBN - 1) / kBN;
  // Q^T and dO^T of the wave's head tile (B operands: lane (g, c) holds head c, dims 32 s + 8 g .. +8)
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
  // dq^T accumulators: acc[m HT + n] = value-dim tile wave + NW m, head tile n;
  // acc[16], acc[17] = rope-dim tile 32 + 2 wave / HT, head tiles n0, n0 + 1.
  // Lane (g, c) holds dims 16 i + 4 g .. +4 of head 16 n + c.
  const int n0 = (2 * wave) % HT;                  // uniform
  const int irope = 32 + (2 * wave) / HT;          // uniform
  f32x4 acc[18];
#pragma unroll
  for (int i = 0; i < 18; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Lane roles are recomputed in each phase from a laundered lane id:
  // hoisted out of the tile loop, the per-step LDS addresses they feed would
  // hold a dozen registers for the whole kernel.
  auto laundered = [&]() {
    int l = lane;
    asm volatile("" : "+v"(l));
    return l;
  };
  // The query's s dS and P rows as bounded buffers: stores of entries >= k are dropped.
  const __amdgpu_buffer_rsrc_t rds =
      __builtin_amdgcn_make_buffer_rsrc((void *)(dsT + tc * k * H), 0, k * H * 2, (int)kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rp =
      __builtin_amdgcn_make_buffer_rsrc((void *)(pT + tc * k * H), 0, k * H * 2, (int)kRsrcWord3);
  // Write-out roles (waves 0 .. HT-1): lane group tid / 16 takes key
  // 16 (group & 1) + c and the group's 8 heads 8 (group >> 1) .. +8, read from
  // the head-major staging with the transposing load (lane c of a group gets
  // column c of a 4 x 16 block).
  auto write_out = [&](int jt) {  // tile jt's staged values to the workspace
    const int l = laundered(), lc = l & 15;
    const int grp = 4 * wave + (l >> 4), okey = 16 * (grp & 1) + lc, oh = 8 * (grp >> 1);
    const int tr_stage = (oh + (lc >> 2)) * kStageRow + (16 * (grp & 1) + 4 * (lc & 3)) * 2;
    const int ooff = (okey * H + hbase + oh) * 2;  // bytes, within a tile's rows
    const uint8_t *sb = stage + (jt & 1) * kStageBuf;
    i16x4 r[4];
    DSA_TR_READ4(r, lds_addr(sb + tr_stage), 0, 4 * kStageRow, kHeads * kStageRow, kHeads * kStageRow + 4 * kStageRow);
    const i16x4 dd[2] = {r[0], r[1]}, pp[2] = {r[2], r[3]};
    const int off = jt * kBN * H * 2 + ooff;
    __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const i32x4 *>(dd), rds, off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const i32x4 *>(pp), rp, off, 0, 0);
  };
  // logits, P, dS of tile jt for the wave's (head tile, key half); s dS and P to staging buffer jt & 1
  auto logits_ds = [&](const uint8_t *ct, int jt) {
    const int l = laundered(), lg = l >> 4, lc = l & 15;
    const int *rv = rows + jt * kBN + 16 * kb + 4 * lg;
    f32x4 x, dp;
    half_tile_dot_pair(ct, qr, gr, kb, lg, lc, x, dp);
    bf16x4 sdb, pb;
    float p4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = rv[r] >= 0 ? __builtin_amdgcn_exp2f(fmaf(x[r], scale_log2, -lse2)) : 0.0f;
      sdb[r] = (__bf16)(sm_scale * (p * (dp[r] - Dh)));
      pb[r] = (__bf16)p;
      p4[r] = p;
    }
    // head-major: row 16 ht + c, keys 16 kb + 4 g .. +4
    uint8_t *sb = stage + (jt & 1) * kStageBuf + (16 * ht + lc) * kStageRow + 32 * kb + 8 * lg;
    *reinterpret_cast<bf16x4 *>(sb) = sdb;
    *reinterpret_cast<bf16x4 *>(sb + kHeads * kStageRow) = pb;
    if (KL) {  // the head tile's sum of P for keys 16 kb + 4 g + r
      f32x4 hs;
#pragma unroll
      for (int r = 0; r < 4; ++r) hs[r] = row16_sum(p4[r]);
      if (lc == 0) *reinterpret_cast<f32x4 *>(hsum + ((jt & 1) * HT + ht) * kBN + 16 * kb + 4 * lg) = hs;
    }
  };
  // KL, wave HT: tile jt's head sums over the group, stored through a buffer
  // bounded to the query's k entries
  auto store_hsum = [&](int jt) {
    const __amdgpu_buffer_rsrc_t rps =
        __builtin_amdgcn_make_buffer_rsrc((void *)(psum + (tc * (H / kHeads) + blockIdx.y) * k), 0, k * 4,
                                          (int)kRsrcWord3);
    if (lane < kBN) {
      float v = 0.0f;
#pragma unroll
      for (int n = 0; n < HT; ++n) v += hsum[((jt & 1) * HT + n) * kBN + lane];
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), rps, (jt * kBN + lane) * 4, 0, 0);
    }
  };
  // dq^T += C^T (s dS)^T for tile jt, s dS from staging buffer jt & 1
  auto dq_tile = [&](const uint8_t *ct, int jt) {
    const int l = laundered(), lg = l >> 4, lc = l & 15;
    const int tr_base = (4 * lg + (lc >> 2)) * kCRow + (lc & 3) * 8;
    const uint8_t *sb = stage + (jt & 1) * kStageBuf;
    // B operand of head tile n: lane (g, c) holds head 16 n + c, keys
    // 4 g .. +4 and 16 + 4 g .. +4, the key order of the transposing A reads
    auto b_operand = [&](int n) {
      const uint8_t *row = sb + (16 * n + lc) * kStageRow + 8 * lg;
      const bf16x4 lohi[2] = {*reinterpret_cast<const bf16x4 *>(row), *reinterpret_cast<const bf16x4 *>(row + 32)};
      return *reinterpret_cast<const bf16x8 *>(lohi);
    };
    {  // the rope-dim pairs first, with their own B operands (n0 is uniform, not a constant)
      const bf16x8 rb0 = b_operand(n0), rb1 = b_operand(n0 + 1);
      i16x4 r[2];
      DSA_TR_READ2(r, lds_addr(ct + tr_base + irope * 32), 0, 16 * kCRow);
      const bf16x8 ar = *reinterpret_cast<const bf16x8 *>(r);
      acc[16] = mfma_bf16_16x16x32(ar, rb0, acc[16]);
      acc[17] = mfma_bf16_16x16x32(ar, rb1, acc[17]);
    }
    bf16x8 bs[HT];
#pragma unroll
    for (int n = 0; n < HT; ++n) bs[n] = b_operand(n);
    const uint32_t trw = lds_addr(ct + tr_base + wave * 32);  // value-dim tile `wave`
#pragma unroll
    for (int m = 0; m < DT; ++m) {
      // A operand of value-dim tile wave + NW m
      i16x4 r[2];
      switch (m) {
        case 0: DSA_TR_READ2(r, trw, 0, 16 * kCRow); break;
        case 1: DSA_TR_READ2(r, trw, NW * 32, NW * 32 + 16 * kCRow); break;
        case 2: DSA_TR_READ2(r, trw, 2 * NW * 32, 2 * NW * 32 + 16 * kCRow); break;
        case 3: DSA_TR_READ2(r, trw, 3 * NW * 32, 3 * NW * 32 + 16 * kCRow); break;
        case 4: DSA_TR_READ2(r, trw, 4 * NW * 32, 4 * NW * 32 + 16 * kCRow); break;
        case 5: DSA_TR_READ2(r, trw, 5 * NW * 32, 5 * NW * 32 + 16 * kCRow); break;
        case 6: DSA_TR_READ2(r, trw, 6 * NW * 32, 6 * NW * 32 + 16 * kCRow); break;
        default: DSA_TR_READ2(r, trw, 7 * NW * 32, 7 * NW * 32 + 16 * kCRow); break;
      }
      const bf16x8 a = *reinterpret_cast<const bf16x8 *>(r);
#pragma unroll
      for (int n = 0; n < HT; ++n) acc[m * HT + n] = mfma_bf16_16x16x32(a, bs[n], acc[m * HT + n]);
    }
  };
  // gather instructions a wave issues per tile (the fewest, over the waves)
  constexpr int kGatherMin = kGatherInsts / NW;
  __syncthreads();
  if (ntiles > 0) gather_tile_fwd<NW, rec>(mla_tile<0>(), rows, 0, kv, N, wave, lane);
  if (ntiles > 1) gather_tile_fwd<NW, rec>(mla_tile<1>(), rows, kBN, kv, N, wave, lane);
  if (ntiles > 0) {
    if (ntiles > 1)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kGatherMin));  // tile 0 landed (tile 1 may be in flight)
    else
      __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();  // every wave's gathers of tile 0
    logits_ds(mla_tile<0>(), 0);
  }
  // Iteration j with tile j in static buffer B = j % 3 (j+1 in B+1, j+2 in
  // B+2), unrolled by three so that every buffer is a fixed object.
  auto step = [&](auto bc, int j) {
    constexpr int B = decltype(bc)::value;
    // This wave's gathers of tile j+1 have landed.  Issued after them: the
    // stores of tile j-1 (j >= 1): two per write-out wave, one for wave HT
    // with KL (its lanes 0..31 always store).
    if (j + 1 < ntiles) {
      if (wave < HT && j >= 1)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2));
      else if (KL && wave == HT && j >= 1)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(1));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    lds_barrier();  // staging j & 1 and tile j+1 complete; tile j-1 and staging (j+1) & 1 no longer read
    if (j + 2 < ntiles) gather_tile_fwd<NW, rec>(mla_tile<(B + 2) % 3>(), rows, (j + 2) * kBN, kv, N, wave, lane);
    if (wave < HT) write_out(j);
    if (KL && wave == HT) store_hsum(j);
    if (j + 1 < ntiles) logits_ds(mla_tile<(B + 1) % 3>(), j + 1);
    dq_tile(mla_tile<B>(), j);
  };
  for (int j = 0; j < ntiles; j += 3) {
    step(std::integral_constant<int, 0>(), j);
    if (j + 1 < ntiles) step(std::integral_constant<int, 1>(), j + 1);
    if (j + 2 < ntiles) step(std::integral_constant<int, 2>(), j + 2);
  }
  // dq of the wave's accumulator tiles
  float *dqq = dq + (t * H + hbase + c) * 576 + 4 * g;
#pragma unroll
  for (int m = 0; m < DT; ++m)
#pragma unroll
    for (int n = 0; n < HT; ++n)
      *reinterpret_cast<f32x4 *>(dqq + (int64_t)16 * n * 576 + 16 * (wave + NW * m)) = acc[m * HT + n];
  *reinterpret_cast<f32x4 *>(dqq + (int64_t)16 * n0 * 576 + 16 * irope) = acc[16];
  *reinterpret_cast<f32x4 *>(dqq + (int64_t)16 * (n0 + 1) * 576 + 16 * irope) = acc[17];
}

// Pair gradients of one query: G[pair, d] = sum_h (s dS)[pair, h] q[h, d] +
// P[pair, h] dO[h, d] (the dO term for d < 512), computed transposed,
// G^T[dims, keys] = q^T (s dS)^T + dO^T P^T: a GEMM over the heads whose
// A operands (q^T and dO^T, 16 dims x 32 heads per step) are constant for the
// query and whose B operands (the key-major s dS and P rows) stream through
// LDS.  One workgroup per query: twelve compute waves, wave w owning the
// 16-dim tiles 3w .. 3w+2 (tiles 32..35 are the rope dims, which have no dO
// term), and four loader waves.
//  * set-up: q[t] and then dO[t] are staged row-major in LDS and read back
//    with the transposing LDS load, so each compute lane holds its A operands
//    (dims 16 i + c, heads 32 s + 8 g .. +8) in registers;
//  * key loop, blocks of 64 keys in three LDS buffers: while the compute
//    waves work on block j, the loader waves fetch block j + 2 straight into
//    LDS and wait only until block j + 1 has landed; one LDS-only barrier a
//    block.  The compute waves issue only stores, so nothing ever makes them
//    wait for memory (loads and stores share one completion counter, and a
//    wait for a load would also wait for every store issued before it; a full
//    __syncthreads would too);
//  * each lane ends a 16 x 16 tile with dims 4 g .. 4 g + 3 of one key, rounds
//    them to bf16 and stores that 8-byte run of the key's G row through a
//    buffer bounded to the query's rows, which drops the stores of keys >= k.
//    (A streaming cache hint on fp32 G stores measured slower: plain 16-byte
//    stores stream at 4.6 TB/s on MI355X, streaming-hinted ones at 4.4.)
constexpr int kGWaves = 12;                   // compute waves
constexpr int kGLoaders = 4;                  // loader waves
constexpr int kGThreads = (kGWaves + kGLoaders) * 64;
constexpr int kGNBuf = 3;                     // key blocks in LDS: computed, landed, in flight
constexpr int kGKeys = 64;                    // keys per LDS block (64 measured 5% faster than 32)
constexpr int kGStageRow = kCRow;             // LDS bytes per staged row of q or dO

template <int H>
struct GShape {
  static constexpr int kRowSlots = H / 4 + 1;  // 16-byte LDS slots per key: s dS | P | pad
  static constexpr int kRow = 16 * kRowSlots;  // stride 4 (mod 64) dwords at H = 32 .. 128: conflict-free reads
  static constexpr int kInsts = (kGKeys * kRowSlots + 63) / 64;  // loader instructions (1 KB each) per block
  static constexpr int kBuf = kInsts * 1024;
  static constexpr int kSmem = H * kGStageRow > kGNBuf * kBuf ? H * kGStageRow : kGNBuf * kBuf;
};

// A operand of a 16x16x32 MFMA from a row-major [K rows][M cols] bf16 matrix
// in LDS: lane (g, c) gets column m0 + c, rows k0 + 8 g .. + 8.
__device__ __forceinline__ bf16x8 tr_operand(const uint8_t *base, int row_bytes, int k0, int m0, int g, int c) {
  const uint8_t *p = base + (k0 + 8 * g + (c >> 2)) * row_bytes + (m0 + 4 * (c & 3)) * 2;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 4 * row_bytes));
  const i16x4 lohi[2] = {lo, hi};
  return *reinterpret_cast<const bf16x8 *>(lohi);
}

// rows [0, H) of `width` bf16 each, from global (contiguous) into LDS rows of kGStageRow bytes
template <int H>
__device__ __forceinline__ void g_stage_rows(uint8_t *lds, const __bf16 *src, int width, int tid) {
  const int chunks = width / 8;  // 16-byte pieces per row
  for (int e = tid; e < H * chunks; e += kGThreads) {
    const int h = e / chunks, ch = e - h * chunks;
    *reinterpret_cast<i32x4 *>(lds + h * kGStageRow + ch * 16) =
        *reinterpret_cast<const i32x4 *>(src + (int64_t)h * width + ch * 8);
  }
}

template <int KS>
__global__ __launch_bounds__(kGThreads, 1) void mla_bwd_g_kernel(const __bf16 *__restrict__ q,
                                                                 const __bf16 *__restrict__ dout,
                                                                 const __bf16 *__restrict__ dsT,
                                                                 const __bf16 *__restrict__ pT, int k, int64_t t0,
                                                                 __bf16 *__restrict__ G) {
  constexpr int H = 32 * KS;
  using S = GShape<H>;
  extern __shared__ __align__(16) uint8_t smem_raw[];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool loader = wave >= kGWaves;  // uniform
  const int li = wave - kGWaves;        // loader index (uniform)
  const int64_t tc = blockIdx.x, t = t0 + tc;
  const int ti0 = 3 * (loader ? 0 : wave);  // uniform
  bf16x8 aq[3][KS], ao[3][KS];
  g_stage_rows<H>(smem_raw, q + t * H * 576, 576, tid);
  __syncthreads();
#pragma unroll
  for (int jt = 0; jt < 3; ++jt)
#pragma unroll
    for (int s = 0; s < KS; ++s) aq[jt][s] = tr_operand(smem_raw, kGStageRow, 32 * s, 16 * (ti0 + jt), g, c);
  __syncthreads();
  g_stage_rows<H>(smem_raw, dout + t * H * 512, 512, tid);
  __syncthreads();
#pragma unroll
  for (int jt = 0; jt < 3; ++jt)
#pragma unroll
    for (int s = 0; s < KS; ++s)
      ao[jt][s] = ti0 + jt < 32 ? tr_operand(smem_raw, kGStageRow, 32 * s, 16 * (ti0 + jt), g, c)
                                : bf16x8{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  __syncthreads();  // the staging area is free for the key blocks
  const __bf16 *dsq = dsT + tc * k * H;
  const __bf16 *pq = pT + tc * k * H;
  const int nblk = (k + kGKeys - 1) / kGKeys;
  // Loader li: instructions li, li + 4, ... of block b into dst.  Instruction
  // i writes slots [64 i, 64 i + 64); slot s holds key s / kRowSlots, piece
  // s % kRowSlots (the pad piece and the slots past the block's keys re-read a
  // valid piece); entries past k re-read entry k - 1, whose results are never
  // stored.
  auto issue_block = [&](int b, uint8_t *dst) {
    int l = lane;
    asm volatile("" : "+v"(l));  // recompute the lane roles per block instead of holding addresses
#pragma unroll
    for (int n = 0; n < (S::kInsts + kGLoaders - 1) / kGLoaders; ++n) {
      const int i = li + kGLoaders * n;  // uniform
      if (i >= S::kInsts) break;
      const int slot = i * 64 + l;
      const int kk = slot / S::kRowSlots;
      const int part = min(slot - kk * S::kRowSlots, H / 4 - 1);
      const int key = min(b * kGKeys + min(kk, kGKeys - 1), k - 1);
      const __bf16 *src = part < H / 8 ? dsq + (int64_t)key * H + part * 8 : pq + (int64_t)key * H + (part - H / 8) * 8;
      __builtin_amdgcn_global_load_lds(src, (lds_void *)(dst + i * 1024), 16, 0, 0);
    }
  };
  // wait until only this loader's newest block may still be in flight
  auto wait_all_but_newest = [&]() {
    constexpr int base = S::kInsts / kGLoaders, rem = S::kInsts % kGLoaders;
    if (rem != 0 && li < rem)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(base + 1));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(base));
  };
  if (loader) {
    if (nblk > 0) issue_block(0, smem_raw);
    if (nblk > 1) {
      issue_block(1, smem_raw + S::kBuf);
      wait_all_but_newest();
    } else {
      __builtin_amdgcn_s_waitcnt(0);
    }
  }
  __syncthreads();
  // G rows of this query (bf16) as a bounded buffer: stores of keys >= k are dropped
  const __amdgpu_buffer_rsrc_t gr =
      __builtin_amdgcn_make_buffer_rsrc((void *)(G + tc * k * 576), 0, k * 576 * 2, (int)kRsrcWord3);
  const int goff = c * 576 * 2 + (16 * ti0 + 4 * g) * 2;  // bytes: key c of a tile, this lane's dims
  // The two roles run loops of their own with the same barriers, so the
  // compute waves' code holds no direct-to-LDS load: the compiler then counts
  // their LDS reads exactly (a flat direct-to-LDS load anywhere on a path
  // makes it wait for every LDS read at each step).
  if (loader) {
    for (int j = 0; j < nblk; ++j) {
      // block j + 2 goes to the buffer last read before the previous barrier
      if (j + 2 < nblk) {
        issue_block(j + 2, smem_raw + ((j + 2) % kGNBuf) * S::kBuf);
        wait_all_but_newest();
      } else {
        __builtin_amdgcn_s_waitcnt(0);
      }
      lds_barrier();
    }
    return;
  }
  for (int j = 0; j < nblk; ++j) {
#pragma unroll 1
    for (int kt = 0; kt < kGKeys / 16; ++kt) {
      const uint8_t *brow = smem_raw + (j % kGNBuf) * S::kBuf + (16 * kt + c) * S::kRow + 16 * g;
      f32x4 acc[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 b = *reinterpret_cast<const bf16x8 *>(brow + 64 * s);
#pragma unroll
        for (int jt = 0; jt < 3; ++jt) acc[jt] = mfma_bf16_16x16x32(aq[jt][s], b, acc[jt]);
      }
      // the dO term (zero operands on the rope tiles)
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 b = *reinterpret_cast<const bf16x8 *>(brow + 2 * H + 64 * s);
#pragma unroll
        for (int jt = 0; jt < 3; ++jt) acc[jt] = mfma_bf16_16x16x32(ao[jt][s], b, acc[jt]);
      }
      const int off = (j * kGKeys + 16 * kt) * 576 * 2 + goff;
#pragma unroll
      for (int jt = 0; jt < 3; ++jt) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (__bf16)acc[jt][r];  // RNE
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, v), gr, off + 32 * jt, 0, 0);
      }
    }
    // Only the key blocks in LDS need ordering: the loaders waited for their
    // own block above, and nothing here reads G, so the G stores stay in
    // flight across the barrier (a full __syncthreads would wait for them).
    lds_barrier();
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

template <int HT, bool KL>
static hipError_t launch_ds_ht(const void *q, const void *kv, const int32_t *idx, const float *lse, const void *dout,
                               const float *D, int64_t N, int32_t H, int32_t k, float sm_scale, int64_t t0, int32_t Tc,
                               float *dq, void *dsT, void *pT, float *psum, hipStream_t s) {
  // LDS: the static tile buffers (g_mla_t*) plus smem_bwd_bytes of dynamic LDS
  const dim3 grid((uint32_t)Tc, H / (16 * HT));
  if (N * (576 * 2) <= (int64_t(1) << 32))  // every row within 4 GiB: record-indexed gathers
    hipLaunchKernelGGL((mla_bwd_ds_kernel<HT, KL, true>), grid, dim3(HT * 128), smem_bwd_bytes<HT>(), s,
                       (const __bf16 *)q, (const __bf16 *)kv, idx, lse, (const __bf16 *)dout, D, N, H, k, sm_scale, t0,
                       dq, (__bf16 *)dsT, (__bf16 *)pT, psum);
  else
    hipLaunchKernelGGL((mla_bwd_ds_kernel<HT, KL, false>), grid, dim3(HT * 128), smem_bwd_bytes<HT>(), s,
                       (const __bf16 *)q, (const __bf16 *)kv, idx, lse, (const __bf16 *)dout, D, N, H, k, sm_scale, t0,
                       dq, (__bf16 *)dsT, (__bf16 *)pT, psum);
  return hipGetLastError();
}

template <int KS>
static hipError_t launch_g_ks(const void *q, const void *dout, const void *dsT, const void *pT, int32_t k, int64_t t0,
                              int32_t Tc, __bf16 *G, hipStream_t s) {
  constexpr int bytes = GShape<32 * KS>::kSmem;
  static bool attr_done = false;  // per process: the attribute holds for every device
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void *)mla_bwd_g_kernel<KS>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       bytes);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  hipLaunchKernelGGL(mla_bwd_g_kernel<KS>, dim3((uint32_t)Tc), dim3(kGThreads), bytes, s, (const __bf16 *)q,
                     (const __bf16 *)dout, (const __bf16 *)dsT, (const __bf16 *)pT, k, t0, G);
  return hipGetLastError();
}

// Queries [t0, t0 + Tc): dq of those queries; s dS and P [Tc, k, H] bf16; then
// the pair gradients G [Tc, k, 576] (fp32 sums rounded to bf16); with psum,
// also each entry's sum of P over each head group, psum [Tc, H / 64 or H / 32,
// k] fp32 (the groups of the dS kernel: 64 heads when 64 divides H, else 32).
// H a multiple of 32, at most 128.
hipError_t launch_mla_bwd_chunk(const void *q, const void *kv, const int32_t *idx, const float *lse, const void *dout,
                                const float *D, int64_t N, int32_t H, int32_t k, float sm_scale, int64_t t0,
                                int32_t Tc, float *dq, void *dsT, void *pT, void *Gv, float *psum, hipStream_t s) {
  if (Tc <= 0) return hipSuccess;
  __bf16 *G = (__bf16 *)Gv;
  hipError_t e;
  if (H % 64 == 0)
    e = psum ? launch_ds_ht<4, true>(q, kv, idx, lse, dout, D, N, H, k, sm_scale, t0, Tc, dq, dsT, pT, psum, s)
             : launch_ds_ht<4, false>(q, kv, idx, lse, dout, D, N, H, k, sm_scale, t0, Tc, dq, dsT, pT, psum, s);
  else
    e = psum ? launch_ds_ht<2, true>(q, kv, idx, lse, dout, D, N, H, k, sm_scale, t0, Tc, dq, dsT, pT, psum, s)
             : launch_ds_ht<2, false>(q, kv, idx, lse, dout, D, N, H, k, sm_scale, t0, Tc, dq, dsT, pT, psum, s);
  if (e != hipSuccess) return e;
  switch (H / 32) {
    case 1:
      return launch_g_ks<1>(q, dout, dsT, pT, k, t0, Tc, G, s);
    case 2:
      return launch_g_ks<2>(q, dout, dsT, pT, k, t0, Tc, G, s);
    case 3:
      return launch_g_ks<3>(q, dout, dsT, pT, k, t0, Tc, G, s);
    case 4:
      return launch_g_ks<4>(q, dout, dsT, pT, k, t0, Tc, G, s);
    default:
      return hipErrorInvalidValue;
  }
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
