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
//    double buffered so the gather of tile i+1 overlaps the MFMAs of tile i;
//    each row is fetched once for all heads of the workgroup;
//  * logits are computed transposed, S^T = C Q^T (keys x heads), with bf16
//    MFMA 16x16x32 and Q^T resident in registers; in that layout each lane
//    holds 8 keys of one head, which is exactly the B operand layout the PV
//    MFMA needs (up to a fixed permutation of the keys), so P never moves
//    between lanes;
//  * the value operand of PV (value dims x keys) is read from the same
//    row-major tile with the transposing LDS load, which hands each lane four
//    keys of one value column;
//  * online softmax in fp32 (base-2 exponent with the scale folded in),
//    output O^T (value dims x heads) accumulated in fp32 registers;
//  * optional split of the selection across workgroups with an LSE-weighted
//    combine (used when there are too few queries to fill the GPU).
#include "dsa_common.h"

namespace {

constexpr int kBN = 32;                  // selected rows per tile
constexpr int kRowSlots = 73;            // 16-byte slots per LDS row: 72 of data + 1 pad (bank spread)
constexpr int kCRow = kRowSlots * 16;    // LDS bytes per gathered row
constexpr int kTileBytes = kBN * kCRow;  // 37376
constexpr int kTileSlots = kBN * kRowSlots;
constexpr int kGatherInsts = (kTileSlots + 63) / 64;  // wave-wide 1 KB direct-to-LDS loads per tile
constexpr int kSmemMla = 2 * kTileBytes + 2048 * 4;

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
// slots [64i, 64i+64); slot s holds row s/73, 16-byte chunk s%73 (chunk 72 is
// padding and reloads chunk 71).
template <int NW>
__device__ __forceinline__ void gather_tile_async(uint8_t *__restrict__ dst, const int *__restrict__ rows,
                                                  int r0, const __bf16 *__restrict__ kv, int wave, int lane) {
#pragma unroll
  for (int i = wave; i < kGatherInsts; i += NW) {
    const int slot = i * 64 + lane;
    if (slot < kTileSlots) {
      const int r = slot / kRowSlots;
      const int j = min(slot - r * kRowSlots, 71);
      const int pr = rows[r0 + r];
      const __bf16 *src = kv + (int64_t)(pr >= 0 ? pr : 0) * 576 + j * 8;
      __builtin_amdgcn_global_load_lds(src, (lds_void *)(dst + i * 1024), 16, 0, 0);
    }
  }
}

template <int NW>
__global__ __launch_bounds__(NW * 64, 1) void sparse_mla_bf16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ kv, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ bt, int max_blocks, int64_t N, int T, int H, int k, float scale_log2,
    __bf16 *__restrict__ out, float *__restrict__ lse, int splits, float *__restrict__ part_o,
    float *__restrict__ part_ml) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  uint8_t *tiles = smem_raw;                                        // 2 x kTileBytes
  int *rows = reinterpret_cast<int *>(smem_raw + 2 * kTileBytes);   // <= 2048 physical rows

  const int n_hg = H / (16 * NW);
  const int bid = blockIdx.x;
  const int sp = bid % splits;
  const int rest = bid / splits;
  const int hg = rest % n_hg;
  const int64_t t = rest / n_hg;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int h0 = (hg * NW + wave) * 16;
  const int ntiles = (k + kBN - 1) / kBN;
  const int per = (ntiles + splits - 1) / splits;
  const int tb = sp * per, te = min(ntiles, tb + per);
  const int32_t *irow = idx + t * k;

  // physical rows of this workgroup's entries [tb*32, te*32)
  for (int e = tid; e < (te - tb) * kBN; e += NW * 64)
    rows[e] = (int)phys_row(irow, bt, max_blocks, N, t, tb * kBN + e, k);
  __syncthreads();
  if (tb < te) gather_tile_async<NW>(tiles, rows, 0, kv, wave, lane);

  // Q^T in registers: lane (g, c) holds head h0+c, dims 32*s + 8*g .. +8 for step s.
  bf16x8 qr[18];
  const __bf16 *qrow = q + (t * H + h0 + c) * 576 + g * 8;
#pragma unroll
  for (int s = 0; s < 18; ++s) qr[s] = *reinterpret_cast<const bf16x8 *>(qrow + s * 32);

  f32x4 o[32];
#pragma unroll
  for (int m = 0; m < 32; ++m) o[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;
  // transposing-load lane roles: row 4g + (c>>2) of each 4-row group, value chunk (c&3)
  const int tr_row = 4 * g + (c >> 2), tr_col = (c & 3) * 4;

  for (int tile = tb; tile < te; ++tile) {
    const int cur = (tile - tb) & 1;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of `tile` have landed in LDS
    __syncthreads();                // ... and every wave's; tile-1 is no longer read
    if (tile + 1 < te)
      gather_tile_async<NW>(tiles + (cur ^ 1) * kTileBytes, rows, (tile + 1 - tb) * kBN, kv, wave, lane);
    const uint8_t *ct = tiles + cur * kTileBytes;
    const int *rv = rows + (tile - tb) * kBN;
    // S^T for keys [0,16) and [16,32) of the tile
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 18; ++s) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(ct + c * kCRow + (s * 32 + g * 8) * 2);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(ct + (16 + c) * kCRow + (s * 32 + g * 8) * 2);
      s0 = mfma_bf16_16x16x32(a0, qr[s], s0);
      s1 = mfma_bf16_16x16x32(a1, qr[s], s1);
    }
    // keep LDS reads close to their MFMAs (bounds live registers)
#pragma unroll
    for (int s = 0; s < 18; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    // lane (g,c): x[r] = key 4g+r, x[4+r] = key 16+4g+r, head c
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = rv[4 * g + r] >= 0 ? s0[r] * scale_log2 : -INFINITY;
      x[4 + r] = rv[16 + 4 * g + r] >= 0 ? s1[r] * scale_log2 : -INFINITY;
    }
    float mx = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float msub = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - m_new);
    float p[8], psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = exp2f(x[i] - msub);
      psum += p[i];
    }
    l_run = l_run * alpha + psum;
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int m = 0; m < 32; ++m) o[m] *= alpha;
    }
    m_run = m_new;
    bf16x8 pb;
#pragma unroll
    for (int i = 0; i < 8; ++i) pb[i] = (__bf16)p[i];
    // O^T[dv, head] += V^T[dv, keys] P^T[keys, head]; key slot order matches pb
    const uint8_t *tr0 = ct + tr_row * kCRow + tr_col * 2;
    const uint8_t *tr1 = tr0 + 16 * kCRow;
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(tr0 + m * 32));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(tr1 + m * 32));
      const i16x4 lohi[2] = {lo, hi};
      const bf16x8 a = *reinterpret_cast<const bf16x8 *>(lohi);
      o[m] = mfma_bf16_16x16x32(a, pb, o[m]);
    }
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    }
  }

  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const int head = h0 + c;
  if (splits == 1) {
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    __bf16 *orow = out + (t * H + head) * 512;
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      bf16x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (__bf16)(o[m][r] * inv);
      *reinterpret_cast<bf16x4 *>(orow + 16 * m + 4 * g) = v;
    }
    if (lse && g == 0)
      lse[t * H + head] = l_tot > 0.0f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  } else {
    float *po = part_o + ((t * splits + sp) * H + head) * 512;
#pragma unroll
    for (int m = 0; m < 32; ++m) *reinterpret_cast<f32x4 *>(po + 16 * m + 4 * g) = o[m];
    if (g == 0) {
      float *pm = part_ml + ((t * splits + sp) * H + head) * 2;
      pm[0] = m_run;
      pm[1] = l_tot;
    }
  }
}

// LSE-weighted combine of split partials.  grid (T*H/4), block 256: 4 heads,
// 64 threads per head, 8 value dims per thread.
__global__ __launch_bounds__(256) void mla_combine_kernel(const float *__restrict__ part_o,
                                                          const float *__restrict__ part_ml, int T, int H,
                                                          int splits, __bf16 *__restrict__ out,
                                                          float *__restrict__ lse) {
  const int64_t th = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (th >= (int64_t)T * H) return;
  const int lane = threadIdx.x & 63;
  const int64_t t = th / H;
  const int h = (int)(th % H);
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, part_ml[((t * splits + s) * H + h) * 2]);
  float Lsum = 0.0f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < splits; ++s) {
    const float *pm = part_ml + ((t * splits + s) * H + h) * 2;
    const float ms = pm[0], ls = pm[1];
    if (ms == -INFINITY) continue;
    const float wgt = exp2f(ms - M);
    Lsum += wgt * ls;
    const float *po = part_o + ((t * splits + s) * H + h) * 512 + lane * 8;
    const f32x4 a = *reinterpret_cast<const f32x4 *>(po);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(po + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] += wgt * a[i];
      acc[4 + i] += wgt * b[i];
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

template <int NW>
hipError_t launch_bf16_nw(const void *q, const void *kv, const int32_t *idx, const int32_t *bt,
                          int max_blocks, int64_t N, int T, int H, int k, float scale_log2, void *out, float *lse,
                          int splits, float *part_o, float *part_ml, hipStream_t s) {
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void *)sparse_mla_bf16_kernel<NW>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kSmemMla);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int64_t blocks = (int64_t)T * (H / (16 * NW)) * splits;
  hipLaunchKernelGGL(sparse_mla_bf16_kernel<NW>, dim3((uint32_t)blocks), dim3(NW * 64), kSmemMla, s,
                     (const __bf16 *)q, (const __bf16 *)kv, idx, bt, max_blocks, N, T, H, k, scale_log2,
                     (__bf16 *)out, lse, splits, part_o, part_ml);
  return hipGetLastError();
}

}  // namespace

namespace dsa {
hipError_t launch_sparse_mla_bf16(const void *q, const void *kv, const int32_t *idx,
                                  const int32_t *block_table, int32_t max_blocks, int64_t N, int32_t T,
                                  int32_t H, int32_t k, float sm_scale, void *out, float *lse,
                                  int32_t splits, float *part_o, float *part_ml, hipStream_t s) {
  if (T == 0) return hipSuccess;
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

hipError_t launch_sparse_mla_f32(const float *q, const float *kv, const int32_t *idx, int64_t N, int32_t T,
                                 int32_t H, int32_t k, float sm_scale, float *out, float *lse,
                                 hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(sparse_mla_f32_kernel, dim3(T), dim3(256), 0, s, q, kv, idx, N, T, H, k, sm_scale,
                     out, lse);
  return hipGetLastError();
}
}  // namespace dsa
