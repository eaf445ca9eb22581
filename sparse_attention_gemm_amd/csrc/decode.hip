// Paged decode pieces: the indexer over each sequence's FP8 key pages, and the
// cache append of one new token per sequence.
//
// The latent KV cache of MLA (jienda.com, section 2.1: keys and values
// compressed into a latent space) is paged in 64-token pages; logical
// position p of sequence b lives in physical row
// block_table[b][p/64]*64 + p%64 of each pool.
//
// Decode indexer: one query (64 heads x 128 E4M3) per sequence against all of
// its ctx keys.  This streams 132 B per key from HBM (the key payload and its
// scale) and is bandwidth bound.  A wavefront keeps the query's 64 heads in
// registers and scores kPagesPerWave pages (64 keys, 8 KB contiguous in the
// pool, each read exactly once), loading the next page's keys while it
// computes the current one.
#include "dsa_common.h"
#include "dsa_launch.h"
#include "indexer_core.h"

namespace {

constexpr int kWavesD = 4;
constexpr int kPagesPerWave = 8;
constexpr int kPagesPerBlock = kWavesD * kPagesPerWave;

// grid: (ceil(max_ctx / (64 * kPagesPerBlock)), B)
__global__ __launch_bounds__(kWavesD * 64) void decode_indexer_kernel(
    const uint8_t *__restrict__ q8, const float *__restrict__ qs, const float *__restrict__ w,
    const uint8_t *__restrict__ k8_pool, const float *__restrict__ ks_pool, const int32_t *__restrict__ bt,
    int max_blocks, const int32_t *__restrict__ ctx_len, int64_t n_pool_rows, float *__restrict__ scores,
    int64_t ld, int max_ctx) {
  __shared__ uint8_t qscratch[kWavesD][kQueryScratch];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t b = blockIdx.y;
  const int ctx = min(ctx_len[b], max_ctx);
  const int npages = min((ctx + 63) >> 6, max_blocks);
  const int p0 = blockIdx.x * kPagesPerBlock + wave * kPagesPerWave;
  const int np = min(kPagesPerWave, npages - p0);  // pages of this wave
  if (np <= 0) return;
  float *srow = scores + b * ld;
  // the wave's block-table entries, one per lane, requested before the query
  // set-up so that their latency overlaps it
  const int32_t blk_l = lane < np ? bt[b * max_blocks + p0 + lane] : -1;
  IdxQuery<4> Q;
  idx_load_query<4>(Q, q8 + b * 64 * 128, w + b * 64, qs[b], lane, qscratch[wave]);
  // physical first row of page p0 + j (j uniform), or -1 when unmapped
  auto page_row = [&](int j) -> int64_t {
    const int32_t blk = __builtin_amdgcn_readlane(blk_l, j);
    const int64_t prow = (int64_t)blk * 64;
    return (blk < 0 || prow + 64 > n_pool_rows) ? -1 : prow;
  };
  // Page loads are unconditional (an unmapped or missing page reads row 0 of
  // the pool and is discarded): with no branch around them the compiler can
  // wait for exactly the loads a key block needs, leaving the next page's
  // loads in flight.
  i32x8 kb[2][4];
  float kscale[2];
  auto load_page = [&](int buf, int64_t prow) {
    const int64_t r = prow < 0 ? 0 : prow;
    idx_load_keys(kb[buf], k8_pool + r * 128, 128, lane);
    kscale[buf] = ks_pool[r + lane];
  };
  int64_t prow = page_row(0);
  load_page(0, prow);
#pragma unroll
  for (int j = 0; j < kPagesPerWave; ++j) {
    if (j >= np) break;  // uniform
    const int cur = j & 1;
    const int64_t next = j + 1 < np ? page_row(j + 1) : -1;
    if (j + 1 < kPagesPerWave) load_page(cur ^ 1, next);
    const int s = (p0 + j) * 64 + lane;
    const float tot = idx_score64<4>(Q, kb[cur]);
    if (s < ctx) srow[s] = prow >= 0 ? canon_zero(tot * kscale[cur]) : -INFINITY;  // unmapped page: nothing to score
    prow = next;
  }
}

// One workgroup per appended token: 72 chunks of latent, 8 of key, 1 scale.
__global__ __launch_bounds__(128) void cache_append_kernel(const __bf16 *__restrict__ latent,
                                                           const uint8_t *__restrict__ k8,
                                                           const float *__restrict__ ks,
                                                           const int32_t *__restrict__ pos, int D_I,
                                                           const int32_t *__restrict__ bt, int max_blocks,
                                                           int64_t n_pool_rows, __bf16 *__restrict__ kv_pool,
                                                           uint8_t *__restrict__ k8_pool,
                                                           float *__restrict__ ks_pool) {
  const int64_t b = blockIdx.x;
  const int p = pos[b];
  if (p < 0 || (p >> 6) >= max_blocks) return;  // position outside the table
  const int32_t blk = bt[b * max_blocks + (p >> 6)];
  const int64_t row = (int64_t)blk * 64 + (p & 63);
  if (blk < 0 || row >= n_pool_rows) return;    // unmapped page
  const int tid = threadIdx.x;
  if (tid < 72) {
    *reinterpret_cast<i32x4 *>(kv_pool + row * 576 + tid * 8) =
        *reinterpret_cast<const i32x4 *>(latent + b * 576 + tid * 8);
  } else if (tid < 72 + D_I / 16) {
    const int c = tid - 72;
    *reinterpret_cast<i32x4 *>(k8_pool + row * D_I + c * 16) =
        *reinterpret_cast<const i32x4 *>(k8 + b * D_I + c * 16);
  } else if (tid == 127) {
    ks_pool[row] = ks[b];
  }
}

}  // namespace

namespace dsa {
hipError_t launch_decode_indexer(const uint8_t *q8, const float *qs, const float *w,
                                 const uint8_t *k8_pool, const float *ks_pool,
                                 const int32_t *block_table, int32_t max_blocks,
                                 const int32_t *ctx_len, int32_t B, int32_t max_ctx, int64_t n_pool_rows,
                                 float *scores, int64_t ld, hipStream_t s) {
  if (B == 0) return hipSuccess;
  dim3 grid((max_ctx + 64 * kPagesPerBlock - 1) / (64 * kPagesPerBlock), B);
  hipLaunchKernelGGL(decode_indexer_kernel, grid, dim3(kWavesD * 64), 0, s, q8, qs, w, k8_pool, ks_pool, block_table,
                     max_blocks, ctx_len, n_pool_rows, scores, ld, max_ctx);
  return hipGetLastError();
}

hipError_t launch_cache_append(const void *latent, const uint8_t *k8, const float *ks,
                               const int32_t *pos, int32_t B, int32_t D_I,
                               const int32_t *block_table, int32_t max_blocks, int64_t n_pool_rows,
                               void *kv_pool, uint8_t *k8_pool, float *ks_pool, hipStream_t s) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(cache_append_kernel, dim3(B), dim3(128), 0, s, (const __bf16 *)latent, k8, ks, pos, D_I,
                     block_table, max_blocks, n_pool_rows, (__bf16 *)kv_pool, k8_pool, ks_pool);
  return hipGetLastError();
}
}  // namespace dsa
