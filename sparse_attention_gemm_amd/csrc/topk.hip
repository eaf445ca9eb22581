// Row-wise top-k selection over a score matrix (fine-grained token selection:
// mizuki-eaf.pages.dev, "How it works"; m.digipub.cc, section 2).
//
// One 1024-thread workgroup per row.  Scores are mapped to order-preserving
// u32 keys.  The row is read from global memory in coalesced passes (each
// thread takes 4 consecutive scores, as one 16-byte load when the row is
// aligned, with several such groups in flight):
//   1. 2048-bin histograms over the window that holds the k-th largest key,
//      starting from the top 11 key bits (sign, exponent and two mantissa
//      bits of the score) and narrowing 11 bits at a time, until the entries
//      at or above the lower edge of that bin fit in LDS (18432 candidates;
//      usually after the first histogram);
//   2. one ordered pass that copies those candidates (key, position) into
//      LDS in position order.
// The exact k-th key tau lies in the last bin of pass 1; narrowing over the
// candidates of that bin in LDS finds it (two more levels).  The output pass
// keeps key > tau plus the most recent (largest-position) ties at tau and
// writes positions in ascending order: each thread owns a contiguous run of
// the position-ordered candidates and one block scan places the runs, so
// results are deterministic.  If a single key value is too frequent to fit
// (massive ties), the output pass runs over the row in global memory instead.
#include <algorithm>

#include "dsa_common.h"
#include "dsa_launch.h"
#include "dsa_sizes.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;
constexpr int kCand = 18432;  // candidates held in LDS
constexpr int kU = 8;         // groups of 4 row elements per thread in flight (32768 elements)
constexpr int kMaxChunks = dsa::kTopkMaxChunks;  // chunks per row of a split selection
static_assert(kMaxChunks * 2048 <= 18432, "a merge's candidates fit in LDS");

struct TopkShared {
  uint32_t hist[kBins];
  uint32_t ckey[kCand];
  int32_t cpos[kCand];
  uint32_t wred[2][kWaves];
  uint32_t upre[kU][kWaves];  // pass 2: exclusive offsets of (group u, wave) in position order
  uint32_t bstar, above, bcnt;
};
constexpr size_t kTopkSmem = sizeof(TopkShared);

__device__ __forceinline__ uint32_t row_key(const float *__restrict__ sc, int i) {
  return score_key(canon_zero(sc[i]));
}

// Block-wide inclusive scan helpers over 1024 threads (16 waves).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive prefix over threads in thread order; also returns the total.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *wred, uint32_t &total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = wave_incl_scan(v, lane);
  if (lane == 63) wred[wave] = inc;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    uint32_t x = wred[w];
    off += (w < wave) ? x : 0;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return off + inc - v;
}

// Keys of the 4 consecutive row elements starting at i0 (those >= n are 0).
__device__ __forceinline__ void load4(const float *__restrict__ sc, bool aligned, int i0, int n, uint32_t (&k4)[4]) {
  if (aligned && i0 + 3 < n) {
    const float4 v = *reinterpret_cast<const float4 *>(sc + i0);
    k4[0] = score_key(canon_zero(v.x));
    k4[1] = score_key(canon_zero(v.y));
    k4[2] = score_key(canon_zero(v.z));
    k4[3] = score_key(canon_zero(v.w));
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) k4[j] = i0 + j < n ? row_key(sc, i0 + j) : 0u;
  }
}

// Visit the row in blocks of 4096 elements (thread t takes elements
// 4t..4t+3 of a block; kU blocks in flight): f(i0, k4) with i0 the first
// element of the thread's group.  Every thread runs every block (the loop
// bounds are uniform), so f may synchronise the workgroup.
template <typename F>
__device__ __forceinline__ void for_row4(const float *__restrict__ sc, bool aligned, int n, F &&f) {
  const int tid = threadIdx.x;
  for (int b0 = 0; b0 < n; b0 += 4 * kThreads * kU) {
    uint32_t kk[kU][4];
#pragma unroll
    for (int u = 0; u < kU; ++u) load4(sc, aligned, b0 + 4 * (u * kThreads + tid), n, kk[u]);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (b0 + 4 * u * kThreads >= n) break;  // uniform
      f(b0 + 4 * (u * kThreads + tid), kk[u]);
    }
  }
}

// Given the histogram in sm.hist, find the bin that holds the remaining-th
// largest element of the window: its index, the count strictly above it and
// its own count (all threads get them).
__device__ __forceinline__ void select_bin(TopkShared &sm, uint32_t remaining, uint32_t &bstar,
                                           uint32_t &above, uint32_t &bcnt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Suffix sums from the top bin.  Thread tid owns bins 2*tid and 2*tid+1;
  // s_hi = number of window elements in bins above 2*tid+1.
  const uint32_t h1 = sm.hist[2 * tid + 1], h0 = sm.hist[2 * tid];
  const uint32_t mine = h0 + h1;
  // inclusive scan over reversed lanes gives, read back reversed, the
  // in-wave suffix sum including the own lane
  const uint32_t inc = wave_incl_scan(__shfl(mine, 63 - lane), lane);
  const uint32_t suffix_in_wave = __shfl(inc, 63 - lane);
  if (lane == 0) sm.wred[0][wave] = suffix_in_wave;  // wave total
  __syncthreads();
  uint32_t above_waves = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) above_waves += (w > wave) ? sm.wred[0][w] : 0;
  const uint32_t s_hi = above_waves + suffix_in_wave - mine;  // count in bins > 2*tid+1
  const uint32_t s1 = s_hi + h1;                               // count in bins >= 2*tid+1
  const uint32_t s0 = s1 + h0;                                 // count in bins >= 2*tid
  if (s1 >= remaining && s_hi < remaining) {
    sm.bstar = 2 * tid + 1;
    sm.above = s_hi;
    sm.bcnt = h1;
  } else if (s0 >= remaining && s1 < remaining) {
    sm.bstar = 2 * tid;
    sm.above = s1;
    sm.bcnt = h0;
  }
  __syncthreads();
  bstar = sm.bstar;
  above = sm.above;
  bcnt = sm.bcnt;
  __syncthreads();
}

// Histogram narrowing state over a window [base, base + (nbins << shift)).
struct Narrow {
  uint32_t base;
  int shift;
  uint32_t nbins;
  uint32_t remaining;  // rank of the target inside the window
  // the whole key space, binned on the top 11 bits
  __device__ __forceinline__ void init_full(uint32_t k) {
    base = 0;
    shift = 21;
    nbins = kBins;
    remaining = k;
  }
  // the window [lo, lo + 2^w) (one bin of an earlier level), rank r inside it
  __device__ __forceinline__ void init_bin(uint32_t lo, int w, uint32_t r) {
    base = lo;
    shift = max(0, w - 11);
    nbins = 1u << (w - shift);
    remaining = r;
  }
  __device__ __forceinline__ void add(TopkShared &sm, uint32_t key) const {
    if (key >= base) {
      const uint32_t d = (key - base) >> shift;
      if (d < nbins) atomicAdd(&sm.hist[d], 1u);
    }
  }
  // narrow to bin bstar (call after select_bin); returns false at a single key
  __device__ __forceinline__ bool descend(uint32_t bstar, uint32_t above) {
    remaining -= above;
    base += bstar << shift;
    if (shift == 0) return false;
    const int nshift = max(0, shift - 11);
    nbins = 1u << (shift - nshift);
    shift = nshift;
    return true;
  }
};

__device__ __forceinline__ void clear_hist(TopkShared &sm) {
  for (int b = threadIdx.x; b < kBins; b += kThreads) sm.hist[b] = 0;
  __syncthreads();
}

// Ordered output of one block of up to 1024 entries (one per thread, thread
// order = position order): keep key > tau, and the ties at tau whose rank
// among all ties (in position order) is >= tie_cut.  dst and tie_seen carry
// across blocks.
__device__ __forceinline__ void emit_block(TopkShared &sm, bool in, uint32_t key, int32_t pos, uint32_t tau,
                                           uint32_t tie_cut, uint32_t &dst, uint32_t &tie_seen,
                                           int32_t *__restrict__ out) {
  const bool tie = in && key == tau;
  uint32_t n_tie, n_gt;
  const uint32_t tie_rank = tie_seen + block_excl_scan(tie ? 1u : 0u, sm.wred[0], n_tie);
  const bool keep = in && (key > tau || (tie && tie_rank >= tie_cut));
  const uint32_t off = block_excl_scan(keep ? 1u : 0u, sm.wred[1], n_gt);
  if (keep) out[dst + off] = pos;
  dst += n_gt;
  tie_seen += n_tie;
}

// Exact k-th key and ordered output of the m candidates (key, position) in
// sm.ckey / sm.cpos, which are in position order and hold every key above
// `edge` plus all keys of the window [edge, edge + 2^width) (width 32: the
// whole key space); the k-th key has rank rank_in_bin inside that window.
__device__ void cut_and_output(TopkShared &sm, uint32_t m, uint32_t edge, int width, uint32_t rank_in_bin,
                               int32_t *__restrict__ out) {
  const int tid = threadIdx.x;
  // ---- exact k-th key: narrow over the window's candidates in LDS
  Narrow nc;
  nc.init_bin(edge, width, rank_in_bin);
  uint32_t tau = edge, ties = 0;
  while (width > 0) {
    clear_hist(sm);
    for (int i = tid; i < (int)m; i += kThreads) nc.add(sm, sm.ckey[i]);
    __syncthreads();
    uint32_t bstar, above, bcnt;
    select_bin(sm, nc.remaining, bstar, above, bcnt);
    if (!nc.descend(bstar, above)) {
      tau = nc.base;
      ties = bcnt;
      break;
    }
  }
  if (width == 0) {  // the window is a single key value
    ties = 0;
    for (int i = tid; i < (int)m; i += kThreads) ties += sm.ckey[i] == tau ? 1u : 0u;
    uint32_t tot;
    block_excl_scan(ties, sm.wred[0], tot);
    ties = tot;
    nc.remaining = rank_in_bin;
  }
  // ---- ordered output from LDS: thread t owns the candidates [t R, t R + R),
  // which are in position order.  One scan of packed (greater, tie) counts
  // gives each thread its output offset: the greater keys before its run plus
  // the ties before its run that rank at or after tie_cut.
  const uint32_t tie_cut = ties - nc.remaining;
  const int R = ((int)m + kThreads - 1) / kThreads;
  const int i0 = min(tid * R, (int)m), i1 = min(i0 + R, (int)m);
  uint32_t n_gt = 0, n_tie = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = sm.ckey[i];
    n_gt += key > tau ? 1u : 0u;
    n_tie += key == tau ? 1u : 0u;
  }
  static_assert(kCand < 65536, "counts pack into 16 bits");
  uint32_t packed_tot;
  const uint32_t pre = block_excl_scan((n_gt << 16) | n_tie, sm.wred[0], packed_tot);
  const uint32_t gt_before = pre >> 16, tie_before = pre & 0xFFFFu;
  uint32_t dst = gt_before + (tie_before > tie_cut ? tie_before - tie_cut : 0u);
  uint32_t tie_rank = tie_before;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = sm.ckey[i];
    const bool tie = key == tau;
    if (key > tau || (tie && tie_rank >= tie_cut)) out[dst++] = sm.cpos[i];
    tie_rank += tie ? 1u : 0u;
  }
}

// One workgroup per (row, chunk): workgroup b takes columns [c chunk,
// (c + 1) chunk) of row b / nch, c = b % nch (nch = 1: the whole row), and
// writes its selection (positions within the chunk) to idx + b k, and, when
// cnt is given, its size to cnt[b].
__global__ __launch_bounds__(kThreads) void topk_rows_kernel(const float *__restrict__ scores, int64_t ld,
                                                             const int32_t *__restrict__ n_valid, int32_t n_cap,
                                                             int32_t nch, int32_t chunk, int32_t k,
                                                             int32_t *__restrict__ idx, int32_t *__restrict__ cnt) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  TopkShared &sm = *reinterpret_cast<TopkShared *>(smem_raw);
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x / nch;
  const int c0 = (int)(blockIdx.x % nch) * chunk;
  const int n = max(0, min(min(n_valid[row], n_cap) - c0, chunk));
  const float *sc = scores + row * ld + c0;
  int32_t *out = idx + (int64_t)blockIdx.x * k;
  if (cnt && tid == 0) cnt[blockIdx.x] = min(n, k);
  if (n <= k) {
    for (int i = tid; i < k; i += kThreads) out[i] = i < n ? i : -1;
    return;
  }
  const bool aligned = (reinterpret_cast<uintptr_t>(sc) & 15) == 0;
  // ---- pass 1: narrow over the row until the candidates fit in LDS
  Narrow nw;
  nw.init_full((uint32_t)k);
  uint32_t above_total = 0, edge = 0, rank_in_bin = 0;
  while (true) {
    clear_hist(sm);
    for_row4(sc, aligned, n, [&](int i0, const uint32_t (&k4)[4]) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (i0 + j < n) nw.add(sm, k4[j]);
    });
    __syncthreads();
    uint32_t bstar, above, bcnt;
    select_bin(sm, nw.remaining, bstar, above, bcnt);
    edge = nw.base + (bstar << nw.shift);
    rank_in_bin = nw.remaining - above;
    if (above_total + above + bcnt <= (uint32_t)kCand) break;
    above_total += above;
    if (!nw.descend(bstar, above)) {
      // one key value too frequent for LDS: output straight from the row
      const uint32_t tie_cut = bcnt - nw.remaining;
      uint32_t dst = 0, tie_seen = 0;
      for (int b0 = 0; b0 < n; b0 += kThreads) {
        const int i = b0 + tid;
        emit_block(sm, i < n, i < n ? row_key(sc, i) : 0u, i, nw.base, tie_cut, dst, tie_seen, out);
      }
      return;
    }
  }
  // ---- pass 2: candidates (key >= edge) into LDS, in position order.  The
  // element order within a batch is (group u, thread); the offsets of all kU
  // groups come from one set of wave scans and one 128-entry scan.
  uint32_t m = 0;
  {
    const int lane = tid & 63, wave = tid >> 6;
    for (int b0 = 0; b0 < n; b0 += 4 * kThreads * kU) {
      uint32_t kk[kU][4], cnt[kU], incl[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) load4(sc, aligned, b0 + 4 * (u * kThreads + tid), n, kk[u]);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i0 = b0 + 4 * (u * kThreads + tid);
        cnt[u] = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) cnt[u] += (i0 + j < n && kk[u][j] >= edge) ? 1u : 0u;
        incl[u] = wave_incl_scan(cnt[u], lane);
        if (lane == 63) sm.upre[u][wave] = incl[u];  // wave total
      }
      __syncthreads();
      if (wave == 0) {
        // exclusive scan of the kU x kWaves totals in (u, wave) order; lane
        // handles entries 2 lane and 2 lane + 1
        uint32_t *flat = &sm.upre[0][0];
        static_assert(kU * kWaves == 128, "two entries per lane");
        const uint32_t a0 = flat[2 * lane], a1 = flat[2 * lane + 1];
        const uint32_t pair = a0 + a1;
        const uint32_t pin = wave_incl_scan(pair, lane);
        flat[2 * lane] = pin - pair;
        flat[2 * lane + 1] = pin - pair + a0;
        if (lane == 63) sm.bcnt = pin;  // batch total
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i0 = b0 + 4 * (u * kThreads + tid);
        uint32_t off = m + sm.upre[u][wave] + incl[u] - cnt[u];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (i0 + j < n && kk[u][j] >= edge) {
            sm.ckey[off] = kk[u][j];
            sm.cpos[off] = i0 + j;
            ++off;
          }
      }
      m += sm.bcnt;
      __syncthreads();  // upre and bcnt are rewritten by the next batch
    }
  }
  __syncthreads();
  // the exact k-th key lies in the last bin of pass 1, [edge, edge + 2^shift),
  // at rank rank_in_bin; the candidates above that bin are all kept
  cut_and_output(sm, m, edge, nw.shift, rank_in_bin, out);
}

// Second pass of a chunked selection: row b's candidates are the nch chunk
// selections of the first pass (positions within their chunk, cnt[b nch + c]
// of them), in position order.  At most nch k <= kCand of them, so they all
// go to LDS and only the exact cut remains.
__global__ __launch_bounds__(kThreads) void topk_merge_kernel(const float *__restrict__ scores, int64_t ld,
                                                              const int32_t *__restrict__ cpos,
                                                              const int32_t *__restrict__ cnt, int32_t nch,
                                                              int32_t chunk, int32_t k, int32_t *__restrict__ idx) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  TopkShared &sm = *reinterpret_cast<TopkShared *>(smem_raw);
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const float *sc = scores + row * ld;
  int32_t *out = idx + row * (int64_t)k;
  int off[kMaxChunks + 1];
  off[0] = 0;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) off[c + 1] = off[c] + (c < nch ? cnt[row * nch + c] : 0);
  const int m = off[kMaxChunks];
  for (int i = tid; i < m; i += kThreads) {
    int c = 0;
#pragma unroll
    for (int j = 1; j < kMaxChunks; ++j) c += i >= off[j] ? 1 : 0;
    const int p = c * chunk + cpos[(row * nch + c) * (int64_t)k + (i - off[c])];
    sm.cpos[i] = p;
    sm.ckey[i] = row_key(sc, p);
  }
  __syncthreads();
  if (m <= k) {
    for (int i = tid; i < k; i += kThreads) out[i] = i < m ? sm.cpos[i] : -1;
    return;
  }
  cut_and_output(sm, (uint32_t)m, 0u, 32, (uint32_t)k, out);
}

__global__ void positions_kernel(int32_t *__restrict__ q_pos, int32_t *__restrict__ n_valid, int32_t L) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < L) {
    q_pos[i] = i;
    n_valid[i] = i + 1;
  }
}

}  // namespace

namespace dsa {
// q_pos[t] = t, n_valid[t] = t + 1: the causal candidate sets of one sequence.
hipError_t launch_positions(int32_t *q_pos, int32_t *n_valid, int32_t L, hipStream_t s) {
  if (L <= 0) return hipSuccess;
  hipLaunchKernelGGL(positions_kernel, dim3((L + 255) / 256), dim3(256), 0, s, q_pos, n_valid, L);
  return hipGetLastError();
}

// Chunks per row for T rows of at most n_cap scores: enough workgroups for
// about one per CU, each chunk at least 16 k long (1: no split).  Measured on
// rows of 32768 (B = 64, k = 2048): chunks of 8192 or 16384 make the two
// launches slower than one workgroup per row (41 and 38 us against 28); on
// rows up to 131072 (B = 128), two chunks per row gain about 10%.
hipError_t launch_topk(const float *scores, int64_t ld, const int32_t *n_valid, int32_t n_cap, int32_t T,
                       int32_t k, int32_t *idx, hipStream_t s, void *ws, size_t ws_bytes) {
  if (T == 0) return hipSuccess;
  static bool attr_done = false;  // per process: the attribute holds for every device
  if (!attr_done) {
    for (const void *f : {(const void *)topk_rows_kernel, (const void *)topk_merge_kernel}) {
      hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kTopkSmem);
      if (e != hipSuccess) return e;
    }
    attr_done = true;
  }
  const int nch = ws ? topk_split_chunks(T, n_cap, k) : 1;
  if (nch > 1 && ws_bytes >= topk_workspace_bytes(T, n_cap, k)) {
    // chunk-wise selections, then one merge per row over their union
    const int chunk = (int)align_up((size_t)((n_cap + nch - 1) / nch), 4);
    int32_t *cpos = (int32_t *)ws;
    int32_t *ccnt = (int32_t *)((char *)ws + align_up((size_t)T * nch * k * 4, 256));
    hipLaunchKernelGGL(topk_rows_kernel, dim3((uint32_t)(T * nch)), dim3(kThreads), kTopkSmem, s, scores, ld, n_valid,
                       n_cap, nch, chunk, k, cpos, ccnt);
    hipLaunchKernelGGL(topk_merge_kernel, dim3(T), dim3(kThreads), kTopkSmem, s, scores, ld, cpos, ccnt, nch, chunk,
                       k, idx);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(topk_rows_kernel, dim3(T), dim3(kThreads), kTopkSmem, s, scores, ld, n_valid, n_cap, 1, n_cap,
                     k, idx, (int32_t *)nullptr);
  return hipGetLastError();
}
}  // namespace dsa
