// Row-wise top-k selection over a score matrix (fine-grained token selection:
// mizuki-eaf.pages.dev, "How it works"; m.digipub.cc, section 2).
//
// One 1024-thread workgroup per row.  Scores are mapped to order-preserving
// u32 keys.  The k-th largest key tau is found exactly by histogram
// narrowing: a 2048-bin histogram over the row's [min, max] key range, then
// repeatedly over the bin that holds the k-th element, 11 bits at a time,
// until a bin is one key wide.  Spreading the first histogram over the
// observed range keeps LDS atomic conflicts low even when all scores share
// sign and exponent.  The output pass keeps key > tau, plus the most recent
// (largest-position) ties at tau, and writes positions in ascending order
// through an ordered block scan, so results are deterministic.
//
// The row is re-read from L2 on every pass; HBM sees it once.
#include "dsa_common.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;

struct TopkShared {
  uint32_t hist[kBins];
  uint32_t wred[2][kWaves];
  uint32_t bstar, above, tie_cnt;
};

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

__global__ __launch_bounds__(kThreads) void topk_rows_kernel(const float *__restrict__ scores, int64_t ld,
                                                             const int32_t *__restrict__ n_valid, int32_t n_cap,
                                                             int32_t k, int32_t *__restrict__ idx) {
  __shared__ TopkShared sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int n = max(0, min(n_valid[row], n_cap));
  const float *sc = scores + row * ld;
  int32_t *out = idx + row * (int64_t)k;
  if (n <= k) {
    for (int i = tid; i < k; i += kThreads) out[i] = i < n ? i : -1;
    return;
  }
  // ---- pass 0: key range
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int i = tid; i < n; i += kThreads) {
    const uint32_t key = row_key(sc, i);
    kmin = key < kmin ? key : kmin;
    kmax = key > kmax ? key : kmax;
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (lane == 0) {
    sm.wred[0][wave] = kmin;
    sm.wred[1][wave] = kmax;
  }
  __syncthreads();
  kmin = 0xFFFFFFFFu;
  kmax = 0u;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    kmin = sm.wred[0][w] < kmin ? sm.wred[0][w] : kmin;
    kmax = sm.wred[1][w] > kmax ? sm.wred[1][w] : kmax;
  }
  __syncthreads();
  // ---- narrowing passes
  uint32_t base = kmin;
  const uint32_t span = kmax - kmin;
  int shift = span == 0 ? 0 : max(0, 32 - __clz(span) - 11);
  uint32_t remaining = (uint32_t)k;
  uint32_t tau = 0, ties = 0;
  // bins in use at this level: the whole digit at level 0 (the window is the
  // key range), afterwards only as many as the previous bin was wide
  uint32_t nbins = kBins;
  while (true) {
    for (int b = tid; b < kBins; b += kThreads) sm.hist[b] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) {
      const uint32_t key = row_key(sc, i);
      if (key >= base) {
        const uint32_t d = (key - base) >> shift;
        if (d < nbins) atomicAdd(&sm.hist[d], 1u);
      }
    }
    __syncthreads();
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
      sm.tie_cnt = h1;
    } else if (s0 >= remaining && s1 < remaining) {
      sm.bstar = 2 * tid;
      sm.above = s1;
      sm.tie_cnt = h0;
    }
    __syncthreads();
    const uint32_t bstar = sm.bstar, above = sm.above, bcnt = sm.tie_cnt;
    __syncthreads();
    remaining -= above;
    base += bstar << shift;
    if (shift == 0) {
      tau = base;
      ties = bcnt;
      break;
    }
    const int nshift = max(0, shift - 11);
    nbins = 1u << (shift - nshift);
    shift = nshift;
  }
  // ---- output pass: contiguous position chunks per thread, ordered scan
  const int chunk = (n + kThreads - 1) / kThreads;
  const int pbeg = min(n, tid * chunk), pend = min(n, pbeg + chunk);
  uint32_t cnt_gt = 0, cnt_eq = 0;
  for (int i = pbeg; i < pend; ++i) {
    const uint32_t key = row_key(sc, i);
    cnt_gt += key > tau;
    cnt_eq += key == tau;
  }
  uint32_t tot_gt, tot_eq;
  const uint32_t off_gt = block_excl_scan(cnt_gt, sm.wred[0], tot_gt);
  const uint32_t off_eq = block_excl_scan(cnt_eq, sm.wred[1], tot_eq);
  (void)ties;
  const uint32_t need = remaining;            // ties to keep, the most recent ones
  const uint32_t tie_cut = tot_eq - need;     // tie rank (ascending position) >= tie_cut is kept
  // kept before my chunk: all gt before + ties before that are kept
  uint32_t tie_rank = off_eq;
  uint32_t dst = off_gt + (off_eq > tie_cut ? off_eq - tie_cut : 0);
  for (int i = pbeg; i < pend; ++i) {
    const uint32_t key = row_key(sc, i);
    bool keep = key > tau;
    if (key == tau) {
      keep = tie_rank >= tie_cut;
      ++tie_rank;
    }
    if (keep) out[dst++] = i;
  }
  // k entries are always written (n > k here)
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

hipError_t launch_topk(const float *scores, int64_t ld, const int32_t *n_valid, int32_t n_cap, int32_t T,
                       int32_t k, int32_t *idx, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_rows_kernel, dim3(T), dim3(kThreads), 0, s, scores, ld, n_valid, n_cap, k, idx);
  return hipGetLastError();
}
}  // namespace dsa
