// Fused prefill indexer + per-query streaming top-k (one causal sequence,
// query t at position t).  The L x L score matrix is never written: scores
// are produced 64 keys at a time in registers and filtered on chip.
//
// Lightning indexer and fine-grained token selection: mizuki-eaf.pages.dev,
// "How it works" (index score of each query against its preceding tokens,
// then the top-k KV entries per query, k = 2048); m.digipub.cc, section 2.
//
// Workgroup = 4 wavefronts = 4 consecutive query tokens, one per wave.  Key
// tiles (64 keys x 128 B of E4M3 + 64 fp32 scales) are staged in LDS once
// and shared by the four waves (double buffered, one barrier per tile).
// Each wave owns a 4096-entry candidate buffer in LDS holding (order key,
// position) pairs in ascending position order, plus a threshold tau:
//   * a key enters the buffer if its order key >= tau (keys arrive in
//     increasing position, so a new key that ties tau outranks it);
//   * when the buffer would overflow, it is compacted in place to exactly
//     the k best entries under (score desc, position desc) by histogram
//     narrowing, and tau becomes the k-th key.
// At the end the buffer is compacted to min(k, t+1) entries and written out
// in ascending position order (deterministic).
//
// Workgroups are issued longest-first (the last query block first) so that
// the causal triangle drains evenly.
#include "indexer_core.h"

namespace {

constexpr int kWaves = 4;
constexpr int kCap = 4096;      // candidate buffer entries per query
constexpr int kTile = 64;       // keys per tile
constexpr int kRowB = 144;      // LDS bytes per key row (128 + 16 pad: spreads banks)
constexpr int kBins = 256;      // compaction histogram

struct PrefillShared {
  uint8_t keys[2][kTile * kRowB];
  float ksc[2][kTile];
  uint32_t bkey[kWaves][kCap];
  uint32_t bpos[kWaves][kCap];
  uint32_t hist[kWaves][kBins];
};

// Compact buf[0..n) to its `keep` best entries (order key desc, position desc),
// preserving ascending position order.  Returns the new threshold (k-th key).
// All 64 lanes of the owning wave call this together.
__device__ uint32_t compact_wave(uint32_t *__restrict__ bk, uint32_t *__restrict__ bp,
                                 uint32_t *__restrict__ hist, int &n, int keep, int lane) {
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int i = lane; i < n; i += 64) {
    const uint32_t key = bk[i];
    mn = key < mn ? key : mn;
    mx = key > mx ? key : mx;
  }
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  uint32_t base = mn;
  const uint32_t span = mx - mn;
  int shift = span == 0 ? 0 : max(0, 32 - __clz(span) - 8);
  uint32_t remaining = (uint32_t)keep;
  uint32_t tau, ties;
  uint32_t nbins = kBins;  // later levels: only as many bins as the window is wide
  while (true) {
#pragma unroll
    for (int b = lane; b < kBins; b += 64) hist[b] = 0;
    __builtin_amdgcn_wave_barrier();
    for (int i = lane; i < n; i += 64) {
      const uint32_t key = bk[i];
      if (key >= base) {
        const uint32_t d = (key - base) >> shift;
        if (d < nbins) atomicAdd(&hist[d], 1u);
      }
    }
    __builtin_amdgcn_wave_barrier();
    // lane owns bins 4*lane .. 4*lane+3
    const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2],
                   h3 = hist[4 * lane + 3];
    const uint32_t mine = h0 + h1 + h2 + h3;
    uint32_t suf = mine;  // sum over lanes >= lane
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t t = __shfl_down(suf, o);
      if (lane + o < 64) suf += t;
    }
    const uint32_t s4 = suf - mine;  // bins > 4*lane+3
    const uint32_t s3 = s4 + h3, s2 = s3 + h2, s1 = s2 + h1, s0 = s1 + h0;
    int bsel = -1;
    uint32_t babove = 0, bcnt = 0;
    if (s3 >= remaining && s4 < remaining) { bsel = 4 * lane + 3; babove = s4; bcnt = h3; }
    else if (s2 >= remaining && s3 < remaining) { bsel = 4 * lane + 2; babove = s3; bcnt = h2; }
    else if (s1 >= remaining && s2 < remaining) { bsel = 4 * lane + 1; babove = s2; bcnt = h1; }
    else if (s0 >= remaining && s1 < remaining) { bsel = 4 * lane; babove = s1; bcnt = h0; }
    const uint64_t who = __ballot(bsel >= 0);
    const int src = __ffsll((unsigned long long)who) - 1;
    const uint32_t bstar = __shfl((uint32_t)bsel, src);
    const uint32_t above = __shfl(babove, src);
    const uint32_t cnt = __shfl(bcnt, src);
    __builtin_amdgcn_wave_barrier();
    remaining -= above;
    base += bstar << shift;
    if (shift == 0) {
      tau = base;
      ties = cnt;
      break;
    }
    const int nshift = max(0, shift - 8);
    nbins = 1u << (shift - nshift);
    shift = nshift;
  }
  // ordered in-place compaction: keep key > tau and the last `remaining` ties
  const uint32_t tie_cut = ties - remaining;
  uint32_t out = 0, tie_seen = 0;
  for (int b0 = 0; b0 < n; b0 += 64) {
    const int i = b0 + lane;
    const bool in = i < n;
    const uint32_t key = in ? bk[i] : 0u;
    const uint32_t pos = in ? bp[i] : 0u;
    const bool tie = in && key == tau;
    const uint64_t tmask = __ballot(tie);
    const uint32_t my_tie = tie_seen + (uint32_t)lanes_below(tmask);
    const bool kp = in && (key > tau || (tie && my_tie >= tie_cut));
    const uint64_t kmask = __ballot(kp);
    if (kp) {
      const uint32_t dst = out + (uint32_t)lanes_below(kmask);
      bk[dst] = key;
      bp[dst] = pos;
    }
    out += (uint32_t)__popcll(kmask);
    tie_seen += (uint32_t)__popcll(tmask);
    __builtin_amdgcn_wave_barrier();
  }
  n = (int)out;
  return tau;
}

__device__ __forceinline__ void load_tile_regs(const uint8_t *__restrict__ k8, const float *__restrict__ ks,
                                               int L, int tile, int tid, i32x4 &r0, i32x4 &r1, float &sv) {
  // thread tid: key tid/4 of the tile, bytes (tid%4)*32 .. +32
  const int key = min(tile * kTile + (tid >> 2), L - 1);
  const uint8_t *src = k8 + (int64_t)key * 128 + (tid & 3) * 32;
  r0 = *reinterpret_cast<const i32x4 *>(src);
  r1 = *reinterpret_cast<const i32x4 *>(src + 16);
  sv = (tid < kTile) ? ks[min(tile * kTile + tid, L - 1)] : 0.0f;
}

__device__ __forceinline__ void store_tile_lds(PrefillShared &sm, int buf, int tid, const i32x4 &r0,
                                               const i32x4 &r1, float sv) {
  uint8_t *dst = sm.keys[buf] + (tid >> 2) * kRowB + (tid & 3) * 32;
  *reinterpret_cast<i32x4 *>(dst) = r0;
  *reinterpret_cast<i32x4 *>(dst + 16) = r1;
  if (tid < kTile) sm.ksc[buf][tid] = sv;
}

__global__ __launch_bounds__(256, 1) void prefill_indexer_topk_kernel(
    const uint8_t *__restrict__ q8, const float *__restrict__ qs, const uint8_t *__restrict__ k8,
    const float *__restrict__ ks, const float *__restrict__ w, int32_t L, int32_t k,
    int32_t *__restrict__ idx) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  PrefillShared &sm = *reinterpret_cast<PrefillShared *>(smem_raw);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = gridDim.x - 1 - blockIdx.x;  // longest rows first
  const int t0 = g * kWaves;
  const int t = t0 + wave;
  const bool active = t < L;
  const int tq = min(t, L - 1);
  const int last = min(t0 + kWaves - 1, L - 1);
  const int ntiles = last / kTile + 1;

  IdxQuery<2> Q;
  idx_load_query<2>(Q, q8 + (int64_t)tq * 64 * 128, w + (int64_t)tq * 64, qs[tq], lane);

  uint32_t *bk = sm.bkey[wave];
  uint32_t *bp = sm.bpos[wave];
  uint32_t *hist = sm.hist[wave];
  int nbuf = 0;
  uint32_t thr = 0u;

  i32x4 r0, r1;
  float sv;
  load_tile_regs(k8, ks, L, 0, tid, r0, r1, sv);
  store_tile_lds(sm, 0, tid, r0, r1, sv);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    if (it + 1 < ntiles) load_tile_regs(k8, ks, L, it + 1, tid, r0, r1, sv);
    const int s0 = it * kTile;
    if (active && s0 <= t) {
      i32x8 b[2][2];
      const uint8_t *kt = sm.keys[buf];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          b[u][kk] = *reinterpret_cast<const i32x8 *>(kt + (u * 32 + (lane & 31)) * kRowB + kk * 64 +
                                                       (lane >> 5) * 32);
      const float tot = idx_score64<2>(Q, b);
      const int s = s0 + lane;
      const float v = canon_zero(tot * sm.ksc[buf][lane]);
      const uint32_t key = score_key(v);
      const bool valid = s <= t;
      bool pass = valid && key >= thr;
      uint64_t mask = __ballot(pass);
      int cnt = __popcll(mask);
      if (nbuf + cnt > kCap) {
        thr = compact_wave(bk, bp, hist, nbuf, k, lane);
        pass = valid && key >= thr;
        mask = __ballot(pass);
        cnt = __popcll(mask);
      }
      if (pass) {
        const int dst = nbuf + lanes_below(mask);
        bk[dst] = key;
        bp[dst] = (uint32_t)s;
      }
      nbuf += cnt;
    }
    if (it + 1 < ntiles) store_tile_lds(sm, buf ^ 1, tid, r0, r1, sv);
    __syncthreads();
  }

  if (!active) return;
  __builtin_amdgcn_wave_barrier();
  if (nbuf > k) compact_wave(bk, bp, hist, nbuf, k, lane);
  int32_t *orow = idx + (int64_t)t * k;
  for (int i = lane; i < k; i += 64) orow[i] = i < nbuf ? (int32_t)bp[i] : -1;
}

}  // namespace

namespace dsa {
hipError_t launch_prefill_indexer_topk(const uint8_t *q8, const float *qs, const uint8_t *k8,
                                       const float *ks, const float *w, int32_t L, int32_t k,
                                       int32_t *idx, hipStream_t s) {
  if (L == 0) return hipSuccess;
  static bool attr_done = false;
  const size_t smem = sizeof(PrefillShared);
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void *)prefill_indexer_topk_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int groups = (L + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(prefill_indexer_topk_kernel, dim3(groups), dim3(256), smem, s, q8, qs, k8, ks, w, L,
                     k, idx);
  return hipGetLastError();
}
}  // namespace dsa
