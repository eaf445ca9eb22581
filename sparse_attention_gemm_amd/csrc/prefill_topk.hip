// Fused prefill indexer + per-query streaming top-k (one causal sequence,
// query t at position t).  The L x L score matrix is never written: scores
// are produced 64 keys at a time in registers and filtered on chip.
//
// Lightning indexer and fine-grained token selection: mizuki-eaf.pages.dev,
// "How it works" (index score of each query against its preceding tokens,
// then the top-k KV entries per query, k = 2048); m.digipub.cc, section 2.
//
// Workgroup = 4 wavefronts = 4 consecutive query tokens, one wave per token
// with all 64 indexer heads in registers (4 MFMA A tiles plus the tile of the
// weighted query sum), so every key block read from LDS feeds five MFMAs.
// Key tiles (64 keys x 128 B of E4M3 + 64 fp32 scales) are loaded straight
// into LDS (direct-to-LDS loads, double buffered, one barrier per tile) and
// shared by the four waves.
//
// Each wave owns its token's 4096-entry candidate buffer in the workspace
// (in L2/MALL; after the first few thousand keys a key enters it only
// rarely), holding (order key, position) pairs in ascending position order,
// plus a threshold tau:
//   * a key enters the buffer if its order key >= tau (keys arrive in
//     increasing position, so a new key that ties tau outranks it);
//   * when a buffer could overflow on the next tile, it is compacted in place
//     by histogram narrowing over the order keys.  The narrowing stops at the
//     first level whose bin holding the k-th key is small enough: every entry
//     at or above that bin's lower edge is kept and tau becomes the edge.
//     (Ties make the narrowing run down to single keys, where the cut is
//     exact.)  The key range is tracked while appending, so a compaction is
//     one histogram pass per level plus one compaction pass, each reading the
//     buffer 16 bytes per lane.
//   * the four tokens see the same keys, so their buffers fill at nearly the
//     same rate: when one wave must compact, every wave whose buffer is past
//     a watermark compacts at the same tile, and the workgroup stalls once
//     instead of once per wave.
// At the end the buffer is compacted exactly to min(k, t+1) entries (score
// desc, position desc) and written out in ascending position order.
//
// Workgroups are issued longest-first (the last query block first) so that
// the causal triangle drains evenly.
#include "dsa_common.h"
#include "dsa_launch.h"
#include "dsa_sizes.h"
#include "indexer_core.h"

namespace {

constexpr int kTok = 4;         // query tokens per workgroup
constexpr int kWaves = kTok;    // one per token
constexpr int kCap = dsa::kPrefillCap;  // candidate buffer entries per query
constexpr int kTile = 64;       // keys per tile
constexpr int kKRow = 160;      // LDS bytes per key row: 128 + 32 pad (40 dwords mod 64: conflict-free reads)
constexpr int kKSlots = kKRow / 16;
constexpr int kKeyInsts = kTile * kKSlots / 64;  // wave-wide 1 KB direct-to-LDS loads per tile
constexpr int kBins = 256;      // compaction histogram
static_assert(kBins * 4 >= kQueryScratch, "the histogram doubles as query scratch");
static_assert(kWaves == 4, "the overflow flags of the four waves are read together");
// An early cut may leave at most this many entries (k <= 2048), so that it
// frees at least a quarter of the buffer; otherwise the narrowing continues.
constexpr int kCutLimit = kCap - kCap / 4;

typedef __attribute__((address_space(3))) void lds_void;

struct PrefillShared {
  uint8_t keys[2][kTile * kKRow];
  float ksc[2][kTile];
  uint32_t hist[kTok][kBins];
  uint32_t full[2][kWaves];  // per tile parity: the wave's buffer could overflow on the next tile
};
// When any wave of the workgroup must compact, every wave whose buffer holds
// more than this compacts at the same tile: the four tokens see the same keys,
// so their buffers fill at nearly the same rate, and compactions that overlap
// cost the workgroup one stall instead of four.
constexpr int kSyncMark = kCap / 2 + kCap / 8;

constexpr int kVec = 4;    // consecutive buffer entries per lane and load (16 bytes)
constexpr int kBatch = 4;  // key loads in flight per lane in a histogram pass (1024 entries)
constexpr int kBatchC = 2; // key + position loads in flight per lane in the compaction pass

// Compact the candidate buffer bk/bp[0..n) (order keys, positions; ascending
// position order, which is preserved), all of whose keys lie in [lo, hi].
// All 64 lanes of the owning wave call this together; hist is its LDS
// histogram.  Returns the new threshold tau.
//   limit == 0 (exact): keep exactly the `keep` best entries under (key desc,
//     position desc); tau is the keep-th key.
//   limit > 0 (early cut): stop narrowing as soon as cutting at the lower edge
//     of the bin that holds the keep-th key leaves at most `limit` entries, and
//     keep every entry >= that edge (tau).  At least `keep` entries survive, all
//     >= tau, so everything dropped (< tau) is outranked by `keep` survivors.
// The buffer is read 16 bytes per lane (4 consecutive entries), 1024 entries
// per batch of loads; it holds kCap entries, so the last group of 4 never
// leaves it (entries past n are masked).
__device__ uint32_t compact_wave(uint32_t *__restrict__ bk, uint32_t *__restrict__ bp,
                                 uint32_t *__restrict__ hist, int &n, int keep, int limit, uint32_t lo,
                                 uint32_t hi, int lane) {
  static_assert(kCap % (64 * kVec) == 0, "whole groups of 4 entries");
  __threadfence_block();  // the wave's earlier appends (other lanes) are visible
  // lane-derived addresses are computed here, not kept live across the caller's loop
  asm volatile("" : "+v"(lane));
  uint32_t base = lo;
  const uint32_t span = hi - lo;
  int shift = span == 0 ? 0 : max(0, 32 - __clz(span) - 8);
  uint32_t remaining = (uint32_t)keep;
  uint32_t tau, ties = 0;
  bool exact_cut = false;
  uint32_t nbins = kBins;  // later levels: only as many bins as the window is wide
  while (true) {
#pragma unroll
    for (int b = lane; b < kBins; b += 64) hist[b] = 0;
    __builtin_amdgcn_wave_barrier();
    for (int b0 = 0; b0 < n; b0 += 64 * kVec * kBatch) {
      uint4 kk[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int i0 = b0 + (u * 64 + lane) * kVec;
        kk[u] = i0 < n ? *reinterpret_cast<const uint4 *>(bk + i0) : uint4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int i0 = b0 + (u * 64 + lane) * kVec;
        const uint32_t k4[4] = {kk[u].x, kk[u].y, kk[u].z, kk[u].w};
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
          const uint32_t d = (k4[j] - base) >> shift;
          if (i0 + j < n && k4[j] >= base && d < nbins) atomicAdd(&hist[d], 1u);
        }
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
    const uint32_t edge = base + (bstar << shift);
    if (limit > 0 && (uint32_t)keep - remaining + above + cnt <= (uint32_t)limit) {
      tau = edge;  // early cut at the bin's lower edge
      break;
    }
    remaining -= above;
    base = edge;
    if (shift == 0) {
      tau = base;
      ties = cnt;
      exact_cut = true;
      break;
    }
    const int nshift = max(0, shift - 8);
    nbins = 1u << (shift - nshift);
    shift = nshift;
  }
  // ordered in-place compaction: keep key > tau, and of the keys equal to tau
  // all (early cut) or the last `remaining` (exact cut).  A batch is loaded
  // whole before any of it is written, and entry i moves to dst <= i, below
  // every entry not yet read.
  const uint32_t tie_cut = exact_cut ? ties - remaining : 0u;
  uint32_t out = 0, tie_seen = 0;
  for (int b0 = 0; b0 < n; b0 += 64 * kVec * kBatchC) {
    uint4 kk[kBatchC], pp[kBatchC];
#pragma unroll
    for (int u = 0; u < kBatchC; ++u) {
      const int i0 = b0 + (u * 64 + lane) * kVec;
      kk[u] = i0 < n ? *reinterpret_cast<const uint4 *>(bk + i0) : uint4{0, 0, 0, 0};
      pp[u] = i0 < n ? *reinterpret_cast<const uint4 *>(bp + i0) : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kBatchC; ++u) {
      if (b0 + u * 64 * kVec >= n) break;  // uniform
      const int i0 = b0 + (u * 64 + lane) * kVec;
      const uint32_t k4[4] = {kk[u].x, kk[u].y, kk[u].z, kk[u].w};
      const uint32_t p4[4] = {pp[u].x, pp[u].y, pp[u].z, pp[u].w};
      // entry (lane l, j) is entry 4l + j of the group: the entries of lower
      // lanes come first, then the lane's own lower j
      bool kp[4];
      if (exact_cut) {
        uint64_t tm[4];
        uint32_t rank = tie_seen;
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
          tm[j] = __ballot(i0 + j < n && k4[j] == tau);
          rank += (uint32_t)lanes_below(tm[j]);
          tie_seen += (uint32_t)__popcll(tm[j]);
        }
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
          const bool tie = (tm[j] >> lane) & 1u;
          kp[j] = i0 + j < n && (k4[j] > tau || (tie && rank >= tie_cut));
          rank += tie ? 1u : 0u;
        }
      } else {
#pragma unroll
        for (int j = 0; j < kVec; ++j) kp[j] = i0 + j < n && k4[j] >= tau;
      }
      uint32_t dst = out;
#pragma unroll
      for (int j = 0; j < kVec; ++j) {
        const uint64_t km = __ballot(kp[j]);
        dst += (uint32_t)lanes_below(km);
        out += (uint32_t)__popcll(km);
      }
#pragma unroll
      for (int j = 0; j < kVec; ++j)
        if (kp[j]) {
          bk[dst] = k4[j];
          bp[dst] = p4[j];
          ++dst;
        }
    }
  }
  __threadfence_block();  // the moved entries are visible to every lane
  n = (int)out;
  return tau;
}

// Issue the direct-to-LDS loads of key tile `tile` into dkeys/dks.
// Instruction i writes slots [64i, 64i+64); slot s holds row s/10, 16-byte
// chunk s%10 (chunks 8, 9 are padding and reload chunk 7).  Addresses are a
// uniform tile base plus a 32-bit lane offset.  In the sequence's last tile,
// keys past L-1 read key L-1 (never selected: they are beyond every query).
__device__ __forceinline__ void load_tile_async(uint8_t *dkeys, float *dks, const uint8_t *__restrict__ k8,
                                                const float *__restrict__ ks, int L, int tile, int wave, int lane) {
  const uint8_t *kbase = k8 + (int64_t)tile * kTile * 128;
  const int nrow = L - tile * kTile;  // rows of this tile inside the sequence
#pragma unroll
  for (int i = wave; i < kKeyInsts; i += kWaves) {
    const int slot = i * 64 + lane;
    const int r = slot / kKSlots;
    const uint32_t off_full = (uint32_t)(r * 128 + min(slot - r * kKSlots, 7) * 16);
    uint32_t off = off_full;
    if (nrow < kTile) {  // uniform: the sequence's last tile; recompute from a fresh lane id
      int l = lane;
      asm volatile("" : "+v"(l));
      const int s2 = i * 64 + l, r2 = s2 / kKSlots;
      off = (uint32_t)(min(r2, nrow - 1) * 128 + min(s2 - r2 * kKSlots, 7) * 16);
    }
    __builtin_amdgcn_global_load_lds(kbase + off, (lds_void *)(dkeys + i * 1024), 16, 0, 0);
  }
  if (wave == kWaves - 1) {
    const float *sbase = ks + (int64_t)tile * kTile;
    __builtin_amdgcn_global_load_lds(sbase + min(lane, nrow - 1), (lds_void *)dks, 4, 0, 0);
  }
}

// Score tile `it` from (ckeys, cks) for one token and prefetch tile it+1
// into (nkeys, nks).  The current tile's LDS reads are issued before the
// prefetch: the compiler cannot tell the direct-to-LDS writes from them and
// would otherwise wait for the prefetch before reading LDS.
// Score tile `it` from (ckeys, cks) for one token and prefetch tile it+1
// into (nkeys, nks).  Every LDS read of the tile is issued before the
// prefetch (the last key block's operand right before it): the compiler
// cannot tell the direct-to-LDS writes from them and would otherwise wait for
// the prefetch before reading LDS.
__device__ __forceinline__ float score_and_prefetch(uint8_t *nkeys, float *nks, const uint8_t *ckeys, const float *cks,
                                                    bool prefetch, bool need, const IdxQuery<4> &Q,
                                                    const uint8_t *__restrict__ k8, const float *__restrict__ ks,
                                                    int L, int next, int wave, int lane) {
  const int g = lane >> 4, c = lane & 15;
  const float ksv = cks[lane];
  auto issue_prefetch = [&] {
    if (prefetch) load_tile_async(nkeys, nks, k8, ks, L, next, wave, lane);
  };
  if (!need) {
    issue_prefetch();
    return 0.0f;
  }
  auto get_b = [&](int u) { return *reinterpret_cast<const i32x8 *>(ckeys + (16 * u + c) * kKRow + 32 * g); };
  return canon_zero(idx_score64<4>(Q, get_b, issue_prefetch) * ksv);
}

__global__ __launch_bounds__(kWaves * 64, 3) void prefill_indexer_topk_kernel(
    const uint8_t *__restrict__ q8, const float *__restrict__ qs, const uint8_t *__restrict__ k8,
    const float *__restrict__ ks, const float *__restrict__ w, int32_t L, int32_t k,
    int32_t *__restrict__ idx, uint32_t *__restrict__ cand) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  PrefillShared &sm = *reinterpret_cast<PrefillShared *>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps per-wave values in SGPRs
  const int grp = gridDim.x - 1 - blockIdx.x;  // longest rows first
  const int t0 = grp * kTok;
  const int t = t0 + wave;
  const bool active = t < L;
  const int tq = min(t, L - 1);
  const int last = min(t0 + kTok - 1, L - 1);
  const int ntiles = last / kTile + 1;

  // the query's 64 heads (and the pieces of its weighted sum); the LDS of its
  // compaction histogram serves as scratch until the first compaction
  IdxQuery<4> Q;
  idx_load_query<4>(Q, q8 + (int64_t)tq * 64 * 128, w + (int64_t)tq * 64, qs[tq], lane,
                    reinterpret_cast<uint8_t *>(sm.hist[wave]));

  uint32_t *bk = cand + (int64_t)tq * 2 * kCap;  // order keys
  uint32_t *bp = bk + kCap;                        // positions
  uint32_t *hist = sm.hist[wave];
  int nbuf = 0;
  uint32_t thr = 0u;
  uint32_t klo = 0xFFFFFFFFu, khi = 0u;  // bounds of the keys this lane appended since the last cut

  load_tile_async(sm.keys[0], sm.ksc[0], k8, ks, L, 0, wave, lane);
  bool appended = false;  // the previous tile's two append stores follow its prefetch
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    // this wave's loads of tile `it` have landed in LDS; the previous tile's
    // appends, issued after them, may still be in flight (loads and stores
    // complete in issue order)
    if (appended)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();  // ... and every wave's; tile it-1's buffer is free
    if (it > 0) {
      const int par = (it - 1) & 1;
      const uint32_t any = __builtin_amdgcn_readfirstlane(sm.full[par][0] | sm.full[par][1] | sm.full[par][2] |
                                                          sm.full[par][3]);
      if (any != 0u && nbuf > kSyncMark) {
        thr = compact_wave(bk, bp, hist, nbuf, k, kCutLimit, wave_min_u32(klo), wave_max_u32(khi), lane);
        klo = thr;  // every survivor is >= tau
      }
    }
    const bool need = active && it * kTile <= t;
    appended = false;
    const float v = score_and_prefetch(sm.keys[buf ^ 1], sm.ksc[buf ^ 1], sm.keys[buf], sm.ksc[buf], it + 1 < ntiles,
                                       need, Q, k8, ks, L, it + 1, wave, lane);
    if (need) {
      // score of key it*64 + lane; the buffer has room for the whole tile
      const int s = it * kTile + lane;
      const uint32_t key = score_key(v);
      const bool pass = s <= t && key >= thr;
      const uint64_t mask = __ballot(pass);
      if (pass) {
        klo = min(klo, key);
        khi = max(khi, key);
        const int dst = nbuf + lanes_below(mask);
        bk[dst] = key;
        bp[dst] = (uint32_t)s;
      }
      nbuf += __popcll(mask);
      appended = mask != 0;  // uniform
    }
    if (lane == 0) sm.full[it & 1][wave] = nbuf > kCap - kTile ? 1u : 0u;
  }

  if (!active) return;
  __threadfence_block();
  if (nbuf > k) compact_wave(bk, bp, hist, nbuf, k, 0, wave_min_u32(klo), wave_max_u32(khi), lane);
  int32_t *orow = idx + (int64_t)t * k;
  for (int i = lane; i < k; i += 64) orow[i] = i < nbuf ? (int32_t)bp[i] : -1;
}

}  // namespace

namespace dsa {

hipError_t launch_prefill_indexer_topk(const uint8_t *q8, const float *qs, const uint8_t *k8,
                                       const float *ks, const float *w, int32_t L, int32_t k,
                                       int32_t *idx, uint32_t *cand, hipStream_t s) {
  if (L == 0) return hipSuccess;
  static bool attr_done = false;
  const size_t smem = sizeof(PrefillShared);
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void *)prefill_indexer_topk_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int groups = (L + kTok - 1) / kTok;
  hipLaunchKernelGGL(prefill_indexer_topk_kernel, dim3(groups), dim3(kWaves * 64), smem, s, q8, qs, k8, ks, w,
                     L, k, idx, cand);
  return hipGetLastError();
}
}  // namespace dsa
