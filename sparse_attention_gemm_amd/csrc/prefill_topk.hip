// Fused prefill indexer + per-query streaming top-k (one causal sequence,
// query t at position t).  The L x L score matrix is never written: scores
// are produced 64 keys at a time in registers and filtered on chip.
//
// Lightning indexer and fine-grained token selection: mizuki-eaf.pages.dev,
// "How it works" (index score of each query against its preceding tokens,
// then the top-k KV entries per query, k = 2048); m.digipub.cc, section 2.
//
// Workgroup = 8 wavefronts = 4 consecutive query tokens; each token's 64
// indexer heads are split over a pair of waves (heads 0..31 and 32..63), so
// one wave's ReLU/weight epilogue (VALU) overlaps the other's MFMAs on the
// same SIMD.  Key tiles (64 keys x 128 B of E4M3 + 64 fp32 scales) are
// loaded straight into LDS (direct-to-LDS loads, double buffered, one
// barrier per tile) and shared by all eight waves.  The first wave of a pair
// publishes its half-score of each key in LDS; one tile later the second
// wave adds it to its own half and runs the selection.
//
// The second wave of each pair owns the token's 4096-entry candidate buffer
// (in the workspace: it stays in L2/MALL, and after the first few thousand
// keys a key enters it only rarely; keeping it out of LDS lets two
// workgroups share a CU) holding (order key, position) pairs in ascending
// position order, plus a threshold tau:
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

constexpr int kTok = 4;         // query tokens per workgroup
constexpr int kWaves = 8;       // two per token
constexpr int kCap = 4096;      // candidate buffer entries per query
constexpr int kTile = 64;       // keys per tile
constexpr int kKRow = 160;      // LDS bytes per key row: 128 + 32 pad (40 dwords mod 64: conflict-free reads)
constexpr int kKSlots = kKRow / 16;
constexpr int kKeyInsts = kTile * kKSlots / 64;  // wave-wide 1 KB direct-to-LDS loads per tile
constexpr int kBins = 256;      // compaction histogram

typedef __attribute__((address_space(3))) void lds_void;

struct PrefillShared {
  uint8_t keys[2][kTile * kKRow];
  float ksc[2][kTile];
  float part[2][kTok][kTile];   // half-scores (heads 0..31) of the current and previous tile
  uint32_t hist[kTok][kBins];
};

// Compact buf[0..n) to its `keep` best entries (order key desc, position desc),
// preserving ascending position order.  Returns the new threshold (k-th key).
// All 64 lanes of the owning wave call this together; bk/bp are the wave's
// own candidate buffer (global memory), hist its LDS histogram.
__device__ uint32_t compact_wave(uint32_t *__restrict__ bk, uint32_t *__restrict__ bp,
                                 uint32_t *__restrict__ hist, int &n, int keep, int lane) {
  __threadfence_block();  // the wave's earlier appends (other lanes) are visible
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
  __threadfence_block();  // the moved entries are visible to every lane
  n = (int)out;
  return tau;
}

// Issue the direct-to-LDS loads of key tile `tile` into buffer `buf`.
// Instruction i writes slots [64i, 64i+64); slot s holds row s/10, 16-byte
// chunk s%10 (chunks 8, 9 are padding and reload chunk 7).  Keys past L-1
// read key L-1 (never selected: they are beyond every query of the sequence).
__device__ __forceinline__ void load_tile_async(PrefillShared &sm, int buf, const uint8_t *__restrict__ k8,
                                                const float *__restrict__ ks, int L, int tile, int wave, int lane) {
#pragma unroll
  for (int i = wave; i < kKeyInsts; i += kWaves) {
    const int slot = i * 64 + lane;
    const int r = slot / kKSlots;
    const int j = min(slot - r * kKSlots, 7);
    const int key = min(tile * kTile + r, L - 1);
    __builtin_amdgcn_global_load_lds(k8 + (int64_t)key * 128 + j * 16, (lds_void *)(sm.keys[buf] + i * 1024), 16, 0,
                                     0);
  }
  if (wave == kWaves - 1) {
    const int key = min(tile * kTile + lane, L - 1);
    __builtin_amdgcn_global_load_lds(ks + key, (lds_void *)sm.ksc[buf], 4, 0, 0);
  }
}

__global__ __launch_bounds__(kWaves * 64, 2) void prefill_indexer_topk_kernel(
    const uint8_t *__restrict__ q8, const float *__restrict__ qs, const uint8_t *__restrict__ k8,
    const float *__restrict__ ks, const float *__restrict__ w, int32_t L, int32_t k,
    int32_t *__restrict__ idx, uint32_t *__restrict__ cand) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  PrefillShared &sm = *reinterpret_cast<PrefillShared *>(smem_raw);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int tok = wave >> 1, half = wave & 1;
  const int grp = gridDim.x - 1 - blockIdx.x;  // longest rows first
  const int t0 = grp * kTok;
  const int t = t0 + tok;
  const bool active = t < L;
  const int tq = min(t, L - 1);
  const int last = min(t0 + kTok - 1, L - 1);
  const int ntiles = last / kTile + 1;

  IdxHalf Q;
  idx_load_half(Q, q8 + (int64_t)tq * 64 * 128, w + (int64_t)tq * 64, qs[tq], 32 * half, lane);

  uint32_t *bk = cand + (int64_t)tq * 2 * kCap;  // order keys
  uint32_t *bp = bk + kCap;                        // positions
  uint32_t *hist = sm.hist[tok];
  int nbuf = 0;
  uint32_t thr = 0u;
  float prev = 0.0f, prev_ks = 0.0f;  // second wave: its half-score and the key scale of the last tile

  load_tile_async(sm, 0, k8, ks, L, 0, wave, lane);
  for (int it = 0; it <= ntiles; ++it) {
    const int buf = it & 1;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of tile `it` have landed in LDS
    __syncthreads();                // ... and every wave's; tile it-1's buffer is free
    if (half == 1 && active && it > 0) {
      // score of key (it-1)*64 + lane = half(0..31) + half(32..63), times its scale
      const int s = (it - 1) * kTile + lane;
      const float v = canon_zero((sm.part[buf ^ 1][tok][lane] + prev) * prev_ks);
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
    if (it == ntiles) break;
    if (it + 1 < ntiles) load_tile_async(sm, buf ^ 1, k8, ks, L, it + 1, wave, lane);
    if (active) {
      i32x8 b[4];
      idx_load_keys(b, sm.keys[buf], kKRow, lane);
      const float part = idx_half_score64(Q, b);
      if (half == 0) {
        sm.part[buf][tok][lane] = part;
      } else {
        prev = part;
        prev_ks = sm.ksc[buf][lane];
      }
    }
  }

  if (!active || half == 0) return;
  __threadfence_block();
  if (nbuf > k) compact_wave(bk, bp, hist, nbuf, k, lane);
  int32_t *orow = idx + (int64_t)t * k;
  for (int i = lane; i < k; i += 64) orow[i] = i < nbuf ? (int32_t)bp[i] : -1;
}

}  // namespace

namespace dsa {
size_t prefill_candidate_bytes(int32_t L) { return (size_t)L * 2 * kCap * sizeof(uint32_t); }

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
