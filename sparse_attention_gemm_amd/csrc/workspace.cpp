// workspace.cpp -- host-side sizes of the scratch space the kernels need.
// Plain C++ on the HIP runtime API: the C ABI layer sizes and carves
// workspaces with these, and the same code runs in the host sanitizer build.
#include <algorithm>

#include "dsa_launch.h"
#include "dsa_sizes.h"

namespace dsa {

// Column chunks per row for a split row top-k: enough chunks to give every CU
// a chunk when the batch is short, each at least 16 k scores long.
int topk_split_chunks(int64_t T, int32_t n_cap, int32_t k) {
  static int n_cu = 0;
  if (n_cu == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) ==
                                                 hipSuccess && v > 0)
      n_cu = v;
    else
      return 1;
  }
  if (T <= 0 || n_cap <= 0 || k <= 0) return 1;
  int nch = (int)std::min<int64_t>(kTopkMaxChunks, n_cu / T);
  while (nch > 1 && (n_cap + nch - 1) / nch < 16 * k) --nch;
  return std::max(nch, 1);
}

// Split top-k: each chunk's k winners [T, chunks, k] int32, then their counts [T, chunks].
size_t topk_workspace_bytes(int64_t T, int32_t n_cap, int32_t k) {
  const int nch = topk_split_chunks(T, n_cap, k);
  if (nch <= 1) return 0;
  return align_up((size_t)T * nch * k * 4, 256) + align_up((size_t)T * nch * 4, 256);
}

// Fused prefill top-k: one candidate buffer of (order key, position) pairs per query.
size_t prefill_candidate_bytes(int32_t L) { return (size_t)L * 2 * kPrefillCap * sizeof(uint32_t); }

// Masked MHA: K_h and V_h [Lp, H, 128] fp16 with Lp = L rounded up to whole
// up-projection blocks, then the bit mask [L, ceil(L/32)] u32.
size_t masked_mha_kv_bytes(int32_t L, int32_t H) {
  const size_t Lp = (size_t)(L + kMhaUpT - 1) / kMhaUpT * kMhaUpT;
  return align_up(Lp * H * kMhaDn * 2, 256);
}
size_t masked_mha_workspace_bytes(int32_t L, int32_t H) {
  return 2 * masked_mha_kv_bytes(L, H) + align_up((size_t)L * ((L + 31) / 32) * 4, 256);
}

}  // namespace dsa
