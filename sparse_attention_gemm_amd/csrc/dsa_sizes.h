// dsa_sizes.h -- the constants that fix workspace sizes, shared by the
// kernels that use the space and by the host code that sizes it.  Host and
// device; no HIP device headers.
#pragma once

namespace dsa {
constexpr int kTopkMaxChunks = 8;    // row top-k: most column chunks per row of a split selection
constexpr int kPrefillCap = 4096;    // fused prefill top-k: candidate buffer entries per query
constexpr int kMhaUpT = 256;         // masked MHA: tokens per up-projection workgroup (K_h, V_h row padding)
constexpr int kMhaDn = 128;          // masked MHA: per-head up-projected key (and value) dims
constexpr int kMhaQB = 128;          // masked MHA: queries per attention workgroup
}  // namespace dsa
