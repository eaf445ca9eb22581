// capi.cpp -- the C ABI of libdsa: argument validation, workspace layout and
// dispatch to the gfx950 kernels.  Validation happens before any HIP call;
// nothing is enqueued on failure.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "dsa_launch.h"

namespace dsa {
static thread_local char g_err[512];

dsa_status fail(dsa_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

dsa_status hip_check(hipError_t e, const char *what) {
  if (e == hipSuccess) return DSA_OK;
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

hipError_t launch_positions(int32_t *q_pos, int32_t *n_valid, int32_t L, hipStream_t s);

// Workgroups of the bf16 sparse-MLA kernel without splitting, and the split
// count that brings a small batch up to about one workgroup per CU.
// heads per workgroup of the bf16 kernel (16 per wave)
static int mla_heads_per_wg(int H) { return H % 128 == 0 ? 128 : H % 64 == 0 ? 64 : H % 32 == 0 ? 32 : 16; }
static int mla_splits(int64_t T, int H, int k) {
  const int hpw = mla_heads_per_wg(H);
  const int64_t base = T * ((H + hpw - 1) / hpw);
  const int ntiles = (k + 31) / 32;
  if (base <= 0 || base >= 256) return 1;
  int s = (int)((256 + base - 1) / base);
  if (s > ntiles) s = ntiles;
  if (s > 32) s = 32;
  return s < 1 ? 1 : s;
}
// Split workspace: bf16 partial outputs [T][splits][H][512] (each normalised
// by its own softmax sum), then fp32 (reference, sum) pairs [T][splits][H][2].
static size_t mla_ws_bytes(int64_t T, int H, int k) {
  const int s = mla_splits(T, H, k);
  if (s <= 1) return 0;
  return align_up((size_t)T * s * H * 512 * 2, 256) + align_up((size_t)T * s * H * 2 * 4, 256);
}
static void mla_ws_split(void *ws, int64_t T, int H, int k, void **po, float **pml) {
  const int s = mla_splits(T, H, k);
  char *p = (char *)ws;
  *po = p;
  p += align_up((size_t)T * s * H * 512 * 2, 256);
  *pml = (float *)p;
}
}  // namespace dsa

using namespace dsa;

#define CLEAR_ERR() (g_err[0] = '\0')
#define REQUIRE(cond, st, ...) \
  do {                         \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

extern "C" {

const char *dsa_last_error(void) { return g_err; }
#ifndef DSA_SOURCE_HASH
#define DSA_SOURCE_HASH "unstamped"
#endif
// the build stamps the hash of the sources it compiled, so a binding can tell
// a library built from other sources
const char *dsa_version(void) { return "libdsa 0.2 gfx950 src=" DSA_SOURCE_HASH; }

dsa_status dsa_quantize_e4m3_per_token(const float *x, int64_t rows, int32_t cols, uint8_t *x8,
                                       float *scale, hipStream_t stream) {
  CLEAR_ERR();
  REQUIRE(rows >= 0, DSA_ERR_INVALID_ARG, "rows must be >= 0 (got %lld)", (long long)rows);
  REQUIRE(cols > 0, DSA_ERR_INVALID_ARG, "cols must be > 0 (got %d)", cols);
  REQUIRE(rows == 0 || (x && x8 && scale), DSA_ERR_INVALID_ARG, "null pointer");
  REQUIRE(cols % 4 == 0 && cols <= 16384, DSA_ERR_UNSUPPORTED, "cols must be a multiple of 4, <= 16384");
  REQUIRE(rows <= 0x7FFFFFFF, DSA_ERR_UNSUPPORTED, "rows must be < 2^31");
  return hip_check(launch_quantize(x, rows, cols, x8, scale, stream), "quantize launch");
}

dsa_status dsa_indexer_scores(const void *q, const float *q_scale, const void *k, const float *k_scale,
                              const float *w, const int32_t *q_pos, int32_t T, int32_t S, int32_t H_I,
                              int32_t D_I, dsa_dtype dt, float *scores, int64_t ld_scores,
                              hipStream_t stream) {
  CLEAR_ERR();
  REQUIRE(T >= 0 && S >= 0, DSA_ERR_INVALID_ARG, "T and S must be >= 0");
  REQUIRE(H_I > 0 && D_I > 0, DSA_ERR_INVALID_ARG, "H_I and D_I must be > 0");
  REQUIRE(ld_scores >= S, DSA_ERR_INVALID_ARG, "ld_scores (%lld) < S (%d)", (long long)ld_scores, S);
  if (T == 0 || S == 0) return DSA_OK;
  REQUIRE(q && k && w && q_pos && scores, DSA_ERR_INVALID_ARG, "null pointer");
  if (dt == DSA_E4M3) {
    REQUIRE(q_scale && k_scale, DSA_ERR_INVALID_ARG, "E4M3 needs q_scale and k_scale");
    REQUIRE((D_I == 64 || D_I == 128) && H_I <= 64, DSA_ERR_UNSUPPORTED,
            "E4M3 indexer needs D_I in {64, 128} and H_I <= 64 (got %d, %d)", D_I, H_I);
    return hip_check(launch_indexer_scores_fp8((const uint8_t *)q, q_scale, (const uint8_t *)k, k_scale, w,
                                               q_pos, T, S, H_I, D_I, scores, ld_scores, stream),
                     "indexer launch");
  }
  if (dt == DSA_F32) {
    REQUIRE(D_I <= 128 && H_I <= 64, DSA_ERR_UNSUPPORTED, "F32 indexer needs D_I <= 128, H_I <= 64");
    return hip_check(launch_indexer_scores_f32((const float *)q, (const float *)k, w, q_pos, T, S, H_I, D_I,
                                               scores, ld_scores, stream),
                     "indexer launch");
  }
  return fail(DSA_ERR_UNSUPPORTED, "indexer dtype must be E4M3 or F32");
}

dsa_status dsa_topk_select(const float *scores, int64_t ld_scores, const int32_t *n_valid, int32_t T,
                           int32_t k, int32_t *idx, void *workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  CLEAR_ERR();
  REQUIRE(T >= 0, DSA_ERR_INVALID_ARG, "T must be >= 0");
  REQUIRE(k >= 1, DSA_ERR_INVALID_ARG, "k must be >= 1 (got %d)", k);
  REQUIRE(k <= DSA_MAX_K, DSA_ERR_UNSUPPORTED, "k must be <= %d (got %d)", DSA_MAX_K, k);
  REQUIRE(ld_scores >= 0, DSA_ERR_INVALID_ARG, "ld_scores must be >= 0");
  if (T == 0) return DSA_OK;
  REQUIRE(scores && n_valid && idx, DSA_ERR_INVALID_ARG, "null pointer");
  // with a workspace, rows are at most ld_scores long and short batches split
  const bool split = workspace && ld_scores > 0;
  const int32_t n_cap = split ? (int32_t)std::min<int64_t>(ld_scores, 0x7FFFFFFF) : 0x7FFFFFFF;
  return hip_check(launch_topk(scores, ld_scores, n_valid, n_cap, T, k, idx, stream, split ? workspace : nullptr,
                               split ? workspace_bytes : 0),
                   "topk launch");
}

size_t dsa_topk_workspace_bytes(int32_t T, int64_t ld_scores, int32_t k) {
  if (T <= 0 || ld_scores <= 0 || k <= 0) return 0;
  return topk_workspace_bytes(T, (int32_t)std::min<int64_t>(ld_scores, 0x7FFFFFFF), std::min<int32_t>(k, DSA_MAX_K));
}

size_t dsa_sparse_mla_workspace_bytes(int32_t T, int32_t H, int32_t k) {
  if (T <= 0 || H <= 0 || k <= 0 || H % 8) return 0;
  return mla_ws_bytes(T, H, k);
}

dsa_status dsa_sparse_mla_fwd(const void *q, const void *kv, dsa_dtype dt, const int32_t *idx, int32_t T,
                              int32_t H, int64_t N, int32_t k, float sm_scale, void *out, float *lse,
                              void *workspace, size_t workspace_bytes, hipStream_t stream) {
  CLEAR_ERR();
  REQUIRE(T >= 0 && N >= 0, DSA_ERR_INVALID_ARG, "T and N must be >= 0");
  REQUIRE(H > 0, DSA_ERR_INVALID_ARG, "H must be > 0");
  REQUIRE(k >= 1, DSA_ERR_INVALID_ARG, "k must be >= 1");
  REQUIRE(k <= DSA_MAX_K, DSA_ERR_UNSUPPORTED, "k must be <= %d", DSA_MAX_K);
  REQUIRE(sm_scale == sm_scale && sm_scale > 0.0f, DSA_ERR_INVALID_ARG, "sm_scale must be > 0");
  if (T == 0) return DSA_OK;
  REQUIRE(q && kv && idx && out, DSA_ERR_INVALID_ARG, "null pointer");
  if (dt == DSA_BF16) {
    REQUIRE(H % 8 == 0, DSA_ERR_UNSUPPORTED, "BF16 sparse MLA needs H a multiple of 8 (got %d)", H);
    const size_t need = mla_ws_bytes(T, H, k);
    int splits = 1;
    void *po = nullptr;
    float *pml = nullptr;
    if (workspace && need > 0) {
      REQUIRE(workspace_bytes >= need, DSA_ERR_WORKSPACE, "workspace %zu < required %zu", workspace_bytes,
              need);
      splits = mla_splits(T, H, k);
      mla_ws_split(workspace, T, H, k, &po, &pml);
    }
    return hip_check(launch_sparse_mla_bf16(q, kv, idx, nullptr, 0, N, T, H, k, sm_scale, out, lse, splits,
                                            po, pml, stream),
                     "sparse mla launch");
  }
  if (dt == DSA_F32) {
    return hip_check(launch_sparse_mla_f32((const float *)q, (const float *)kv, idx, N, T, H, k, sm_scale,
                                           (float *)out, lse, stream),
                     "sparse mla launch");
  }
  return fail(DSA_ERR_UNSUPPORTED, "sparse MLA dtype must be BF16 or F32");
}

dsa_status dsa_indexer_scores_at(const uint8_t *q8, const float *q_scale, const uint8_t *k8, const float *k_scale,
                                 const float *w, const int32_t *idx, int32_t T, int32_t S, int32_t H_I, int32_t D_I,
                                 int32_t k, float *out, hipStream_t stream) {
  CLEAR_ERR();
  REQUIRE(T >= 0 && S >= 1 && k >= 1, DSA_ERR_INVALID_ARG, "need T >= 0, S >= 1, k >= 1");
  REQUIRE(D_I == 128 && (H_I == 32 || H_I == 64), DSA_ERR_UNSUPPORTED, "E4M3 index scores need D_I = 128 and H_I 32 or 64");
  if (T == 0) return DSA_OK;
  REQUIRE(q8 && q_scale && k8 && k_scale && w && idx && out, DSA_ERR_INVALID_ARG, "null pointer");
  return hip_check(launch_indexer_scores_at(q8, q_scale, k8, k_scale, w, idx, T, S, H_I, k, out, stream),
                   "indexer scores-at launch");
}

dsa_status dsa_indexer_kl_fwd(const void *q, const void *kv, const int32_t *idx, const float *idx_scores,
                              const float *lse, int32_t T, int32_t H, int64_t N, int32_t k, float sm_scale, float *kl,
                              hipStream_t stream) {
  CLEAR_ERR();
  REQUIRE(T >= 0 && N >= 0, DSA_ERR_INVALID_ARG, "T and N must be >= 0");
  REQUIRE(k >= 1, DSA_ERR_INVALID_ARG, "k must be >= 1");
  REQUIRE(k <= DSA_MAX_K, DSA_ERR_UNSUPPORTED, "k must be <= %d", DSA_MAX_K);
  REQUIRE(H == 16 || H == 32 || H == 64 || H == 128, DSA_ERR_UNSUPPORTED, "KL loss needs H in {16, 32, 64, 128} (got %d)", H);
  REQUIRE(sm_scale == sm_scale && sm_scale > 0.0f, DSA_ERR_INVALID_ARG, "sm_scale must be > 0");
  if (T == 0) return DSA_OK;
  REQUIRE(q && kv && idx && idx_scores && lse && kl, DSA_ERR_INVALID_ARG, "null pointer");
  return hip_check(launch_indexer_kl(q, kv, idx, idx_scores, lse, N, T, H, k, sm_scale, kl, stream),
                   "indexer KL launch");
}

dsa_status dsa_indexer_kl_bwd(const void *q, const void *kv, const int32_t *idx, const float *idx_scores,
                              const float *lse, const float *dkl, int32_t T, int32_t H, int64_t N, int32_t k,
                              float sm_scale, float *grad_scores, hipStream_t stream) {
  CLEAR_ERR();
  REQUIRE(T >= 0 && N >= 0, DSA_ERR_INVALID_ARG, "T and N must be >= 0");
  REQUIRE(k >= 1, DSA_ERR_INVALID_ARG, "k must be >= 1");
  REQUIRE(k <= DSA_MAX_K, DSA_ERR_UNSUPPORTED, "k must be <= %d", DSA_MAX_K);
  REQUIRE(H == 16 || H == 32 || H == 64 || H == 128, DSA_ERR_UNSUPPORTED,
          "KL gradient needs H in {16, 32, 64, 128} (got %d)", H);
  REQUIRE(sm_scale == sm_scale && sm_scale > 0.0f, DSA_ERR_INVALID_ARG, "sm_scale must be > 0");
  if (T == 0) return DSA_OK;
  REQUIRE(q && kv && idx && idx_scores && lse && dkl && grad_scores, DSA_ERR_INVALID_ARG, "null pointer");
  return hip_check(launch_indexer_kl_grad(q, kv, idx, idx_scores, lse, dkl, N, T, H, k, sm_scale, grad_scores, stream),
                   "indexer KL gradient launch");
}

// Indexer backward workspace for one chunk of up to kIdxBwdChunk queries:
// u [Tc, k, 128] fp32, then the inverted selection (cnt, start [S + 1], list [Tc k]).
static constexpr int32_t kIdxBwdChunk = 1024;
static int32_t idx_bwd_chunk(int32_t T) { return T < kIdxBwdChunk ? T : kIdxBwdChunk; }
static size_t idx_bwd_ws(int32_t T, int32_t S, int32_t k) {
  const size_t tc = (size_t)idx_bwd_chunk(T);
  return align_up(tc * k * 128 * 4, 256) + 2 * align_up(((size_t)S + 1) * 4, 256) + align_up(tc * k * 4, 256);
}

size_t dsa_indexer_bwd_workspace_bytes(int32_t T, int32_t S, int32_t k) {
  if (T <= 0 || S <= 0 || k <= 0) return 0;
  return idx_bwd_ws(T, S, std::min<int32_t>(k, DSA_MAX_K));
}

dsa_status dsa_indexer_bwd(const uint8_t *q8, const float *q_scale, const uint8_t *k8, const float *k_scale,
                           const float *w, const int32_t *idx, const float *grad_scores, int32_t T, int32_t S,
                           int32_t H_I, int32_t D_I, int32_t k, float *dw, float *dq, float *dk, void *workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  CLEAR_ERR();
  REQUIRE(T >= 0 && S >= 1 && k >= 1, DSA_ERR_INVALID_ARG, "need T >= 0, S >= 1, k >= 1");
  REQUIRE(k <= DSA_MAX_K, DSA_ERR_UNSUPPORTED, "k must be <= %d", DSA_MAX_K);
  REQUIRE(H_I == 64 && D_I == 128, DSA_ERR_UNSUPPORTED, "indexer backward needs H_I = 64, D_I = 128 (got %d, %d)",
          H_I, D_I);
  if (T == 0) return DSA_OK;
  REQUIRE(q8 && q_scale && k8 && k_scale && w && idx && grad_scores && dw && dq && dk, DSA_ERR_INVALID_ARG,
          "null pointer");
  const size_t need = idx_bwd_ws(T, S, k);
  REQUIRE(workspace && workspace_bytes >= need, DSA_ERR_WORKSPACE, "workspace %zu < required %zu",
          workspace ? workspace_bytes : (size_t)0, need);
  const int32_t tc_max = idx_bwd_chunk(T);
  char *p = (char *)workspace;
  float *u = (float *)p;
  p += align_up((size_t)tc_max * k * 128 * 4, 256);
  int32_t *cnt = (int32_t *)p;
  p += align_up(((size_t)S + 1) * 4, 256);
  int32_t *start = (int32_t *)p;
  p += align_up(((size_t)S + 1) * 4, 256);
  int32_t *list = (int32_t *)p;
  dsa_status st = hip_check(launch_fill_zero_f32(dk, (int64_t)S * 128, stream), "fill launch");
  for (int32_t t0 = 0; t0 < T && st == DSA_OK; t0 += tc_max) {
    const int32_t tc = std::min(tc_max, T - t0);
    const int32_t *idx_c = idx + (int64_t)t0 * k;
    st = hip_check(launch_indexer_bwd_chunk(q8, q_scale, k8, k_scale, w, idx, grad_scores, t0, tc, S, k, dw, dq, u,
                                            stream),
                   "indexer backward launch");
    if (st == DSA_OK)
      st = hip_check(launch_scatter_build(idx_c, (int64_t)tc * k, S, cnt, start, list, stream), "scatter launch");
    if (st == DSA_OK) st = hip_check(launch_scatter_add(start, list, S, u, 128, dk, stream), "scatter launch");
  }
  return st;
}

// Sparse MLA backward workspace: D [T, H] fp32, then for one chunk of up to
// kMlaBwdChunk queries s dS and P [Tc, k, H] bf16, the pair gradients
// G [Tc, k, 576] bf16 and the inverted selection (cnt, start [N + 1], list [Tc k]).
static constexpr int32_t kMlaBwdChunk = 512;
static int32_t mla_bwd_chunk(int32_t T) { return T < kMlaBwdChunk ? T : kMlaBwdChunk; }
// Head groups of the dS kernel: 64 heads when 64 divides H, else 32.
static int32_t mla_bwd_head_groups(int32_t H) { return H % 64 == 0 ? H / 64 : H / 32; }
static size_t mla_bwd_ws(int32_t T, int32_t H, int64_t N, int32_t k) {
  const size_t tc = (size_t)mla_bwd_chunk(T);
  return align_up((size_t)T * H * 4, 256) + 2 * align_up(tc * k * H * 2, 256) + align_up(tc * k * 576 * 2, 256) +
         2 * align_up(((size_t)N + 1) * 4, 256) + align_up(tc * k * 4, 256) +
         align_up(tc * mla_bwd_head_groups(H) * k * 4, 256);
}

size_t dsa_sparse_mla_bwd_workspace_bytes(int32_t T, int32_t H, int64_t N, int32_t k) {
  if (T <= 0 || H <= 0 || N <= 0 || k <= 0) return 0;
  return mla_bwd_ws(T, H, N, std::min<int32_t>(k, DSA_MAX_K));
}

// The sparse-MLA backward; with grad_scores, also the indexer KL score
// gradient from the same P (idx_scores and dkl then required).
static dsa_status mla_bwd_run(const void *q, const void *kv, const int32_t *idx, const void *out, const float *lse,
                              const void *dout, const float *idx_scores, const float *dkl, int32_t T, int32_t H,
                              int64_t N, int32_t k, float sm_scale, float *dq, float *dkv, float *grad_scores,
                              void *workspace, size_t workspace_bytes, hipStream_t stream) {
  REQUIRE(T >= 0 && N >= 1, DSA_ERR_INVALID_ARG, "need T >= 0 and N >= 1");
  REQUIRE(k >= 1, DSA_ERR_INVALID_ARG, "k must be >= 1");
  REQUIRE(k <= DSA_MAX_K, DSA_ERR_UNSUPPORTED, "k must be <= %d", DSA_MAX_K);
  REQUIRE(H > 0 && H % 32 == 0 && H <= 128, DSA_ERR_UNSUPPORTED,
          "sparse MLA backward needs H a multiple of 32, at most 128 (got %d)", H);
  REQUIRE(N <= 0x7FFFFFFF, DSA_ERR_UNSUPPORTED, "N must be < 2^31");
  REQUIRE(sm_scale == sm_scale && sm_scale > 0.0f, DSA_ERR_INVALID_ARG, "sm_scale must be > 0");
  if (T == 0) return DSA_OK;
  REQUIRE(q && kv && idx && out && lse && dout && dq && dkv, DSA_ERR_INVALID_ARG, "null pointer");
  REQUIRE(!grad_scores || (idx_scores && dkl), DSA_ERR_INVALID_ARG, "null pointer");
  const size_t need = mla_bwd_ws(T, H, N, k);
  REQUIRE(workspace && workspace_bytes >= need, DSA_ERR_WORKSPACE, "workspace %zu < required %zu",
          workspace ? workspace_bytes : (size_t)0, need);
  const int32_t tc_max = mla_bwd_chunk(T);
  const int32_t nhg = mla_bwd_head_groups(H);
  char *p = (char *)workspace;
  float *D = (float *)p;
  p += align_up((size_t)T * H * 4, 256);
  void *dsT = p;
  p += align_up((size_t)tc_max * k * H * 2, 256);
  void *pT = p;
  p += align_up((size_t)tc_max * k * H * 2, 256);
  void *G = p;
  p += align_up((size_t)tc_max * k * 576 * 2, 256);
  int32_t *cnt = (int32_t *)p;
  p += align_up(((size_t)N + 1) * 4, 256);
  int32_t *start = (int32_t *)p;
  p += align_up(((size_t)N + 1) * 4, 256);
  int32_t *list = (int32_t *)p;
  p += align_up((size_t)tc_max * k * 4, 256);
  float *psum = grad_scores ? (float *)p : nullptr;
  dsa_status st = hip_check(launch_mla_bwd_delta(out, dout, (int64_t)T * H, D, stream), "delta launch");
  if (st == DSA_OK) st = hip_check(launch_fill_zero_f32(dkv, N * 576, stream), "fill launch");
  for (int32_t t0 = 0; t0 < T && st == DSA_OK; t0 += tc_max) {
    const int32_t tc = std::min(tc_max, T - t0);
    st = hip_check(
        launch_mla_bwd_chunk(q, kv, idx, lse, dout, D, N, H, k, sm_scale, t0, tc, dq, dsT, pT, G, psum, stream),
        "sparse mla backward launch");
    if (st == DSA_OK && psum)
      st = hip_check(launch_kl_grad_from_head_sums(idx, idx_scores, dkl, psum, N, k, nhg, t0, tc, grad_scores,
                                                   stream),
                     "kl gradient launch");
    if (st == DSA_OK)
      st = hip_check(launch_scatter_build(idx + (int64_t)t0 * k, (int64_t)tc * k, N, cnt, start, list, stream),
                     "scatter launch");
    if (st == DSA_OK) st = hip_check(launch_scatter_add_bf16(start, list, N, G, 576, dkv, stream), "scatter launch");
  }
  return st;
}

dsa_status dsa_sparse_mla_bwd(const void *q, const void *kv, const int32_t *idx, const void *out, const float *lse,
                              const void *dout, int32_t T, int32_t H, int64_t N, int32_t k, float sm_scale, float *dq,
                              float *dkv, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  CLEAR_ERR();
  return mla_bwd_run(q, kv, idx, out, lse, dout, nullptr, nullptr, T, H, N, k, sm_scale, dq, dkv, nullptr, workspace,
                     workspace_bytes, stream);
}

dsa_status dsa_sparse_mla_bwd_kl(const void *q, const void *kv, const int32_t *idx, const void *out,
                                 const float *lse, const void *dout, const float *idx_scores, const float *dkl,
                                 int32_t T, int32_t H, int64_t N, int32_t k, float sm_scale, float *dq, float *dkv,
                                 float *grad_scores, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  CLEAR_ERR();
  REQUIRE(T == 0 || grad_scores, DSA_ERR_INVALID_ARG, "null pointer");
  return mla_bwd_run(q, kv, idx, out, lse, dout, idx_scores, dkl, T, H, N, k, sm_scale, dq, dkv, grad_scores,
                     workspace, workspace_bytes, stream);
}

size_t dsa_masked_mha_workspace_bytes(int32_t L, int32_t H) {
  if (L <= 0 || H <= 0) return 0;
  return masked_mha_workspace_bytes(L, H);
}

dsa_status dsa_masked_mha_prefill(const void *q, const void *kv, const void *w_uk, const void *w_uv,
                                  const int32_t *idx, int32_t L, int32_t H, int32_t k, float sm_scale,
                                  void *out, float *lse, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  CLEAR_ERR();
  REQUIRE(L >= 0, DSA_ERR_INVALID_ARG, "L must be >= 0 (got %d)", L);
  REQUIRE(H > 0, DSA_ERR_INVALID_ARG, "H must be > 0");
  REQUIRE(k >= 1, DSA_ERR_INVALID_ARG, "k must be >= 1");
  REQUIRE(L <= DSA_MHA_MAX_L, DSA_ERR_UNSUPPORTED, "masked MHA needs L <= %d (got %d)", DSA_MHA_MAX_L, L);
  REQUIRE(sm_scale == sm_scale && sm_scale > 0.0f, DSA_ERR_INVALID_ARG, "sm_scale must be > 0");
  if (L == 0) return DSA_OK;
  REQUIRE(q && kv && w_uk && w_uv && idx && out && workspace, DSA_ERR_INVALID_ARG, "null pointer");
  const size_t need = masked_mha_workspace_bytes(L, H);
  REQUIRE(workspace_bytes >= need, DSA_ERR_WORKSPACE, "workspace %zu < required %zu", workspace_bytes, need);
  return hip_check(launch_masked_mha(q, kv, w_uk, w_uv, idx, L, H, k, sm_scale, out, lse, workspace, stream),
                   "masked mha launch");
}

// The fused indexer + streaming top-k covers the full-size E4M3 indexer (64
// heads of 128 dims); every other indexer shape scores the L x L matrix into
// the workspace and selects rows from it.
static bool prefill_fused(const dsa_prefill_args *a) {
  return a->idx_dt == DSA_E4M3 && a->H_I == 64 && a->D_I == 128;
}

static dsa_status check_prefill(const dsa_prefill_args *a, bool attention) {
  REQUIRE(a, DSA_ERR_INVALID_ARG, "null args");
  REQUIRE(a->L >= 1, DSA_ERR_INVALID_ARG, "L must be >= 1");
  REQUIRE(a->H > 0 && a->H_I > 0 && a->D_I > 0, DSA_ERR_INVALID_ARG, "head counts and D_I must be > 0");
  REQUIRE(a->k >= 1, DSA_ERR_INVALID_ARG, "k must be >= 1");
  REQUIRE(a->k <= DSA_MAX_K, DSA_ERR_UNSUPPORTED, "k must be <= %d", DSA_MAX_K);
  REQUIRE(a->q_idx && a->k_idx && a->w && a->idx, DSA_ERR_INVALID_ARG, "null pointer");
  if (attention) {
    REQUIRE(a->q && a->kv && a->out, DSA_ERR_INVALID_ARG, "null pointer");
    REQUIRE(a->sm_scale == a->sm_scale && a->sm_scale > 0.0f, DSA_ERR_INVALID_ARG, "sm_scale must be > 0");
  }
  if (a->idx_dt == DSA_E4M3) {
    REQUIRE(a->q_scale && a->k_scale, DSA_ERR_INVALID_ARG, "E4M3 needs q_scale and k_scale");
    REQUIRE((a->D_I == 64 || a->D_I == 128) && a->H_I <= 64, DSA_ERR_UNSUPPORTED,
            "E4M3 prefill needs D_I in {64, 128} and H_I <= 64 (got %d, %d)", a->D_I, a->H_I);
  } else if (a->idx_dt == DSA_F32) {
    REQUIRE(a->D_I <= 128 && a->H_I <= 64, DSA_ERR_UNSUPPORTED, "F32 indexer needs D_I <= 128, H_I <= 64");
  } else {
    return fail(DSA_ERR_UNSUPPORTED, "indexer dtype must be E4M3 or F32");
  }
  if (!prefill_fused(a))
    REQUIRE((int64_t)a->L * a->L <= (int64_t)1 << 28, DSA_ERR_UNSUPPORTED,
            "this indexer shape keeps the L x L scores in the workspace; L must be <= 16384 (only E4M3 with "
            "H_I = 64, D_I = 128 streams them)");
  if (!attention) return DSA_OK;
  if (a->attn_dt == DSA_BF16)
    REQUIRE(a->H % 8 == 0, DSA_ERR_UNSUPPORTED, "BF16 sparse MLA needs H a multiple of 8");
  else
    REQUIRE(a->attn_dt == DSA_F32, DSA_ERR_UNSUPPORTED, "attention dtype must be BF16 or F32");
  return DSA_OK;
}

size_t dsa_prefill_workspace_bytes(const dsa_prefill_args *a) {
  if (!a || a->L < 1) return 0;
  if (!prefill_fused(a)) {
    const size_t L = (size_t)a->L;
    return align_up(L * L * 4, 256) + 2 * align_up(L * 4, 256);
  }
  return align_up(prefill_candidate_bytes(a->L), 256);  // per-query candidate buffers of the streaming top-k
}

// indexer + top-k of one prefill sequence into a->idx
static dsa_status prefill_select(const dsa_prefill_args *a, void *workspace, hipStream_t stream) {
  const int L = a->L;
  if (prefill_fused(a))
    return hip_check(launch_prefill_indexer_topk((const uint8_t *)a->q_idx, a->q_scale, (const uint8_t *)a->k_idx,
                                                 a->k_scale, a->w, L, a->k, a->idx, (uint32_t *)workspace, stream),
                     "prefill indexer/top-k launch");
  float *sc = (float *)workspace;
  int32_t *qpos = (int32_t *)((char *)workspace + align_up((size_t)L * L * 4, 256));
  int32_t *nval = (int32_t *)((char *)qpos + align_up((size_t)L * 4, 256));
  dsa_status st = hip_check(launch_positions(qpos, nval, L, stream), "positions launch");
  if (st == DSA_OK && a->idx_dt == DSA_E4M3)
    st = hip_check(launch_indexer_scores_fp8((const uint8_t *)a->q_idx, a->q_scale, (const uint8_t *)a->k_idx,
                                             a->k_scale, a->w, qpos, L, L, a->H_I, a->D_I, sc, L, stream),
                   "indexer launch");
  else if (st == DSA_OK)
    st = hip_check(launch_indexer_scores_f32((const float *)a->q_idx, (const float *)a->k_idx, a->w, qpos, L, L,
                                             a->H_I, a->D_I, sc, L, stream),
                   "indexer launch");
  if (st == DSA_OK) st = hip_check(launch_topk(sc, L, nval, L, L, a->k, a->idx, stream), "topk launch");
  return st;
}

dsa_status dsa_prefill_select(const dsa_prefill_args *a, void *workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  CLEAR_ERR();
  dsa_status st = check_prefill(a, false);
  if (st != DSA_OK) return st;
  const size_t need = dsa_prefill_workspace_bytes(a);
  REQUIRE(workspace && workspace_bytes >= need, DSA_ERR_WORKSPACE, "workspace %zu < required %zu",
          workspace ? workspace_bytes : (size_t)0, need);
  return prefill_select(a, workspace, stream);
}

dsa_status dsa_prefill(const dsa_prefill_args *a, void *workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  CLEAR_ERR();
  dsa_status st = check_prefill(a, true);
  if (st != DSA_OK) return st;
  const size_t need = dsa_prefill_workspace_bytes(a);
  REQUIRE(workspace && workspace_bytes >= need, DSA_ERR_WORKSPACE, "workspace %zu < required %zu",
          workspace ? workspace_bytes : (size_t)0, need);
  const int L = a->L;
  st = prefill_select(a, workspace, stream);
  if (st != DSA_OK) return st;
  if (a->attn_dt == DSA_BF16)
    return hip_check(launch_sparse_mla_bf16(a->q, a->kv, a->idx, nullptr, 0, L, L, a->H, a->k, a->sm_scale,
                                            a->out, a->lse, 1, nullptr, nullptr, stream),
                     "sparse mla launch");
  return hip_check(launch_sparse_mla_f32((const float *)a->q, (const float *)a->kv, a->idx, L, L, a->H, a->k,
                                         a->sm_scale, (float *)a->out, a->lse, stream),
                   "sparse mla launch");
}

static dsa_status check_decode(const dsa_decode_args *a, bool attention) {
  REQUIRE(a, DSA_ERR_INVALID_ARG, "null args");
  REQUIRE(a->B >= 0, DSA_ERR_INVALID_ARG, "B must be >= 0");
  REQUIRE(a->k >= 1, DSA_ERR_INVALID_ARG, "k must be >= 1");
  REQUIRE(a->k <= DSA_MAX_K, DSA_ERR_UNSUPPORTED, "k must be <= %d", DSA_MAX_K);
  REQUIRE(a->max_ctx >= 1, DSA_ERR_INVALID_ARG, "max_ctx must be >= 1");
  REQUIRE(a->max_blocks >= (a->max_ctx + DSA_PAGE - 1) / DSA_PAGE, DSA_ERR_INVALID_ARG,
          "max_blocks (%d) too small for max_ctx (%d)", a->max_blocks, a->max_ctx);
  REQUIRE(a->n_pool_rows > 0 && a->n_pool_rows % DSA_PAGE == 0, DSA_ERR_INVALID_ARG,
          "n_pool_rows must be a positive multiple of 64");
  REQUIRE(a->H_I == 64 && a->D_I == 128, DSA_ERR_UNSUPPORTED, "decode indexer needs H_I = 64, D_I = 128");
  if (attention) {
    REQUIRE(a->H > 0 && a->H % 8 == 0, DSA_ERR_UNSUPPORTED, "decode attention needs H a multiple of 8");
    REQUIRE(a->sm_scale == a->sm_scale && a->sm_scale > 0.0f, DSA_ERR_INVALID_ARG, "sm_scale must be > 0");
  }
  if (a->B == 0) return DSA_OK;
  REQUIRE(a->q8 && a->q_scale && a->w && a->k8_pool && a->ks_pool && a->block_table && a->ctx_len,
          DSA_ERR_INVALID_ARG, "null pointer");
  if (attention) REQUIRE(a->q && a->kv_pool && a->out, DSA_ERR_INVALID_ARG, "null pointer");
  return DSA_OK;
}

static int64_t decode_ld(const dsa_decode_args *a) { return (int64_t)align_up((size_t)a->max_ctx, 64); }

size_t dsa_decode_workspace_bytes(const dsa_decode_args *a) {
  if (!a || a->B <= 0 || a->max_ctx <= 0 || a->k <= 0) return 0;
  size_t n = align_up((size_t)a->B * decode_ld(a) * 4, 256);
  if (!a->idx_out) n += align_up((size_t)a->B * a->k * 4, 256);
  // one region, used first by a split top-k and then by the split attention
  const size_t mla = (a->H > 0 && a->H % 8 == 0) ? mla_ws_bytes(a->B, a->H, a->k) : 0;
  n += std::max(mla, topk_workspace_bytes(a->B, a->max_ctx, a->k));
  return n;
}

dsa_status dsa_decode_indexer_scores(const dsa_decode_args *a, float *scores, int64_t ld_scores,
                                     hipStream_t stream) {
  CLEAR_ERR();
  dsa_status st = check_decode(a, false);
  if (st != DSA_OK) return st;
  REQUIRE(ld_scores >= a->max_ctx, DSA_ERR_INVALID_ARG, "ld_scores < max_ctx");
  if (a->B == 0) return DSA_OK;
  REQUIRE(scores, DSA_ERR_INVALID_ARG, "null pointer");
  return hip_check(launch_decode_indexer(a->q8, a->q_scale, a->w, a->k8_pool, a->ks_pool, a->block_table,
                                         a->max_blocks, a->ctx_len, a->B, a->max_ctx, a->n_pool_rows, scores,
                                         ld_scores, stream),
                   "decode indexer launch");
}

dsa_status dsa_sparse_mla_paged_fwd(const void *q, const void *kv_pool, int64_t n_pool_rows,
                                    const int32_t *block_table, int32_t max_blocks, const int32_t *idx,
                                    int32_t T, int32_t H, int32_t k, float sm_scale, void *out, float *lse,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream) {
  CLEAR_ERR();
  REQUIRE(T >= 0, DSA_ERR_INVALID_ARG, "T must be >= 0");
  REQUIRE(n_pool_rows > 0 && n_pool_rows % DSA_PAGE == 0, DSA_ERR_INVALID_ARG,
          "n_pool_rows must be a positive multiple of 64");
  REQUIRE(max_blocks >= 1, DSA_ERR_INVALID_ARG, "max_blocks must be >= 1");
  REQUIRE(k >= 1, DSA_ERR_INVALID_ARG, "k must be >= 1");
  REQUIRE(k <= DSA_MAX_K, DSA_ERR_UNSUPPORTED, "k must be <= %d", DSA_MAX_K);
  REQUIRE(H > 0 && H % 8 == 0, DSA_ERR_UNSUPPORTED, "paged sparse MLA needs H a multiple of 8");
  REQUIRE(sm_scale == sm_scale && sm_scale > 0.0f, DSA_ERR_INVALID_ARG, "sm_scale must be > 0");
  if (T == 0) return DSA_OK;
  REQUIRE(q && kv_pool && block_table && idx && out, DSA_ERR_INVALID_ARG, "null pointer");
  const size_t need = mla_ws_bytes(T, H, k);
  int splits = 1;
  void *po = nullptr;
    float *pml = nullptr;
  if (workspace && need > 0) {
    REQUIRE(workspace_bytes >= need, DSA_ERR_WORKSPACE, "workspace %zu < required %zu", workspace_bytes, need);
    splits = mla_splits(T, H, k);
    mla_ws_split(workspace, T, H, k, &po, &pml);
  }
  return hip_check(launch_sparse_mla_bf16(q, kv_pool, idx, block_table, max_blocks, n_pool_rows, T, H, k,
                                          sm_scale, out, lse, splits, po, pml, stream),
                   "sparse mla launch");
}

// The decode steps on a validated request, with scratch carved from `ws`
// (at least dsa_decode_workspace_bytes(a) bytes): fp32 score rows [B, ld],
// then the selection [B, k] unless the caller takes it in idx_out, then one
// region used first by a split top-k and then by the split attention.
static dsa_status decode_run(const dsa_decode_args *a, void *ws, hipStream_t stream) {
  const int64_t ld = decode_ld(a);
  char *p = (char *)ws;
  float *scores = (float *)p;
  p += align_up((size_t)a->B * ld * 4, 256);
  int32_t *idx = a->idx_out;
  if (!idx) {
    idx = (int32_t *)p;
    p += align_up((size_t)a->B * a->k * 4, 256);
  }
  void *po = nullptr;
  float *pml = nullptr;
  const int splits = mla_splits(a->B, a->H, a->k);
  if (splits > 1) mla_ws_split(p, a->B, a->H, a->k, &po, &pml);
  const size_t topk_ws = topk_workspace_bytes(a->B, a->max_ctx, a->k);  // the same region, before the attention
  dsa_status st = hip_check(launch_decode_indexer(a->q8, a->q_scale, a->w, a->k8_pool, a->ks_pool, a->block_table,
                                                  a->max_blocks, a->ctx_len, a->B, a->max_ctx, a->n_pool_rows, scores,
                                                  ld, stream),
                            "decode indexer launch");
  if (st != DSA_OK) return st;
  st = hip_check(launch_topk(scores, ld, a->ctx_len, a->max_ctx, a->B, a->k, idx, stream, topk_ws ? p : nullptr,
                             topk_ws),
                 "topk launch");
  if (st != DSA_OK) return st;
  return hip_check(launch_sparse_mla_bf16(a->q, a->kv_pool, idx, a->block_table, a->max_blocks, a->n_pool_rows,
                                          a->B, a->H, a->k, a->sm_scale, a->out, a->lse, splits, po, pml, stream),
                   "sparse mla launch");
}

dsa_status dsa_decode(const dsa_decode_args *a, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  CLEAR_ERR();
  dsa_status st = check_decode(a, true);
  if (st != DSA_OK) return st;
  if (a->B == 0) return DSA_OK;
  const size_t need = dsa_decode_workspace_bytes(a);
  REQUIRE(workspace && workspace_bytes >= need, DSA_ERR_WORKSPACE, "workspace %zu < required %zu",
          workspace ? workspace_bytes : (size_t)0, need);
  return decode_run(a, workspace, stream);
}

size_t dsa_decode_static_scratch_bytes(void) { return static_scratch_bytes(); }

dsa_status dsa_decode_noalloc(const dsa_decode_args *a, hipStream_t stream) {
  CLEAR_ERR();
  dsa_status st = check_decode(a, true);
  if (st != DSA_OK) return st;
  if (a->B == 0) return DSA_OK;
  const size_t need = dsa_decode_workspace_bytes(a);
  REQUIRE(need <= static_scratch_bytes(), DSA_ERR_UNSUPPORTED,
          "this decode needs %zu bytes of scratch; the library's static scratch holds %zu (use dsa_decode with a "
          "workspace)",
          need, static_scratch_bytes());
  void *scratch = nullptr;
  st = hip_check(static_scratch(stream, &scratch), "static scratch");
  if (st != DSA_OK) return st;
  return decode_run(a, scratch, stream);
}

dsa_status dsa_paged_cache_append(const void *latent, const uint8_t *k8, const float *ks, const int32_t *pos,
                                  int32_t B, int32_t D_I, const int32_t *block_table, int32_t max_blocks,
                                  void *kv_pool, uint8_t *k8_pool, float *ks_pool, int64_t n_pool_rows,
                                  hipStream_t stream) {
  CLEAR_ERR();
  REQUIRE(B >= 0, DSA_ERR_INVALID_ARG, "B must be >= 0");
  REQUIRE(max_blocks >= 1, DSA_ERR_INVALID_ARG, "max_blocks must be >= 1");
  REQUIRE(n_pool_rows > 0 && n_pool_rows % DSA_PAGE == 0, DSA_ERR_INVALID_ARG,
          "n_pool_rows must be a positive multiple of 64");
  // the decode indexer reads the key pool with a 128-byte row stride
  REQUIRE(D_I == 128, DSA_ERR_UNSUPPORTED, "the paged key pool needs D_I = 128 (got %d)", D_I);
  if (B == 0) return DSA_OK;
  REQUIRE(latent && k8 && ks && pos && block_table && kv_pool && k8_pool && ks_pool, DSA_ERR_INVALID_ARG,
          "null pointer");
  return hip_check(launch_cache_append(latent, k8, ks, pos, B, D_I, block_table, max_blocks, n_pool_rows, kv_pool,
                                       k8_pool, ks_pool, stream),
                   "cache append launch");
}

}  // extern "C"
