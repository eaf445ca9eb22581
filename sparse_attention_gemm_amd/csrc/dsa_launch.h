// dsa_launch.h -- host-side launchers of the library's kernels and the
// C ABI layer's helpers (status, messages).  Each launcher enqueues its
// kernels on the given stream and validates nothing: the C ABI layer does.
// Host-only: it needs the HIP runtime API, not the device headers, so the
// C ABI layer also compiles as plain C++ (the host sanitizer build).
#pragma once
#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "dsa.h"

namespace dsa {
dsa_status fail(dsa_status st, const char *fmt, ...);
dsa_status hip_check(hipError_t e, const char *what);
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Launchers (each validates nothing: the C ABI layer does).
hipError_t launch_quantize(const float *x, int64_t rows, int32_t cols, uint8_t *x8, float *scale,
                           hipStream_t s);
hipError_t launch_indexer_scores_fp8(const uint8_t *q, const float *qs, const uint8_t *k,
                                     const float *ks, const float *w, const int32_t *q_pos,
                                     int32_t T, int32_t S, int32_t H_I, int32_t D_I, float *scores, int64_t ld,
                                     hipStream_t s);
hipError_t launch_indexer_scores_f32(const float *q, const float *k, const float *w,
                                     const int32_t *q_pos, int32_t T, int32_t S, int32_t H_I,
                                     int32_t D_I, float *scores, int64_t ld, hipStream_t s);
// Rows take min(n_valid[t], n_cap) candidates (n_cap guards the row length).
// Row top-k over rows of at most n_cap scores.  With a workspace of at least
// topk_workspace_bytes(T, n_cap, k) bytes a short batch is split into column
// chunks (one selection per chunk, then a merge per row).
int topk_split_chunks(int64_t T, int32_t n_cap, int32_t k);
size_t topk_workspace_bytes(int64_t T, int32_t n_cap, int32_t k);
hipError_t launch_topk(const float *scores, int64_t ld, const int32_t *n_valid, int32_t n_cap, int32_t T,
                       int32_t k, int32_t *idx, hipStream_t s, void *ws = nullptr, size_t ws_bytes = 0);
// Fused prefill selection; cand: prefill_candidate_bytes(L) of scratch.
size_t prefill_candidate_bytes(int32_t L);
hipError_t launch_prefill_indexer_topk(const uint8_t *q8, const float *qs, const uint8_t *k8,
                                       const float *ks, const float *w, int32_t L, int32_t k,
                                       int32_t *idx, uint32_t *cand, hipStream_t s);
// Sparse MLA.  block_table != NULL: idx holds logical positions of sequence
// t (page size 64); otherwise idx holds rows of kv.  Entries that do not map
// to a row in [0, N) are skipped like -1.  splits > 1 needs the
// partial buffers (part_o [T,splits,H,512] bf16, part_ml [T,splits,H,2] f32).
hipError_t launch_sparse_mla_bf16(const void *q, const void *kv, const int32_t *idx,
                                  const int32_t *block_table, int32_t max_blocks, int64_t N, int32_t T,
                                  int32_t H, int32_t k, float sm_scale, void *out, float *lse,
                                  int32_t splits, void *part_o, float *part_ml, hipStream_t s);
hipError_t launch_sparse_mla_f32(const float *q, const float *kv, const int32_t *idx, int64_t N, int32_t T,
                                 int32_t H, int32_t k, float sm_scale, float *out, float *lse,
                                 hipStream_t s);
hipError_t launch_decode_indexer(const uint8_t *q8, const float *qs, const float *w,
                                 const uint8_t *k8_pool, const float *ks_pool,
                                 const int32_t *block_table, int32_t max_blocks,
                                 const int32_t *ctx_len, int32_t B, int32_t max_ctx, int64_t n_pool_rows,
                                 float *scores, int64_t ld, hipStream_t s);
// Masked MHA in MLA's multi-head form (BF16; per head 128 + 64 logit dims,
// 128 value dims, latent 512 + 64).  workspace: masked_mha_workspace_bytes(L, H).
size_t masked_mha_workspace_bytes(int32_t L, int32_t H);
size_t masked_mha_kv_bytes(int32_t L, int32_t H);  // bytes of K_h (and of V_h) at the workspace's start
hipError_t launch_masked_mha(const void *q, const void *kv, const void *w_uk, const void *w_uv,
                             const int32_t *idx, int32_t L, int32_t H, int32_t k, float sm_scale, void *out,
                             float *lse, void *workspace, hipStream_t s);
// Index scores at listed positions (E4M3, D_I = 128, H_I 32 or 64) and the
// indexer KL-alignment loss (H / 16 in {1, 2, 4, 8}, k <= 2048).
hipError_t launch_indexer_scores_at(const uint8_t *q8, const float *qs, const uint8_t *k8, const float *ks,
                                    const float *w, const int32_t *idx, int32_t T, int32_t S, int32_t H_I, int32_t k,
                                    float *out, hipStream_t s);
hipError_t launch_indexer_kl(const void *q, const void *kv, const int32_t *idx, const float *scores, const float *lse,
                             int64_t N, int32_t T, int32_t H, int32_t k, float sm_scale, float *kl, hipStream_t s);
hipError_t launch_positions(int32_t *q_pos, int32_t *n_valid, int32_t L, hipStream_t s);
// Backward.  The KL loss's gradient with respect to the index scores
// (grad [T, k]); the indexer's backward for queries [t0, t0 + Tc) (dw, dq of
// those queries, and each pair's share u [Tc, k, 128] of dk).
hipError_t launch_indexer_kl_grad(const void *q, const void *kv, const int32_t *idx, const float *scores,
                                  const float *lse, const float *dkl, int64_t N, int32_t T, int32_t H, int32_t k,
                                  float sm_scale, float *grad, hipStream_t s);
hipError_t launch_indexer_bwd_chunk(const uint8_t *q8, const float *qs, const uint8_t *k8, const float *ks,
                                    const float *w, const int32_t *idx, const float *grad, int64_t t0, int32_t Tc,
                                    int32_t S, int32_t k, float *dw, float *dq, float *u, hipStream_t s);
// The selection of npairs pairs (idx entries in [0, N) are rows) inverted:
// cnt, start [N + 1] and list [npairs] of workspace; then
// Y[r, :] += sum over r's pairs, in increasing pair index, of X[pair, :] (W <= 768).
hipError_t launch_scatter_build(const int32_t *idx, int64_t npairs, int64_t N, int32_t *cnt, int32_t *start,
                                int32_t *list, hipStream_t s);
hipError_t launch_scatter_add(const int32_t *start, const int32_t *list, int64_t N, const float *X, int32_t W, float *Y,
                              hipStream_t s);
// The same with bf16 X [npairs, W] (W even, at most 768), summed in fp32.
hipError_t launch_scatter_add_bf16(const int32_t *start, const int32_t *list, int64_t N, const void *X, int32_t W,
                                   float *Y, hipStream_t s);
hipError_t launch_fill_zero_f32(float *p, int64_t n, hipStream_t s);
// Sparse MLA backward: D = dO . o per (token, head); then for queries
// [t0, t0 + Tc): dq, s dS and P [Tc, k, H] bf16, and the pair gradients
// G [Tc, k, 576] bf16 (H a multiple of 32, at most 128).
hipError_t launch_mla_bwd_delta(const void *out, const void *dout, int64_t TH, float *D, hipStream_t s);
hipError_t launch_mla_bwd_chunk(const void *q, const void *kv, const int32_t *idx, const float *lse, const void *dout,
                                const float *D, int64_t N, int32_t H, int32_t k, float sm_scale, int64_t t0,
                                int32_t Tc, float *dq, void *dsT, void *pT, void *G, float *psum, hipStream_t s);
// The KL score gradient of queries [t0, t0 + Tc) from psum (launch_mla_bwd_chunk's
// head-group sums of P, nhg groups): grad[t, a] = dkl[t] (softmax(scores[t])_a
// - P_a / Z), P_a the sum over the groups, Z its sum over the valid entries.
hipError_t launch_kl_grad_from_head_sums(const int32_t *idx, const float *scores, const float *dkl, const float *psum,
                                         int64_t N, int32_t k, int32_t nhg, int64_t t0, int32_t Tc, float *grad,
                                         hipStream_t s);
// The library's static device scratch (scratch.hip): its size, and its
// address on the device that owns `stream` (which must be the current device),
// looked up once per device.
size_t static_scratch_bytes();
hipError_t static_scratch(hipStream_t stream, void **ptr);
hipError_t launch_cache_append(const void *latent, const uint8_t *k8, const float *ks,
                               const int32_t *pos, int32_t B, int32_t D_I,
                               const int32_t *block_table, int32_t max_blocks, int64_t n_pool_rows,
                               void *kv_pool, uint8_t *k8_pool, float *ks_pool, hipStream_t s);
}  // namespace dsa
