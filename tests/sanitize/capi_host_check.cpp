// capi_host_check.cpp -- the C ABI layer (capi.cpp, workspace.cpp) on the
// host, built with AddressSanitizer and UndefinedBehaviorSanitizer and no
// GPU: every kernel launcher is replaced by a stub that writes each byte of
// every output and scratch region the launcher is handed, at the size the
// kernel's contract gives it.  A workspace carved past the caller's buffer,
// or an output sized wrong, is then a heap overflow that ASan reports; size
// arithmetic that overflows is reported by UBSan.  The three HIP runtime
// queries the layer makes are answered here (a 256-CU device).
//
// Exit status 0 and "capi host check ok" on success; any failed expectation
// prints its line and aborts.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "dsa_launch.h"

#define EXPECT(c)                                                                \
  do {                                                                           \
    if (!(c)) {                                                                  \
      std::fprintf(stderr, "%s:%d: expectation failed: %s (%s)\n", __FILE__, __LINE__, #c, \
                   dsa_last_error());                                            \
      std::abort();                                                              \
    }                                                                            \
  } while (0)

// ------------------------------------------------------------ HIP runtime
extern "C" {
hipError_t hipGetDevice(int *d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int *v, hipDeviceAttribute_t a, int) {
  *v = a == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
  return hipSuccess;
}
const char *hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "stubbed error"; }
}

// ------------------------------------------------------------ launcher stubs
static int g_launches = 0;
static void touch(void *p, size_t bytes) {
  if (bytes) {
    EXPECT(p != nullptr);
    std::memset(p, 0x5A, bytes);
  }
}
static void read_all(const void *p, size_t bytes) {
  volatile unsigned char acc = 0;
  const unsigned char *b = (const unsigned char *)p;
  for (size_t i = 0; i < bytes; i += 61) acc ^= b[i];
  if (bytes) acc ^= b[bytes - 1];
  (void)acc;
}

namespace dsa {
hipError_t launch_quantize(const float *x, int64_t rows, int32_t cols, uint8_t *x8, float *scale, hipStream_t) {
  ++g_launches;
  read_all(x, (size_t)rows * cols * 4);
  touch(x8, (size_t)rows * cols);
  touch(scale, (size_t)rows * 4);
  return hipSuccess;
}
hipError_t launch_indexer_scores_fp8(const uint8_t *q, const float *qs, const uint8_t *k, const float *ks,
                                     const float *w, const int32_t *q_pos, int32_t T, int32_t S, int32_t H_I,
                                     int32_t D_I, float *scores, int64_t ld, hipStream_t) {
  ++g_launches;
  read_all(q, (size_t)T * H_I * D_I);
  read_all(k, (size_t)S * D_I);
  read_all(qs, (size_t)T * 4);
  read_all(ks, (size_t)S * 4);
  read_all(w, (size_t)T * H_I * 4);
  read_all(q_pos, (size_t)T * 4);
  for (int32_t t = 0; t < T; ++t) touch(scores + (size_t)t * ld, (size_t)S * 4);
  return hipSuccess;
}
hipError_t launch_indexer_scores_f32(const float *q, const float *k, const float *w, const int32_t *q_pos,
                                     int32_t T, int32_t S, int32_t H_I, int32_t D_I, float *scores, int64_t ld,
                                     hipStream_t) {
  ++g_launches;
  read_all(q, (size_t)T * H_I * D_I * 4);
  read_all(k, (size_t)S * D_I * 4);
  read_all(w, (size_t)T * H_I * 4);
  read_all(q_pos, (size_t)T * 4);
  for (int32_t t = 0; t < T; ++t) touch(scores + (size_t)t * ld, (size_t)S * 4);
  return hipSuccess;
}
hipError_t launch_topk(const float *scores, int64_t ld, const int32_t *n_valid, int32_t n_cap, int32_t T,
                       int32_t k, int32_t *idx, hipStream_t, void *ws, size_t ws_bytes) {
  ++g_launches;
  read_all(n_valid, (size_t)T * 4);
  // each row reads at most min(n_cap, ld) scores: the callers here keep n_valid <= that
  const int64_t row = std::min<int64_t>(n_cap, ld > 0 ? ld : n_cap);
  if (ld > 0)
    for (int32_t t = 0; t < T; ++t) read_all(scores + (size_t)t * ld, (size_t)row * 4);
  touch(idx, (size_t)T * k * 4);
  if (ws) {
    const size_t need = topk_workspace_bytes(T, n_cap, k);
    if (topk_split_chunks(T, n_cap, k) > 1 && ws_bytes >= need) touch(ws, need);
  }
  return hipSuccess;
}
hipError_t launch_prefill_indexer_topk(const uint8_t *q8, const float *qs, const uint8_t *k8, const float *ks,
                                       const float *w, int32_t L, int32_t k, int32_t *idx, uint32_t *cand,
                                       hipStream_t) {
  ++g_launches;
  read_all(q8, (size_t)L * 64 * 128);
  read_all(k8, (size_t)L * 128);
  read_all(qs, (size_t)L * 4);
  read_all(ks, (size_t)L * 4);
  read_all(w, (size_t)L * 64 * 4);
  touch(idx, (size_t)L * k * 4);
  touch(cand, prefill_candidate_bytes(L));
  return hipSuccess;
}
hipError_t launch_sparse_mla_bf16(const void *q, const void *kv, const int32_t *idx, const int32_t *bt,
                                  int32_t max_blocks, int64_t N, int32_t T, int32_t H, int32_t k, float,
                                  void *out, float *lse, int32_t splits, void *part_o, float *part_ml,
                                  hipStream_t) {
  ++g_launches;
  EXPECT(splits >= 1);
  read_all(q, (size_t)T * H * 576 * 2);
  read_all(kv, (size_t)N * 576 * 2);
  read_all(idx, (size_t)T * k * 4);
  if (bt) read_all(bt, (size_t)T * max_blocks * 4);
  touch(out, (size_t)T * H * 512 * 2);
  if (lse) touch(lse, (size_t)T * H * 4);
  if (splits > 1) {
    touch(part_o, (size_t)T * splits * H * 512 * 2);
    touch(part_ml, (size_t)T * splits * H * 2 * 4);
  }
  return hipSuccess;
}
hipError_t launch_sparse_mla_f32(const float *q, const float *kv, const int32_t *idx, int64_t N, int32_t T,
                                 int32_t H, int32_t k, float, float *out, float *lse, hipStream_t) {
  ++g_launches;
  read_all(q, (size_t)T * H * 576 * 4);
  read_all(kv, (size_t)N * 576 * 4);
  read_all(idx, (size_t)T * k * 4);
  touch(out, (size_t)T * H * 512 * 4);
  if (lse) touch(lse, (size_t)T * H * 4);
  return hipSuccess;
}
hipError_t launch_decode_indexer(const uint8_t *q8, const float *qs, const float *w, const uint8_t *k8_pool,
                                 const float *ks_pool, const int32_t *bt, int32_t max_blocks, const int32_t *ctx_len,
                                 int32_t B, int32_t max_ctx, int64_t n_pool_rows, float *scores, int64_t ld,
                                 hipStream_t) {
  ++g_launches;
  read_all(q8, (size_t)B * 64 * 128);
  read_all(qs, (size_t)B * 4);
  read_all(w, (size_t)B * 64 * 4);
  read_all(k8_pool, (size_t)n_pool_rows * 128);
  read_all(ks_pool, (size_t)n_pool_rows * 4);
  read_all(bt, (size_t)B * max_blocks * 4);
  read_all(ctx_len, (size_t)B * 4);
  EXPECT(ld >= max_ctx);
  for (int32_t b = 0; b < B; ++b) touch(scores + (size_t)b * ld, (size_t)max_ctx * 4);
  return hipSuccess;
}
hipError_t launch_masked_mha(const void *q, const void *kv, const void *w_uk, const void *w_uv, const int32_t *idx,
                             int32_t L, int32_t H, int32_t k, float, void *out, float *lse, void *workspace,
                             hipStream_t) {
  ++g_launches;
  read_all(q, (size_t)L * H * 192 * 2);
  read_all(kv, (size_t)L * 576 * 2);
  read_all(w_uk, (size_t)H * 128 * 512 * 2);
  read_all(w_uv, (size_t)H * 128 * 512 * 2);
  read_all(idx, (size_t)L * k * 4);
  touch(out, (size_t)L * H * 128 * 2);
  if (lse) touch(lse, (size_t)L * H * 4);
  touch(workspace, masked_mha_workspace_bytes(L, H));
  return hipSuccess;
}
hipError_t launch_indexer_scores_at(const uint8_t *q8, const float *qs, const uint8_t *k8, const float *ks,
                                    const float *w, const int32_t *idx, int32_t T, int32_t S, int32_t H_I, int32_t k,
                                    float *out, hipStream_t) {
  ++g_launches;
  read_all(q8, (size_t)T * H_I * 128);
  read_all(k8, (size_t)S * 128);
  read_all(qs, (size_t)T * 4);
  read_all(ks, (size_t)S * 4);
  read_all(w, (size_t)T * H_I * 4);
  read_all(idx, (size_t)T * k * 4);
  touch(out, (size_t)T * k * 4);
  return hipSuccess;
}
hipError_t launch_indexer_kl(const void *q, const void *kv, const int32_t *idx, const float *scores,
                             const float *lse, int64_t N, int32_t T, int32_t H, int32_t k, float, float *kl,
                             hipStream_t) {
  ++g_launches;
  read_all(q, (size_t)T * H * 576 * 2);
  read_all(kv, (size_t)N * 576 * 2);
  read_all(idx, (size_t)T * k * 4);
  read_all(scores, (size_t)T * k * 4);
  read_all(lse, (size_t)T * H * 4);
  touch(kl, (size_t)T * 4);
  return hipSuccess;
}
hipError_t launch_positions(int32_t *q_pos, int32_t *n_valid, int32_t L, hipStream_t) {
  ++g_launches;
  touch(q_pos, (size_t)L * 4);
  touch(n_valid, (size_t)L * 4);
  return hipSuccess;
}
hipError_t launch_cache_append(const void *latent, const uint8_t *k8, const float *ks, const int32_t *pos, int32_t B,
                               int32_t D_I, const int32_t *bt, int32_t max_blocks, int64_t n_pool_rows, void *kv_pool,
                               uint8_t *k8_pool, float *ks_pool, hipStream_t) {
  ++g_launches;
  read_all(latent, (size_t)B * 576 * 2);
  read_all(k8, (size_t)B * D_I);
  read_all(ks, (size_t)B * 4);
  read_all(pos, (size_t)B * 4);
  read_all(bt, (size_t)B * max_blocks * 4);
  read_all(kv_pool, (size_t)n_pool_rows * 576 * 2);
  read_all(k8_pool, (size_t)n_pool_rows * D_I);
  read_all(ks_pool, (size_t)n_pool_rows * 4);
  return hipSuccess;
}
hipError_t launch_indexer_kl_grad(const void *q, const void *kv, const int32_t *idx, const float *scores,
                                  const float *lse, const float *dkl, int64_t N, int32_t T, int32_t H, int32_t k, float,
                                  float *grad, hipStream_t) {
  ++g_launches;
  read_all(q, (size_t)T * H * 576 * 2);
  read_all(kv, (size_t)N * 576 * 2);
  read_all(idx, (size_t)T * k * 4);
  read_all(scores, (size_t)T * k * 4);
  read_all(lse, (size_t)T * H * 4);
  read_all(dkl, (size_t)T * 4);
  touch(grad, (size_t)T * k * 4);
  return hipSuccess;
}
hipError_t launch_indexer_bwd_chunk(const uint8_t *q8, const float *qs, const uint8_t *k8, const float *ks,
                                    const float *w, const int32_t *idx, const float *grad, int64_t t0, int32_t Tc,
                                    int32_t S, int32_t k, float *dw, float *dq, float *u, hipStream_t) {
  ++g_launches;
  read_all(q8 + t0 * 64 * 128, (size_t)Tc * 64 * 128);
  read_all(qs + t0, (size_t)Tc * 4);
  read_all(k8, (size_t)S * 128);
  read_all(ks, (size_t)S * 4);
  read_all(w + t0 * 64, (size_t)Tc * 64 * 4);
  read_all(idx + t0 * k, (size_t)Tc * k * 4);
  read_all(grad + t0 * k, (size_t)Tc * k * 4);
  touch(dw + t0 * 64, (size_t)Tc * 64 * 4);
  touch(dq + t0 * 64 * 128, (size_t)Tc * 64 * 128 * 4);
  touch(u, (size_t)Tc * k * 128 * 4);
  return hipSuccess;
}
hipError_t launch_scatter_build(const int32_t *idx, int64_t npairs, int64_t N, int32_t *cnt, int32_t *start,
                                int32_t *list, hipStream_t) {
  ++g_launches;
  read_all(idx, (size_t)npairs * 4);
  touch(cnt, (size_t)N * 4);
  touch(start, (size_t)(N + 1) * 4);
  touch(list, (size_t)npairs * 4);
  return hipSuccess;
}
hipError_t launch_scatter_add_bf16(const int32_t *start, const int32_t *list, int64_t N, const void *X, int32_t W,
                                   float *Y, hipStream_t) {
  ++g_launches;
  EXPECT(W % 2 == 0 && W <= 768);
  read_all(start, (size_t)(N + 1) * 4);
  (void)list;
  (void)X;
  touch(Y, (size_t)N * W * 4);
  return hipSuccess;
}
hipError_t launch_scatter_add(const int32_t *start, const int32_t *list, int64_t N, const float *X, int32_t W, float *Y,
                              hipStream_t) {
  ++g_launches;
  read_all(start, (size_t)(N + 1) * 4);
  (void)list;
  (void)X;
  touch(Y, (size_t)N * W * 4);
  return hipSuccess;
}
hipError_t launch_fill_zero_f32(float *p, int64_t n, hipStream_t) {
  ++g_launches;
  touch(p, (size_t)n * 4);
  return hipSuccess;
}
hipError_t launch_mla_bwd_delta(const void *out, const void *dout, int64_t TH, float *D, hipStream_t) {
  ++g_launches;
  read_all(out, (size_t)TH * 512 * 2);
  read_all(dout, (size_t)TH * 512 * 2);
  touch(D, (size_t)TH * 4);
  return hipSuccess;
}
hipError_t launch_mla_bwd_chunk(const void *q, const void *kv, const int32_t *idx, const float *lse, const void *dout,
                                const float *D, int64_t N, int32_t H, int32_t k, float, int64_t t0, int32_t Tc,
                                float *dq, void *dsT, void *pT, void *G, float *psum, hipStream_t) {
  ++g_launches;
  EXPECT(H % 32 == 0 && H <= 128);
  if (psum) touch(psum, (size_t)Tc * (H % 64 == 0 ? H / 64 : H / 32) * k * 4);
  read_all((const char *)q + t0 * H * 576 * 2, (size_t)Tc * H * 576 * 2);
  read_all(kv, (size_t)N * 576 * 2);
  read_all(idx + t0 * k, (size_t)Tc * k * 4);
  read_all(lse + t0 * H, (size_t)Tc * H * 4);
  read_all((const char *)dout + t0 * H * 512 * 2, (size_t)Tc * H * 512 * 2);
  read_all(D + t0 * H, (size_t)Tc * H * 4);
  touch(dq + t0 * H * 576, (size_t)Tc * H * 576 * 4);
  touch(dsT, (size_t)Tc * k * H * 2);
  touch(pT, (size_t)Tc * k * H * 2);
  touch(G, (size_t)Tc * k * 576 * 2);
  return hipSuccess;
}
hipError_t launch_kl_grad_from_head_sums(const int32_t *idx, const float *scores, const float *dkl, const float *psum,
                                         int64_t N, int32_t k, int32_t nhg, int64_t t0, int32_t Tc, float *grad,
                                         hipStream_t) {
  ++g_launches;
  EXPECT(N >= 1 && nhg >= 1);
  read_all(idx + t0 * k, (size_t)Tc * k * 4);
  read_all(scores + t0 * k, (size_t)Tc * k * 4);
  read_all(dkl + t0, (size_t)Tc * 4);
  read_all(psum, (size_t)Tc * nhg * k * 4);
  touch(grad + t0 * k, (size_t)Tc * k * 4);
  return hipSuccess;
}
// the static scratch: a host buffer of the same size, so a request carved past it overflows
static std::vector<unsigned char> g_scratch(size_t(128) << 20);
size_t static_scratch_bytes() { return g_scratch.size(); }
hipError_t static_scratch(hipStream_t, void **ptr) {
  *ptr = g_scratch.data();
  return hipSuccess;
}
}  // namespace dsa

// ------------------------------------------------------------ driver
// Exact-size host buffers: one byte past the end is a redzone.
struct Buf {
  std::vector<unsigned char> v;
  explicit Buf(size_t n) : v(n ? n : 1) {}
  void *p() { return v.size() ? v.data() : nullptr; }
  size_t n() const { return v.size(); }
};

static void check_quantize_and_indexer() {
  Buf x(1000 * 8192 * 4), x8(1000 * 8192), sc(1000 * 4);
  EXPECT(dsa_quantize_e4m3_per_token((float *)x.p(), 1000, 8192, (uint8_t *)x8.p(), (float *)sc.p(), 0) == DSA_OK);
  EXPECT(dsa_quantize_e4m3_per_token((float *)x.p(), 1000, 8190, (uint8_t *)x8.p(), (float *)sc.p(), 0) ==
         DSA_ERR_UNSUPPORTED);
  const int T = 37, S = 1000, HI = 64;
  Buf q(T * HI * 128), k(S * 128), qs(T * 4), ks(S * 4), w(T * HI * 4), pos(T * 4), out((size_t)T * 1005 * 4);
  EXPECT(dsa_indexer_scores(q.p(), (float *)qs.p(), k.p(), (float *)ks.p(), (float *)w.p(), (int32_t *)pos.p(), T, S,
                            HI, 128, DSA_E4M3, (float *)out.p(), 1005, 0) == DSA_OK);
  EXPECT(dsa_indexer_scores(q.p(), (float *)qs.p(), k.p(), (float *)ks.p(), (float *)w.p(), (int32_t *)pos.p(), T, S,
                            HI, 128, DSA_E4M3, (float *)out.p(), 999, 0) == DSA_ERR_INVALID_ARG);
  Buf q4(T * 4 * 64), k4(S * 64), w4(T * 4 * 4);  // the tiny workload's E4M3 indexer: 4 heads of 64 dims
  EXPECT(dsa_indexer_scores(q4.p(), (float *)qs.p(), k4.p(), (float *)ks.p(), (float *)w4.p(), (int32_t *)pos.p(), T,
                            S, 4, 64, DSA_E4M3, (float *)out.p(), 1005, 0) == DSA_OK);
  Buf qf(T * 4 * 64 * 4), kf(S * 64 * 4);
  EXPECT(dsa_indexer_scores(qf.p(), nullptr, kf.p(), nullptr, (float *)w.p(), (int32_t *)pos.p(), T, S, 4, 64,
                            DSA_F32, (float *)out.p(), 1005, 0) == DSA_OK);
}

static void check_topk() {
  for (int T : {1, 4, 64, 512}) {
    for (int64_t n : {(int64_t)300, (int64_t)32768, (int64_t)131072}) {
      Buf sc((size_t)T * n * 4), nv(T * 4), idx((size_t)T * 2048 * 4);
      const size_t wsb = dsa_topk_workspace_bytes(T, n, 2048);
      Buf ws(wsb);
      EXPECT(dsa_topk_select((float *)sc.p(), n, (int32_t *)nv.p(), T, 2048, (int32_t *)idx.p(), wsb ? ws.p() : nullptr,
                             wsb, 0) == DSA_OK);
      EXPECT(dsa_topk_select((float *)sc.p(), n, (int32_t *)nv.p(), T, 2048, (int32_t *)idx.p(), nullptr, 0, 0) ==
             DSA_OK);
    }
  }
  Buf one(4);
  EXPECT(dsa_topk_select((float *)one.p(), 1, (int32_t *)one.p(), 1, 2049, (int32_t *)one.p(), nullptr, 0, 0) ==
         DSA_ERR_UNSUPPORTED);
}

static void check_sparse_mla() {
  const int N = 5000;
  for (int T : {1, 6, 300}) {
    for (int H : {16, 64, 128}) {
      for (int k : {48, 2048}) {
        Buf q((size_t)T * H * 576 * 2), kv((size_t)N * 576 * 2), idx((size_t)T * k * 4), out((size_t)T * H * 512 * 2),
            lse((size_t)T * H * 4);
        const size_t wsb = dsa_sparse_mla_workspace_bytes(T, H, k);
        Buf ws(wsb);
        EXPECT(dsa_sparse_mla_fwd(q.p(), kv.p(), DSA_BF16, (int32_t *)idx.p(), T, H, N, k, 0.07f, out.p(),
                                  (float *)lse.p(), wsb ? ws.p() : nullptr, wsb, 0) == DSA_OK);
        if (wsb)
          EXPECT(dsa_sparse_mla_fwd(q.p(), kv.p(), DSA_BF16, (int32_t *)idx.p(), T, H, N, k, 0.07f, out.p(),
                                    (float *)lse.p(), ws.p(), wsb - 1, 0) == DSA_ERR_WORKSPACE);
      }
    }
  }
}

static dsa_prefill_args prefill_args(int L, dsa_dtype idt, Buf &qi, Buf &qs, Buf &ki, Buf &ks, Buf &w, Buf &q, Buf &kv,
                                     Buf &idx, Buf &out, Buf &lse, int H, int k) {
  dsa_prefill_args a;
  std::memset(&a, 0, sizeof a);
  a.L = L;
  a.H_I = idt == DSA_E4M3 ? 64 : 4;
  a.D_I = idt == DSA_E4M3 ? 128 : 64;
  a.H = H;
  a.k = k;
  a.idx_dt = idt;
  a.q_idx = qi.p();
  a.q_scale = idt == DSA_E4M3 ? (float *)qs.p() : nullptr;
  a.k_idx = ki.p();
  a.k_scale = idt == DSA_E4M3 ? (float *)ks.p() : nullptr;
  a.w = (float *)w.p();
  a.attn_dt = idt == DSA_E4M3 ? DSA_BF16 : DSA_F32;
  a.q = q.p();
  a.kv = kv.p();
  a.sm_scale = 0.07f;
  a.idx = (int32_t *)idx.p();
  a.out = out.p();
  a.lse = (float *)lse.p();
  return a;
}

static void check_prefill() {
  for (int L : {130, 2500}) {
    // E4M3 64 x 128 (fused), F32 4 x 64, and E4M3 4 x 64 (the unfused path with fp32 attention)
    for (int mode = 0; mode < 3; ++mode) {
      const dsa_dtype idt = mode == 1 ? DSA_F32 : DSA_E4M3;
      const bool bf = mode == 0;
      const int H = 16, k = 256, e = idt == DSA_E4M3 ? 1 : 4, HI = mode == 0 ? 64 : 4, DI = mode == 0 ? 128 : 64;
      Buf qi((size_t)L * HI * DI * e), qs(L * 4), ki((size_t)L * DI * e), ks(L * 4), w((size_t)L * HI * 4),
          q((size_t)L * H * 576 * (bf ? 2 : 4)), kv((size_t)L * 576 * (bf ? 2 : 4)), idx((size_t)L * k * 4),
          out((size_t)L * H * 512 * (bf ? 2 : 4)), lse((size_t)L * H * 4);
      dsa_prefill_args a = prefill_args(L, idt, qi, qs, ki, ks, w, q, kv, idx, out, lse, H, k);
      a.H_I = HI;
      a.D_I = DI;
      a.attn_dt = bf ? DSA_BF16 : DSA_F32;
      const size_t wsb = dsa_prefill_workspace_bytes(&a);
      Buf ws(wsb);
      EXPECT(dsa_prefill(&a, ws.p(), wsb, 0) == DSA_OK);
      EXPECT(dsa_prefill_select(&a, ws.p(), wsb, 0) == DSA_OK);
      EXPECT(dsa_prefill(&a, ws.p(), wsb - 1, 0) == DSA_ERR_WORKSPACE);
    }
  }
}

static void check_decode() {
  struct Case {
    int B, max_ctx, H, k;
    bool with_idx;
  };
  for (Case c : {Case{3, 900, 32, 64, false}, Case{64, 32768, 128, 2048, true}, Case{64, 32768, 128, 2048, false},
                 Case{128, 131072, 128, 2048, false}, Case{1, 70, 16, 2048, true}}) {
    const int max_blocks = (c.max_ctx + 63) / 64;
    const int64_t rows = (int64_t)c.B * max_blocks * 64;
    Buf q8((size_t)c.B * 64 * 128), qs(c.B * 4), w((size_t)c.B * 64 * 4), q((size_t)c.B * c.H * 576 * 2),
        k8p((size_t)rows * 128), ksp((size_t)rows * 4), kvp((size_t)rows * 576 * 2), bt((size_t)c.B * max_blocks * 4),
        ctx(c.B * 4), idx((size_t)c.B * c.k * 4), out((size_t)c.B * c.H * 512 * 2), lse((size_t)c.B * c.H * 4);
    dsa_decode_args a;
    std::memset(&a, 0, sizeof a);
    a.B = c.B;
    a.H_I = 64;
    a.D_I = 128;
    a.H = c.H;
    a.k = c.k;
    a.q8 = (uint8_t *)q8.p();
    a.q_scale = (float *)qs.p();
    a.w = (float *)w.p();
    a.q = q.p();
    a.k8_pool = (uint8_t *)k8p.p();
    a.ks_pool = (float *)ksp.p();
    a.kv_pool = kvp.p();
    a.n_pool_rows = rows;
    a.block_table = (int32_t *)bt.p();
    a.max_blocks = max_blocks;
    a.ctx_len = (int32_t *)ctx.p();
    a.max_ctx = c.max_ctx;
    a.sm_scale = 0.07f;
    a.idx_out = c.with_idx ? (int32_t *)idx.p() : nullptr;
    a.out = out.p();
    a.lse = (float *)lse.p();
    const size_t wsb = dsa_decode_workspace_bytes(&a);
    Buf ws(wsb);
    EXPECT(dsa_decode(&a, ws.p(), wsb, 0) == DSA_OK);
    EXPECT(dsa_decode(&a, ws.p(), wsb - 1, 0) == DSA_ERR_WORKSPACE);
    EXPECT(dsa_decode_noalloc(&a, 0) == (wsb <= dsa_decode_static_scratch_bytes() ? DSA_OK : DSA_ERR_UNSUPPORTED));
    Buf sc((size_t)c.B * c.max_ctx * 4);
    EXPECT(dsa_decode_indexer_scores(&a, (float *)sc.p(), c.max_ctx, 0) == DSA_OK);
    const size_t mwsb = dsa_sparse_mla_workspace_bytes(c.B, c.H, c.k);
    Buf mws(mwsb);
    EXPECT(dsa_sparse_mla_paged_fwd(q.p(), kvp.p(), rows, (int32_t *)bt.p(), max_blocks, (int32_t *)idx.p(), c.B, c.H,
                                    c.k, 0.07f, out.p(), (float *)lse.p(), mwsb ? mws.p() : nullptr, mwsb,
                                    0) == DSA_OK);
    Buf lat((size_t)c.B * 576 * 2), tk8((size_t)c.B * 128), tks(c.B * 4), pos(c.B * 4);
    EXPECT(dsa_paged_cache_append(lat.p(), (uint8_t *)tk8.p(), (float *)tks.p(), (int32_t *)pos.p(), c.B, 128,
                                  (int32_t *)bt.p(), max_blocks, kvp.p(), (uint8_t *)k8p.p(), (float *)ksp.p(), rows,
                                  0) == DSA_OK);
  }
}

static void check_indexer_backward() {
  for (int T : {1, 37, 1500}) {
    const int S = 3000, k = 2048;
    Buf q_att((size_t)T * 128 * 576 * 2), kv((size_t)S * 576 * 2), idx((size_t)T * k * 4), sc((size_t)T * k * 4),
        lse((size_t)T * 128 * 4), dkl(T * 4), grad((size_t)T * k * 4), q8((size_t)T * 64 * 128), qs(T * 4),
        k8((size_t)S * 128), ks(S * 4), w((size_t)T * 64 * 4), dw((size_t)T * 64 * 4), dq((size_t)T * 64 * 128 * 4),
        dk((size_t)S * 128 * 4);
    EXPECT(dsa_indexer_kl_bwd(q_att.p(), kv.p(), (int32_t *)idx.p(), (float *)sc.p(), (float *)lse.p(),
                              (float *)dkl.p(), T, 128, S, k, 0.07f, (float *)grad.p(), 0) == DSA_OK);
    const size_t wsb = dsa_indexer_bwd_workspace_bytes(T, S, k);
    Buf ws(wsb);
    EXPECT(dsa_indexer_bwd((uint8_t *)q8.p(), (float *)qs.p(), (uint8_t *)k8.p(), (float *)ks.p(), (float *)w.p(),
                           (int32_t *)idx.p(), (float *)grad.p(), T, S, 64, 128, k, (float *)dw.p(), (float *)dq.p(),
                           (float *)dk.p(), ws.p(), wsb, 0) == DSA_OK);
    EXPECT(dsa_indexer_bwd((uint8_t *)q8.p(), (float *)qs.p(), (uint8_t *)k8.p(), (float *)ks.p(), (float *)w.p(),
                           (int32_t *)idx.p(), (float *)grad.p(), T, S, 64, 128, k, (float *)dw.p(), (float *)dq.p(),
                           (float *)dk.p(), ws.p(), wsb - 1, 0) == DSA_ERR_WORKSPACE);
  }
}

static void check_mla_backward() {
  for (int T : {1, 6, 700}) {
    for (int H : {32, 96, 128}) {
      const int N = 2500, k = 2048;
      Buf q((size_t)T * H * 576 * 2), kv((size_t)N * 576 * 2), idx((size_t)T * k * 4), out((size_t)T * H * 512 * 2),
          lse((size_t)T * H * 4), dout((size_t)T * H * 512 * 2), dq((size_t)T * H * 576 * 4), dkv((size_t)N * 576 * 4);
      const size_t wsb = dsa_sparse_mla_bwd_workspace_bytes(T, H, N, k);
      Buf ws(wsb);
      EXPECT(dsa_sparse_mla_bwd(q.p(), kv.p(), (int32_t *)idx.p(), out.p(), (float *)lse.p(), dout.p(), T, H, N, k,
                                0.07f, (float *)dq.p(), (float *)dkv.p(), ws.p(), wsb, 0) == DSA_OK);
      EXPECT(dsa_sparse_mla_bwd(q.p(), kv.p(), (int32_t *)idx.p(), out.p(), (float *)lse.p(), dout.p(), T, H, N, k,
                                0.07f, (float *)dq.p(), (float *)dkv.p(), ws.p(), wsb - 1, 0) == DSA_ERR_WORKSPACE);
      // the same with the KL score gradient from the same P
      Buf sc((size_t)T * k * 4), dkl((size_t)T * 4), grad((size_t)T * k * 4);
      EXPECT(dsa_sparse_mla_bwd_kl(q.p(), kv.p(), (int32_t *)idx.p(), out.p(), (float *)lse.p(), dout.p(),
                                   (float *)sc.p(), (float *)dkl.p(), T, H, N, k, 0.07f, (float *)dq.p(),
                                   (float *)dkv.p(), (float *)grad.p(), ws.p(), wsb, 0) == DSA_OK);
      EXPECT(dsa_sparse_mla_bwd_kl(q.p(), kv.p(), (int32_t *)idx.p(), out.p(), (float *)lse.p(), dout.p(),
                                   (float *)sc.p(), (float *)dkl.p(), T, H, N, k, 0.07f, (float *)dq.p(),
                                   (float *)dkv.p(), (float *)grad.p(), ws.p(), wsb - 1, 0) == DSA_ERR_WORKSPACE);
      EXPECT(dsa_sparse_mla_bwd_kl(q.p(), kv.p(), (int32_t *)idx.p(), out.p(), (float *)lse.p(), dout.p(), nullptr,
                                   (float *)dkl.p(), T, H, N, k, 0.07f, (float *)dq.p(), (float *)dkv.p(),
                                   (float *)grad.p(), ws.p(), wsb, 0) == DSA_ERR_INVALID_ARG);
    }
  }
  Buf one(64);
  EXPECT(dsa_sparse_mla_bwd(one.p(), one.p(), (int32_t *)one.p(), one.p(), (float *)one.p(), one.p(), 1, 16, 1, 1,
                            0.07f, (float *)one.p(), (float *)one.p(), one.p(), 64, 0) == DSA_ERR_UNSUPPORTED);
}

static void check_training_side() {
  const int T = 50, H = 128, k = 2048, S = 3000, L = 700;
  Buf q8((size_t)T * 64 * 128), qs(T * 4), k8((size_t)S * 128), ks(S * 4), w((size_t)T * 64 * 4),
      idx((size_t)T * k * 4), sc((size_t)T * k * 4), q((size_t)T * H * 576 * 2), kv((size_t)S * 576 * 2),
      lse((size_t)T * H * 4), kl(T * 4);
  EXPECT(dsa_indexer_scores_at((uint8_t *)q8.p(), (float *)qs.p(), (uint8_t *)k8.p(), (float *)ks.p(), (float *)w.p(),
                               (int32_t *)idx.p(), T, S, 64, 128, k, (float *)sc.p(), 0) == DSA_OK);
  EXPECT(dsa_indexer_kl_fwd(q.p(), kv.p(), (int32_t *)idx.p(), (float *)sc.p(), (float *)lse.p(), T, H, S, k, 0.07f,
                            (float *)kl.p(), 0) == DSA_OK);
  Buf mq((size_t)L * H * 192 * 2), mkv((size_t)L * 576 * 2), wuk((size_t)H * 128 * 512 * 2),
      wuv((size_t)H * 128 * 512 * 2), midx((size_t)L * k * 4), mout((size_t)L * H * 128 * 2), mlse((size_t)L * H * 4);
  const size_t wsb = dsa_masked_mha_workspace_bytes(L, H);
  Buf ws(wsb);
  EXPECT(dsa_masked_mha_prefill(mq.p(), mkv.p(), wuk.p(), wuv.p(), (int32_t *)midx.p(), L, H, k, 0.07f, mout.p(),
                                (float *)mlse.p(), ws.p(), wsb, 0) == DSA_OK);
}

int main() {
  check_quantize_and_indexer();
  check_topk();
  check_sparse_mla();
  check_prefill();
  check_decode();
  check_training_side();
  check_indexer_backward();
  check_mla_backward();
  {  // a decode too large for the static scratch is refused before any launch
    dsa_decode_args a;
    std::memset(&a, 0, sizeof a);
    a.B = 1024;
    a.H_I = 64;
    a.D_I = 128;
    a.H = 128;
    a.k = 2048;
    a.max_ctx = 131072;
    a.max_blocks = 2048;
    a.n_pool_rows = 64;
    a.sm_scale = 0.07f;
    Buf fake(64);
    a.q8 = (uint8_t *)fake.p(), a.q_scale = (float *)fake.p(), a.w = (float *)fake.p(), a.q = fake.p();
    a.k8_pool = (uint8_t *)fake.p(), a.ks_pool = (float *)fake.p(), a.kv_pool = fake.p();
    a.block_table = (int32_t *)fake.p(), a.ctx_len = (int32_t *)fake.p(), a.out = fake.p();
    const int before = g_launches;
    EXPECT(dsa_decode_workspace_bytes(&a) > dsa_decode_static_scratch_bytes());
    EXPECT(dsa_decode_noalloc(&a, 0) == DSA_ERR_UNSUPPORTED);
    EXPECT(std::strstr(dsa_last_error(), "static scratch") != nullptr);
    EXPECT(g_launches == before);
  }
  EXPECT(g_launches > 50);
  std::printf("capi host check ok: %d stubbed launches\n", g_launches);
  return 0;
}
