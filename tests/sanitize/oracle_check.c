/*
 * oracle_check.c -- runs every function of oracle/dsa_oracle.c on small
 * inputs, edge cases included (empty and padded selections, k above the row
 * length, a query at position 0, entries outside the table, zero rows), in a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer.  Each output
 * buffer is exactly as large as the function's contract says, so a write past
 * it is a heap overflow that ASan reports.  The values are not checked here
 * (the pins in tests/test_oracle_pins.py do that); only memory safety and
 * defined behaviour.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

enum { F32 = 0, BF16 = 1, E4M3 = 2, F64 = 3 };

double ora_e4m3_decode(uint8_t c);
double ora_bf16_decode(uint16_t h);
uint8_t ora_e4m3_encode(float x);
void ora_quantize_rows(const float *x, int64_t rows, int32_t cols, uint8_t *x8, float *scale);
void ora_indexer_rows(int dtype, const void *q, const float *q_scale, const void *k, const float *k_scale,
                      const float *w, const int32_t *q_pos, int64_t T, int64_t S, int32_t H_I, int32_t D_I,
                      const int64_t *rows, int64_t nrows, double *out);
int64_t ora_topk_row(const double *scores, int64_t n, int32_t k, int32_t *idx, double *tau);
void ora_topk_rows(const double *scores, int64_t ld, const int64_t *n_valid, int64_t nrows, int32_t k, int32_t *idx,
                   double *tau);
void ora_sparse_mla_rows(int dtype, const void *q, const void *kv, const int32_t *idx, int64_t T, int32_t H, int64_t N,
                         int32_t k, int32_t Dqk, int32_t Dv, double sm_scale, const int64_t *rows, int64_t nrows,
                         double *o, double *lse);
void ora_indexer_kl_rows(int dtype, const void *q, const void *kv, const int32_t *idx, const double *scores, int32_t H,
                         int32_t k, int32_t Dqk, double sm_scale, const int64_t *rows, int64_t nrows, double *kl,
                         double *mag);
void ora_decode(const uint8_t *q8, const float *qs, const float *w, const uint16_t *q, const uint8_t *k8_pool,
                const float *ks_pool, const uint16_t *kv_pool, const int32_t *block_table, int32_t max_blocks,
                const int32_t *ctx, int32_t B, int32_t H_I, int32_t D_I, int32_t H, int32_t k, int32_t Dqk, int32_t Dv,
                double sm_scale, const int64_t *seqs, int64_t nseq, int32_t *idx, double *tau, double *o, double *lse);
void ora_paged_cache_append(const uint16_t *latent, const uint8_t *k8, const float *ks, const int32_t *pos, int32_t B,
                            int32_t D_I, int32_t Dqk, const int32_t *block_table, int32_t max_blocks,
                            int64_t n_pool_rows, uint16_t *kv_pool, uint8_t *k8_pool, float *ks_pool);
void ora_masked_mha_rows(int dtype, const void *q, const void *kv, const void *w_uk, const void *w_uv,
                         const int32_t *idx, int32_t H, int32_t k, int32_t Dc, int32_t Dr, int32_t Dn, int32_t Dvh,
                         double sm_scale, const int64_t *rows, int64_t nrows, double *o, double *lse);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return (uint32_t)(g_state >> 11);
}
static float rndf(void) { return (float)((int)(rnd() % 2001) - 1000) / 500.0f; }
static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) abort();
    return p;
}
static float *rand_f32(size_t n) {
    float *p = (float *)xmalloc(n * sizeof(float));
    for (size_t i = 0; i < n; ++i) p[i] = rndf();
    return p;
}
static uint16_t *rand_bf16(size_t n) {
    uint16_t *p = (uint16_t *)xmalloc(n * sizeof(uint16_t));
    for (size_t i = 0; i < n; ++i) {
        float f = rndf() * 0.05f;
        uint32_t b;
        memcpy(&b, &f, 4);
        p[i] = (uint16_t)(b >> 16);
    }
    return p;
}
static uint8_t *rand_e4m3(size_t n) {
    uint8_t *p = (uint8_t *)xmalloc(n);
    for (size_t i = 0; i < n; ++i) p[i] = ora_e4m3_encode(rndf() * 3.0f);
    return p;
}

static void check_codecs(void) {
    volatile double acc = 0.0;
    for (int c = 0; c < 256; ++c) acc += isnan(ora_e4m3_decode((uint8_t)c)) ? 0.0 : ora_e4m3_decode((uint8_t)c);
    for (int h = 0; h < 65536; h += 7) acc += isfinite(ora_bf16_decode((uint16_t)h)) ? 1.0 : 0.0;
    const float special[] = {0.0f, -0.0f, 1e30f, -1e30f, 448.0f, 464.0f, 1e-10f, INFINITY, -INFINITY};
    for (size_t i = 0; i < sizeof special / sizeof *special; ++i) acc += ora_e4m3_encode(special[i]);
    (void)acc;
    float x[3 * 12];
    for (int i = 0; i < 36; ++i) x[i] = rndf();
    memset(x + 12, 0, 12 * sizeof(float)); /* an all-zero row */
    uint8_t *x8 = (uint8_t *)xmalloc(36);
    float *sc = (float *)xmalloc(3 * sizeof(float));
    ora_quantize_rows(x, 3, 12, x8, sc);
    free(x8);
    free(sc);
}

static void check_indexer_topk(void) {
    const int T = 9, S = 70, HI = 4, DI = 16, K = 32;
    uint8_t *q8 = rand_e4m3((size_t)T * HI * DI), *k8 = rand_e4m3((size_t)S * DI);
    float *qs = rand_f32(T), *ks = rand_f32(S), *w = rand_f32((size_t)T * HI);
    float *qf = rand_f32((size_t)T * HI * DI), *kf = rand_f32((size_t)S * DI);
    for (int i = 0; i < T; ++i) qs[i] = fabsf(qs[i]) + 0.5f;
    for (int i = 0; i < S; ++i) ks[i] = fabsf(ks[i]) + 0.5f;
    int32_t pos[9] = {0, 1, 5, 31, 32, 33, 60, 69, 69};
    int64_t rows[4] = {0, 3, 7, 8};
    double *out = (double *)xmalloc(sizeof(double) * 4 * S);
    ora_indexer_rows(E4M3, q8, qs, k8, ks, w, pos, T, S, HI, DI, rows, 4, out);
    ora_indexer_rows(F32, qf, NULL, kf, NULL, w, pos, T, S, HI, DI, rows, 4, out);
    /* top-k of each row: n below, at and above k; n = 0 */
    int32_t *idx = (int32_t *)xmalloc(sizeof(int32_t) * 4 * K);
    double tau[4];
    int64_t nv[4] = {0, 4, 32, 70};
    for (int r = 0; r < 4; ++r) out[r * S + 3] = out[r * S + 5]; /* a tie */
    ora_topk_rows(out, S, nv, 4, K, idx, tau);
    (void)ora_topk_row(out, 1, K, idx, tau);
    (void)ora_topk_row(out, 0, 1, idx, tau);
    free(q8), free(k8), free(qs), free(ks), free(w), free(qf), free(kf), free(out), free(idx);
}

static void check_attention(void) {
    const int T = 5, H = 3, N = 50, K = 40, Dqk = 24, Dv = 16;
    uint16_t *q = rand_bf16((size_t)T * H * Dqk), *kv = rand_bf16((size_t)N * Dqk);
    int32_t *idx = (int32_t *)xmalloc(sizeof(int32_t) * T * K);
    for (int t = 0; t < T; ++t)
        for (int a = 0; a < K; ++a) idx[t * K + a] = (int32_t)(rnd() % N);
    for (int a = 0; a < K; ++a) idx[1 * K + a] = -1; /* empty selection */
    for (int a = K / 2; a < K; ++a) idx[2 * K + a] = -1;
    int64_t rows[3] = {0, 1, 2};
    double *o = (double *)xmalloc(sizeof(double) * 3 * H * Dv), *lse = (double *)xmalloc(sizeof(double) * 3 * H);
    ora_sparse_mla_rows(BF16, q, kv, idx, T, H, N, K, Dqk, Dv, 0.125, rows, 3, o, lse);
    float *qf = rand_f32((size_t)T * H * Dqk), *kvf = rand_f32((size_t)N * Dqk);
    ora_sparse_mla_rows(F32, qf, kvf, idx, T, H, N, K, Dqk, Dv, 0.125, rows, 3, o, lse);
    double *sc = (double *)xmalloc(sizeof(double) * T * K), kl[3], mag[3];
    for (int i = 0; i < T * K; ++i) sc[i] = rndf();
    ora_indexer_kl_rows(BF16, q, kv, idx, sc, H, K, Dqk, 0.125, rows, 3, kl, mag);
    /* masked MHA: Dc = 16 compressed + Dr = 8 rope dims, per-head Dn = 8, Dvh = 8.  This oracle takes
     * every non-negative entry as a row of kv (it is given no row count): entries the mode ignores are
     * handed to it as -1, as the parity tests do. */
    const int Dc = 16, Dr = 8, Dn = 8, Dvh = 8, L = 20, MK = 12;
    uint16_t *mq = rand_bf16((size_t)L * H * (Dn + Dr)), *mkv = rand_bf16((size_t)L * (Dc + Dr));
    uint16_t *wuk = rand_bf16((size_t)H * Dn * Dc), *wuv = rand_bf16((size_t)H * Dvh * Dc);
    int32_t *midx = (int32_t *)xmalloc(sizeof(int32_t) * L * MK);
    for (int t = 0; t < L; ++t)
        for (int a = 0; a < MK; ++a) midx[t * MK + a] = a <= t ? t - a : -1; /* causal, then padding */
    int64_t mrows[4] = {0, 1, 11, 19};
    double *mo = (double *)xmalloc(sizeof(double) * 4 * H * Dvh), *ml = (double *)xmalloc(sizeof(double) * 4 * H);
    ora_masked_mha_rows(BF16, mq, mkv, wuk, wuv, midx, H, MK, Dc, Dr, Dn, Dvh, 0.2, mrows, 4, mo, ml);
    free(q), free(kv), free(idx), free(o), free(lse), free(qf), free(kvf), free(sc);
    free(mq), free(mkv), free(wuk), free(wuv), free(midx), free(mo), free(ml);
}

static void check_decode_and_append(void) {
    const int B = 3, HI = 4, DI = 16, H = 2, K = 40, Dqk = 24, Dv = 16, MAXB = 3;
    const int32_t ctx[3] = {1, 64, 130};
    int32_t bt[9] = {4, -1, -1, 2, -1, -1, 0, 3, 1}; /* 5 pages, one unused */
    const int64_t nrows = 5 * 64;
    uint8_t *q8 = rand_e4m3((size_t)B * HI * DI), *k8p = rand_e4m3((size_t)nrows * DI);
    float *qs = rand_f32(B), *w = rand_f32((size_t)B * HI), *ksp = rand_f32(nrows);
    for (int i = 0; i < B; ++i) qs[i] = fabsf(qs[i]) + 0.5f;
    for (int i = 0; i < nrows; ++i) ksp[i] = fabsf(ksp[i]) + 0.5f;
    uint16_t *q = rand_bf16((size_t)B * H * Dqk), *kvp = rand_bf16((size_t)nrows * Dqk);
    int64_t seqs[3] = {0, 1, 2};
    int32_t *idx = (int32_t *)xmalloc(sizeof(int32_t) * B * K);
    double tau[3], *o = (double *)xmalloc(sizeof(double) * B * H * Dv), *lse = (double *)xmalloc(sizeof(double) * B * H);
    ora_decode(q8, qs, w, q, k8p, ksp, kvp, bt, MAXB, ctx, B, HI, DI, H, K, Dqk, Dv, 0.125, seqs, 3, idx, tau, o, lse);
    uint16_t *lat = rand_bf16((size_t)B * Dqk);
    uint8_t *tk8 = rand_e4m3((size_t)B * DI);
    float *tks = rand_f32(B);
    int32_t pos[3] = {1, 64, 3 * 64}; /* in the table, a new page, past the table */
    int32_t bt2[9] = {4, -1, -1, 2, -1, -1, 0, 3, 1};
    ora_paged_cache_append(lat, tk8, tks, pos, B, DI, Dqk, bt2, MAXB, nrows, kvp, k8p, ksp);
    int32_t pos2[3] = {-5, 70, 10};
    ora_paged_cache_append(lat, tk8, tks, pos2, B, DI, Dqk, bt2, MAXB, nrows, kvp, k8p, ksp);
    free(q8), free(k8p), free(qs), free(w), free(ksp), free(q), free(kvp), free(idx), free(o), free(lse);
    free(lat), free(tk8), free(tks);
}

int main(void) {
    check_codecs();
    check_indexer_topk();
    check_attention();
    check_decode_and_append();
    printf("oracle check ok\n");
    return 0;
}
