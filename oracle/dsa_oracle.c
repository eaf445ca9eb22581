/*
 * dsa_oracle.c -- plain, slow, fp64 CPU oracle for the DeepSeek Sparse Attention
 * (DSA) hot path: lightning indexer -> per-query top-k -> sparse MLA (MQA mode).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library shares
 * no code, header, table or helper with it.
 *
 * What is computed, and where it is stated:
 *  - The indexer gives every query token an "index score" against each
 *    preceding token, with few heads, a ReLU activation and FP8 operands
 *    (mizuki-eaf.pages.dev, "DeepSeek Sparse Attention" / "How it works";
 *    m.digipub.cc, section 2).  The score formula
 *        I[t,s] = sum_j w[t,j] * ReLU( q_I[t,j] . k_I[s] )
 *    and the per-token fp32 scales of the FP8 operands are the workload's
 *    definition; the pages name only "few heads, ReLU, FP8".
 *  - Each query keeps the key/value entries with the top-k index scores,
 *    k = 2048 (mizuki-eaf.pages.dev, same section, and its "DSA key
 *    parameters" table; m.36881.com.cn, "Fine-grained Token Selection").
 *  - Main attention is MLA in MQA mode: one latent vector per token is shared
 *    by all query heads of a query token (mizuki-eaf.pages.dev, "built on
 *    MLA"); the latent is 576-dim (512 + 64 rope) and its first 512 dims are
 *    the value.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of the repository):
 *  - "preceding tokens" includes the query's own position: candidates of the
 *    query at position p are s in [0, p], so a query selects min(k, p+1).
 *  - ties in the index score are broken toward the larger (more recent)
 *    position; the order is (score descending, position descending).
 *  - -0 scores are canonicalised to +0.
 *  - FP8 is OCP E4M3FN (bias 7, max 448, no infinities, S.1111.111 = NaN).
 *  - per-token quantisation: scale = amax(|x_row|)/448 in fp32 (1 when the
 *    row is all zero); payload = RNE-to-E4M3, saturating at +-448, of the fp32
 *    quotient x/scale.
 *  - an empty selected set gives o = 0 and lse = -inf.
 *  - the masked-MHA mode for short prefill (mizuki-eaf.pages.dev, "parity
 *    evaluation"; m.digipub.cc, section 2) is read as MLA in its multi-head
 *    form: every head gets its own key (the latent's 512 dims up-projected to
 *    128, plus the shared 64 rope dims) and value (the latent up-projected to
 *    128), and attends densely over its causal positions with every position
 *    outside the query's top-k selection masked out.
 *  - the indexer's KL-alignment loss (mizuki-eaf.pages.dev, two-stage
 *    continued pre-training; m.36881.com.cn, dense warm-up and sparse
 *    training; m.digipub.cc, section 2) is read per query token t as
 *    KL(p_t || pi_t) over a set S_t of positions: p_t is the main attention
 *    distribution of t over S_t aggregated over heads (the heads' softmaxes
 *    summed and L1-normalised, i.e. averaged), pi_t the softmax of t's index
 *    scores over S_t.  S_t is the top-k selection in sparse training and all
 *    causal positions in the dense warm-up.  The loss value is per token; how
 *    tokens are summed or averaged is left to the caller.
 *
 * Every floating-point accumulation here is fp64, in the plain loop order of
 * the definition; nothing is blocked, fused or reordered.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ codecs */

/* OCP 8-bit floating point spec v1.0, E4M3: bias 7; e=0 is subnormal with
 * value m/8 * 2^-6; e=15,m=7 is NaN; no infinities. */
double ora_e4m3_decode(uint8_t c)
{
    int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* bf16 is the top half of an IEEE binary32. */
double ora_bf16_decode(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* fp32 -> E4M3 with round-to-nearest-even and saturation at +-448. */
uint8_t ora_e4m3_encode(float x)
{
    uint8_t sign;
    double a, step, q, v;
    int E;
    if (isnan(x))
        return 0x7F;
    sign = signbit(x) ? 0x80 : 0x00;
    a = fabs((double)x);
    if (a >= 448.0)
        return sign | 0x7E;
    if (a == 0.0)
        return sign;
    /* exponent of a; below the smallest normal (2^-6) the grid step is 2^-9 */
    E = ilogb(a);
    if (E < -6)
        E = -6;
    step = ldexp(1.0, E - 3);       /* 3 mantissa bits */
    q = rint(a / step);             /* exact quotient, RNE (default rounding mode) */
    v = q * step;                   /* rounded magnitude, on the E4M3 grid */
    if (v >= 448.0)
        return sign | 0x7E;
    if (v == 0.0)
        return sign;
    if (v < ldexp(1.0, -6))         /* subnormal: m * 2^-9 */
        return sign | (uint8_t)(v / ldexp(1.0, -9));
    E = ilogb(v);
    return sign | (uint8_t)(((E + 7) << 3) | ((int)(v / ldexp(1.0, E - 3)) - 8));
}

/* Per-row quantisation of an fp32 matrix [rows, cols] to E4M3 + fp32 scale. */
void ora_quantize_rows(const float *x, int64_t rows, int32_t cols, uint8_t *x8, float *scale)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        const float *xr = x + r * (int64_t)cols;
        float amax = 0.0f, s;
        int32_t c;
        for (c = 0; c < cols; ++c) {
            float a = fabsf(xr[c]);
            if (a > amax)
                amax = a;
        }
        s = amax / 448.0f;          /* fp32 division, correctly rounded */
        if (!(s > 0.0f))
            s = 1.0f;
        scale[r] = s;
        for (c = 0; c < cols; ++c) {
            float qf = xr[c] / s;   /* fp32 quotient, then one rounding to E4M3 */
            x8[r * (int64_t)cols + c] = ora_e4m3_encode(qf);
        }
    }
}

/* ----------------------------------------------------------------- indexer */

enum { ORA_F32 = 0, ORA_BF16 = 1, ORA_E4M3 = 2, ORA_F64 = 3 };

static double elem(int dtype, const void *p, int64_t i)
{
    if (dtype == ORA_E4M3)
        return ora_e4m3_decode(((const uint8_t *)p)[i]);
    if (dtype == ORA_BF16)
        return ora_bf16_decode(((const uint16_t *)p)[i]);
    if (dtype == ORA_F64)
        return ((const double *)p)[i];
    return (double)((const float *)p)[i];
}

/*
 * Index scores of selected query rows.
 *   q  [T, H_I, D_I]  (E4M3 payload with q_scale[T], or F32 with no scale)
 *   k  [S, D_I]       (same dtype; k_scale[S] for E4M3)
 *   w  [T, H_I] fp32, q_pos[T]
 * For each i < nrows, t = rows[i]:
 *   out[i, s] = sum_j w[t,j] * max(0, sum_d (qs[t] q[t,j,d]) * (ks[s] k[s,d]))
 *               for s <= q_pos[t]   (and s < S),
 *   out[i, s] = -inf otherwise.
 */
void ora_indexer_rows(int dtype, const void *q, const float *q_scale, const void *k,
                      const float *k_scale, const float *w, const int32_t *q_pos, int64_t T,
                      int64_t S, int32_t H_I, int32_t D_I, const int64_t *rows, int64_t nrows,
                      double *out)
{
    int64_t i;
    (void)T;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < nrows; ++i) {
        int64_t t = rows[i], s;
        int64_t p = q_pos[t];
        double *o = out + i * S;
        double *qv = (double *)malloc(sizeof(double) * (size_t)H_I * (size_t)D_I);
        double *kv = (double *)malloc(sizeof(double) * (size_t)D_I);
        double qs = (dtype == ORA_E4M3) ? (double)q_scale[t] : 1.0;
        int32_t j, d;
        for (j = 0; j < H_I; ++j)
            for (d = 0; d < D_I; ++d)
                qv[j * D_I + d] = qs * elem(dtype, q, (t * H_I + j) * (int64_t)D_I + d);
        for (s = 0; s < S; ++s) {
            double ks, acc = 0.0;
            if (s > p) {
                o[s] = -INFINITY;
                continue;
            }
            ks = (dtype == ORA_E4M3) ? (double)k_scale[s] : 1.0;
            for (d = 0; d < D_I; ++d)
                kv[d] = ks * elem(dtype, k, s * (int64_t)D_I + d);
            for (j = 0; j < H_I; ++j) {
                double dot = 0.0;
                for (d = 0; d < D_I; ++d)
                    dot += qv[j * D_I + d] * kv[d];
                acc += (double)w[t * H_I + j] * (dot > 0.0 ? dot : 0.0);
            }
            o[s] = (acc == 0.0) ? 0.0 : acc;   /* -0 -> +0 */
        }
        free(qv);
        free(kv);
    }
}

/* ------------------------------------------------------------------- top-k */

typedef struct {
    double v;
    int64_t pos;
} cand_t;

/* (score descending, position descending) */
static int cand_cmp(const void *a, const void *b)
{
    const cand_t *x = (const cand_t *)a, *y = (const cand_t *)b;
    if (x->v > y->v)
        return -1;
    if (x->v < y->v)
        return 1;
    if (x->pos > y->pos)
        return -1;
    if (x->pos < y->pos)
        return 1;
    return 0;
}

static int i32_cmp(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/*
 * Top-k of one row of n candidate scores (positions 0..n-1).  Writes the
 * K = min(k, n) kept positions to idx[0..K) in ascending position order,
 * -1 to idx[K..k), and returns K.  *tau = score of the K-th kept candidate
 * (-inf if K = 0).
 */
int64_t ora_topk_row(const double *scores, int64_t n, int32_t k, int32_t *idx, double *tau)
{
    int64_t K = n < k ? n : k, i;
    cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)(n > 0 ? n : 1));
    for (i = 0; i < n; ++i) {
        c[i].v = scores[i];
        c[i].pos = i;
    }
    qsort(c, (size_t)n, sizeof(cand_t), cand_cmp);
    for (i = 0; i < K; ++i)
        idx[i] = (int32_t)c[i].pos;
    qsort(idx, (size_t)K, sizeof(int32_t), i32_cmp);
    for (i = K; i < k; ++i)
        idx[i] = -1;
    *tau = K > 0 ? c[K - 1].v : -INFINITY;
    free(c);
    return K;
}

/* Row-wise top-k over a [nrows, ld] score matrix with per-row candidate counts. */
void ora_topk_rows(const double *scores, int64_t ld, const int64_t *n_valid, int64_t nrows,
                   int32_t k, int32_t *idx, double *tau)
{
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < nrows; ++i)
        ora_topk_row(scores + i * ld, n_valid[i], k, idx + i * (int64_t)k, tau + i);
}

/* ------------------------------------------------------------- sparse MLA */

/*
 * Sparse MLA in MQA mode for selected query rows.
 *   q   [T, H, Dqk]  (F32 or BF16)
 *   kv  [N, Dqk]     (same dtype); the value of row r is kv[r, 0..Dv)
 *   idx [T, k]       row indices into kv; -1 entries are skipped
 * For t = rows[i] and every head h, over the valid entries r_1..r_m of idx[t]:
 *   z_a = sm_scale * sum_d q[t,h,d] kv[r_a,d]
 *   o[i,h,:] = sum_a softmax(z)_a kv[r_a, 0..Dv)
 *   lse[i,h] = log sum_a exp(z_a)       (natural log)
 * with m = 0 giving o = 0, lse = -inf.
 */
void ora_sparse_mla_rows(int dtype, const void *q, const void *kv, const int32_t *idx, int64_t T,
                         int32_t H, int64_t N, int32_t k, int32_t Dqk, int32_t Dv, double sm_scale,
                         const int64_t *rows, int64_t nrows, double *o, double *lse)
{
    int64_t i;
    (void)T;
    (void)N;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < nrows; ++i) {
        int64_t t = rows[i];
        const int32_t *sel = idx + t * (int64_t)k;
        double *z = (double *)malloc(sizeof(double) * (size_t)k);
        double *qh = (double *)malloc(sizeof(double) * (size_t)Dqk);
        int32_t h;
        for (h = 0; h < H; ++h) {
            double *oh = o + (i * H + h) * (int64_t)Dv;
            double mx = -INFINITY, sum = 0.0;
            int32_t a, d, m = 0;
            for (d = 0; d < Dqk; ++d)
                qh[d] = elem(dtype, q, (t * H + h) * (int64_t)Dqk + d);
            for (d = 0; d < Dv; ++d)
                oh[d] = 0.0;
            for (a = 0; a < k; ++a) {
                double dot = 0.0;
                int64_t r = sel[a];
                if (r < 0) {
                    z[a] = -INFINITY;
                    continue;
                }
                for (d = 0; d < Dqk; ++d)
                    dot += qh[d] * elem(dtype, kv, r * Dqk + d);
                z[a] = sm_scale * dot;
                if (z[a] > mx)
                    mx = z[a];
                ++m;
            }
            if (m == 0) {
                lse[i * H + h] = -INFINITY;
                continue;
            }
            for (a = 0; a < k; ++a)
                if (sel[a] >= 0)
                    sum += exp(z[a] - mx);
            for (a = 0; a < k; ++a) {
                double p;
                int64_t r = sel[a];
                if (r < 0)
                    continue;
                p = exp(z[a] - mx) / sum;
                for (d = 0; d < Dv; ++d)
                    oh[d] += p * elem(dtype, kv, r * Dqk + d);
            }
            lse[i * H + h] = mx + log(sum);
        }
        free(z);
        free(qh);
    }
}

/* --------------------------------------------------- sparse MLA backward */

/*
 * Gradient of sparse MLA in MQA mode.  In sparse training the main model is
 * trained on the language-modelling loss through the attention over the
 * selected entries (mizuki-eaf.pages.dev, two-stage continued pre-training /
 * sparse training; m.36881.com.cn, sparse training); the selection itself
 * carries no gradient.  With the forward of ora_sparse_mla_rows, for every
 * query t and head h, over the valid entries r_a of idx[t]:
 *   z_a = s q.c_a,  P_a = softmax(z)_a,  o = sum_a P_a v_a     (c_a = kv[r_a], v_a = c_a[0..Dv))
 * and an upstream gradient dout[t,h] = dL/do, the chain rule gives
 *   dP_a   = dout . v_a
 *   D      = sum_a P_a dP_a  (= dout . o)
 *   dz_a   = P_a (dP_a - D)
 *   dq     = s sum_a dz_a c_a
 *   dkv[r_a] += s dz_a q  +  P_a dout   (the second term on the value dims 0..Dv only)
 * where dkv sums over every query and head that selected the row (an entry
 * listed twice counts twice, as in the forward).  All T queries are taken;
 * dq [T,H,Dqk], dkv [N,Dqk] (zeroed here), fp64.  Inputs q, kv, dout share
 * one dtype (F32, BF16 or F64).
 * The magnitudes that bound rounding in an evaluation whose dz and P are held
 * in a short format, and whose D comes from a rounded o, are returned too:
 *   mD          = sum_d |dout_d| |o_d|
 *   mag_dq      = s sum_a (|dz_a| + P_a mD) |c_a|
 *   mag_dkv[r]  = sum over the same terms of s (|dz_a| + P_a mD) |q| + P_a |dout|
 */
void ora_sparse_mla_bwd(int dtype, const void *q, const void *kv, const int32_t *idx, const void *dout, int64_t T,
                        int32_t H, int64_t N, int32_t k, int32_t Dqk, int32_t Dv, double sm_scale, double *dq,
                        double *dkv, double *mag_dq, double *mag_dkv)
{
    int64_t t, i;
    double *z = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
    double *pr = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
    double *dpa = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
    double *qh = (double *)malloc(sizeof(double) * (size_t)Dqk);
    double *gh = (double *)malloc(sizeof(double) * (size_t)Dv);
    double *oh = (double *)malloc(sizeof(double) * (size_t)Dv);
    for (i = 0; i < N * Dqk; ++i) {
        dkv[i] = 0.0;
        mag_dkv[i] = 0.0;
    }
    for (t = 0; t < T; ++t) {
        const int32_t *sel = idx + t * (int64_t)k;
        int32_t h;
        for (h = 0; h < H; ++h) {
            double *dqh = dq + (t * H + h) * (int64_t)Dqk, *mqh = mag_dq + (t * H + h) * (int64_t)Dqk;
            double mx = -INFINITY, sum = 0.0, D = 0.0, mD = 0.0;
            int32_t a, d, m = 0;
            for (d = 0; d < Dqk; ++d) {
                qh[d] = elem(dtype, q, (t * H + h) * (int64_t)Dqk + d);
                dqh[d] = 0.0;
                mqh[d] = 0.0;
            }
            for (d = 0; d < Dv; ++d) {
                gh[d] = elem(dtype, dout, (t * H + h) * (int64_t)Dv + d);
                oh[d] = 0.0;
            }
            for (a = 0; a < k; ++a) {
                double dot = 0.0;
                const int64_t r = sel[a];
                if (r < 0)
                    continue;
                for (d = 0; d < Dqk; ++d)
                    dot += qh[d] * elem(dtype, kv, r * Dqk + d);
                z[a] = sm_scale * dot;
                if (z[a] > mx)
                    mx = z[a];
                ++m;
            }
            if (m == 0)
                continue;
            for (a = 0; a < k; ++a)
                if (sel[a] >= 0)
                    sum += exp(z[a] - mx);
            /* probabilities, the output, and dP */
            for (a = 0; a < k; ++a) {
                const int64_t r = sel[a];
                double dp = 0.0;
                if (r < 0)
                    continue;
                pr[a] = exp(z[a] - mx) / sum;
                for (d = 0; d < Dv; ++d) {
                    const double v = elem(dtype, kv, r * Dqk + d);
                    oh[d] += pr[a] * v;
                    dp += gh[d] * v;
                }
                dpa[a] = dp;
            }
            for (d = 0; d < Dv; ++d) {
                D += gh[d] * oh[d];
                mD += fabs(gh[d]) * fabs(oh[d]);
            }
            for (a = 0; a < k; ++a) {
                const int64_t r = sel[a];
                double dz, adz;
                if (r < 0)
                    continue;
                dz = pr[a] * (dpa[a] - D);
                adz = fabs(dz) + pr[a] * mD;
                for (d = 0; d < Dqk; ++d) {
                    const double c = elem(dtype, kv, r * Dqk + d);
                    dqh[d] += sm_scale * dz * c;
                    mqh[d] += sm_scale * adz * fabs(c);
                    dkv[r * Dqk + d] += sm_scale * dz * qh[d];
                    mag_dkv[r * Dqk + d] += sm_scale * adz * fabs(qh[d]);
                }
                for (d = 0; d < Dv; ++d) {
                    dkv[r * Dqk + d] += pr[a] * gh[d];
                    mag_dkv[r * Dqk + d] += pr[a] * fabs(gh[d]);
                }
            }
        }
    }
    (void)N;
    free(z);
    free(pr);
    free(dpa);
    free(qh);
    free(gh);
    free(oh);
}

/* ------------------------------------------------ indexer KL-alignment loss */

/*
 * Per-token KL(p_t || pi_t) for selected query rows.
 *   q [T, H, Dqk], kv [N, Dqk] (F32, BF16 or F64); idx [T, k] rows of kv
 *   (-1 entries are skipped); scores [T, k] fp64: the index score of each
 *   entry (ignored where idx is -1).
 * For t = rows[i], over the valid entries r_1..r_m of idx[t]:
 *   z_{h,a}  = sm_scale * q[t,h,:] . kv[r_a,:]
 *   p_a      = (1/H) sum_h softmax_a(z_{h,.})        (main attention, heads averaged)
 *   pi_a     = softmax_a(scores[t,a])                 (indexer distribution)
 *   kl[i]    = sum_a p_a (log p_a - log pi_a)         (natural log; terms with p_a = 0 add 0)
 *   mag[i]   = sum_a p_a |log p_a - log pi_a|         (the same sum of magnitudes)
 * m = 0 gives kl = mag = 0.
 */
void ora_indexer_kl_rows(int dtype, const void *q, const void *kv, const int32_t *idx, const double *scores,
                         int32_t H, int32_t k, int32_t Dqk, double sm_scale, const int64_t *rows, int64_t nrows,
                         double *kl, double *mag)
{
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < nrows; ++i) {
        const int64_t t = rows[i];
        const int32_t *sel = idx + t * (int64_t)k;
        const double *sc = scores + t * (int64_t)k;
        double *z = (double *)malloc(sizeof(double) * (size_t)k);
        double *pa = (double *)calloc((size_t)k, sizeof(double));
        double smax = -INFINITY, ssum = 0.0, lse_i, acc = 0.0, accm = 0.0;
        int32_t a, h, d, m = 0;
        for (a = 0; a < k; ++a)
            if (sel[a] >= 0)
                ++m;
        if (m == 0) {
            kl[i] = 0.0;
            mag[i] = 0.0;
            free(z);
            free(pa);
            continue;
        }
        /* main attention: each head's softmax over the valid entries, averaged */
        for (h = 0; h < H; ++h) {
            double mx = -INFINITY, sum = 0.0;
            for (a = 0; a < k; ++a) {
                double dot = 0.0;
                const int64_t r = sel[a];
                if (r < 0)
                    continue;
                for (d = 0; d < Dqk; ++d)
                    dot += elem(dtype, q, (t * H + h) * (int64_t)Dqk + d) * elem(dtype, kv, r * Dqk + d);
                z[a] = sm_scale * dot;
                if (z[a] > mx)
                    mx = z[a];
            }
            for (a = 0; a < k; ++a)
                if (sel[a] >= 0)
                    sum += exp(z[a] - mx);
            for (a = 0; a < k; ++a)
                if (sel[a] >= 0)
                    pa[a] += exp(z[a] - mx) / sum / H;
        }
        /* indexer distribution: log-softmax of the scores over the valid entries */
        for (a = 0; a < k; ++a)
            if (sel[a] >= 0 && sc[a] > smax)
                smax = sc[a];
        for (a = 0; a < k; ++a)
            if (sel[a] >= 0)
                ssum += exp(sc[a] - smax);
        lse_i = smax + log(ssum);
        for (a = 0; a < k; ++a) {
            double term;
            if (sel[a] < 0 || pa[a] == 0.0)
                continue;
            term = pa[a] * (log(pa[a]) - (sc[a] - lse_i));
            acc += term;
            accm += fabs(term);
        }
        kl[i] = acc;
        mag[i] = accm;
        free(z);
        free(pa);
    }
}

/*
 * Gradient of the indexer's KL-alignment loss.  In sparse training the
 * indexer's input is detached from the main model and the indexer is trained
 * by the KL loss alone (mizuki-eaf.pages.dev, two-stage continued
 * pre-training; m.36881.com.cn, sparse training): the target p (the main
 * attention, heads averaged) carries no gradient, and the loss reaches only
 * the indexer's queries, keys and head weights.  Two steps, then their
 * composition:
 *
 * ora_indexer_kl_grad -- the gradient of sum_t dkl[t] KL_t with respect to
 * the index scores of the entries.  For query t, over the valid entries r_a
 * of idx[t] (rows of kv):
 *   pi_a = softmax_a(scores[t, a]),   p_a = (1/H) sum_h softmax_a(sm_scale q[t,h] . kv[r_a])
 *   g[t, a] = dkl[t] (pi_a - p_a)          (d KL(p || pi) / d I_a, since p sums to one)
 * and 0 at invalid entries.  q, kv: F32, BF16 or F64; scores, dkl, g fp64.
 */
void ora_indexer_kl_grad(int att_dtype, const void *q_att, const void *kv, const int32_t *idx, const double *scores,
                         const double *dkl, int64_t T, int32_t H, int32_t k, int32_t Dqk, double sm_scale, double *g)
{
    int64_t t;
#pragma omp parallel for schedule(dynamic, 1)
    for (t = 0; t < T; ++t) {
        const int32_t *sel = idx + t * (int64_t)k;
        const double *sc = scores + t * (int64_t)k;
        double *z = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
        double *pa = (double *)calloc((size_t)(k > 0 ? k : 1), sizeof(double));
        double smax = -INFINITY, ssum = 0.0;
        int32_t a, h, d, m = 0;
        for (a = 0; a < k; ++a) {
            g[t * (int64_t)k + a] = 0.0;
            if (sel[a] >= 0)
                ++m;
        }
        if (m > 0) {
            for (h = 0; h < H; ++h) {
                double mx = -INFINITY, sum = 0.0;
                for (a = 0; a < k; ++a) {
                    double dot = 0.0;
                    const int64_t r = sel[a];
                    if (r < 0)
                        continue;
                    for (d = 0; d < Dqk; ++d)
                        dot += elem(att_dtype, q_att, (t * H + h) * (int64_t)Dqk + d) * elem(att_dtype, kv, r * Dqk + d);
                    z[a] = sm_scale * dot;
                    if (z[a] > mx)
                        mx = z[a];
                }
                for (a = 0; a < k; ++a)
                    if (sel[a] >= 0)
                        sum += exp(z[a] - mx);
                for (a = 0; a < k; ++a)
                    if (sel[a] >= 0)
                        pa[a] += exp(z[a] - mx) / sum / H;
            }
            for (a = 0; a < k; ++a)
                if (sel[a] >= 0 && sc[a] > smax)
                    smax = sc[a];
            for (a = 0; a < k; ++a)
                if (sel[a] >= 0)
                    ssum += exp(sc[a] - smax);
            for (a = 0; a < k; ++a)
                if (sel[a] >= 0)
                    g[t * (int64_t)k + a] = dkl[t] * (exp(sc[a] - smax) / ssum - pa[a]);
        }
        free(z);
        free(pa);
    }
}

/*
 * ora_indexer_bwd -- the indexer's gradients from the score gradient g [T,k].
 * For query t and valid entry r_a (a row of the indexer keys):
 *   x_ja   = qh_j . kh_a          qh_j = qs[t] q[t,j,:], kh_a = ks[r_a] k[r_a,:]  (dequantised)
 *   (I_a   = sum_j w_j max(0, x_ja))
 *   dw[t,j]    = sum_a g_a max(0, x_ja)
 *   dq[t,j,:]  = sum_a g_a w_j [x_ja > 0] kh_a
 *   dk[r_a,:] += g_a sum_j w_j [x_ja > 0] qh_j        (summed over every query selecting the row)
 * ([x > 0] is 0 at the kink.)  q, k: E4M3 payloads with per-token scales, or
 * F32 / F64 values (scales ignored); w, g fp64.  Outputs fp64: dw [T,H_I],
 * dq [T,H_I,D_I], dk [N,D_I] (zeroed here).  For tolerances: mag_dq, mag_dk
 * are the same sums over |terms|, mag_dw sums |g_a| sum_d |qh_jd kh_ad| (which
 * bounds |g_a x_ja| and the rounding of x_ja), and amb_* collect the terms
 * whose dot product lies within kink_rel sum_d |qh_jd kh_ad| of the kink,
 * where an evaluation of that accuracy may take either side (an IEEE fp32
 * sum: kink_rel = (D_I + 2) 2^-24; kink_rel <= 0 selects that value).
 */
void ora_indexer_bwd(int idx_dtype, const void *q_idx, const float *q_scale, const void *k_idx, const float *k_scale,
                     const double *w, const int32_t *idx, const double *g, int64_t T, int64_t N, int32_t H_I,
                     int32_t D_I, int32_t k, double *dw, double *dq, double *dk, double *mag_dw, double *mag_dq,
                     double *mag_dk, double *amb_dq, double *amb_dk, double kink_rel)
{
    const double win = kink_rel > 0.0 ? kink_rel : (D_I + 2) * ldexp(1.0, -24);
    int64_t t, i;
    double *qh = (double *)malloc(sizeof(double) * (size_t)H_I * (size_t)D_I);
    double *kh = (double *)malloc(sizeof(double) * (size_t)D_I);
    for (i = 0; i < N * D_I; ++i) {
        dk[i] = 0.0;
        mag_dk[i] = 0.0;
        amb_dk[i] = 0.0;
    }
    for (t = 0; t < T; ++t) {
        const int32_t *sel = idx + t * (int64_t)k;
        const double qs = idx_dtype == ORA_E4M3 ? (double)q_scale[t] : 1.0;
        int32_t a, j, d;
        for (j = 0; j < H_I; ++j) {
            dw[t * H_I + j] = 0.0;
            mag_dw[t * H_I + j] = 0.0;
            for (d = 0; d < D_I; ++d) {
                qh[j * D_I + d] = qs * elem(idx_dtype, q_idx, (t * H_I + j) * (int64_t)D_I + d);
                dq[(t * H_I + j) * (int64_t)D_I + d] = 0.0;
                mag_dq[(t * H_I + j) * (int64_t)D_I + d] = 0.0;
                amb_dq[(t * H_I + j) * (int64_t)D_I + d] = 0.0;
            }
        }
        for (a = 0; a < k; ++a) {
            const int64_t r = sel[a];
            const double ga = g[t * (int64_t)k + a], gm = fabs(ga);
            if (r < 0 || r >= N)
                continue;
            for (d = 0; d < D_I; ++d)
                kh[d] = (idx_dtype == ORA_E4M3 ? (double)k_scale[r] : 1.0) * elem(idx_dtype, k_idx, r * D_I + d);
            for (j = 0; j < H_I; ++j) {
                const double wj = w[t * H_I + j];
                double x = 0.0, xm = 0.0;
                int amb;
                for (d = 0; d < D_I; ++d) {
                    x += qh[j * D_I + d] * kh[d];
                    xm += fabs(qh[j * D_I + d] * kh[d]);
                }
                amb = fabs(x) <= win * xm;
                if (x > 0.0)
                    dw[t * H_I + j] += ga * x;
                mag_dw[t * H_I + j] += gm * xm;   /* bounds |g x| and the rounding of x itself */
                for (d = 0; d < D_I; ++d) {
                    const int64_t qi = (t * H_I + j) * (int64_t)D_I + d;
                    if (x > 0.0) {
                        dq[qi] += ga * wj * kh[d];
                        mag_dq[qi] += gm * fabs(wj * kh[d]);
                        dk[r * D_I + d] += ga * wj * qh[j * D_I + d];
                        mag_dk[r * D_I + d] += gm * fabs(wj * qh[j * D_I + d]);
                    }
                    if (amb) {
                        amb_dq[qi] += gm * fabs(wj * kh[d]);
                        amb_dk[r * D_I + d] += gm * fabs(wj * qh[j * D_I + d]);
                    }
                }
            }
        }
    }
    free(qh);
    free(kh);
}

/*
 * ora_indexer_kl_bwd -- the two steps composed: the index scores of the
 * entries from the indexer's inputs (I_a = sum_j w_j max(0, x_ja)), their
 * gradient g, then dw, dq, dk.  Entries of idx index both kv and the keys.
 * kink_rel: as for ora_indexer_bwd.
 */
void ora_indexer_kl_bwd(int att_dtype, const void *q_att, const void *kv, int idx_dtype, const void *q_idx,
                        const float *q_scale, const void *k_idx, const float *k_scale, const double *w,
                        const int32_t *idx, const double *dkl, int64_t T, int64_t N, int32_t H, int32_t H_I,
                        int32_t D_I, int32_t k, int32_t Dqk, double sm_scale, double *g, double *dw, double *dq,
                        double *dk, double *mag_dw, double *mag_dq, double *mag_dk, double *amb_dq, double *amb_dk,
                        double kink_rel)
{
    double *sc = (double *)malloc(sizeof(double) * (size_t)(T * k > 0 ? T * k : 1));
    double *kh = (double *)malloc(sizeof(double) * (size_t)D_I);
    int64_t t;
    for (t = 0; t < T; ++t) {
        const double qs = idx_dtype == ORA_E4M3 ? (double)q_scale[t] : 1.0;
        int32_t a, j, d;
        for (a = 0; a < k; ++a) {
            const int64_t r = idx[t * (int64_t)k + a];
            double acc = 0.0;
            sc[t * (int64_t)k + a] = 0.0;
            if (r < 0 || r >= N)
                continue;
            for (d = 0; d < D_I; ++d)
                kh[d] = (idx_dtype == ORA_E4M3 ? (double)k_scale[r] : 1.0) * elem(idx_dtype, k_idx, r * D_I + d);
            for (j = 0; j < H_I; ++j) {
                double x = 0.0;
                for (d = 0; d < D_I; ++d)
                    x += qs * elem(idx_dtype, q_idx, (t * H_I + j) * (int64_t)D_I + d) * kh[d];
                acc += w[t * H_I + j] * (x > 0.0 ? x : 0.0);
            }
            sc[t * (int64_t)k + a] = acc;
        }
    }
    ora_indexer_kl_grad(att_dtype, q_att, kv, idx, sc, dkl, T, H, k, Dqk, sm_scale, g);
    ora_indexer_bwd(idx_dtype, q_idx, q_scale, k_idx, k_scale, w, idx, g, T, N, H_I, D_I, k, dw, dq, dk, mag_dw,
                    mag_dq, mag_dk, amb_dq, amb_dk, kink_rel);
    free(sc);
    free(kh);
}

/* ------------------------------------------------------------ paged decode */

/*
 * One decode query per sequence over a paged cache of 64-token pages.
 * Sequence b has ctx[b] cached tokens; its query sits at position ctx[b]-1
 * (its own key and latent are already in the cache), so candidates are
 * positions 0..ctx[b]-1.  Logical position p of sequence b lives in physical
 * row  block_table[b*max_blocks + p/64]*64 + p%64  of the pools:
 *   k8 pool [nrows_phys, D_I] E4M3 + ks pool [nrows_phys] fp32 (indexer keys)
 *   kv pool [nrows_phys, Dqk] BF16 (latent; value = first Dv dims)
 * Query side per sequence: q8 [B, H_I, D_I] E4M3 + qs [B], w [B, H_I],
 * q [B, H, Dqk] BF16.
 * Outputs for sequences seqs[0..nseq): idx [nseq, k] logical positions
 * (ascending, -1 padded), tau [nseq], o [nseq, H, Dv], lse [nseq, H].
 */
void ora_decode(const uint8_t *q8, const float *qs, const float *w, const uint16_t *q,
                const uint8_t *k8_pool, const float *ks_pool, const uint16_t *kv_pool,
                const int32_t *block_table, int32_t max_blocks, const int32_t *ctx, int32_t B,
                int32_t H_I, int32_t D_I, int32_t H, int32_t k, int32_t Dqk, int32_t Dv,
                double sm_scale, const int64_t *seqs, int64_t nseq, int32_t *idx, double *tau,
                double *o, double *lse)
{
    int64_t i;
    (void)B;
    for (i = 0; i < nseq; ++i) {
        int64_t b = seqs[i], n = ctx[b], p;
        double *sc = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        int32_t *phys = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
        int32_t *lidx = idx + i * (int64_t)k;
        int32_t a;
        double qsv = (double)qs[b];
#pragma omp parallel for schedule(static)
        for (p = 0; p < n; ++p) {
            int64_t row = (int64_t)block_table[b * max_blocks + p / 64] * 64 + p % 64;
            double ksv = (double)ks_pool[row], acc = 0.0;
            int32_t j, d;
            for (j = 0; j < H_I; ++j) {
                double dot = 0.0;
                for (d = 0; d < D_I; ++d)
                    dot += (qsv * ora_e4m3_decode(q8[(b * H_I + j) * (int64_t)D_I + d])) *
                           (ksv * ora_e4m3_decode(k8_pool[row * D_I + d]));
                acc += (double)w[b * H_I + j] * (dot > 0.0 ? dot : 0.0);
            }
            sc[p] = (acc == 0.0) ? 0.0 : acc;
        }
        ora_topk_row(sc, n, k, lidx, tau + i);
        /* selected logical positions -> physical latent rows */
        for (a = 0; a < k; ++a) {
            int32_t lp = lidx[a];
            phys[a] = lp < 0 ? -1 : block_table[b * max_blocks + lp / 64] * 64 + lp % 64;
        }
        {
            int64_t one = 0;
            /* q row b viewed as a single-row problem whose idx row is phys */
            ora_sparse_mla_rows(ORA_BF16, q + b * (int64_t)H * Dqk, kv_pool, phys, 1, H, 0, k, Dqk,
                                Dv, sm_scale, &one, 1, o + i * (int64_t)H * Dv, lse + i * H);
        }
        free(sc);
        free(phys);
    }
}

/*
 * Paged cache append: the latent KV cache of MLA holds one compressed latent
 * row per token (jienda.com, section 2.1), and the indexer keeps one FP8 key
 * with its scale per token; decode adds the new token of each sequence to
 * both.  Token b goes to logical position pos[b] of sequence b, i.e. physical
 * row  block_table[b*max_blocks + pos[b]/64]*64 + pos[b]%64  of each pool:
 *   kv pool [n_pool_rows, Dqk] BF16 <- latent [B, Dqk]
 *   k8 pool [n_pool_rows, D_I] E4M3 <- k8 [B, D_I]
 *   ks pool [n_pool_rows] fp32      <- ks [B]
 * A position outside the table (negative, page past max_blocks), an unmapped
 * page (-1) or a row past the pool writes nothing.  Every other pool row is
 * left as it was.
 */
void ora_paged_cache_append(const uint16_t *latent, const uint8_t *k8, const float *ks, const int32_t *pos,
                            int32_t B, int32_t D_I, int32_t Dqk, const int32_t *block_table, int32_t max_blocks,
                            int64_t n_pool_rows, uint16_t *kv_pool, uint8_t *k8_pool, float *ks_pool)
{
    int32_t b, d;
    for (b = 0; b < B; ++b) {
        int32_t p = pos[b], blk;
        int64_t row;
        if (p < 0 || p / 64 >= max_blocks)
            continue;
        blk = block_table[(int64_t)b * max_blocks + p / 64];
        if (blk < 0)
            continue;
        row = (int64_t)blk * 64 + p % 64;
        if (row >= n_pool_rows)
            continue;
        for (d = 0; d < Dqk; ++d)
            kv_pool[row * Dqk + d] = latent[(int64_t)b * Dqk + d];
        for (d = 0; d < D_I; ++d)
            k8_pool[row * D_I + d] = k8[(int64_t)b * D_I + d];
        ks_pool[row] = ks[b];
    }
}

/* ------------------------------------------------- masked MHA (short prefill) */

/*
 * Masked multi-head attention in MLA's multi-head form.  Latent rows kv
 * [N, Dc + Dr] (Dc compressed dims, Dr rope dims); per head h the up-projections
 * w_uk [H, Dn, Dc] and w_uv [H, Dvh, Dc]:
 *   K_h[s] = ( sum_c w_uk[h,e,c] kv[s,c]  for e < Dn ,  kv[s, Dc + j]  for j < Dr )
 *   V_h[s] =   sum_c w_uv[h,e,c] kv[s,c]  for e < Dvh
 * Query q [T, H, Dn + Dr].  For t = rows[i], head h, over the positions allowed
 * by the query's mask -- the valid entries r_1..r_m of idx[t] --
 *   z_a = sm_scale * q[t,h,:] . K_h[r_a]
 *   o[i,h,:] = sum_a softmax(z)_a V_h[r_a],  lse[i,h] = log sum_a exp(z_a)
 * with m = 0 giving o = 0, lse = -inf.  Head by head, K_h and V_h are formed
 * from their definition once for each position that a requested row selects
 * and then read by every row that selects it.
 */
void ora_masked_mha_rows(int dtype, const void *q, const void *kv, const void *w_uk, const void *w_uv,
                         const int32_t *idx, int32_t H, int32_t k, int32_t Dc, int32_t Dr, int32_t Dn,
                         int32_t Dvh, double sm_scale, const int64_t *rows, int64_t nrows, double *o,
                         double *lse)
{
    const int32_t Dq = Dn + Dr, Dl = Dc + Dr;
    int64_t i, p, npos = 0, top = -1;
    int64_t *slot, *pos;
    double *K, *V;
    int32_t h;
    /* the positions the requested rows select, each given a table slot */
    for (i = 0; i < nrows; ++i) {
        int32_t a;
        for (a = 0; a < k; ++a)
            if (idx[rows[i] * (int64_t)k + a] > top)
                top = idx[rows[i] * (int64_t)k + a];
    }
    slot = (int64_t *)malloc(sizeof(int64_t) * (size_t)(top + 1 > 0 ? top + 1 : 1));
    pos = (int64_t *)malloc(sizeof(int64_t) * (size_t)(top + 1 > 0 ? top + 1 : 1));
    for (p = 0; p <= top; ++p)
        slot[p] = -1;
    for (i = 0; i < nrows; ++i) {
        int32_t a;
        for (a = 0; a < k; ++a) {
            int64_t r = idx[rows[i] * (int64_t)k + a];
            if (r >= 0 && slot[r] < 0) {
                slot[r] = npos;
                pos[npos++] = r;
            }
        }
    }
    K = (double *)malloc(sizeof(double) * (size_t)(npos > 0 ? npos : 1) * (size_t)Dq);
    V = (double *)malloc(sizeof(double) * (size_t)(npos > 0 ? npos : 1) * (size_t)Dvh);
    for (h = 0; h < H; ++h) {
#pragma omp parallel for schedule(static)
        for (p = 0; p < npos; ++p) {
            const int64_t r = pos[p];
            double *key = K + p * Dq, *val = V + p * Dvh;
            int32_t c, e;
            for (e = 0; e < Dn; ++e) {
                double acc = 0.0;
                for (c = 0; c < Dc; ++c)
                    acc += elem(dtype, w_uk, ((int64_t)h * Dn + e) * Dc + c) * elem(dtype, kv, r * Dl + c);
                key[e] = acc;
            }
            for (e = 0; e < Dr; ++e)
                key[Dn + e] = elem(dtype, kv, r * Dl + Dc + e);
            for (e = 0; e < Dvh; ++e) {
                double acc = 0.0;
                for (c = 0; c < Dc; ++c)
                    acc += elem(dtype, w_uv, ((int64_t)h * Dvh + e) * Dc + c) * elem(dtype, kv, r * Dl + c);
                val[e] = acc;
            }
        }
#pragma omp parallel for schedule(dynamic, 1)
        for (i = 0; i < nrows; ++i) {
            const int64_t t = rows[i];
            const int32_t *sel = idx + t * (int64_t)k;
            double *oh = o + (i * H + h) * (int64_t)Dvh;
            double *z = (double *)malloc(sizeof(double) * (size_t)k);
            double mx = -INFINITY, sum = 0.0;
            int32_t a, e, m = 0;
            for (e = 0; e < Dvh; ++e)
                oh[e] = 0.0;
            for (a = 0; a < k; ++a) {
                double dot = 0.0;
                const double *key;
                if (sel[a] < 0) {
                    z[a] = -INFINITY;
                    continue;
                }
                key = K + slot[sel[a]] * Dq;
                for (e = 0; e < Dq; ++e)
                    dot += elem(dtype, q, (t * H + h) * (int64_t)Dq + e) * key[e];
                z[a] = sm_scale * dot;
                if (z[a] > mx)
                    mx = z[a];
                ++m;
            }
            if (m == 0) {
                lse[i * H + h] = -INFINITY;
                free(z);
                continue;
            }
            for (a = 0; a < k; ++a)
                if (sel[a] >= 0)
                    sum += exp(z[a] - mx);
            for (a = 0; a < k; ++a) {
                double pr;
                const double *val;
                if (sel[a] < 0)
                    continue;
                pr = exp(z[a] - mx) / sum;
                val = V + slot[sel[a]] * Dvh;
                for (e = 0; e < Dvh; ++e)
                    oh[e] += pr * val[e];
            }
            lse[i * H + h] = mx + log(sum);
            free(z);
        }
    }
    free(slot);
    free(pos);
    free(K);
    free(V);
}
