/*
 * dsa.h -- C ABI of libdsa, the MI355X (gfx950) implementation of the
 * DeepSeek Sparse Attention (DSA) hot path:
 *
 *   lightning indexer  ->  per-query top-k selection  ->  sparse MLA (MQA mode)
 *
 * The method (DeepSeek-V3.2; mizuki-eaf.pages.dev, section "DeepSeek Sparse
 * Attention", "How it works" and "built on MLA"; m.digipub.cc, section 2):
 * a light indexer with few heads, ReLU and FP8 operands scores every query
 * token against each preceding token; each query keeps the key/value entries
 * with the top-k scores (k = 2048); main attention runs over only those
 * entries, as MLA in MQA mode, where one latent vector per token is shared by
 * all query heads of a query token.
 *
 * Conventions (all entry points)
 *  - Tensor pointers are DEVICE pointers owned by the caller; tensors are
 *    dense, row-major, with the shapes given below.  The library never
 *    allocates device memory: scratch space comes from a caller-provided
 *    workspace sized by the matching *_workspace_bytes() query.
 *  - Calls only validate and enqueue work on `stream`; they return before the
 *    GPU finishes.  Results are deterministic run to run.
 *  - Every call returns a dsa_status.  Host-side validation runs before any
 *    HIP call; on failure nothing is enqueued and dsa_last_error() returns a
 *    message (thread-local, valid until the next call on the same thread).
 *  - Offsets are 64-bit; the 128K-token shapes are supported.
 *  - Positions: the query at position p may select keys at positions
 *    0..p inclusive, so it selects min(k, p+1) of them.  Equal index scores
 *    are ordered by position, the larger (more recent) position first.
 *  - FP8 is OCP E4M3FN (bias 7, max 448, no infinities).  bf16 is the top 16
 *    bits of an IEEE binary32.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSA_OK = 0,
    DSA_ERR_INVALID_ARG = 1,  /* null pointer, negative or inconsistent size   */
    DSA_ERR_UNSUPPORTED = 2,  /* valid but outside what the kernels implement  */
    DSA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required     */
    DSA_ERR_HIP = 4           /* a HIP call (launch, query) failed              */
} dsa_status;

typedef enum { DSA_F32 = 0, DSA_BF16 = 1, DSA_E4M3 = 2 } dsa_dtype;

enum {
    DSA_D_QK = 576,    /* latent width: 512 no-rope + 64 rope               */
    DSA_D_V = 512,     /* value width: the first 512 dims of the latent     */
    DSA_MAX_K = 2048,  /* largest supported top-k                           */
    DSA_PAGE = 64,     /* tokens per page of the paged decode cache         */
    DSA_MHA_DN = 128,  /* masked MHA: per-head no-rope key dims             */
    DSA_MHA_DR = 64,   /* masked MHA: rope dims (shared by every head)      */
    DSA_MHA_DV = 128,  /* masked MHA: per-head value dims                   */
    DSA_MHA_MAX_L = 65536  /* masked MHA: longest sequence                  */
};

/* Message of the last failed call on this thread ("" if none). */
const char *dsa_last_error(void);

/* Library version string: "libdsa <version> gfx950 src=<hash>", where <hash>
 * identifies the sources the library was built from. */
const char *dsa_version(void);

/* ---------------------------------------------------------------------------
 * Per-token E4M3 quantisation of indexer operands (the indexer "can run in
 * FP8": mizuki-eaf.pages.dev, "How it works"; m.digipub.cc, section 2).
 *   x      [rows, cols] fp32
 *   x8     [rows, cols] E4M3 out;  scale [rows] fp32 out
 * scale[r] = amax_c |x[r,c]| / 448 (fp32 division; 1 if the row is all zero);
 * x8[r,c] = E4M3 of the fp32 quotient x[r,c]/scale[r], round-to-nearest-even,
 * saturating at +-448.  cols must be a multiple of 4 and at most 16384;
 * rows at most 2^31 - 1.  x must be 16-byte aligned, x8 4-byte aligned.
 */
dsa_status dsa_quantize_e4m3_per_token(const float *x, int64_t rows, int32_t cols, uint8_t *x8,
                                       float *scale, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Lightning indexer scores (mizuki-eaf.pages.dev, "How it works":
 * "index score" of a query token against every preceding token).
 *   I[t,s] = sum_{j<H_I} w[t,j] * ReLU( (qs[t] q[t,j,:]) . (ks[s] k[s,:]) )
 *   q       [T, H_I, D_I]  E4M3 (with q_scale [T]) or F32 (q_scale NULL)
 *   k       [S, D_I]       same dtype (with k_scale [S] for E4M3)
 *   w       [T, H_I] fp32 head weights
 *   q_pos   [T] int32: query t may see keys s in [0, q_pos[t]]
 *   scores  [T, ld_scores] fp32 out; s > q_pos[t] (s < S) is written -inf.
 * E4M3: products are exact; scales must be > 0.  H_I 32 or 64 with
 *   D_I = 128 runs on the FP8 MFMA, whose fp32 result comes from a coarser
 *   internal sum of the 128 products (measured on gfx950: within 2^-12 of the
 *   sum of their magnitudes); every other E4M3 shape sums the exact products
 *   with IEEE fp32 fused multiply-adds.
 * Limits: E4M3 needs D_I in {64, 128} and H_I <= 64;
 *         F32 needs D_I <= 128 and H_I <= 64.
 */
dsa_status dsa_indexer_scores(const void *q, const float *q_scale, const void *k,
                              const float *k_scale, const float *w, const int32_t *q_pos,
                              int32_t T, int32_t S, int32_t H_I, int32_t D_I, dsa_dtype dt,
                              float *scores, int64_t ld_scores, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Fine-grained token selection (mizuki-eaf.pages.dev, "How it works";
 * m.digipub.cc, section 2): per row keep the k largest scores.
 *   scores  [T, ld_scores] fp32; row t has candidates s in [0, n_valid[t])
 *   n_valid [T] int32 (device)
 *   idx     [T, k] int32 out: the min(k, n_valid[t]) selected positions in
 *           ascending order, then -1.
 * Order: score descending, then position descending.  k <= 2048.
 * Without a workspace (NULL, 0) rows may be of any length up to 2^31-1 and
 * each row is one workgroup.  With a workspace of at least
 * dsa_topk_workspace_bytes(T, ld_scores, k) bytes (ld_scores > 0), rows are
 * taken to be at most ld_scores long, and a batch too short to fill the GPU
 * is split: each row's column chunks are selected separately, then merged
 * (same result).  The workspace is scratch, overwritten by the call.
 */
dsa_status dsa_topk_select(const float *scores, int64_t ld_scores, const int32_t *n_valid,
                           int32_t T, int32_t k, int32_t *idx, void *workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes for a split dsa_topk_select of T rows of at most
 * ld_scores scores (0: the batch is never split). */
size_t dsa_topk_workspace_bytes(int32_t T, int64_t ld_scores, int32_t k);

/* ---------------------------------------------------------------------------
 * Sparse MLA forward in MQA mode (mizuki-eaf.pages.dev, "built on MLA";
 * jienda.com, section 2.1): one latent row per token, shared by all heads.
 *   q    [T, H, 576]   BF16 or F32
 *   kv   [N, 576]      same dtype; the value of row r is kv[r, 0:512]
 *   idx  [T, k] int32  rows of kv attended by query t; -1 entries are skipped
 *   out  [T, H, 512]   same dtype as q;  lse [T, H] fp32 (natural log), may be NULL
 *   o[t,h] = sum_i softmax_i(sm_scale * q[t,h].kv[idx[t,i]]) kv[idx[t,i], :512]
 * A query with no valid entry gets o = 0 and lse = -inf.
 * BF16: bf16 MFMA, fp32 softmax and accumulation, output rounded (RNE) to bf16.
 * Limits: BF16 needs H a multiple of 8 (the kernel works in tiles of 16
 * heads; a last, partial tile is padded with zero queries whose outputs are
 * never written); F32 needs H <= 128; k <= 2048.
 * workspace (optional) lets the kernel split long selections across more
 * workgroups when T is small; size it with dsa_sparse_mla_workspace_bytes().
 * Each split's output is then held in bf16, normalised by its own softmax
 * sum, and merged by LSE weighting in fp32 (one extra bf16 rounding).  The
 * workspace needs no initialisation; calls that share one must not overlap.
 */
size_t dsa_sparse_mla_workspace_bytes(int32_t T, int32_t H, int32_t k);
dsa_status dsa_sparse_mla_fwd(const void *q, const void *kv, dsa_dtype dt, const int32_t *idx,
                              int32_t T, int32_t H, int64_t N, int32_t k, float sm_scale,
                              void *out, float *lse, void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Sparse MLA backward.  In sparse training the main model is trained by the
 * language-modelling loss through the attention over the selected entries
 * (mizuki-eaf.pages.dev, two-stage continued pre-training / sparse training;
 * m.36881.com.cn, sparse training); the selection carries no gradient.  With
 * the forward of dsa_sparse_mla_fwd (its out and lse) and the upstream
 * gradient dout, for every query t, head h and valid entry a (row r = idx[t,a],
 * c = kv[r], v = c[0:512], P_a the forward's probability):
 *   dS_a = P_a (dout . v_a - dout . o)
 *   dq[t,h]  = sm_scale sum_a dS_a c_a
 *   dkv[r]  += sm_scale dS_a q[t,h] + P_a dout[t,h]   (the second term on dims 0..511)
 * summed over every query and head that selected the row (an entry listed
 * twice counts twice).
 *   q [T,H,576], kv [N,576], out [T,H,512], dout [T,H,512] BF16; idx [T,k];
 *   lse [T,H] fp32 (the forward's); dq [T,H,576], dkv [N,576] fp32 out, fully
 *   overwritten.
 * bf16 MFMA with fp32 sums; sm_scale dS and P enter the products rounded to bf16, and
 * dout . o uses the forward's bf16 output.  Each pair's contribution to dkv
 * (its sum over the heads) is rounded to bf16 once; dkv is summed in fp32 per
 * row over its pairs in increasing (t, a) order (an inverted selection, no
 * atomics), so
 * it is deterministic as long as no idx row lists one row more than 4096
 * times.
 * workspace: dsa_sparse_mla_bwd_workspace_bytes(T, H, N, k), required.
 * Limits: H a multiple of 32, at most 128; k <= 2048. */
size_t dsa_sparse_mla_bwd_workspace_bytes(int32_t T, int32_t H, int64_t N, int32_t k);
dsa_status dsa_sparse_mla_bwd(const void *q, const void *kv, const int32_t *idx, const void *out, const float *lse,
                              const void *dout, int32_t T, int32_t H, int64_t N, int32_t k, float sm_scale, float *dq,
                              float *dkv, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* dsa_sparse_mla_bwd_kl: one sparse-training backward for both losses.  In
 * sparse training the main model is trained by the language-modelling loss
 * and the indexer, on the same selection, by the KL loss against the main
 * attention (the pages cited at dsa_sparse_mla_bwd and dsa_indexer_kl_bwd).
 * The attention's backward already forms every probability P of the
 * selection with the forward's lse, and the KL target is their head average,
 * so this call returns dsa_sparse_mla_bwd's dq and dkv and, from the same P,
 * dsa_indexer_kl_bwd's score gradient, without a second pass over the
 * logits:
 *   grad_scores[t, a] = dkl[t] (pi_a - p_a),  pi = softmax(idx_scores[t]),
 *   p_a = P_a / sum_a P_a,  P_a = sum over the heads of P[t, a, h]
 * (0 where the entry has no row).  P_a is summed in fp32 per group of 64
 * heads (32 when 64 does not divide H), the groups then added in order.
 *   idx_scores [T, k] fp32 (dsa_indexer_scores_at on this idx), dkl [T] fp32,
 *   grad_scores [T, k] fp32 out; every other argument, the workspace size and
 *   the limits as dsa_sparse_mla_bwd (dq and dkv are bit-identical to its).
 */
dsa_status dsa_sparse_mla_bwd_kl(const void *q, const void *kv, const int32_t *idx, const void *out,
                                 const float *lse, const void *dout, const float *idx_scores, const float *dkl,
                                 int32_t T, int32_t H, int64_t N, int32_t k, float sm_scale, float *dq, float *dkv,
                                 float *grad_scores, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Index scores at listed positions: the scores a selection ranked, as the
 * indexer's KL loss needs them.  out[t, a] = I[t, idx[t, a]] with the E4M3
 * arithmetic of dsa_indexer_scores (same expression, bit-identical values),
 * and -inf where idx[t, a] is outside [0, S).  No causal check is made.
 *   q8 [T, H_I, D_I] E4M3 + q_scale [T], k8 [S, D_I] E4M3 + k_scale [S],
 *   w [T, H_I] fp32, idx [T, k] int32, out [T, k] fp32.
 * Limits: D_I = 128, H_I 32 or 64, S >= 1.
 */
dsa_status dsa_indexer_scores_at(const uint8_t *q8, const float *q_scale, const uint8_t *k8, const float *k_scale,
                                 const float *w, const int32_t *idx, int32_t T, int32_t S, int32_t H_I, int32_t D_I,
                                 int32_t k, float *out, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Indexer KL-alignment loss, forward.  In both continued-pre-training
 * stages a KL loss aligns the indexer's output distribution with the main
 * attention's (mizuki-eaf.pages.dev, two-stage continued pre-training;
 * m.36881.com.cn, dense warm-up and sparse training).  Per query t, over the
 * valid entries a of idx[t] (the top-k selection in sparse training; all
 * causal positions in the dense warm-up):
 *   p_a  = (1/H) sum_h softmax_a(sm_scale q[t,h] . kv[idx[t,a]])   heads averaged
 *   pi_a = softmax_a(idx_scores[t, a])
 *   kl[t] = sum_a p_a (log p_a - log pi_a)   (natural log; 0 with no valid entry)
 *   q [T, H, 576] BF16, kv [N, 576] BF16, idx [T, k] rows of kv (entries
 *   outside [0, N) are skipped), idx_scores [T, k] fp32 (dsa_indexer_scores_at),
 *   lse [T, H] fp32: each head's natural-log log-sum-exp over the same
 *   entries (the lse output of dsa_sparse_mla_fwd on this idx), kl [T] fp32.
 * Each head's softmax is taken against lse; the head sum is then normalised
 * by its own total, so p sums to one whatever small error lse carries.
 * Logits are bf16 MFMA with fp32 sums; exponentials, logs and sums are fp32.
 * How the per-token values are summed or averaged is left to the caller.
 * Limits: H one of 16, 32, 64, 128; k <= 2048.
 */
dsa_status dsa_indexer_kl_fwd(const void *q, const void *kv, const int32_t *idx, const float *idx_scores,
                              const float *lse, int32_t T, int32_t H, int64_t N, int32_t k, float sm_scale, float *kl,
                              hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Backward of the indexer's KL-alignment loss.  In sparse training the
 * indexer's input is detached and the indexer is trained by the KL loss
 * alone (mizuki-eaf.pages.dev, two-stage continued pre-training / sparse
 * training; m.36881.com.cn, sparse training): the target p (the main
 * attention) carries no gradient.
 *
 * dsa_indexer_kl_bwd: the gradient of sum_t dkl[t] KL_t with respect to the
 * index scores of the entries, with the inputs of dsa_indexer_kl_fwd and
 *   dkl [T] fp32 (upstream gradient of each token's loss), grad_scores [T, k]
 *   fp32 out: grad[t, a] = dkl[t] (pi_a - p_a), 0 where the entry has no row.
 * Limits as dsa_indexer_kl_fwd.
 */
dsa_status dsa_indexer_kl_bwd(const void *q, const void *kv, const int32_t *idx, const float *idx_scores,
                              const float *lse, const float *dkl, int32_t T, int32_t H, int64_t N, int32_t k,
                              float sm_scale, float *grad_scores, hipStream_t stream);

/* dsa_indexer_bwd: the indexer's own gradients from the score gradient.
 * With I[t,a] = sum_j w[t,j] ReLU(x_ja), x_ja = (qs[t] q8[t,j]) . (ks[r] k8[r]),
 * r = idx[t,a] (the FP8 encoding passed straight through):
 *   dw [T, H_I]         dw[t,j]  = sum_a g[t,a] ReLU(x_ja)
 *   dq [T, H_I, D_I]    dq[t,j]  = sum_a g[t,a] w[t,j] [x_ja > 0] ks[r] k8[r]
 *   dk [S, D_I]         dk[r]    = sum over the (t, a) with idx[t,a] = r of
 *                                  g[t,a] qs[t] sum_j w[t,j] [x_ja > 0] q8[t,j]
 * (gradients with respect to the dequantised q and k; [x > 0] is 0 at the
 * kink).  q8 [T,H_I,D_I] E4M3 + q_scale [T], k8 [S,D_I] E4M3 + k_scale [S],
 * w [T,H_I], idx [T,k] (entries outside [0,S) skipped), grad_scores [T,k]; all
 * outputs fp32, fully overwritten.  Products come from the FP8 MFMA as in the
 * forward; sums are fp32.  dk is summed per key over its pairs in increasing
 * (t, a) order (an inverted selection, no atomics), so it is deterministic
 * as long as no idx row lists one key more than 4096 times.
 * workspace: dsa_indexer_bwd_workspace_bytes(T, S, k) bytes, required.
 * Limits: H_I = 64, D_I = 128, k <= 2048. */
size_t dsa_indexer_bwd_workspace_bytes(int32_t T, int32_t S, int32_t k);
dsa_status dsa_indexer_bwd(const uint8_t *q8, const float *q_scale, const uint8_t *k8, const float *k_scale,
                           const float *w, const int32_t *idx, const float *grad_scores, int32_t T, int32_t S,
                           int32_t H_I, int32_t D_I, int32_t k, float *dw, float *dq, float *dk, void *workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Masked multi-head attention for short prefill (the mode that stands in for
 * DSA on short sequences: mizuki-eaf.pages.dev, "parity evaluation";
 * m.digipub.cc, section 2).  MLA in its multi-head form over one causal
 * sequence (query t sits at position t): per head h
 *   K_h[s] = ( W_uk[h] kv[s, 0:512] ,  kv[s, 512:576] )       (128 + 64 dims)
 *   V_h[s] =   W_uv[h] kv[s, 0:512]                           (128 dims)
 *   o[t,h] = sum_s softmax_s(sm_scale * q[t,h].K_h[s]) V_h[s]
 * over the positions s <= t that idx[t] selects (the top-k mask); entries
 * outside [0, t] (-1 padding among them) are ignored and a position listed
 * twice counts once.  It equals dsa_sparse_mla_fwd on the same selection with
 * the up-projections absorbed into the query (out = W_uv[h] o_MQA, same lse).
 *   q    [L, H, 192] BF16 (128 no-rope dims, then the 64 rope dims)
 *   kv   [L, 576]    BF16 latent rows (512 compressed + 64 rope)
 *   w_uk [H, 128, 512] BF16,  w_uv [H, 128, 512] BF16 (row e of head h maps
 *        the 512 compressed dims to output dim e)
 *   idx  [L, k] int32;  out [L, H, 128] BF16;  lse [L, H] fp32 (natural log,
 *        may be NULL).  A query with nothing selected gets o = 0, lse = -inf.
 * K_h and V_h are formed once per call with fp32 accumulation and held in
 * fp16 (one round-to-nearest-even, saturating at +-65504); the no-rope part
 * of q enters the logits in fp16 and the rope part in bf16; logits, softmax
 * and the output accumulate in fp32, probabilities enter the value sum in
 * fp16.  Values of q, K_h or V_h beyond fp16's range (|x| > 65504) are
 * outside what this mode supports.
 * workspace: dsa_masked_mha_workspace_bytes(L, H) bytes (K, V and the L x L
 * bit mask), required, no initialisation; calls sharing one must not overlap.
 * Limits: L <= DSA_MHA_MAX_L.
 */
size_t dsa_masked_mha_workspace_bytes(int32_t L, int32_t H);
dsa_status dsa_masked_mha_prefill(const void *q, const void *kv, const void *w_uk, const void *w_uv,
                                  const int32_t *idx, int32_t L, int32_t H, int32_t k, float sm_scale,
                                  void *out, float *lse, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Fused prefill of one causal sequence (query t sits at position t):
 * indexer scores are computed tile by tile and fed straight into a per-query
 * streaming top-k held on chip, so the L x L score matrix is never written;
 * then sparse MLA over the selected rows.
 *   idx_dt E4M3: q_idx [L,H_I,D_I] + q_scale [L], k_idx [L,D_I] + k_scale [L]
 *          (D_I in {64, 128}, H_I <= 64).  H_I = 64 with D_I = 128 is the
 *          fused streaming path; any other E4M3 shape runs like F32;
 *   idx_dt F32 : same shapes in fp32, scales NULL; runs the three unfused
 *          calls with the L x L scores in the workspace (small L only:
 *          L <= 16384).
 *   w [L,H_I] fp32;  q [L,H,576], kv [L,576] in attn_dt (BF16 or F32);
 *   idx [L,k] int32 out (selected positions, ascending, -1 padded);
 *   out [L,H,512] in attn_dt;  lse [L,H] fp32 (may be NULL).
 */
typedef struct {
    int32_t L, H_I, D_I, H, k;
    dsa_dtype idx_dt;
    const void *q_idx;
    const float *q_scale;
    const void *k_idx;
    const float *k_scale;
    const float *w;
    dsa_dtype attn_dt;
    const void *q;
    const void *kv;
    float sm_scale;
    int32_t *idx;
    void *out;
    float *lse;
} dsa_prefill_args;

size_t dsa_prefill_workspace_bytes(const dsa_prefill_args *a);
dsa_status dsa_prefill(const dsa_prefill_args *a, void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* The selection stage of dsa_prefill alone (indexer + top-k into a->idx;
 * q, kv, out, lse are not touched and may be NULL).  dsa_prefill is exactly
 * this call followed by dsa_sparse_mla_fwd on a->idx with no workspace.
 * Both need dsa_prefill_workspace_bytes(a) of workspace: for E4M3 the
 * streaming top-k keeps a 4096-entry candidate buffer per query there
 * (32 KiB per query: 4 GiB at L = 131072); for F32 and the other E4M3
 * shapes, the L x L scores. */
dsa_status dsa_prefill_select(const dsa_prefill_args *a, void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Paged decode: one query per sequence at position ctx_len[b]-1, whose own
 * key and latent are already in the cache.  The cache is paged in 64-token
 * pages; logical position p of sequence b lives in physical row
 *     block_table[b*max_blocks + p/64]*64 + p%64
 * of every pool.  Steps: indexer over the sequence's FP8 keys -> top-k ->
 * sparse MLA gathering the selected latent rows through the block table.
 *   q8 [B,H_I,D_I] E4M3, q_scale [B], w [B,H_I] fp32, q [B,H,576] BF16
 *   k8_pool [n_pool_rows, D_I] E4M3, ks_pool [n_pool_rows] fp32,
 *   kv_pool [n_pool_rows, 576] BF16, with n_pool_rows a multiple of 64
 *   block_table [B, max_blocks] int32, ctx_len [B] int32 (device)
 *   max_ctx: host-side upper bound of ctx_len (sizes grids and workspace)
 *   idx_out [B,k] int32 (optional, logical positions ascending, -1 padded)
 *   out [B,H,512] BF16, lse [B,H] fp32 (may be NULL)
 * Limits: D_I = 128, H_I = 64, H a multiple of 8, 1 <= ctx_len <= max_ctx.
 */
typedef struct {
    int32_t B, H_I, D_I, H, k;
    const uint8_t *q8;
    const float *q_scale;
    const float *w;
    const void *q;
    const uint8_t *k8_pool;
    const float *ks_pool;
    const void *kv_pool;
    int64_t n_pool_rows;
    const int32_t *block_table;
    int32_t max_blocks;
    const int32_t *ctx_len;
    int32_t max_ctx;
    float sm_scale;
    int32_t *idx_out;
    void *out;
    float *lse;
} dsa_decode_args;

size_t dsa_decode_workspace_bytes(const dsa_decode_args *a);
dsa_status dsa_decode(const dsa_decode_args *a, void *workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* Allocation-free dsa_decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same steps and kernels as dsa_decode, bit-identical
 * results, with the workspace carved from a static device array inside the
 * library instead of a caller buffer.  No allocation of any kind is made.
 *   - The array holds dsa_decode_static_scratch_bytes() bytes (128 MiB) on
 *     every GPU the library runs on, from its first use until the process
 *     ends.  A request whose dsa_decode_workspace_bytes() exceeds it fails
 *     with DSA_ERR_UNSUPPORTED before anything is enqueued.
 *   - `stream` must belong to the current device (the array's address is
 *     looked up once per device, on the current device).
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents; nothing in it needs to start at zero.  Calls that
 *     overlap in time on one GPU (other streams, other threads) race. */
size_t dsa_decode_static_scratch_bytes(void);
dsa_status dsa_decode_noalloc(const dsa_decode_args *a, hipStream_t stream);

/* The stages of dsa_decode, callable one by one.  dsa_decode is exactly
 *   dsa_decode_indexer_scores -> dsa_topk_select (n_valid = ctx_len) ->
 *   dsa_sparse_mla_paged_fwd
 * on buffers carved from its workspace.
 *
 * Indexer scores of each sequence's query against its cached keys:
 *   scores [B, ld_scores] fp32 out, ld_scores >= max_ctx; positions
 *   p < ctx_len[b] are written, the rest of the row is left untouched.
 *   (q, kv_pool, out, lse, idx_out of a are not used.) */
dsa_status dsa_decode_indexer_scores(const dsa_decode_args *a, float *scores, int64_t ld_scores,
                                     hipStream_t stream);

/* Sparse MLA over a paged latent pool: idx [T, k] holds LOGICAL positions of
 * sequence t (-1 = skip); row = block_table[t*max_blocks + p/64]*64 + p%64
 * of kv_pool [n_pool_rows, 576] BF16.  q [T,H,576] BF16, out [T,H,512] BF16,
 * lse [T,H] fp32 or NULL.  Entries whose page is unmapped (or outside the
 * pool) are skipped.  workspace as for dsa_sparse_mla_fwd (optional). */
dsa_status dsa_sparse_mla_paged_fwd(const void *q, const void *kv_pool, int64_t n_pool_rows,
                                    const int32_t *block_table, int32_t max_blocks,
                                    const int32_t *idx, int32_t T, int32_t H, int32_t k,
                                    float sm_scale, void *out, float *lse, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Paged cache append (MLA's latent cache: jienda.com, section 2.1): write one
 * token per sequence into the pools at logical position pos[b].
 *   latent [B,576] BF16, k8 [B,D_I] E4M3, ks [B] fp32, pos [B] int32 (device)
 *   pools and block_table as for dsa_decode; D_I must be 128 (the row stride
 *   of the key pool that dsa_decode reads).  A position that the block table
 *   does not map (negative, past max_blocks, an unmapped page, a row past the
 *   pool) writes nothing; rows of different b must differ.
 * dsa_decode does not append: a serving step calls this, then dsa_decode
 * with ctx_len grown by one, so the new token is its own query's candidate.
 */
dsa_status dsa_paged_cache_append(const void *latent, const uint8_t *k8, const float *ks,
                                  const int32_t *pos, int32_t B, int32_t D_I,
                                  const int32_t *block_table, int32_t max_blocks, void *kv_pool,
                                  uint8_t *k8_pool, float *ks_pool, int64_t n_pool_rows,
                                  hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
