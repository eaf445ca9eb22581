"""GPU parity of the backward entries against the fp64 oracle, through the C ABI.

Tolerances (each derived from the arithmetic of the kernel it checks):
  * score gradient of the KL loss, g = dkl (pi - p): pi is an fp32 softmax of
    the given scores and p sums each head's exp(z - lse) with z from bf16 MFMA
    logits (fp32 sums) and lse from the sparse-MLA forward; both carry relative
    errors far below 1e-4, so |dg| <= 1e-4 dkl (pi + p) + 1e-9.
  * indexer gradients from a given score gradient: the dot products are
    exact (E4M3 x E4M3) with fp32 sums; the dq and dk products take their fp32
    coefficient (g ks w, or w) as the sum of two bf16 terms (hi = RNE(v),
    lo = RNE(v - hi)), which leaves at most 2^-18 |v| of it out, times an
    operand exact in bf16; every sum is fp32, over at most k keys (dw, dq),
    H_I heads and T pairs (dk).  The a-priori bound
    ((k + H_I + T + 8) 2^-24 + 2^-18) mag covers this, with mag the oracle's
    sum of |terms| (for dw, |g| times the magnitude of each dot product, which
    also bounds its own rounding), plus amb: the terms whose dot product lies
    within the FP8 MFMA's accuracy (FP8_MFMA_SUM_REL of the sum of the
    products' magnitudes; the kernel forms x with that MFMA) of the ReLU kink,
    where the GPU may take the other side.
Each test prints its case before touching the GPU.
"""
import math

import numpy as np
import pytest
import torch

import synth
from tests.parity import FP8_MFMA_SUM_REL

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
U = 2.0 ** -24
SPLIT = 2.0 ** -18   # residue of a coefficient held as two bf16 terms


def _say(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def dsa():
    from sparse_attention_gemm_amd import dsa as d
    d.load()
    return d


def _selection(seed, T, N, k, causal=False):
    """Sorted selections with padding, an empty row and out-of-range entries."""
    rows = []
    for t in range(T):
        n = min(k, (t + 1) if causal else N)
        pool = (t + 1) if causal else N
        sel = torch.sort(synth.permutation(seed, 100 + t, pool)[:n]).values
        rows.append(torch.cat([sel, torch.full((k - n,), -1, dtype=torch.int64)]))
    idx = torch.stack(rows).to(torch.int32)
    if T > 3:
        idx[1, k // 3:] = -1          # ragged
        idx[2, :] = -1                # empty
    return idx


def _pi_p(scores, idx, g_ref, dkl):
    """pi = softmax of the scores over the valid entries, and p = pi - g / dkl
    (the oracle's target), the scales of the score gradient's tolerance."""
    sc = np.where(idx >= 0, scores, -np.inf)
    mx = np.max(np.where(np.isfinite(sc), sc, -1e300), axis=1, keepdims=True)
    e = np.where(np.isfinite(sc), np.exp(np.minimum(sc - mx, 0.0)), 0.0)
    tot = e.sum(axis=1, keepdims=True)
    pi = np.divide(e, tot, out=np.zeros_like(e), where=tot > 0)
    return pi, pi - g_ref / np.asarray(dkl)[:, None]


def _check(name, gpu, ref, tol):
    gpu = np.asarray(gpu, np.float64)
    err = np.abs(gpu - ref)
    bad = err > tol
    worst = float((err / np.maximum(tol, 1e-300)).max()) if err.size else 0.0
    print(f"[grad] {name}: worst err/bound {worst:.3g}, max|ref| {np.abs(ref).max():.3g}", flush=True)
    assert not bad.any(), f"{name}: {bad.sum()} of {bad.size} out of tolerance; worst err/bound {worst:.3g}"


@pytest.mark.parametrize("H,k,sstd", [(128, 2048, 1.0), (16, 256, 4.0), (64, 100, 0.3)])
def test_indexer_kl_grad(dsa, ora, H, k, sstd):
    T, N = 12, 3000
    _say(f"indexer KL score gradient H={H} k={k} sstd={sstd}")
    q = synth.normal(41, 1, (T, H, 576)).to(torch.bfloat16)
    kv = synth.normal(41, 2, (N, 576), std=1 / 24).to(torch.bfloat16)
    idx = _selection(41, T, N, k)
    idx[3, 7] = N + 5                 # out of range: no row
    scores = synth.normal(41, 3, (T, k), std=sstd)
    dkl = synth.uniform(41, 4, (T,), lo=0.5, hi=1.5)
    d = {n: x.to(DEV) for n, x in dict(q=q, kv=kv, idx=idx, sc=scores, dkl=dkl).items()}
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, H), dtype=torch.float32, device=DEV)
    dsa.dsa_sparse_mla_fwd(d["q"], d["kv"], d["idx"], 1 / math.sqrt(192), out, lse)
    grad = torch.full((T, k), 7.0, dtype=torch.float32, device=DEV)
    dsa.dsa_indexer_kl_bwd(d["q"], d["kv"], d["idx"], d["sc"], lse, d["dkl"], 1 / math.sqrt(192), grad)
    torch.cuda.synchronize()
    ref_idx = idx.clone()
    ref_idx[3, 7] = -1
    g_ref = ora.indexer_kl_grad(q, kv, ref_idx.numpy(), scores.double().numpy(), dkl.double().numpy(),
                                1 / math.sqrt(192))
    pi, p = _pi_p(scores.double().numpy(), ref_idx.numpy(), g_ref, dkl.double().numpy())
    tol = 1e-4 * dkl.double().numpy()[:, None] * (pi + np.abs(p)) + 1e-9
    _check("score gradient", grad.cpu().numpy(), g_ref, tol)
    assert torch.all(grad.cpu()[2] == 0) and grad.cpu()[3, 7] == 0
    np.testing.assert_allclose(grad.cpu().double().sum(dim=1).numpy(), 0, atol=1e-5)


def _indexer_inputs(seed, T, S):
    q = synth.normal(seed, synth.T_QI, (T, 64, 128))
    kk = synth.normal(seed, synth.T_KI, (S, 128))
    w = synth.normal(seed, synth.T_W, (T, 64), std=0.5)
    return q, kk, w


@pytest.mark.parametrize("T,S,k,causal", [(40, 3000, 2048, False), (300, 300, 256, True), (1100, 2500, 64, False),
                                          (24, 40000, 2048, False)])
def test_indexer_bwd_from_score_gradient(dsa, ora, T, S, k, causal):
    """dw, dq, dk from a given score gradient; T = 1100 spans two query chunks
    of the inverted-selection reduce; S = 40000 keys take three pages of its
    prefix scan."""
    _say(f"indexer backward T={T} S={S} k={k} causal={causal}")
    q, kk, w = _indexer_inputs(43, T, S)
    q8, qs = ora.quantize_rows(q.view(T, -1).numpy())
    k8, ks = ora.quantize_rows(kk.numpy())
    q8 = q8.reshape(T, 64, 128)
    idx = _selection(43, T, S, k, causal=causal)
    idx[0, 1] = S + 7                 # out of range: skipped
    g = synth.normal(43, 5, (T, k), std=1e-2)
    d = {n: torch.from_numpy(np.ascontiguousarray(x)).to(DEV) if isinstance(x, np.ndarray) else x.to(DEV)
         for n, x in dict(q8=q8, qs=qs, k8=k8, ks=ks, w=w, idx=idx, g=g).items()}
    dw = torch.full((T, 64), 7.0, device=DEV)
    dq = torch.full((T, 64, 128), 7.0, device=DEV)
    dk = torch.full((S, 128), 7.0, device=DEV)
    ws = torch.empty(dsa.dsa_indexer_bwd_workspace_bytes(T, S, k), dtype=torch.uint8, device=DEV)
    dsa.dsa_indexer_bwd(d["q8"], d["qs"], d["k8"], d["ks"], d["w"], d["idx"], d["g"], dw, dq, dk, ws)
    torch.cuda.synchronize()
    ref_idx = idx.clone()
    ref_idx[0, 1] = -1
    r = ora.indexer_bwd(q8, k8, w.double().numpy(), ref_idx.numpy(), g.double().numpy(), q_scale=qs, k_scale=ks,
                        kink_rel=FP8_MFMA_SUM_REL)
    f = (k + 64 + T + 8) * U
    fs = f + SPLIT  # dq, dk: the coefficient enters as two bf16 terms
    _check("dw", dw.cpu().numpy(), r["dw"], f * r["mag_dw"] + 1e-30)
    _check("dq", dq.cpu().numpy(), r["dq"], fs * r["mag_dq"] + r["amb_dq"] + 1e-30)
    _check("dk", dk.cpu().numpy(), r["dk"], fs * r["mag_dk"] + r["amb_dk"] + 1e-30)
    # keys nobody selected get exactly zero
    chosen = np.zeros(S, bool)
    chosen[ref_idx.numpy()[ref_idx.numpy() >= 0]] = True
    assert torch.all(dk.cpu()[torch.from_numpy(~chosen)] == 0)


def test_indexer_bwd_row_past_the_sort(dsa, ora):
    """Every query lists key 7 eight times: 8192 pairs of one key in the first
    chunk of 1024 queries, more than the reduce sorts in LDS (4096), so that
    key is summed in arrival order; the rest as usual."""
    T, S, k = 1100, 500, 64
    _say(f"indexer backward, a key listed past the sort capacity T={T} S={S} k={k}")
    q, kk, w = _indexer_inputs(45, T, S)
    q8, qs = ora.quantize_rows(q.view(T, -1).numpy())
    k8, ks = ora.quantize_rows(kk.numpy())
    q8 = q8.reshape(T, 64, 128)
    idx = _selection(45, T, S, k)
    idx[:, :8] = 7
    g = synth.normal(45, 5, (T, k), std=1e-2)
    d = {n: torch.from_numpy(np.ascontiguousarray(x)).to(DEV) if isinstance(x, np.ndarray) else x.to(DEV)
         for n, x in dict(q8=q8, qs=qs, k8=k8, ks=ks, w=w, idx=idx, g=g).items()}
    dw, dq, dk = (torch.empty((T, 64), device=DEV), torch.empty((T, 64, 128), device=DEV),
                  torch.empty((S, 128), device=DEV))
    ws = torch.empty(dsa.dsa_indexer_bwd_workspace_bytes(T, S, k), dtype=torch.uint8, device=DEV)
    dsa.dsa_indexer_bwd(d["q8"], d["qs"], d["k8"], d["ks"], d["w"], d["idx"], d["g"], dw, dq, dk, ws)
    torch.cuda.synchronize()
    r = ora.indexer_bwd(q8, k8, w.double().numpy(), idx.numpy(), g.double().numpy(), q_scale=qs, k_scale=ks,
                        kink_rel=FP8_MFMA_SUM_REL)
    # key 7's dk sums up to 8 T pairs, so the fp32 term count grows accordingly
    f = (k + 64 + 8 * T + 8) * U
    _check("dw", dw.cpu().numpy(), r["dw"], f * r["mag_dw"] + 1e-30)
    _check("dq", dq.cpu().numpy(), r["dq"], (f + SPLIT) * r["mag_dq"] + r["amb_dq"] + 1e-30)
    _check("dk", dk.cpu().numpy(), r["dk"], (f + SPLIT) * r["mag_dk"] + r["amb_dk"] + 1e-30)


def test_indexer_bwd_is_deterministic(dsa):
    """The dk reduce sums each key's pairs in a fixed order: two runs agree bit for bit."""
    T, S, k = 700, 2000, 512
    _say("indexer backward determinism")
    q, kk, w = _indexer_inputs(44, T, S)
    q8 = synth.to_e4m3_bits(q).to(DEV)
    k8 = synth.to_e4m3_bits(kk).to(DEV)
    qs, ks = torch.ones(T, device=DEV), torch.ones(S, device=DEV)
    idx = _selection(44, T, S, k).to(DEV)
    g = synth.normal(44, 5, (T, k), std=1e-2).to(DEV)
    ws = torch.empty(dsa.dsa_indexer_bwd_workspace_bytes(T, S, k), dtype=torch.uint8, device=DEV)
    res = []
    for _ in range(2):
        dw, dq, dk = torch.empty((T, 64), device=DEV), torch.empty((T, 64, 128), device=DEV), torch.empty((S, 128),
                                                                                                            device=DEV)
        dsa.dsa_indexer_bwd(q8, qs, k8, ks, w.to(DEV), idx, g, dw, dq, dk, ws)
        torch.cuda.synchronize()
        res.append((dw.cpu(), dq.cpu(), dk.cpu()))
    for a, b in zip(*res):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_indexer_kl_backward_after_prefill_selection(dsa, ora):
    """The sparse-training indexer step end to end on the library's own fused
    selection: quantise -> fused indexer + top-k -> sparse MLA (lse) ->
    scores at the selection -> KL score gradient -> indexer backward, against
    the oracle's composed KL backward on the same selection."""
    L, k, H = 700, 128, 16
    _say(f"KL backward after the fused selection L={L} k={k} H={H}")
    cfg = synth.scaled_down(synth.CONFIGS["prefill16k"], L=L, k=k, H=H, seed=45)
    q_i, k_i, w = synth.prefill_indexer_inputs(cfg)
    q, kv = synth.prefill_attn_q(cfg), synth.prefill_latent(cfg)
    q8, qs = ora.quantize_rows(q_i.view(L, -1).numpy())
    k8, ks = ora.quantize_rows(k_i.numpy())
    q8 = q8.reshape(L, 64, 128)
    d = {n: torch.from_numpy(np.ascontiguousarray(x)).to(DEV) if isinstance(x, np.ndarray) else x.to(DEV)
         for n, x in dict(q8=q8, qs=qs, k8=k8, ks=ks, w=w, q=q, kv=kv).items()}
    idx = torch.empty((L, k), dtype=torch.int32, device=DEV)
    out = torch.empty((L, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((L, H), dtype=torch.float32, device=DEV)
    args = dsa.make_prefill_args(L, 64, 128, H, k, dsa.DSA_E4M3, d["q8"], d["qs"], d["k8"], d["ks"], d["w"],
                                 dsa.DSA_BF16, d["q"], d["kv"], cfg.sm_scale, idx, out, lse)
    pws = torch.empty(dsa.dsa_prefill_workspace_bytes(args), dtype=torch.uint8, device=DEV)
    dsa.dsa_prefill(args, pws)
    sc = torch.empty((L, k), dtype=torch.float32, device=DEV)
    dsa.dsa_indexer_scores_at(d["q8"], d["qs"], d["k8"], d["ks"], d["w"], idx, sc)
    dkl = torch.full((L,), 1.0 / L, dtype=torch.float32, device=DEV)   # the mean over tokens
    grad = torch.empty((L, k), dtype=torch.float32, device=DEV)
    dsa.dsa_indexer_kl_bwd(d["q"], d["kv"], idx, sc, lse, dkl, cfg.sm_scale, grad)
    dw, dq, dk = (torch.empty((L, 64), device=DEV), torch.empty((L, 64, 128), device=DEV),
                  torch.empty((L, 128), device=DEV))
    ws = torch.empty(dsa.dsa_indexer_bwd_workspace_bytes(L, L, k), dtype=torch.uint8, device=DEV)
    dsa.dsa_indexer_bwd(d["q8"], d["qs"], d["k8"], d["ks"], d["w"], idx, grad, dw, dq, dk, ws)
    torch.cuda.synchronize()
    gidx = idx.cpu().numpy()
    # step 1, the score gradient, against the oracle on the GPU's own scores
    dklv = np.full(L, 1.0 / L)
    g_ref = ora.indexer_kl_grad(q, kv, gidx, sc.cpu().double().numpy(), dklv, cfg.sm_scale)
    pi, p = _pi_p(sc.cpu().double().numpy(), gidx, g_ref, dklv)
    _check("score gradient (pipeline)", grad.cpu().numpy(), g_ref, 1e-4 * dklv[:, None] * (pi + np.abs(p)) + 1e-12)
    # step 2, the indexer gradients, on the GPU's own score gradient
    r = ora.indexer_bwd(q8, k8, w.double().numpy(), gidx, grad.cpu().double().numpy(), q_scale=qs, k_scale=ks,
                        kink_rel=FP8_MFMA_SUM_REL)
    f = (k + 64 + L + 8) * U
    fs = f + SPLIT  # dq, dk: the coefficient enters as two bf16 terms
    _check("dw (pipeline)", dw.cpu().numpy(), r["dw"], f * r["mag_dw"] + 1e-30)
    _check("dq (pipeline)", dq.cpu().numpy(), r["dq"], fs * r["mag_dq"] + r["amb_dq"] + 1e-30)
    _check("dk (pipeline)", dk.cpu().numpy(), r["dk"], fs * r["mag_dk"] + r["amb_dk"] + 1e-30)
    # and the composition: the GPU's steps reproduce the oracle's KL backward of the indexer's own
    # scores, up to those scores' fp32 rounding (pi moves by at most 2 pi |dI|)
    full = ora.indexer_kl_bwd(q, kv, q8, k8, w.double().numpy(), gidx, dklv, cfg.sm_scale, q_scale=qs, k_scale=ks,
                              kink_rel=FP8_MFMA_SUM_REL)
    sco = np.take_along_axis(ora.indexer_rows(q8, k8, w, np.arange(L, dtype=np.int32), q_scale=qs, k_scale=ks),
                             np.maximum(gidx, 0).astype(np.int64), axis=1)
    dI = float(np.abs(sc.cpu().double().numpy() - sco)[gidx >= 0].max())
    _check("score gradient vs the oracle's own scores", grad.cpu().numpy(), full["g"],
           (1e-4 + 2 * dI) * dklv[:, None] * (pi + np.abs(p)) + 1e-12)


# ------------------------------------------------------------------ sparse MLA backward
# dS and P enter the products rounded to bf16 (unit roundoff 2^-8 each), and
# D = dout . o uses the forward's bf16 output; the oracle's magnitudes carry
# the matching terms (|dS| + P sum|dout||o|, and P |dout|), so the error is
# within 2^-8 of them per rounding.  A dkv term also meets the bf16 rounding
# of its pair's sum over the heads (at most 2^-9 of that sum's magnitude), so
# 3 * 2^-8 mag covers the roundings a term meets plus the fp32 sums.
MLA_BWD_RTOL = 3 * 2.0 ** -8


def _mla_bwd_gpu(dsa, q, kv, idx, dout, sm):
    T, H = q.shape[0], q.shape[1]
    N, k = kv.shape[0], idx.shape[1]
    d = {n: x.to(DEV) for n, x in dict(q=q, kv=kv, idx=idx, dout=dout).items()}
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, H), dtype=torch.float32, device=DEV)
    dsa.dsa_sparse_mla_fwd(d["q"], d["kv"], d["idx"], sm, out, lse)
    dq = torch.full((T, H, 576), 7.0, device=DEV)
    dkv = torch.full((N, 576), 7.0, device=DEV)
    ws = torch.empty(dsa.dsa_sparse_mla_bwd_workspace_bytes(T, H, N, k), dtype=torch.uint8, device=DEV)
    dsa.dsa_sparse_mla_bwd(d["q"], d["kv"], d["idx"], out, lse, d["dout"], sm, dq, dkv, ws)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dkv.cpu().numpy()


@pytest.mark.parametrize("T,H,N,k,qstd", [(6, 128, 5000, 2048, 1.0), (600, 64, 3000, 256, 1.0),
                                          (9, 32, 2000, 100, 40.0), (5, 96, 1500, 512, 3.0),
                                          (6, 32, 40000, 2048, 1.0)])
def test_sparse_mla_bwd(dsa, ora, T, H, N, k, qstd):
    """dq and dkv against the oracle; T = 600 spans two query chunks; a sharp
    softmax (q x 40); N = 40000 rows take three pages of the reduce's prefix
    scan; a ragged, an empty and a duplicated entry, and an entry outside the
    latent rows."""
    _say(f"sparse mla backward T={T} H={H} N={N} k={k} qstd={qstd}")
    sm = 1 / math.sqrt(192)
    q = synth.normal(51, 1, (T, H, 576), std=qstd).to(torch.bfloat16)
    kv = synth.normal(51, 2, (N, 576), std=1 / 24).to(torch.bfloat16)
    dout = synth.normal(51, 3, (T, H, 512)).to(torch.bfloat16)
    idx = _selection(51, T, N - 1, k)          # row N-1 is never selected
    idx[0, 5] = N + 3                          # outside the rows: skipped
    idx[4, 1] = idx[4, 0]                      # one row listed twice
    dq, dkv = _mla_bwd_gpu(dsa, q, kv, idx, dout, sm)
    ref_idx = idx.clone()
    ref_idx[0, 5] = -1
    r = ora.sparse_mla_bwd(q, kv, ref_idx.numpy(), dout, sm)
    _check("dq", dq, r["dq"], MLA_BWD_RTOL * r["mag_dq"] + 1e-30)
    _check("dkv", dkv, r["dkv"], MLA_BWD_RTOL * r["mag_dkv"] + 1e-30)
    assert np.all(dkv[N - 1] == 0) and np.all(dq[2] == 0)


def test_sparse_mla_bwd_row_past_the_sort(dsa, ora):
    """Every query lists latent row 7 ten times: 5120 pairs of one row in the
    first chunk of 512 queries, more than the reduce sorts in LDS (4096), so
    that row is summed in arrival order (and the forward weighs the row ten
    times); the rest as usual."""
    T, H, N, k = 600, 32, 500, 64
    _say(f"sparse mla backward, a row listed past the sort capacity T={T} H={H} N={N} k={k}")
    sm = 1 / math.sqrt(192)
    q = synth.normal(54, 1, (T, H, 576)).to(torch.bfloat16)
    kv = synth.normal(54, 2, (N, 576), std=1 / 24).to(torch.bfloat16)
    dout = synth.normal(54, 3, (T, H, 512)).to(torch.bfloat16)
    idx = _selection(54, T, N, k)
    idx[:, :10] = 7
    dq, dkv = _mla_bwd_gpu(dsa, q, kv, idx, dout, sm)
    r = ora.sparse_mla_bwd(q, kv, idx.numpy(), dout, sm)
    _check("dq", dq, r["dq"], MLA_BWD_RTOL * r["mag_dq"] + 1e-30)
    _check("dkv", dkv, r["dkv"], MLA_BWD_RTOL * r["mag_dkv"] + 1e-30)


def test_sparse_mla_bwd_is_deterministic(dsa):
    T, H, N, k = 700, 128, 4000, 512
    _say("sparse mla backward determinism")
    q = synth.normal(52, 1, (T, H, 576)).to(torch.bfloat16)
    kv = synth.normal(52, 2, (N, 576), std=1 / 24).to(torch.bfloat16)
    dout = synth.normal(52, 3, (T, H, 512)).to(torch.bfloat16)
    idx = _selection(52, T, N, k)
    a = _mla_bwd_gpu(dsa, q, kv, idx, dout, 0.07)
    b = _mla_bwd_gpu(dsa, q, kv, idx, dout, 0.07)
    assert np.array_equal(a[0].view(np.int32), b[0].view(np.int32))
    assert np.array_equal(a[1].view(np.int32), b[1].view(np.int32))


@pytest.mark.parametrize("T,H,N,k,sstd", [(600, 128, 3000, 256, 1.0), (9, 32, 2000, 100, 4.0),
                                          (5, 96, 1500, 512, 0.3), (6, 128, 5000, 2048, 1.0)])
def test_sparse_mla_bwd_kl(dsa, ora, T, H, N, k, sstd):
    """The backward of both losses from one pass: dq and dkv bit-identical to
    dsa_sparse_mla_bwd's, and the KL score gradient from the same P against the
    oracle, with the tolerance of the standalone KL gradient (and against
    dsa_indexer_kl_bwd where it takes H).  T = 600 spans two query chunks and
    two head groups of 64; H = 32 and 96 take groups of 32; a ragged row, an
    empty row and an entry outside the latent rows."""
    _say(f"sparse mla backward with the KL score gradient T={T} H={H} N={N} k={k} sstd={sstd}")
    sm = 1 / math.sqrt(192)
    q = synth.normal(55, 1, (T, H, 576)).to(torch.bfloat16)
    kv = synth.normal(55, 2, (N, 576), std=1 / 24).to(torch.bfloat16)
    dout = synth.normal(55, 3, (T, H, 512)).to(torch.bfloat16)
    idx = _selection(55, T, N, k)
    idx[0, 5] = N + 3                          # outside the rows: no row
    scores = synth.normal(55, 4, (T, k), std=sstd)
    dkl = synth.uniform(55, 5, (T,), lo=0.5, hi=1.5)
    d = {n: x.to(DEV) for n, x in dict(q=q, kv=kv, idx=idx, dout=dout, sc=scores, dkl=dkl).items()}
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, H), dtype=torch.float32, device=DEV)
    dsa.dsa_sparse_mla_fwd(d["q"], d["kv"], d["idx"], sm, out, lse)
    ws = torch.empty(dsa.dsa_sparse_mla_bwd_workspace_bytes(T, H, N, k), dtype=torch.uint8, device=DEV)
    dq1, dkv1 = torch.full((T, H, 576), 7.0, device=DEV), torch.full((N, 576), 7.0, device=DEV)
    dsa.dsa_sparse_mla_bwd(d["q"], d["kv"], d["idx"], out, lse, d["dout"], sm, dq1, dkv1, ws)
    dq2, dkv2 = torch.full((T, H, 576), 7.0, device=DEV), torch.full((N, 576), 7.0, device=DEV)
    grad = torch.full((T, k), 7.0, device=DEV)
    dsa.dsa_sparse_mla_bwd_kl(d["q"], d["kv"], d["idx"], out, lse, d["dout"], d["sc"], d["dkl"], sm, dq2, dkv2, grad,
                              ws)
    standalone = None
    if H in (16, 32, 64, 128):
        standalone = torch.full((T, k), 7.0, device=DEV)
        dsa.dsa_indexer_kl_bwd(d["q"], d["kv"], d["idx"], d["sc"], lse, d["dkl"], sm, standalone)
    torch.cuda.synchronize()
    assert torch.equal(dq1.view(torch.int32), dq2.view(torch.int32))
    assert torch.equal(dkv1.view(torch.int32), dkv2.view(torch.int32))
    ref_idx = idx.clone()
    ref_idx[0, 5] = -1
    g_ref = ora.indexer_kl_grad(q, kv, ref_idx.numpy(), scores.double().numpy(), dkl.double().numpy(), sm)
    pi, p = _pi_p(scores.double().numpy(), ref_idx.numpy(), g_ref, dkl.double().numpy())
    tol = 1e-4 * dkl.double().numpy()[:, None] * (pi + np.abs(p)) + 1e-9
    g = grad.cpu()
    _check("score gradient (fused)", g.numpy(), g_ref, tol)
    if standalone is not None:
        _check("score gradient (fused) vs dsa_indexer_kl_bwd", g.numpy(), standalone.cpu().double().numpy(), 2 * tol)
    assert torch.all(g[2] == 0) and g[0, 5] == 0
    np.testing.assert_allclose(g.double().sum(dim=1).numpy(), 0, atol=1e-5)


def test_sparse_mla_bwd_after_prefill_selection(dsa, ora):
    """The sparse-training attention step on the library's own fused causal
    selection: fused prefill -> backward, against the oracle on that selection."""
    L, k, H = 1200, 256, 64
    _say(f"sparse mla backward after the fused selection L={L} k={k} H={H}")
    cfg = synth.scaled_down(synth.CONFIGS["prefill16k"], L=L, k=k, H=H, seed=53)
    q_i, k_i, w = synth.prefill_indexer_inputs(cfg)
    q, kv = synth.prefill_attn_q(cfg), synth.prefill_latent(cfg)
    q8, qs = ora.quantize_rows(q_i.view(L, -1).numpy())
    k8, ks = ora.quantize_rows(k_i.numpy())
    d = {n: torch.from_numpy(np.ascontiguousarray(x)).to(DEV) if isinstance(x, np.ndarray) else x.to(DEV)
         for n, x in dict(q8=q8.reshape(L, 64, 128), qs=qs, k8=k8, ks=ks, w=w, q=q, kv=kv).items()}
    idx = torch.empty((L, k), dtype=torch.int32, device=DEV)
    args = dsa.make_prefill_args(L, 64, 128, H, k, dsa.DSA_E4M3, d["q8"], d["qs"], d["k8"], d["ks"], d["w"],
                                 dsa.DSA_BF16, None, None, cfg.sm_scale, idx, None, None)
    ws = torch.empty(dsa.dsa_prefill_workspace_bytes(args), dtype=torch.uint8, device=DEV)
    dsa.dsa_prefill_select(args, ws)
    torch.cuda.synchronize()
    dout = synth.normal(53, 9, (L, H, 512), std=0.01).to(torch.bfloat16)
    gidx = idx.cpu()
    dq, dkv = _mla_bwd_gpu(dsa, q, kv, gidx, dout, cfg.sm_scale)
    r = ora.sparse_mla_bwd(q, kv, gidx.numpy(), dout, cfg.sm_scale)
    _check("dq (pipeline)", dq, r["dq"], MLA_BWD_RTOL * r["mag_dq"] + 1e-30)
    _check("dkv (pipeline)", dkv, r["dkv"], MLA_BWD_RTOL * r["mag_dkv"] + 1e-30)
