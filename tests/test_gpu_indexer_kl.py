"""GPU parity of the indexer's KL-alignment loss (forward) and of the index
scores at listed positions, against the fp64 oracle, through the C ABI.

The KL kernel takes each head's log-sum-exp from the library's sparse-MLA
forward on the same selection, as a training step would.  Tolerance: with
lse_h off by at most e (the sparse-MLA lse bound, 1e-3), each head's
softmax moves by at most a factor exp(e), the renormalised head average p by
at most 2e in log, and KL = sum p (log p - log pi) by at most 2e * M, with
M = sum p |log p - log pi| from the oracle; 1e-4 more covers fp32 logits,
exponentials and sums.  Each test prints its case before touching the GPU.
"""
import math

import numpy as np
import pytest
import torch

import synth
from tests.parity import check_scores, check_topk_row, oracle_score_bounds

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LSE_EPS = 1e-3
KL_ABS = 1e-4


def _say(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def dsa():
    from sparse_attention_gemm_amd import dsa as d
    d.load()
    return d


def _check_kl(gpu, ora_kl, ora_mag, label):
    gpu = np.asarray(gpu, np.float64)
    assert np.isfinite(gpu).all(), f"{label}: non-finite loss"
    err = np.abs(gpu - ora_kl)
    bound = 2 * LSE_EPS * ora_mag + KL_ABS
    bad = err > bound
    assert not bad.any(), (f"{label}: {bad.sum()} losses out of tolerance; worst err {err.max():.3e} "
                           f"(bound there {bound[np.argmax(err)]:.3e})")
    return float(err.max())


def _mla_lse(dsa, q, kv, idx, scale):
    T, H = q.shape[0], q.shape[1]
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, H), dtype=torch.float32, device=DEV)
    dsa.dsa_sparse_mla_fwd(q, kv, idx, scale, out, lse)
    return lse


def _kl_gpu(dsa, q, kv, idx, sc, scale):
    qd, kvd, idd, scd = q.to(DEV), kv.to(DEV), idx.to(DEV), sc.to(DEV)
    lse = _mla_lse(dsa, qd, kvd, idd, scale)
    kl = torch.empty(q.shape[0], dtype=torch.float32, device=DEV)
    dsa.dsa_indexer_kl_fwd(qd, kvd, idd, scd, lse, scale, kl)
    torch.cuda.synchronize()
    return kl.cpu().double().numpy()


def _quant(dsa, x):
    rows, cols = x.numel() // x.shape[-1], x.shape[-1]
    x8 = torch.empty(x.shape, dtype=torch.uint8, device=DEV)
    sc = torch.empty(x.shape[:-1], dtype=torch.float32, device=DEV)
    dsa.dsa_quantize_e4m3_per_token(x.to(DEV).contiguous(), x8, sc, rows=rows, cols=cols)
    return x8, sc


@pytest.mark.parametrize("H_I", [64, 32])
def test_indexer_scores_at_positions(dsa, ora, H_I):
    """Bit-identical to the unfused score matrix at the listed positions, and
    within the score tolerance of the oracle; -inf outside [0, S)."""
    T, S, k = 37, 900, 300
    _say(f"indexer scores at positions T={T} S={S} k={k} H_I={H_I}")
    q = synth.normal(41, 1, (T, H_I, 128))
    kk = synth.normal(41, 2, (S, 128))
    w = synth.normal(41, 3, (T, H_I), std=0.5)
    q8, qs = _quant(dsa, q)
    k8, ks = _quant(dsa, kk)
    wd = w.to(DEV)
    idx = synth.randint(41, 4, (T, k), 0, S - 1).to(torch.int32)
    idx[3, :10] = -1
    idx[4, 5] = S + 7
    idd = idx.to(DEV)
    out = torch.empty((T, k), dtype=torch.float32, device=DEV)
    dsa.dsa_indexer_scores_at(q8, qs, k8, ks, wd, idd, out)
    full = torch.empty((T, S), dtype=torch.float32, device=DEV)
    pos = torch.full((T,), S - 1, dtype=torch.int32, device=DEV)  # every key visible
    dsa.dsa_indexer_scores(q8, qs, k8, ks, wd, pos, full, dsa.DSA_E4M3)
    torch.cuda.synchronize()
    g = out.cpu()
    valid = (idx >= 0) & (idx < S)
    ref = torch.gather(full.cpu(), 1, idx.clamp(0, S - 1).long())
    assert torch.equal(g[valid].view(torch.int32), ref[valid].view(torch.int32))
    assert torch.all(torch.isneginf(g[~valid]))
    rows = np.array([0, 5, 17, T - 1])
    o, m = oracle_score_bounds(ora, q8.cpu().numpy(), k8.cpu().numpy(), w.numpy(),
                                  np.full(T, S - 1, np.int32), rows=rows, q_scale=qs.cpu().numpy(),
                                  k_scale=ks.cpu().numpy())
    for j, r in enumerate(rows):
        sel = idx[r][valid[r]].long().numpy()
        check_scores(g[r][valid[r]].numpy(), o[j][sel], m[j][sel], 128 + H_I, f"row {r}")


@pytest.mark.parametrize("H,k,qstd,sstd", [(128, 2048, 1.0, 1.0), (16, 256, 1.0, 3.0), (64, 100, 40.0, 1.0),
                                           (32, 37, 1.0, 0.0)])
def test_indexer_kl_random_selection(dsa, ora, H, k, qstd, sstd):
    N, T = 3000, 24
    _say(f"indexer KL random selection H={H} k={k} qstd={qstd} sstd={sstd}")
    q = synth.normal(42, 1, (T, H, 576), std=qstd).to(torch.bfloat16)
    kv = synth.normal(42, 2, (N, 576), std=1 / 24).to(torch.bfloat16)
    idx = torch.stack([synth.permutation(42, 10 + t, N)[:k] for t in range(T)]).to(torch.int32)
    idx[1, k // 2:] = -1          # ragged selection
    idx[2, :] = -1                # empty selection: loss 0
    idx[3, 0] = N + 3             # out of range: skipped
    sc = synth.normal(42, 3, (T, k), std=max(sstd, 1e-30)) if sstd > 0 else torch.zeros((T, k))
    g = _kl_gpu(dsa, q, kv, idx, sc, 1 / math.sqrt(192))
    ref_idx = idx.clone()
    ref_idx[3, 0] = -1
    kl, mag = ora.indexer_kl_rows(q, kv, ref_idx.numpy(), sc.double().numpy(), 1 / math.sqrt(192))
    assert g[2] == 0.0
    _check_kl(g, kl, mag, f"KL H={H} k={k}")


def test_indexer_kl_dense_causal(dsa, ora):
    """The dense warm-up form: every causal position is in S_t."""
    L, H = 300, 32
    _say(f"indexer KL dense causal L={L} H={H}")
    q = synth.normal(43, 1, (L, H, 576), std=4.0).to(torch.bfloat16)
    kv = synth.normal(43, 2, (L, 576), std=1 / 24).to(torch.bfloat16)
    k = 320
    idx = torch.full((L, k), -1, dtype=torch.int32)
    for t in range(L):
        idx[t, :t + 1] = torch.arange(t + 1)
    sc = synth.normal(43, 3, (L, k), std=2.0)
    g = _kl_gpu(dsa, q, kv, idx, sc, 1 / math.sqrt(192))
    kl, mag = ora.indexer_kl_rows(q, kv, idx.numpy(), sc.double().numpy(), 1 / math.sqrt(192))
    assert g[0] == pytest.approx(0.0, abs=1e-6)  # one position: p = pi = 1
    _check_kl(g, kl, mag, "KL dense")


def _selection_pipeline(dsa, cfg):
    """Quantise -> fused selection -> scores at the selection -> sparse MLA lse -> KL."""
    L = cfg.L
    q_i, k_i, w = synth.prefill_indexer_inputs(cfg, device=DEV)
    q8, qs = _quant(dsa, q_i)
    k8, ks = _quant(dsa, k_i)
    idx = torch.empty((L, cfg.k), dtype=torch.int32, device=DEV)
    args = dsa.make_prefill_args(L, cfg.H_I, cfg.D_I, cfg.H, cfg.k, dsa.DSA_E4M3, q8, qs, k8, ks, w, dsa.DSA_BF16,
                                 None, None, cfg.sm_scale, idx, None, None)
    ws = torch.empty(dsa.dsa_prefill_workspace_bytes(args), dtype=torch.uint8, device=DEV)
    dsa.dsa_prefill_select(args, ws)
    del ws
    sc = torch.empty((L, cfg.k), dtype=torch.float32, device=DEV)
    dsa.dsa_indexer_scores_at(q8, qs, k8, ks, w, idx, sc)
    q = synth.prefill_attn_q(cfg, device=DEV)
    kv = synth.prefill_latent(cfg, device=DEV)
    lse = _mla_lse(dsa, q, kv, idx, cfg.sm_scale)
    kl = torch.empty(L, dtype=torch.float32, device=DEV)
    dsa.dsa_indexer_kl_fwd(q, kv, idx, sc, lse, cfg.sm_scale, kl)
    torch.cuda.synchronize()
    return dict(q8=q8, qs=qs, k8=k8, ks=ks, w=w, idx=idx, sc=sc, q=q, kv=kv, kl=kl)


def _check_pipeline(ora, cfg, r, rows, label):
    rt = torch.from_numpy(rows).to(DEV)
    # the selection ranks the scores the KL kernel receives
    osc = ora.indexer_rows(r["q8"][rt].cpu().numpy(), r["k8"].cpu().numpy(), r["w"][rt].cpu().numpy(),
                           rows.astype(np.int32), q_scale=r["qs"][rt].cpu().numpy(), k_scale=r["ks"].cpu().numpy())
    gidx = r["idx"][rt].cpu().numpy()
    for j, t in enumerate(rows):
        check_topk_row(gidx[j], osc[j], int(t) + 1, cfg.k, f"{label} row {t}")
    kl, mag = ora.indexer_kl_rows(r["q"][rt].cpu(), r["kv"].cpu(), gidx, r["sc"][rt].cpu().double().numpy(),
                                  cfg.sm_scale)
    return _check_kl(r["kl"][rt].cpu().numpy(), kl, mag, label)


def test_indexer_kl_after_prefill_selection(dsa, ora):
    cfg = synth.scaled_down(synth.CONFIGS["prefill16k"], L=2500, H=16, k=1024, seed=9)
    _say(f"indexer KL pipeline L={cfg.L} H={cfg.H} k={cfg.k}")
    r = _selection_pipeline(dsa, cfg)
    rows = np.unique(np.concatenate([np.arange(0, cfg.L, 97), [0, 1, cfg.k - 1, cfg.k, cfg.L - 1]]))
    _check_pipeline(ora, cfg, r, rows, "KL pipeline")


def test_indexer_kl_prefill16k_sampled(dsa, ora):
    """The L = 16384 prefill workload (H = 128, k = 2048), sampled rows."""
    cfg = synth.CONFIGS["prefill16k"]
    _say(f"indexer KL pipeline L={cfg.L} H={cfg.H} k={cfg.k}")
    r = _selection_pipeline(dsa, cfg)
    rows = np.array([0, 1, 2047, 2048, 9000, cfg.L - 1], dtype=np.int64)
    _check_pipeline(ora, cfg, r, rows, "KL L=16384")
