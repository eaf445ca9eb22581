"""GPU parity of the masked-MHA short-prefill mode (MLA in its multi-head form
under the top-k mask) against the fp64 oracle, through the C ABI.

Selections are either drawn at random (with padding, empty rows, and entries
the mask ignores: non-causal, out of range, repeated) or produced by the
library's own fused FP8 indexer + top-k, as in the short-prefill pipeline.
Each test prints its case before touching the GPU.
"""
import math

import numpy as np
import pytest
import torch

import synth
from tests.parity import check_attention, check_topk_row

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DN = synth.MHA_DN


def _say(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def dsa():
    from sparse_attention_gemm_amd import dsa as d
    d.load()
    return d


def _selector_weights(H, seed):
    """Up-projections with one weight of 32 per output dim (a seeded choice of
    latent dim): every K_h and V_h element is 32 times a bf16 latent value,
    exact in fp16, so the kernel's one rounding of K_h and V_h vanishes and
    sharp softmaxes test the attention arithmetic alone."""
    ws = []
    for m in range(2):
        w = torch.zeros((H, DN, synth.MHA_DC), dtype=torch.bfloat16)
        for h in range(H):
            pick = synth.permutation(seed, 40 + 2 * h + m, synth.MHA_DC)[:DN]
            w[h, torch.arange(DN), pick] = 32.0
        ws.append(w)
    return ws


def _inputs(L, H, seed, q_std=1.0, selector=False):
    cfg = synth.PrefillConfig(f"mha_L{L}", L, 64, 128, H, 2048, seed, "bf16", True, q_std=q_std)
    q = synth.mha_query(cfg)
    kv = synth.prefill_latent(cfg)
    w_uk, w_uv = _selector_weights(H, seed) if selector else synth.mha_up_weights(cfg)
    return cfg, q, kv, w_uk, w_uv


def _run(dsa, q, kv, w_uk, w_uv, idx, scale):
    L, H = q.shape[0], q.shape[1]
    out = torch.empty((L, H, synth.MHA_DV), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((L, H), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(dsa.dsa_masked_mha_workspace_bytes(L, H), 1), dtype=torch.uint8, device=DEV)
    dsa.dsa_masked_mha_prefill(q.to(DEV), kv.to(DEV), w_uk.to(DEV), w_uv.to(DEV), idx.to(DEV), scale, out, ws, lse)
    torch.cuda.synchronize()
    return out.float().cpu().double().numpy(), lse.cpu().double().numpy()


def _lse_slack(q, kv, w_uk, idx, rows, heads, scale):
    """2 * 2^-11 * sm_scale * max over the row's selected keys of sum_e |q_e K_e|
    over the up-projected (no-rope) dims; see tests/parity.py."""
    c = kv[:, :synth.MHA_DC].double().numpy()
    out = np.zeros((len(rows), len(heads)))
    for j, h in enumerate(heads):
        kabs = np.abs(c @ w_uk[h].double().numpy().T)             # [L, 128]
        qabs = np.abs(q[rows, h, :DN].double().numpy())           # [n, 128]
        for i, r in enumerate(rows):
            sel = idx[r][idx[r] >= 0]
            if sel.size:
                out[i, j] = (kabs[sel] @ qabs[i]).max()
    return 2.0 * 2.0 ** -11 * scale * out


def _reference_idx(idx):
    """The oracle's view of a selection: entries the mask ignores (outside
    [0, t], or repeated) become -1."""
    ref = idx.copy()
    for t in range(ref.shape[0]):
        row = ref[t]
        row[(row < 0) | (row > t)] = -1
        seen = set()
        for a in range(row.size):
            if row[a] >= 0:
                if row[a] in seen:
                    row[a] = -1
                else:
                    seen.add(int(row[a]))
    return ref


def _random_selection(L, k, seed):
    """Rows pick min(k, t+1) random causal positions, in random order."""
    u = synth.uniform(seed, 20, (L, L))
    u = torch.where(torch.arange(L)[None, :] <= torch.arange(L)[:, None], u, torch.full_like(u, -1.0))
    kk = min(k, L)
    v, i = torch.topk(u, kk, dim=1)
    idx = torch.where(v >= 0, i, torch.full_like(i, -1)).to(torch.int32)
    if kk < k:
        idx = torch.cat([idx, torch.full((L, k - kk), -1, dtype=torch.int32)], dim=1)
    return idx


def _check(ora, q, kv, w_uk, w_uv, idx_np, g, gl, rows, scale, label, heads=None):
    heads = np.arange(q.shape[1]) if heads is None else np.asarray(heads)
    ref = _reference_idx(idx_np)
    hsel = torch.from_numpy(heads)
    o, l = ora.masked_mha_rows(q[:, hsel].contiguous(), kv, w_uk[hsel].contiguous(), w_uv[hsel].contiguous(), ref,
                               scale, rows=rows)
    slack = _lse_slack(q, kv, w_uk, ref, rows, heads, scale)
    return check_attention(g[rows][:, heads], gl[rows][:, heads], o, l, "bf16", label, lse_slack=slack)


# q_std 1, 2 and 4 give logits of about 0.8, 1.6 and 3.1 nats std with the
# random up-projections; the selector cases reach about 4 and 9 nats.
@pytest.mark.parametrize("L,H,k,q_std,selector", [(2000, 16, 256, 1.0, False), (2000, 16, 256, 4.0, False),
                                                  (1100, 8, 2048, 2.0, False), (2000, 16, 256, 4.0, True),
                                                  (1100, 8, 2048, 8.0, True)])
def test_masked_mha_random_selection(dsa, ora, L, H, k, q_std, selector):
    _say(f"masked mha random selection L={L} H={H} k={k} q_std={q_std} selector={selector}")
    cfg, q, kv, w_uk, w_uv = _inputs(L, H, 31, q_std, selector)
    idx = _random_selection(L, k, 31)
    idx[5] = -1                                   # empty selection
    idx[300, k // 2:] = -1                        # ragged
    idx[400, 0], idx[400, 1] = 401, L - 1         # non-causal: ignored
    idx[500, 2], idx[500, 3] = L + 5, -7          # out of range: ignored
    idx[600, 4] = idx[600, 0]                     # repeated: counts once
    idx[700] = torch.flip(idx[700], [0])          # order does not matter
    g, gl = _run(dsa, q, kv, w_uk, w_uv, idx, cfg.sm_scale)
    assert np.all(g[5] == 0) and np.all(np.isneginf(gl[5]))
    rows = np.unique(np.concatenate([np.arange(0, L, L // 30), [0, 1, 5, 63, 64, 300, 400, 500, 600, 700, L - 1]]))
    _check(ora, q, kv, w_uk, w_uv, idx.numpy(), g, gl, rows, cfg.sm_scale, f"masked mha L={L} k={k}")


@pytest.mark.parametrize("L,H", [(1, 4), (33, 3), (64, 16), (65, 8), (130, 2)])
def test_masked_mha_dense_small(dsa, ora, L, H):
    """k >= t+1 everywhere: dense causal MHA; single token, sub-tile and
    ragged lengths, head counts that are not multiples of anything."""
    _say(f"masked mha dense L={L} H={H}")
    cfg, q, kv, w_uk, w_uv = _inputs(L, H, 32, 2.0)
    k = 160
    idx = torch.full((L, k), -1, dtype=torch.int32)
    for t in range(L):
        idx[t, :t + 1] = torch.arange(t + 1)
    g, gl = _run(dsa, q, kv, w_uk, w_uv, idx, cfg.sm_scale)
    _check(ora, q, kv, w_uk, w_uv, idx.numpy(), g, gl, np.arange(L), cfg.sm_scale, f"masked mha dense L={L}")


def test_masked_mha_reference_overshoot(dsa, ora):
    """The first 64 latent rows scaled by 2^-6: a query's first tile of keys
    sits tens of nats below its later keys, so probabilities against the
    first tile's max leave fp16's range and the workgroups take the exact
    two-walk path (maxima first, then the sums)."""
    L, H = 700, 4
    _say(f"masked mha reference overshoot L={L} H={H}")
    cfg, q, kv, w_uk, w_uv = _inputs(L, H, 33, 8.0, selector=True)
    kv = kv.clone()
    kv[:64] = (kv[:64].float() * 2.0 ** -6).to(torch.bfloat16)
    k = 1024
    idx = torch.full((L, k), -1, dtype=torch.int32)
    for t in range(L):
        idx[t, :t + 1] = torch.arange(t + 1)
    g, gl = _run(dsa, q, kv, w_uk, w_uv, idx, cfg.sm_scale)
    assert np.isfinite(g).all() and np.isfinite(gl).all()
    rows = np.unique(np.concatenate([np.arange(0, L, 23), [0, 31, 32, 63, 64, 127, 128, L - 1]]))
    _check(ora, q, kv, w_uk, w_uv, idx.numpy(), g, gl, rows, cfg.sm_scale, "masked mha overshoot")


def _prefill_selection(dsa, cfg):
    """The library's fused FP8 indexer + top-k selection of one sequence."""
    L = cfg.L
    q_i, k_i, w = synth.prefill_indexer_inputs(cfg, device=DEV)
    q8 = torch.empty((L, cfg.H_I, cfg.D_I), dtype=torch.uint8, device=DEV)
    qs = torch.empty(L, dtype=torch.float32, device=DEV)
    k8 = torch.empty((L, cfg.D_I), dtype=torch.uint8, device=DEV)
    ks = torch.empty(L, dtype=torch.float32, device=DEV)
    dsa.dsa_quantize_e4m3_per_token(q_i, q8, qs, rows=L, cols=cfg.H_I * cfg.D_I)
    dsa.dsa_quantize_e4m3_per_token(k_i, k8, ks, rows=L, cols=cfg.D_I)
    idx = torch.empty((L, cfg.k), dtype=torch.int32, device=DEV)
    args = dsa.make_prefill_args(L, cfg.H_I, cfg.D_I, cfg.H, cfg.k, dsa.DSA_E4M3, q8, qs, k8, ks, w, dsa.DSA_BF16,
                                 None, None, cfg.sm_scale, idx, None, None)
    ws = torch.empty(dsa.dsa_prefill_workspace_bytes(args), dtype=torch.uint8, device=DEV)
    dsa.dsa_prefill_select(args, ws)
    torch.cuda.synchronize()
    return idx, (q8, qs, k8, ks, w)


def _check_selection(ora, cfg, idx, quant, rows):
    q8, qs, k8, ks, w = quant
    rt = torch.from_numpy(rows).to(DEV)
    sc = ora.indexer_rows(q8[rt].cpu().numpy(), k8.cpu().numpy(), w[rt].cpu().numpy(), rows.astype(np.int32),
                          q_scale=qs[rt].cpu().numpy(), k_scale=ks.cpu().numpy())
    gidx = idx[rt].cpu().numpy()
    for j, r in enumerate(rows):
        check_topk_row(gidx[j], sc[j], int(r) + 1, cfg.k, f"{cfg.name} row {r}")


def test_masked_mha_after_prefill_selection(dsa, ora):
    """Short-prefill pipeline at a reduced size: fused FP8 indexer + top-k,
    then masked MHA over that selection."""
    cfg = synth.scaled_down(synth.CONFIGS["mha4k"], L=2500, H=16, k=1024)
    _say(f"masked mha after prefill selection L={cfg.L} H={cfg.H} k={cfg.k}")
    idx, quant = _prefill_selection(dsa, cfg)
    q = synth.mha_query(cfg)
    kv = synth.prefill_latent(cfg)
    w_uk, w_uv = synth.mha_up_weights(cfg)
    g, gl = _run(dsa, q, kv, w_uk, w_uv, idx, cfg.sm_scale)
    rows = np.unique(np.concatenate([np.arange(0, cfg.L, cfg.L // 25), [0, cfg.k - 1, cfg.k, cfg.L - 1]]))
    _check_selection(ora, cfg, idx, quant, rows)
    _check(ora, q, kv, w_uk, w_uv, idx.cpu().numpy(), g, gl, rows, cfg.sm_scale, "masked mha after selection")


def test_masked_mha_full_size_sampled(dsa, ora):
    """The benchmarked short-prefill workload (L = 4096, H = 128, k = 2048):
    selection and attention checked on sampled rows and heads."""
    cfg = synth.CONFIGS["mha4k"]
    _say(f"masked mha full size L={cfg.L} H={cfg.H} k={cfg.k}")
    idx, quant = _prefill_selection(dsa, cfg)
    q = synth.mha_query(cfg)
    kv = synth.prefill_latent(cfg)
    w_uk, w_uv = synth.mha_up_weights(cfg)
    g, gl = _run(dsa, q, kv, w_uk, w_uv, idx, cfg.sm_scale)
    assert np.isfinite(g).all() and np.isfinite(gl).all()
    rows = np.array(sorted({0, 1, 63, 2047, 2048, 2049, 3001, cfg.L - 1}), dtype=np.int64)
    heads = sorted({0, 1, 37, 64, 100, cfg.H - 1})
    _check_selection(ora, cfg, idx, quant, rows)
    _check(ora, q, kv, w_uk, w_uv, idx.cpu().numpy(), g, gl, rows, cfg.sm_scale, "masked mha full size", heads)
