"""GPU parity of every hot-path step against the fp64 oracle, through the C ABI.

Sizes here finish in seconds on the oracle yet span several tiles and ragged
tails; the full-size workloads (marked slow) are at the end of this file,
checked on sampled rows.  Each test prints its case before touching the GPU.
"""
import math

import numpy as np
import pytest
import torch

import synth
from tests.parity import check_attention, check_scores, check_topk_row, oracle_score_bounds

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def dsa():
    from sparse_attention_gemm_amd import dsa as d
    d.load()
    return d


def _quant_gpu(dsa, x):
    rows, cols = x.numel() // x.shape[-1], x.shape[-1]
    x8 = torch.empty(x.shape, dtype=torch.uint8, device=DEV)
    sc = torch.empty(x.shape[:-1], dtype=torch.float32, device=DEV)
    xd = x.to(DEV).contiguous()
    dsa.dsa_quantize_e4m3_per_token(xd, x8, sc, rows=rows, cols=cols)
    torch.cuda.synchronize()
    return x8.cpu(), sc.cpu()


# ------------------------------------------------------------------ A0
def test_quantize_bit_exact(dsa, ora):
    _say("quantize 300x8192 + 1000x128 + sweep")
    for shape in ((300, 64 * 128), (1000, 128), (7, 4)):
        x = synth.normal(21, 1, shape) * 3.0
        x[3 % shape[0]] = 0.0
        g8, gs = _quant_gpu(dsa, x)
        o8, os_ = ora.quantize_rows(x.numpy())
        assert np.array_equal(gs.numpy(), os_), f"scales differ for {shape}"
        assert np.array_equal(g8.numpy(), o8), f"payload differs for {shape}: {(g8.numpy() != o8).sum()}"
    # sweep the encoder: rows whose amax is 448 (scale 1) carry arbitrary values
    grid = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float()
    grid = grid[torch.isfinite(grid) & (grid >= 0)].unique().double()
    mids = (grid[1:] + grid[:-1]) / 2
    vals = torch.cat([grid, mids, -mids, synth.normal(5, 9, (20000,)).double() * 30]).float()
    vals = vals[vals.abs() < 448]
    n = (vals.numel() + 126) // 127
    rows = torch.zeros(n * 127, dtype=torch.float32)
    rows[:vals.numel()] = vals
    rows = torch.cat([rows.view(n, 127), torch.full((n, 1), 448.0)], dim=1)
    g8, gs = _quant_gpu(dsa, rows)
    o8, os_ = ora.quantize_rows(rows.numpy())
    assert np.all(os_ == 1.0) and np.array_equal(gs.numpy(), os_)
    assert np.array_equal(g8.numpy(), o8)


# ------------------------------------------------------------------ A1
def _indexer_case(seed, T, S, H_I, fp8=True, pos_offset=0, D_I=128):
    q = synth.normal(seed, synth.T_QI, (T, H_I, D_I))
    k = synth.normal(seed, synth.T_KI, (S, D_I))
    w = synth.normal(seed, synth.T_W, (T, H_I), std=0.5)
    pos = (torch.arange(T, dtype=torch.int32) * max(1, S // max(T, 1)) + pos_offset).clamp(max=S - 1)
    return q, k, w, pos


def _gpu_scores(dsa, q8, qs, k8, ks, w, pos, S, dt):
    T = q8.shape[0]
    sc = torch.full((T, S + 5), 7.0, dtype=torch.float32, device=DEV)  # ld > S, tail untouched
    args = [t.to(DEV).contiguous() if t is not None else None for t in (q8, qs, k8, ks, w, pos)]
    dsa.dsa_indexer_scores(args[0], args[1], args[2], args[3], args[4], args[5], sc, dt, S=S)
    torch.cuda.synchronize()
    out = sc.cpu()
    assert torch.all(out[:, S:] == 7.0), "wrote past S"
    return out[:, :S].double().numpy()


# (64, 128) and (32, 128) are the full-size FP8 MFMA kernel; the rest sum the
# exact E4M3 products in fp32 ((4, 64) is the tiny workload's indexer)
FP8_SHAPES = [(64, 128), (32, 128), (4, 64), (20, 64), (48, 128), (1, 128), (64, 64)]


@pytest.mark.parametrize("H_I,D_I", FP8_SHAPES)
def test_indexer_fp8_scores(dsa, ora, H_I, D_I):
    T, S = 37, 1000  # ragged: S not a multiple of 64 or 512
    _say(f"indexer fp8 T={T} S={S} H_I={H_I} D_I={D_I}")
    q, k, w, pos = _indexer_case(3, T, S, H_I, D_I=D_I)
    q8, qs = ora.quantize_rows(q.view(T, -1).numpy())
    k8, ks = ora.quantize_rows(k.numpy())
    q8 = torch.from_numpy(q8).view(T, H_I, D_I)
    g = _gpu_scores(dsa, q8, torch.from_numpy(qs), torch.from_numpy(k8), torch.from_numpy(ks), w, pos, S,
                    dsa.DSA_E4M3)
    o, m = oracle_score_bounds(ora, q8.numpy(), k8, w.numpy(), pos, q_scale=qs, k_scale=ks)
    check_scores(g, o, m, D_I + H_I, "fp8 scores")


@pytest.mark.parametrize("H_I,D_I", [(64, 128), (4, 64), (20, 64), (36, 128)])
def test_indexer_fp8_exact_arithmetic(dsa, ora, H_I, D_I):
    """E4M3 payloads in {0,+-1,+-2}, scales 1, w in {+-1,+-0.5}: every partial
    sum is exact in fp32, so scores must be bit-identical and the top-k
    (full of exact ties) identical under the position tie rule.  For the
    other shapes this also pins the head and dim bounds: a stray head or dim
    would change some sum."""
    T, S = 70, 700
    _say(f"indexer exact arithmetic H_I={H_I} D_I={D_I}")
    lut = torch.tensor([0xC0, 0xB8, 0x00, 0x38, 0x40], dtype=torch.uint8)  # -2,-1,0,1,2
    qi = synth.randint(4, 1, (T, H_I, D_I), 0, 4)
    ki = synth.randint(4, 2, (S, D_I), 0, 4)
    q8, k8 = lut[qi], lut[ki]
    w = torch.tensor([-1.0, -0.5, 0.5, 1.0])[synth.randint(4, 3, (T, H_I), 0, 3)]
    ones_t, ones_s = torch.ones(T), torch.ones(S)
    pos = torch.arange(T, dtype=torch.int32) * 10
    g = _gpu_scores(dsa, q8, ones_t, k8, ones_s, w, pos, S, dsa.DSA_E4M3)
    o = ora.indexer_rows(q8.numpy(), k8.numpy(), w, pos, q_scale=ones_t, k_scale=ones_s)
    assert np.array_equal(g, o)
    # top-k over these exactly tied scores: identical sets
    sc = torch.from_numpy(g).float().to(DEV)
    nval = (pos + 1).to(DEV)
    for kk in (5, 64, 256):
        idx = torch.empty((T, kk), dtype=torch.int32, device=DEV)
        dsa.dsa_topk_select(sc, nval, kk, idx)
        torch.cuda.synchronize()
        ref, _ = ora.topk_rows(np.where(np.isinf(o), 0, o), (pos + 1).numpy(), kk)
        assert np.array_equal(idx.cpu().numpy(), ref)


def test_indexer_f32_tiny_config(dsa, ora):
    cfg = synth.CONFIGS["tiny"]
    _say("indexer f32 tiny config L=2048")
    q, k, w = synth.prefill_indexer_inputs(cfg)
    pos = torch.arange(cfg.L, dtype=torch.int32)
    g = _gpu_scores(dsa, q, None, k, None, w, pos, cfg.L, dsa.DSA_F32)
    rows = np.arange(0, cfg.L, 7)
    o, m = oracle_score_bounds(ora, q.numpy(), k.numpy(), w.numpy(), pos, rows=rows)
    check_scores(g[rows], o, m, cfg.D_I + cfg.H_I, "f32 scores")


# ------------------------------------------------------------------ A2
@pytest.mark.parametrize("n,k", [(5000, 2048), (40000, 2048), (3000, 256), (2047, 2048), (131072, 2048),
                                 (700, 1)])
def test_topk_matches_oracle_on_same_scores(dsa, ora, n, k):
    """Same fp32 scores on both sides: the selection must be identical."""
    _say(f"topk n={n} k={k}")
    T = 3
    sc = synth.normal(7, 1, (T, n))
    sc[1] = torch.round(sc[1] * 4) / 4  # heavy ties
    sc[2, : n // 2] = 0.0                # a block of exact zeros
    nv = torch.tensor([n, n - 17, max(1, n // 3)], dtype=torch.int32)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    scd, nvd = sc.to(DEV), nv.to(DEV)
    dsa.dsa_topk_select(scd, nvd, k, idx)
    torch.cuda.synchronize()
    ref, _ = ora.topk_rows(sc.double().numpy(), nv.numpy(), k)
    assert np.array_equal(idx.cpu().numpy(), ref)


@pytest.mark.parametrize("n,k", [(70000, 2048), (131072, 2048), (33000, 256), (20000, 1)])
def test_topk_split_rows_match_oracle(dsa, ora, n, k):
    """With a workspace, a short batch splits each row into column chunks and
    merges their selections: the result must still be the oracle's exactly
    (ties across chunk boundaries, -inf scores, a row shorter than k)."""
    T = 4
    _say(f"topk split n={n} k={k}")
    sc = synth.normal(9, 1, (T, n))
    sc[0, :100] = -float("inf")
    sc[1] = torch.round(sc[1] * 4) / 4  # heavy ties, across every chunk
    sc[2] = 0.25                         # one tie class
    nv = torch.tensor([n, n - 17, max(1, n // 3), max(1, k - 5)], dtype=torch.int32)
    nbytes = dsa.dsa_topk_workspace_bytes(T, n, k)
    assert nbytes > 0, "this batch should be split"
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    dsa.dsa_topk_select(sc.to(DEV), nv.to(DEV), k, idx, workspace=ws)
    torch.cuda.synchronize()
    ref, _ = ora.topk_rows(sc.double().numpy(), nv.numpy(), k)
    assert np.array_equal(idx.cpu().numpy(), ref)


def test_topk_negative_zero_and_all_equal(dsa, ora):
    _say("topk -0 / all equal")
    n, k = 5000, 300
    sc = torch.zeros((2, n))
    sc[0, ::2] = -0.0
    sc[1] = -3.5
    idx = torch.empty((2, k), dtype=torch.int32, device=DEV)
    scd, nvd = sc.to(DEV), torch.tensor([n, n], dtype=torch.int32, device=DEV)
    dsa.dsa_topk_select(scd, nvd, k, idx)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    assert np.array_equal(got[0], np.arange(n - k, n))
    assert np.array_equal(got[1], np.arange(n - k, n))


def test_topk_tie_class_larger_than_lds(dsa, ora):
    """A tie class at the k-th score bigger than the LDS candidate buffer:
    the output pass runs over the row itself and must keep the most recent
    ties."""
    _say("topk massive ties")
    n, k = 40000, 2048
    base = torch.cat([10.0 + torch.arange(1000, dtype=torch.float32) / 1000.0,
                      torch.full((30000,), 0.5),
                      -1.0 - torch.arange(9000, dtype=torch.float32) / 1000.0])
    perm = synth.permutation(8, 1, n)
    sc = torch.stack([base[perm], torch.full((n,), 0.25), base.flip(0)])
    nv = torch.tensor([n, 20000, n], dtype=torch.int32)
    idx = torch.empty((3, k), dtype=torch.int32, device=DEV)
    dsa.dsa_topk_select(sc.to(DEV), nv.to(DEV), k, idx)
    torch.cuda.synchronize()
    ref, _ = ora.topk_rows(sc.double().numpy(), nv.numpy(), k)
    got = idx.cpu().numpy()
    assert np.array_equal(got, ref)
    assert np.array_equal(got[1], np.arange(20000 - k, 20000))


# ------------------------------------------------------------------ A3
def _mla_gpu(dsa, q, kv, idx, scale, dtype, use_ws=False):
    T, H = q.shape[0], q.shape[1]
    qd, kvd, idd = q.to(DEV), kv.to(DEV), idx.to(DEV)
    out = torch.empty((T, H, 512), dtype=q.dtype, device=DEV)
    lse = torch.empty((T, H), dtype=torch.float32, device=DEV)
    ws = None
    if use_ws:
        nb = dsa.dsa_sparse_mla_workspace_bytes(T, H, idx.shape[1])
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=DEV)
    dsa.dsa_sparse_mla_fwd(qd, kvd, idd, scale, out, lse, workspace=ws)
    torch.cuda.synchronize()
    return out.float().cpu().double().numpy(), lse.cpu().double().numpy()


@pytest.mark.parametrize("H,k,use_ws,qstd", [(128, 2048, False, 1.0), (128, 2048, True, 40.0), (16, 256, False, 1.0),
                                             (64, 100, True, 40.0), (32, 48, False, 1.0),
                                             # H a multiple of 8 but not of 16: a padded last head tile
                                             (8, 256, False, 1.0), (24, 2048, True, 40.0), (40, 100, False, 1.0)])
def test_sparse_mla_bf16(dsa, ora, H, k, use_ws, qstd):
    N, T = 5000, 6
    _say(f"sparse mla bf16 H={H} k={k} ws={use_ws} qstd={qstd}")
    q = synth.normal(11, 1, (T, H, 576), std=qstd).to(torch.bfloat16)
    kv = synth.normal(11, 2, (N, 576), std=1 / 24).to(torch.bfloat16)
    idx = torch.stack([synth.permutation(11, 10 + t, N)[:k] for t in range(T)]).to(torch.int32)
    idx[1, k // 2:] = -1          # ragged selection
    idx[2, :] = -1                # empty selection
    idx[3, 5] = N + 3             # out of range: skipped
    idx[4] = torch.sort(idx[4]).values
    g, gl = _mla_gpu(dsa, q, kv, idx, 1 / math.sqrt(192), "bf16", use_ws)
    ref_idx = idx.clone()
    ref_idx[3, 5] = -1
    o, l = ora.sparse_mla_rows(q, kv, ref_idx.numpy(), 1 / math.sqrt(192))
    assert np.all(g[2] == 0) and np.all(np.isneginf(gl[2]))
    check_attention(g, gl, o, l, "bf16", "mla bf16")


def test_sparse_mla_f32_tiny_config(dsa, ora):
    cfg = synth.CONFIGS["tiny"]
    _say("sparse mla f32 tiny config")
    q = synth.prefill_attn_q(cfg)
    kv = synth.prefill_latent(cfg)
    # selections: causal windows of varied length
    L, k = cfg.L, cfg.k
    idx = torch.full((L, k), -1, dtype=torch.int32)
    for t in range(L):
        n = min(k, t + 1)
        idx[t, :n] = torch.arange(t + 1 - n, t + 1)
    g, gl = _mla_gpu(dsa, q, kv, idx, cfg.sm_scale, "f32")
    rows = np.arange(0, L, 13)
    o, l = ora.sparse_mla_rows(q, kv, idx.numpy(), cfg.sm_scale, rows=rows)
    check_attention(g[rows], gl[rows], o, l, "f32", "mla f32")


# ------------------------------------------------------------------ prefill
def _prefill_inputs(cfg, dev=DEV):
    q_i, k_i, w = synth.prefill_indexer_inputs(cfg)
    q = synth.prefill_attn_q(cfg)
    kv = synth.prefill_latent(cfg)
    return q_i, k_i, w, q, kv


def _run_prefill(dsa, cfg, q_i, k_i, w, q, kv):
    L = cfg.L
    t = {}
    t["w"] = w.to(DEV)
    t["q"], t["kv"] = q.to(DEV), kv.to(DEV)
    if cfg.fp8_indexer:
        t["q8"] = torch.empty((L, cfg.H_I, cfg.D_I), dtype=torch.uint8, device=DEV)
        t["qs"] = torch.empty(L, dtype=torch.float32, device=DEV)
        t["k8"] = torch.empty((L, cfg.D_I), dtype=torch.uint8, device=DEV)
        t["ks"] = torch.empty(L, dtype=torch.float32, device=DEV)
        qi_d, ki_d = q_i.to(DEV), k_i.to(DEV)
        dsa.dsa_quantize_e4m3_per_token(qi_d, t["q8"], t["qs"], rows=L, cols=cfg.H_I * cfg.D_I)
        dsa.dsa_quantize_e4m3_per_token(ki_d, t["k8"], t["ks"], rows=L, cols=cfg.D_I)
        qa, qsa, ka, ksa, idt = t["q8"], t["qs"], t["k8"], t["ks"], dsa.DSA_E4M3
    else:
        t["qi"], t["ki"] = q_i.to(DEV), k_i.to(DEV)
        qa, qsa, ka, ksa, idt = t["qi"], None, t["ki"], None, dsa.DSA_F32
    adt = dsa.DSA_BF16 if cfg.attn_dtype == "bf16" else dsa.DSA_F32
    t["idx"] = torch.empty((L, cfg.k), dtype=torch.int32, device=DEV)
    t["out"] = torch.empty((L, cfg.H, 512), dtype=q.dtype, device=DEV)
    t["lse"] = torch.empty((L, cfg.H), dtype=torch.float32, device=DEV)
    args = dsa.make_prefill_args(L, cfg.H_I, cfg.D_I, cfg.H, cfg.k, idt, qa, qsa, ka, ksa, t["w"], adt, t["q"],
                                 t["kv"], cfg.sm_scale, t["idx"], t["out"], t["lse"])
    nb = dsa.dsa_prefill_workspace_bytes(args)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=DEV) if nb else None
    dsa.dsa_prefill(args, ws)
    torch.cuda.synchronize()
    return t


def _check_prefill_rows(ora, cfg, q_i, k_i, w, q, kv, t, rows, label):
    L = cfg.L
    pos = np.arange(L, dtype=np.int32)
    if cfg.fp8_indexer:
        q8, qs = ora.quantize_rows(q_i.view(L, -1).numpy())
        k8, ks = ora.quantize_rows(k_i.numpy())
        assert np.array_equal(t["q8"].cpu().view(L, -1).numpy(), q8)
        assert np.array_equal(t["k8"].cpu().numpy(), k8)
        sc = ora.indexer_rows(q8.reshape(L, cfg.H_I, cfg.D_I), k8, w, pos, rows=rows, q_scale=qs, k_scale=ks)
    else:
        sc = ora.indexer_rows(q_i.numpy(), k_i.numpy(), w, pos, rows=rows)
    gidx = t["idx"].cpu().numpy()
    diffs = 0
    for i, r in enumerate(rows):
        diffs += check_topk_row(gidx[r], sc[i], r + 1, cfg.k, f"{label} row {r}")
    o, l = ora.sparse_mla_rows(q, kv, gidx, cfg.sm_scale, rows=rows)
    g = t["out"].float().cpu().double().numpy()[rows]
    gl = t["lse"].cpu().double().numpy()[rows]
    check_attention(g, gl, o, l, cfg.attn_dtype, label)
    return diffs


def test_prefill_tiny_fp32_config(dsa, ora):
    cfg = synth.CONFIGS["tiny"]
    _say("prefill tiny fp32 L=2048 (unfused path)")
    ins = _prefill_inputs(cfg)
    t = _run_prefill(dsa, cfg, *ins)
    rows = np.unique(np.concatenate([np.arange(0, cfg.L, 37), [0, 1, 255, 256, 257, 2047]]))
    _check_prefill_rows(ora, cfg, *ins, t, rows, "tiny fp32")


@pytest.mark.parametrize("attn", ["f32", "bf16"])
def test_prefill_tiny_fp8_config(dsa, ora, attn):
    """The tiny workload with its 4 x 64 indexer in E4M3 (zero-padded FP8
    scores, row top-k) and the attention in fp32 or bf16."""
    cfg = synth.scaled_down(synth.CONFIGS["tiny_fp8"], attn_dtype=attn)
    _say(f"prefill tiny fp8 indexer L=2048 attention {attn}")
    ins = _prefill_inputs(cfg)
    t = _run_prefill(dsa, cfg, *ins)
    rows = np.unique(np.concatenate([np.arange(0, cfg.L, 37), [0, 1, 255, 256, 257, 2047]]))
    _check_prefill_rows(ora, cfg, *ins, t, rows, f"tiny fp8/{attn}")


@pytest.mark.parametrize("L,k,H", [(1000, 256, 16), (777, 64, 32), (4500, 2048, 128), (130, 2048, 16)])
def test_prefill_fused_fp8(dsa, ora, L, k, H):
    cfg = synth.scaled_down(synth.CONFIGS["prefill16k"], L=L, k=k, H=H, seed=5)
    _say(f"prefill fused fp8 L={L} k={k} H={H}")
    ins = _prefill_inputs(cfg)
    t = _run_prefill(dsa, cfg, *ins)
    rows = np.unique(np.concatenate([np.arange(0, L, max(1, L // 40)), [0, 1, k - 1, k, k + 1, L - 1]]))
    rows = rows[rows < L]
    _check_prefill_rows(ora, cfg, *ins, t, rows, f"prefill L={L}")
    # the fused selection equals top-k of the unfused score matrix
    sc = torch.empty((L, L), dtype=torch.float32, device=DEV)
    pos = torch.arange(L, dtype=torch.int32, device=DEV)
    dsa.dsa_indexer_scores(t["q8"], t["qs"], t["k8"], t["ks"], t["w"], pos, sc, dsa.DSA_E4M3)
    idx2 = torch.empty((L, k), dtype=torch.int32, device=DEV)
    nval = pos + 1
    dsa.dsa_topk_select(sc, nval, k, idx2)
    torch.cuda.synchronize()
    bad = (idx2 != t["idx"]).any(dim=1).nonzero().flatten().tolist()
    assert not bad, f"fused and unfused selections differ in {len(bad)} rows, first {bad[:5]}"



def _fused_vs_unfused(dsa, q8, qs, k8, ks, w, k):
    """Run the fused selection and top-k of the unfused score matrix on device
    inputs of one causal sequence; returns both index matrices (CPU)."""
    L, H_I = q8.shape[0], q8.shape[1]
    idx = torch.empty((L, k), dtype=torch.int32, device=DEV)
    args = dsa.make_prefill_args(L, H_I, 128, 16, k, dsa.DSA_E4M3, q8, qs, k8, ks, w, dsa.DSA_BF16, None, None,
                                 0.1, idx, None, None)
    ws = torch.empty(dsa.dsa_prefill_workspace_bytes(args), dtype=torch.uint8, device=DEV)
    dsa.dsa_prefill_select(args, ws)
    sc = torch.empty((L, L), dtype=torch.float32, device=DEV)
    pos = torch.arange(L, dtype=torch.int32, device=DEV)
    dsa.dsa_indexer_scores(q8, qs, k8, ks, w, pos, sc, dsa.DSA_E4M3)
    idx2 = torch.empty((L, k), dtype=torch.int32, device=DEV)
    dsa.dsa_topk_select(sc, pos + 1, k, idx2)
    torch.cuda.synchronize()
    return idx.cpu(), idx2.cpu(), sc


def test_prefill_select_fused_long(dsa, ora):
    """Rows long enough for many buffer compactions (early and exact cuts)."""
    L, k = 20000, 2048
    _say(f"fused select long L={L}")
    cfg = synth.scaled_down(synth.CONFIGS["prefill16k"], L=L, k=k, H=16, seed=11)
    q_i, k_i, w = synth.prefill_indexer_inputs(cfg)
    q8 = torch.empty((L, 64, 128), dtype=torch.uint8, device=DEV)
    qs = torch.empty(L, dtype=torch.float32, device=DEV)
    k8 = torch.empty((L, 128), dtype=torch.uint8, device=DEV)
    ks = torch.empty(L, dtype=torch.float32, device=DEV)
    dsa.dsa_quantize_e4m3_per_token(q_i.to(DEV), q8, qs, rows=L, cols=8192)
    dsa.dsa_quantize_e4m3_per_token(k_i.to(DEV), k8, ks, rows=L, cols=128)
    a, b, sc = _fused_vs_unfused(dsa, q8, qs, k8, ks, w.to(DEV), k)
    bad = (a != b).any(dim=1).nonzero().flatten().tolist()
    assert not bad, f"fused and unfused selections differ in {len(bad)} rows, first {bad[:5]}"
    # sampled rows against the oracle's scores and selection
    rows = np.array([0, k - 1, k, 4095, 4096, 4097, 9000, L - 2, L - 1])
    o, _ = oracle_score_bounds(ora, q8.cpu().numpy(), k8.cpu().numpy(), w.numpy(),
                                  torch.arange(L, dtype=torch.int32), q_scale=qs.cpu().numpy(),
                                  k_scale=ks.cpu().numpy(), rows=rows)
    for j, r in enumerate(rows):
        check_topk_row(a[r].numpy(), o[j], r + 1, k, f"fused long row {r}")


def test_prefill_select_fused_ties(dsa, ora):
    """E4M3 payloads in {0,+-1,+-2} and unit scales: exact scores with huge
    tie classes, so compactions must fall through to the exact tie cut."""
    L, H_I, k = 9000, 64, 2048
    _say(f"fused select ties L={L}")
    lut = torch.tensor([0xC0, 0xB8, 0x00, 0x38, 0x40], dtype=torch.uint8)
    q8 = lut[synth.randint(6, 1, (L, H_I, 128), 0, 4)]
    k8 = lut[synth.randint(6, 2, (L, 128), 0, 4)]
    w = torch.tensor([-1.0, -0.5, 0.5, 1.0])[synth.randint(6, 3, (L, H_I), 0, 3)]
    ones = torch.ones(L)
    a, b, sc = _fused_vs_unfused(dsa, q8.to(DEV), ones.to(DEV), k8.to(DEV), ones.to(DEV), w.to(DEV), k)
    bad = (a != b).any(dim=1).nonzero().flatten().tolist()
    assert not bad, f"fused and unfused selections differ in {len(bad)} rows, first {bad[:5]}"
    rows = np.array([100, 2047, 2048, 5000, 8191, L - 1])
    pos = torch.arange(L, dtype=torch.int32)
    o = ora.indexer_rows(q8[rows].numpy(), k8.numpy(), w[rows], pos[rows], q_scale=ones[rows], k_scale=ones)
    ref, _ = ora.topk_rows(np.where(np.isinf(o), 0, o), (pos[rows] + 1).numpy(), k)
    assert np.array_equal(a[rows].numpy(), ref)


# ------------------------------------------------------------------ decode
def _decode_case(cfg, seqs=None):
    ctx = synth.decode_ctx(cfg)
    bt, nb = synth.decode_block_table(cfg, ctx)
    k8p, ksp, kvp = synth.build_decode_pools(cfg, ctx, bt, nb, seqs=seqs)
    q8, qs, w, q = synth.decode_queries(cfg)
    return ctx, bt, nb, (k8p, ksp, kvp), (q8, qs, w, q)


def _run_decode(dsa, cfg, ctx, bt, nb, pools, qside, with_idx=True):
    k8p, ksp, kvp = [p.to(DEV) for p in pools]
    q8, qs, w, q = [x.to(DEV) for x in qside]
    ctxd, btd = ctx.to(torch.int32).to(DEV), bt.to(DEV)
    out = torch.empty((cfg.B, cfg.H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((cfg.B, cfg.H), dtype=torch.float32, device=DEV)
    idx = torch.empty((cfg.B, cfg.k), dtype=torch.int32, device=DEV) if with_idx else None
    args = dsa.make_decode_args(cfg.B, cfg.H_I, cfg.D_I, cfg.H, cfg.k, q8, qs, w, q, k8p, ksp, kvp, nb * 64, btd,
                                bt.shape[1], ctxd, int(ctx.max()), cfg.sm_scale, out, lse, idx)
    ws = torch.empty(dsa.dsa_decode_workspace_bytes(args), dtype=torch.uint8, device=DEV)
    dsa.dsa_decode(args, ws)
    torch.cuda.synchronize()
    keep = (k8p, ksp, kvp, q8, qs, w, q, ctxd, btd, ws)
    del keep
    return out, lse, idx


@pytest.mark.parametrize("B,lo,hi,k,shuffled,H", [(5, 100, 3000, 256, True, 128), (4, 2000, 2100, 2048, False, 128),
                                                  (3, 1, 70, 64, True, 128), (6, 4096, 9000, 2048, True, 128),
                                                  (4, 3000, 5000, 2048, True, 24)])
def test_decode_paged(dsa, ora, B, lo, hi, k, shuffled, H):
    cfg = synth.DecodeConfig("t", B, lo, hi, 64, 128, H, k, 9, shuffled)
    _say(f"decode B={B} ctx=[{lo},{hi}] k={k} shuffled={shuffled} H={H}")
    ctx, bt, nb, pools, qside = _decode_case(cfg)
    out, lse, idx = _run_decode(dsa, cfg, ctx, bt, nb, pools, qside)
    gidx = idx.cpu().numpy()
    q8, qs, w, q = qside
    for b in range(B):
        c = int(ctx[b])
        kb, sb = synth.decode_seq_keys(cfg, b, c)
        sc = ora.indexer_rows(q8[b:b + 1], kb, w[b:b + 1], np.array([c - 1], np.int32), q_scale=qs[b:b + 1],
                              k_scale=sb)
        check_topk_row(gidx[b], sc[0], c, k, f"decode b={b}")
        lat = synth.decode_seq_latent(cfg, b, c)
        o, l = ora.sparse_mla_rows(q[b:b + 1], lat, gidx[b:b + 1], cfg.sm_scale)
        check_attention(out[b:b + 1].float().cpu().double().numpy(), lse[b:b + 1].cpu().double().numpy(), o, l,
                        "bf16", f"decode b={b}")


def test_decode_block_shuffle_invariance(dsa):
    _say("decode shuffle invariance")
    res = []
    for sh in (False, True):
        cfg = synth.DecodeConfig("t", 4, 500, 5000, 64, 128, 128, 512, 3, sh)
        ctx, bt, nb, pools, qside = _decode_case(cfg)
        out, lse, idx = _run_decode(dsa, cfg, ctx, bt, nb, pools, qside)
        res.append((out.cpu(), lse.cpu(), idx.cpu()))
    assert torch.equal(res[0][2], res[1][2])
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


def test_paged_cache_append(dsa, ora):
    """The pools after a GPU append equal the oracle's append, byte for byte,
    including tokens aimed at positions the block table does not map."""
    _say("paged cache append vs oracle")
    cfg = synth.DecodeConfig("t", 6, 100, 1000, 64, 128, 128, 64, 12, True)
    ctx = synth.decode_ctx(cfg)
    bt, nb = synth.decode_block_table(cfg, ctx + 1)
    k8p, ksp, kvp = synth.build_decode_pools(cfg, ctx, bt, nb)
    lat, k8, ks = synth.new_token_rows(cfg, 0)
    pos = ctx.to(torch.int32).clone()
    pos[1] = -1                       # nothing written
    pos[4] = bt.shape[1] * 64 + 3     # past the table: nothing written
    dk8, dks, dkv = k8p.to(DEV), ksp.to(DEV), kvp.to(DEV)
    dl, d8, ds, dp, dbt = lat.to(DEV), k8.to(DEV), ks.to(DEV), pos.to(DEV), bt.to(DEV)
    dsa.dsa_paged_cache_append(dl, d8, ds, dp, dbt, dkv, dk8, dks, n_pool_rows=nb * 64)
    torch.cuda.synchronize()
    ekv, ek8, eks = ora.paged_cache_append(lat, k8, ks, pos, bt, kvp.view(-1, 576), k8p.view(-1, 128), ksp.view(-1))
    assert np.array_equal(dk8.cpu().view(-1, 128).numpy(), ek8)
    assert np.array_equal(dks.cpu().view(-1).numpy(), eks)
    assert np.array_equal(dkv.cpu().view(-1, 576).view(torch.int16).numpy().view(np.uint16), ekv)
    assert not np.array_equal(ekv, kvp.view(-1, 576).view(torch.int16).numpy().view(np.uint16))


@pytest.mark.parametrize("shuffled", [True, False])
def test_append_then_decode(dsa, ora, shuffled):
    """A serving step: append each sequence's new token at position ctx, then
    decode with ctx + 1 (the new token is its own query's candidate).  The
    pools match the oracle's append byte for byte, and the decode matches the
    oracle's decode of the appended pools (contexts ending on a page boundary
    open a new page)."""
    _say(f"append then decode shuffled={shuffled}")
    cfg = synth.DecodeConfig("t", 5, 60, 3000, 64, 128, 128, 2048, 14, shuffled)
    ctx = synth.decode_ctx(cfg)
    ctx[0], ctx[1] = 64, 2048         # page boundary; the new token is the 2049th
    bt, nb = synth.decode_block_table(cfg, ctx + 1)
    pools = synth.build_decode_pools(cfg, ctx, bt, nb)
    qside = synth.decode_queries(cfg)
    lat, k8, ks = synth.new_token_rows(cfg, 3)
    pos = ctx.to(torch.int32)
    dk8, dks, dkv = [p.to(DEV) for p in pools]
    dsa.dsa_paged_cache_append(lat.to(DEV), k8.to(DEV), ks.to(DEV), pos.to(DEV), bt.to(DEV), dkv, dk8, dks,
                               n_pool_rows=nb * 64)
    torch.cuda.synchronize()
    ekv, ek8, eks = ora.paged_cache_append(lat, k8, ks, pos, bt, pools[2].view(-1, 576), pools[0].view(-1, 128),
                                           pools[1].view(-1))
    assert np.array_equal(dk8.cpu().view(-1, 128).numpy(), ek8)
    assert np.array_equal(dks.cpu().view(-1).numpy(), eks)
    assert np.array_equal(dkv.cpu().view(-1, 576).view(torch.int16).numpy().view(np.uint16), ekv)
    ctx1 = ctx + 1
    out, lse, idx = _run_decode(dsa, cfg, ctx1, bt, nb, (dk8, dks, dkv), qside)
    gidx = idx.cpu().numpy()
    q8, qs, w, q = qside
    ridx, rtau, _, _ = ora.decode(q8, qs, w, q, ek8, eks, ekv, bt, ctx1, cfg.k, cfg.sm_scale)
    for b in range(cfg.B):
        c = int(ctx1[b])
        kb, sb = synth.decode_seq_keys(cfg, b, c - 1)
        kb = torch.cat([kb, k8[b:b + 1]])
        sb = torch.cat([sb, ks[b:b + 1]])
        sc = ora.indexer_rows(q8[b:b + 1], kb, w[b:b + 1], np.array([c - 1], np.int32), q_scale=qs[b:b + 1],
                              k_scale=sb)
        check_topk_row(gidx[b], sc[0], c, cfg.k, f"append+decode b={b}")
        check_topk_row(ridx[b], sc[0], c, cfg.k, f"oracle append+decode b={b}")
        lat_b = torch.cat([synth.decode_seq_latent(cfg, b, c - 1), lat[b:b + 1]])
        o, l = ora.sparse_mla_rows(q[b:b + 1], lat_b, gidx[b:b + 1], cfg.sm_scale)
        check_attention(out[b:b + 1].float().cpu().double().numpy(), lse[b:b + 1].cpu().double().numpy(), o, l,
                        "bf16", f"append+decode b={b}")


def test_decode_equals_its_stages(dsa):
    """dsa_decode == indexer scores -> top-k -> paged sparse MLA, bit for bit."""
    _say("decode stages compose")
    cfg = synth.DecodeConfig("t", 5, 300, 6000, 64, 128, 128, 1024, 8, True)
    ctx, bt, nb, pools, qside = _decode_case(cfg)
    out, lse, idx = _run_decode(dsa, cfg, ctx, bt, nb, pools, qside)
    k8p, ksp, kvp = [p.to(DEV) for p in pools]
    q8, qs, w, q = [x.to(DEV) for x in qside]
    ctxd, btd = ctx.to(torch.int32).to(DEV), bt.to(DEV)
    max_ctx = int(ctx.max())
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    args = dsa.make_decode_args(cfg.B, 64, 128, cfg.H, cfg.k, q8, qs, w, q, k8p, ksp, kvp, nb * 64, btd,
                                bt.shape[1], ctxd, max_ctx, cfg.sm_scale, out2, lse2, None)
    sc = torch.full((cfg.B, max_ctx + 3), -7.0, dtype=torch.float32, device=DEV)
    dsa.dsa_decode_indexer_scores(args, sc)
    idx2 = torch.empty((cfg.B, cfg.k), dtype=torch.int32, device=DEV)
    dsa.dsa_topk_select(sc, ctxd, cfg.k, idx2)
    ws = torch.empty(max(1, dsa.dsa_sparse_mla_workspace_bytes(cfg.B, cfg.H, cfg.k)), dtype=torch.uint8,
                     device=DEV)
    dsa.dsa_sparse_mla_paged_fwd(q, kvp, btd, idx2, cfg.sm_scale, out2, lse2, workspace=ws, n_pool_rows=nb * 64)
    torch.cuda.synchronize()
    assert torch.equal(idx2, idx)
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16)) and torch.equal(lse2, lse)
    # positions past each context are left untouched
    scc = sc.cpu()
    for b in range(cfg.B):
        assert torch.all(scc[b, int(ctx[b]):] == -7.0)


def test_prefill_select_equals_prefill_selection(dsa):
    _say("prefill select stage")
    cfg = synth.scaled_down(synth.CONFIGS["prefill16k"], L=600, k=128, H=16, seed=6)
    ins = _prefill_inputs(cfg)
    t = _run_prefill(dsa, cfg, *ins)
    idx2 = torch.full_like(t["idx"], 12345)
    args = dsa.make_prefill_args(cfg.L, 64, 128, cfg.H, cfg.k, dsa.DSA_E4M3, t["q8"], t["qs"], t["k8"], t["ks"],
                                 t["w"], dsa.DSA_BF16, None, None, cfg.sm_scale, idx2, None, None)
    ws = torch.empty(dsa.dsa_prefill_workspace_bytes(args), dtype=torch.uint8, device=DEV)
    dsa.dsa_prefill_select(args, ws)
    torch.cuda.synchronize()
    assert torch.equal(idx2, t["idx"])


@pytest.mark.parametrize("H,use_ws", [(128, True), (16, True), (128, False), (16, False)])
def test_sparse_mla_bf16_late_large_logits(dsa, ora, H, use_ws):
    """Logits in a late tile far above the first tile's (over 2^64 in base 2)
    for some heads: the result must still be the exact softmax.  With a
    workspace the short batch is split across workgroups; without one every
    query is a single workgroup (the path every prefill takes).  The large
    component sits in a rope dim, which enters the logits but not the value,
    so the outputs keep the workload's magnitude."""
    _say(f"sparse mla bf16 late large logits H={H} ws={use_ws}")
    N, T, k = 3000, 3, 2048
    q = synth.normal(13, 1, (T, H, 576)) * 0.5
    kv = synth.normal(13, 2, (N, 576), std=1 / 24)
    q[:, ::3, 512] = 30.0          # every third head looks along rope dim 0
    kv[:, 512] = 0.01
    late = torch.arange(2500, 2520)
    kv[late, 512] = 100.0          # logit 3000 * sm_scale for those heads, only in late rows
    q, kv = q.to(torch.bfloat16), kv.to(torch.bfloat16)
    # ascending selections whose last tile holds the late rows
    idx = torch.stack([torch.cat([torch.arange(k - 20) + t * 100, late]) for t in range(T)]).to(torch.int32)
    g, gl = _mla_gpu(dsa, q, kv, idx, 1 / math.sqrt(192), "bf16", use_ws=use_ws)
    o, l = ora.sparse_mla_rows(q, kv, idx.numpy(), 1 / math.sqrt(192))
    assert np.isfinite(g).all() and np.isfinite(gl).all()
    assert l[:, ::3].min() > 150.0 and np.abs(l[:, 1::3]).max() < 20.0   # the spike decides those heads only
    check_attention(g, gl, o, l, "bf16", "mla late large logits")


def test_prefill_late_large_logits(dsa, ora):
    """The fused prefill with a few late latent rows that give some heads
    logits far above anything in their first tile (through a rope dim, so
    the values keep the workload's scale): those queries take the recompute
    path of the unsplit kernel."""
    L, k, H = 3000, 2048, 16
    _say(f"prefill late large logits L={L} H={H}")
    cfg = synth.scaled_down(synth.CONFIGS["prefill16k"], L=L, k=k, H=H, seed=17)
    q_i, k_i, w, q, kv = _prefill_inputs(cfg)
    q, kv = q.float(), kv.float()
    q[:, ::3, 512] = 30.0
    kv[:, 512] = 0.01
    kv[2500:2520, 512] = 100.0
    q, kv = q.to(torch.bfloat16), kv.to(torch.bfloat16)
    t = _run_prefill(dsa, cfg, q_i, k_i, w, q, kv)
    rows = np.array([0, 100, 2047, 2499, 2519, 2520, 2600, 2800, 2999])
    _check_prefill_rows(ora, cfg, q_i, k_i, w, q, kv, t, rows, "prefill late large logits")
    # the later queries select some of the late rows, past their first tile
    gidx = t["idx"].cpu().numpy()
    assert np.isin(np.arange(2500, 2520), gidx[2999]).any()
    assert (t["lse"].cpu()[2999, ::3] > 150.0).all()


# ------------------------------------------------------------------ full-size workloads
def _sample_rows(L, extra, seed):
    fixed = [0, 1, 2046, 2047, 2048, 2049, 4095, L // 2 - 1, L - 1]
    drawn = synth.randint(seed, 1, (extra,), 0, L).tolist()
    return np.array(sorted(set(r for r in fixed + drawn if 0 <= r < L)), dtype=np.int64)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["prefill128k", "prefill16k"])
def test_prefill_full_size_sampled_rows(dsa, ora, name):
    """The full-size prefill workloads (L = 131072, the benchmarked one, and
    L = 16384), each through the pipeline the benchmark times (quantise ->
    fused indexer + top-k -> sparse MLA), checked against the oracle on 64
    sampled query rows: nine fixed rows at the selection's edges plus 55
    drawn ones."""
    cfg = synth.CONFIGS[name]
    L, k = cfg.L, cfg.k
    _say(f"prefill full size L={L}")
    q_i, k_i, w = synth.prefill_indexer_inputs(cfg, device=DEV)
    q = synth.prefill_attn_q(cfg, device=DEV)
    kv = synth.prefill_latent(cfg, device=DEV)
    q8 = torch.empty((L, cfg.H_I, cfg.D_I), dtype=torch.uint8, device=DEV)
    qs = torch.empty(L, dtype=torch.float32, device=DEV)
    k8 = torch.empty((L, cfg.D_I), dtype=torch.uint8, device=DEV)
    ks = torch.empty(L, dtype=torch.float32, device=DEV)
    dsa.dsa_quantize_e4m3_per_token(q_i, q8, qs, rows=L, cols=cfg.H_I * cfg.D_I)
    dsa.dsa_quantize_e4m3_per_token(k_i, k8, ks, rows=L, cols=cfg.D_I)
    idx = torch.empty((L, k), dtype=torch.int32, device=DEV)
    out = torch.empty((L, cfg.H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((L, cfg.H), dtype=torch.float32, device=DEV)
    args = dsa.make_prefill_args(L, cfg.H_I, cfg.D_I, cfg.H, k, dsa.DSA_E4M3, q8, qs, k8, ks, w, dsa.DSA_BF16, q, kv,
                                 cfg.sm_scale, idx, out, lse)
    ws = torch.empty(dsa.dsa_prefill_workspace_bytes(args), dtype=torch.uint8, device=DEV)
    dsa.dsa_prefill_select(args, ws)
    dsa.dsa_sparse_mla_fwd(q, kv, idx, cfg.sm_scale, out, lse)
    torch.cuda.synchronize()
    del ws
    rows = _sample_rows(L, 55, 21)
    assert len(rows) >= 60
    rt = torch.from_numpy(rows).to(DEV)
    # quantiser: bit-exact on the sampled query rows and on every key
    o8, os_ = ora.quantize_rows(q_i[rt].view(len(rows), -1).cpu().numpy())
    assert np.array_equal(q8[rt].view(len(rows), -1).cpu().numpy(), o8)
    assert np.array_equal(qs[rt].cpu().numpy(), os_)
    ok8, oks = ora.quantize_rows(k_i.cpu().numpy())
    k8c, ksc = k8.cpu().numpy(), ks.cpu().numpy()
    assert np.array_equal(k8c, ok8) and np.array_equal(ksc, oks)
    del q_i, k_i
    # selection: oracle scores of the sampled rows
    sc = ora.indexer_rows(q8[rt].cpu().numpy(), k8c, w[rt].cpu().numpy(), rows.astype(np.int32),
                          q_scale=qs[rt].cpu().numpy(), k_scale=ksc)
    gidx = idx[rt].cpu().numpy()
    for j, r in enumerate(rows):
        check_topk_row(gidx[j], sc[j], int(r) + 1, k, f"L={L} row {r}")
    # attention over the GPU's own selection
    o, l = ora.sparse_mla_rows(q[rt].cpu(), kv.cpu(), gidx, cfg.sm_scale)
    check_attention(out[rt].float().cpu().double().numpy(), lse[rt].cpu().double().numpy(), o, l, "bf16",
                    f"L={L}")


@pytest.mark.slow
@pytest.mark.parametrize("name", ["decode", "paged"])
def test_decode_full_size_sampled_sequences(dsa, ora, name):
    """The benchmarked decode batches (B = 64 at context 32768; B = 128 ragged
    with shuffled pages), checked against the oracle on sampled sequences."""
    cfg = synth.CONFIGS[name]
    _say(f"decode full size {cfg.name}")
    ctx = synth.decode_ctx(cfg)
    bt, nb = synth.decode_block_table(cfg, ctx)
    pools = synth.build_decode_pools(cfg, ctx, bt, nb, device=DEV)
    qside = synth.decode_queries(cfg)
    out, lse, idx = _run_decode(dsa, cfg, ctx, bt, nb, pools, qside)
    del pools
    gidx = idx.cpu().numpy()
    q8, qs, w, q = qside
    seqs = sorted({0, cfg.B - 1, int(torch.argmax(ctx)), int(torch.argmin(ctx)),
                   int(synth.randint(22, 1, (1,), 0, cfg.B)[0])})
    for b in seqs:
        c = int(ctx[b])
        kb, sb = synth.decode_seq_keys(cfg, b, c)
        sc = ora.indexer_rows(q8[b:b + 1], kb, w[b:b + 1], np.array([c - 1], np.int32), q_scale=qs[b:b + 1],
                              k_scale=sb)
        check_topk_row(gidx[b], sc[0], c, cfg.k, f"{cfg.name} b={b}")
        lat = synth.decode_seq_latent(cfg, b, c)
        o, l = ora.sparse_mla_rows(q[b:b + 1], lat, gidx[b:b + 1], cfg.sm_scale)
        check_attention(out[b:b + 1].float().cpu().double().numpy(), lse[b:b + 1].cpu().double().numpy(), o, l,
                        "bf16", f"{cfg.name} b={b}")
