"""Pins of the fp64 CPU oracle against facts fixed outside the oracle itself:
library routines on special cases, closed forms, invariants, exact arithmetic
and brute force on tiny inputs.  CPU only.

Each pin is chosen so that a plausible slip in the oracle (a dropped ReLU or
scale, a wrong sign or index, a transposed operand, the wrong value width, a
tie broken the wrong way, a paging slip) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def _bf16_bits(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ codecs
def test_e4m3_decode_all_codes_match_torch(ora):
    codes = np.arange(256, dtype=np.uint8)
    mine = ora.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(mine[~nan], ref[~nan])


def test_e4m3_decode_closed_forms(ora):
    # OCP E4M3: max normal 1.75*2^8, min normal 2^-6, min subnormal 2^-9, 1.0 = 0x38
    vals = ora.e4m3_decode(np.array([0x7E, 0x08, 0x01, 0x38, 0xB8, 0x80, 0x07], np.uint8))
    assert list(vals) == [448.0, 2.0 ** -6, 2.0 ** -9, 1.0, -1.0, 0.0, 7 * 2.0 ** -9]
    assert math.copysign(1.0, vals[5]) == -1.0


def _e4m3_grid():
    codes = np.arange(256, dtype=np.uint8)
    v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return np.unique(v[np.isfinite(v) & (v >= 0)])


def test_e4m3_encode_matches_torch_rne(ora):
    grid = _e4m3_grid()
    mids = (grid[1:] + grid[:-1]) / 2  # exact ties: RNE decides
    pts = np.concatenate([grid, mids])
    f32 = pts.astype(np.float32)
    # one fp32 ulp either side of every point
    up = np.nextafter(f32, np.float32(np.inf))
    dn = np.nextafter(f32, np.float32(0))
    rng = np.random.default_rng(0)
    rnd = (rng.standard_normal(4000) * np.exp2(rng.integers(-12, 9, 4000))).astype(np.float32)
    x = np.concatenate([f32, up, dn, rnd])
    x = x[np.abs(x) < 448.0]
    x = np.concatenate([x, -x])
    mine = ora.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)


def test_e4m3_encode_saturates_and_signed_zero(ora):
    x = np.array([448.0, 460.0, 464.0, 1e6, -1e30, -0.0, 0.0], np.float32)
    assert list(ora.e4m3_encode(x)) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00]


def test_bf16_decode_matches_torch(ora):
    x = torch.randn(3000, generator=torch.Generator().manual_seed(1)) * 100
    bits = _bf16_bits(x)
    ref = x.to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ora.bf16_decode(bits), ref)


def test_quantize_rows(ora):
    x = synth.normal(3, 1, (64, 128)).numpy()
    x[5] = 0.0
    x8, sc = ora.quantize_rows(x)
    amax = np.abs(x).max(axis=1)
    exp_scale = np.where(amax > 0, (amax.astype(np.float32) / np.float32(448.0)), np.float32(1.0))
    assert np.array_equal(sc, exp_scale.astype(np.float32))
    # the payload is torch's RNE cast of the fp32 quotient
    quot = (x / sc[:, None]).astype(np.float32)
    ref = torch.from_numpy(quot).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(x8, ref)
    # the largest element of each non-zero row lands on +-448
    dec = ora.e4m3_decode(x8)
    for r in range(64):
        if r == 5:
            assert not dec[r].any()
            continue
        assert np.abs(dec[r]).max() == 448.0
    # E4M3 keeps 3 mantissa bits: relative error at most 2^-4 for normals
    big = np.abs(quot) >= 2 ** -6
    assert np.all(np.abs(dec[big] - quot[big]) <= 2.0 ** -4 * np.abs(quot[big]))


# ------------------------------------------------------------------ indexer
def test_indexer_single_head_is_relu_of_matmul(ora):
    """H_I = 1, w = 1: I = ReLU(q k^T) masked causally (library matmul)."""
    T, S, D = 40, 56, 16
    q = synth.normal(5, 1, (T, 1, D)).numpy()
    k = synth.normal(5, 2, (S, D)).numpy()
    pos = np.arange(T, dtype=np.int32) + 9  # rows see s <= t + 9
    got = ora.indexer_rows(q, k, np.ones((T, 1), np.float32), pos)
    ref = torch.relu(torch.from_numpy(q[:, 0].astype(np.float64)) @
                     torch.from_numpy(k.astype(np.float64)).T).numpy()
    mask = np.arange(S)[None, :] > pos[:, None]
    ref[mask] = -np.inf
    assert np.array_equal(np.isinf(got), mask)
    np.testing.assert_allclose(got[~mask], ref[~mask], rtol=1e-13, atol=1e-13)


def test_indexer_exact_integers(ora):
    """E4M3 payloads in {0, +-1, +-2}, scales 1, w in {+-1, +-0.5}: all exact.
    Check against integer arithmetic written per pair."""
    rng = np.random.default_rng(7)
    T, S, H, D = 9, 9, 3, 8
    lut = {0: 0x00, 1: 0x38, -1: 0xB8, 2: 0x40, -2: 0xC0}
    qi = rng.integers(-2, 3, (T, H, D))
    ki = rng.integers(-2, 3, (S, D))
    wv = rng.choice([-1.0, -0.5, 0.5, 1.0], (T, H)).astype(np.float32)
    q8 = np.vectorize(lut.get)(qi).astype(np.uint8)
    k8 = np.vectorize(lut.get)(ki).astype(np.uint8)
    pos = np.arange(T, dtype=np.int32)
    got = ora.indexer_rows(q8, k8, wv, pos, q_scale=np.ones(T, np.float32),
                           k_scale=np.ones(S, np.float32))
    for t in range(T):
        for s in range(S):
            if s > t:
                assert got[t, s] == -np.inf
                continue
            twice = 0  # 2*I as an integer
            for j in range(H):
                dot = int(sum(int(qi[t, j, d]) * int(ki[s, d]) for d in range(D)))
                twice += int(2 * wv[t, j]) * max(dot, 0)
            assert got[t, s] == twice / 2
            if got[t, s] == 0:
                assert math.copysign(1.0, got[t, s]) == 1.0  # -0 canonicalised


def test_indexer_scales_pull_out(ora):
    """Positive scales factor out of the ReLU: doubling k_scale[s] doubles
    column s exactly and no other; doubling q_scale[t] doubles row t."""
    T, H, D = 6, 4, 32
    x = synth.normal(11, 1, (T, H, D))
    kx = synth.normal(11, 2, (T, D))
    q8, qs = ora.quantize_rows(x.view(T, H * D).numpy())  # one scale per token
    q8 = q8.reshape(T, H, D)
    k8, ks = ora.quantize_rows(kx.numpy())
    w = synth.normal(11, 3, (T, H)).numpy()
    pos = np.full(T, T - 1, np.int32)
    base = ora.indexer_rows(q8, k8, w, pos, q_scale=qs, k_scale=ks)
    ks2 = ks.copy()
    ks2[2] *= 2
    col = ora.indexer_rows(q8, k8, w, pos, q_scale=qs, k_scale=ks2)
    assert np.array_equal(col[:, 2], 2 * base[:, 2])
    assert np.array_equal(np.delete(col, 2, 1), np.delete(base, 2, 1))
    qs2 = qs.copy()
    qs2[4] *= 2
    row = ora.indexer_rows(q8, k8, w, pos, q_scale=qs2, k_scale=ks)
    assert np.array_equal(row[4], 2 * base[4])
    # with unit scales the E4M3 path equals the fp32 path on the decoded values
    dq = ora.e4m3_decode(q8).astype(np.float32)
    dk = ora.e4m3_decode(k8).astype(np.float32)
    f = ora.indexer_rows(dq, dk, w, pos)
    u = ora.indexer_rows(q8, k8, w, pos, q_scale=np.ones(T, np.float32), k_scale=np.ones(T, np.float32))
    np.testing.assert_allclose(f, u, rtol=1e-14)


def test_indexer_relu_drops_negative_heads(ora):
    """A head whose query is the negated key contributes nothing, whatever w."""
    D = 16
    k = synth.normal(2, 2, (1, D)).numpy()
    q = np.stack([np.stack([-k[0], k[0]])])  # [1, 2, D]: head 0 anti-aligned, head 1 aligned
    for w0 in (-3.0, 0.0, 5.0):
        got = ora.indexer_rows(q.astype(np.float32), k, np.array([[w0, 1.0]], np.float32),
                               np.array([0], np.int32))
        assert got[0, 0] == pytest.approx(float(np.dot(k[0].astype(np.float64), k[0])), rel=1e-12)


def test_indexer_linear_in_w_and_head_order(ora):
    T, H, D = 12, 5, 24
    q = synth.normal(4, 1, (T, H, D)).numpy()
    k = synth.normal(4, 2, (T, D)).numpy()
    w1 = synth.normal(4, 3, (T, H)).numpy()
    w2 = synth.normal(4, 4, (T, H)).numpy()
    pos = np.arange(T, dtype=np.int32)
    a = ora.indexer_rows(q, k, w1, pos)
    b = ora.indexer_rows(q, k, w2, pos)
    c = ora.indexer_rows(q, k, (w1 + w2).astype(np.float32), pos)
    fin = np.isfinite(c)
    np.testing.assert_allclose(c[fin], a[fin] + b[fin], rtol=1e-6, atol=1e-5)
    perm = np.array([3, 0, 4, 1, 2])
    d = ora.indexer_rows(np.ascontiguousarray(q[:, perm]), k, np.ascontiguousarray(w1[:, perm]), pos)
    np.testing.assert_allclose(d[fin], a[fin], rtol=1e-12, atol=1e-12)
    # w = 0 gives exactly zero on and below the diagonal
    z = ora.indexer_rows(q, k, np.zeros((T, H), np.float32), pos)
    assert np.all(z[fin] == 0.0)


# ------------------------------------------------------------------ top-k
def test_topk_distinct_matches_torch_topk(ora):
    rng = np.random.default_rng(3)
    for n, k in ((100, 7), (5000, 2048), (300, 300), (10, 50)):
        s = rng.standard_normal(n)
        idx, K, tau = ora.topk_row(s, k)
        assert K == min(n, k)
        assert np.all(idx[K:] == -1)
        ref = torch.topk(torch.from_numpy(s), K).indices.numpy()
        assert np.array_equal(idx[:K], np.sort(ref))
        assert tau == np.sort(s)[::-1][K - 1]


def test_topk_all_tied_selects_most_recent_window(ora):
    n, k = 1000, 256
    idx, K, tau = ora.topk_row(np.zeros(n), k)
    assert K == k and tau == 0.0
    assert np.array_equal(idx, np.arange(n - k, n))


def test_topk_rank_bruteforce_with_ties(ora):
    """Selected iff fewer than k candidates beat it under (score desc, pos desc)."""
    rng = np.random.default_rng(5)
    for trial in range(200):
        n = int(rng.integers(1, 14))
        k = int(rng.integers(1, 10))
        s = rng.integers(-2, 3, n).astype(np.float64)
        idx, K, _ = ora.topk_row(s, k)
        chosen = set(idx[:K].tolist())
        for p in range(n):
            beats = sum(1 for o in range(n) if s[o] > s[p] or (s[o] == s[p] and o > p))
            assert (beats < k) == (p in chosen)


def test_topk_rows_counts(ora):
    s = synth.normal(1, 1, (6, 50)).double().numpy()
    nv = np.array([0, 1, 2, 49, 50, 30])
    idx, tau = ora.topk_rows(s, nv, 8)
    for r in range(6):
        K = min(8, nv[r])
        assert np.all(idx[r, :K] >= 0) and np.all(idx[r, :K] < max(nv[r], 1))
        assert np.all(idx[r, K:] == -1)
        assert len(set(idx[r, :K].tolist())) == K
    assert tau[0] == -np.inf


# --------------------------------------------------------------- attention
def _sdpa(q, kv, mask, scale, Dv=512):
    """torch SDPA in fp64: q [T,H,D], kv [N,D], mask [T,N] bool (True = attend)."""
    qt = torch.from_numpy(q).permute(1, 0, 2)            # [H, T, D]
    K = torch.from_numpy(kv)[None].expand(qt.shape[0], -1, -1)
    V = torch.from_numpy(kv[:, :Dv].copy())[None].expand(qt.shape[0], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, K, V, attn_mask=torch.from_numpy(mask),
                                                         scale=scale)
    logits = (qt @ K.transpose(1, 2)) * scale
    logits = logits.masked_fill(~torch.from_numpy(mask), -math.inf)
    return o.permute(1, 0, 2).numpy(), torch.logsumexp(logits, -1).T.numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mla_full_selection_equals_dense_causal_sdpa(ora, dtype):
    """k >= L: every causal position is selected, so sparse = dense causal."""
    L, H, k = 48, 4, 64
    q = synth.normal(9, 1, (L, H, 576))
    kv = synth.normal(9, 2, (L, 576), std=1.0 / 24)
    if dtype == "bf16":
        q, kv = q.to(torch.bfloat16), kv.to(torch.bfloat16)
    idx = np.full((L, k), -1, np.int32)
    for t in range(L):
        idx[t, :t + 1] = np.arange(t + 1)[::-1]
    scale = 1 / math.sqrt(192)
    o, lse = ora.sparse_mla_rows(q, kv, idx, scale)
    mask = np.tril(np.ones((L, L), bool))
    ro, rl = _sdpa(q.double().numpy(), kv.double().numpy(), mask, scale)
    np.testing.assert_allclose(o, ro, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=1e-12, atol=1e-12)


def test_pipeline_all_tied_equals_band_sdpa(ora):
    """w = 0 ties every score; the (score, position) order then selects the
    window [t-k+1, t], and sparse MLA equals dense attention over that band."""
    L, HI, DI, H, k = 80, 2, 16, 4, 16
    q_i = synth.normal(8, 1, (L, HI, DI)).numpy()
    k_i = synth.normal(8, 2, (L, DI)).numpy()
    pos = np.arange(L, dtype=np.int32)
    sc = ora.indexer_rows(q_i, k_i, np.zeros((L, HI), np.float32), pos)
    idx, tau = ora.topk_rows(np.where(np.isinf(sc), 0, sc), pos + 1, k)
    for t in range(L):
        lo = max(0, t - k + 1)
        assert np.array_equal(idx[t, :t + 1 - lo], np.arange(lo, t + 1))
    q = synth.normal(8, 3, (L, H, 576), std=40.0)  # sharp softmax
    kv = synth.normal(8, 4, (L, 576), std=1.0 / 24)
    scale = 1 / math.sqrt(192)
    o, lse = ora.sparse_mla_rows(q, kv, idx, scale)
    band = np.tril(np.ones((L, L), bool)) & ~np.tril(np.ones((L, L), bool), -k)
    ro, rl = _sdpa(q.double().numpy(), kv.double().numpy(), band, scale)
    np.testing.assert_allclose(o, ro, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=1e-12, atol=1e-12)


def test_mla_zero_query_is_mean_of_values(ora):
    N, k = 64, 16
    kv = synth.normal(1, 2, (N, 576)).numpy()
    idx = np.array([[3, 60, 7, 7, 0, 33, -1, -1, 12, 5, 9, 41, 2, 8, 18, 63]], np.int32)
    o, lse = ora.sparse_mla_rows(np.zeros((1, 2, 576), np.float32), kv, idx, 0.3)
    sel = idx[0][idx[0] >= 0]
    np.testing.assert_allclose(o[0, 0], kv[sel, :512].astype(np.float64).mean(0), rtol=1e-12, atol=1e-14)
    assert lse[0, 1] == pytest.approx(math.log(len(sel)), rel=1e-14)


def test_mla_one_hot_rows_closed_form(ora):
    """Row a = c_a * e_a (one-hot): logits z_a = s c_a q[a]; the value of row a
    is c_a e_a, so o[a] = c_a softmax(z)_a in closed form."""
    m = 10
    c = np.linspace(0.5, 2.0, m)
    kv = np.zeros((m, 576), np.float32)
    kv[np.arange(m), np.arange(m)] = c
    q = np.zeros((1, 1, 576), np.float32)
    q[0, 0, :m] = np.linspace(-3, 3, m)
    s = 0.7
    o, lse = ora.sparse_mla_rows(q, kv, np.arange(m, dtype=np.int32)[None], s)
    z = s * c.astype(np.float32).astype(np.float64) * q[0, 0, :m].astype(np.float64)
    p = np.exp(z - z.max()) / np.exp(z - z.max()).sum()
    np.testing.assert_allclose(o[0, 0, :m], c.astype(np.float32) * p, rtol=1e-13)
    assert np.all(o[0, 0, m:] == 0)
    assert lse[0, 0] == pytest.approx(z.max() + math.log(np.exp(z - z.max()).sum()), rel=1e-14)


def test_mla_order_and_padding_invariance(ora):
    N, T, H, k = 200, 3, 4, 32
    q = synth.normal(2, 1, (T, H, 576)).to(torch.bfloat16)
    kv = synth.normal(2, 2, (N, 576), std=1 / 24).to(torch.bfloat16)
    idx = synth.permutation(2, 3, N)[:T * 24].view(T, 24).to(torch.int32).numpy()
    pad = np.full((T, k), -1, np.int32)
    pad[:, 4:28] = idx
    a, la = ora.sparse_mla_rows(q, kv, pad, 0.1)
    b, lb = ora.sparse_mla_rows(q, kv, np.ascontiguousarray(idx[:, ::-1]), 0.1)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(la, lb, rtol=1e-14)
    e, le = ora.sparse_mla_rows(q, kv, np.full((T, k), -1, np.int32), 0.1)
    assert np.all(e == 0) and np.all(np.isneginf(le))


# ------------------------------------------------------ masked MHA (short prefill)
def _mha_inputs(seed, T, N, H, Dc=32, Dr=8, Dn=16, Dvh=12, dtype=torch.float64):
    q = synth.normal(seed, 1, (T, H, Dn + Dr)).to(dtype)
    kv = synth.normal(seed, 2, (N, Dc + Dr), std=0.5).to(dtype)
    w_uk = synth.normal(seed, 3, (H, Dn, Dc), std=1 / math.sqrt(Dc)).to(dtype)
    w_uv = synth.normal(seed, 4, (H, Dvh, Dc), std=1 / math.sqrt(Dc)).to(dtype)
    return q, kv, w_uk, w_uv


def test_masked_mha_equals_absorbed_mqa(ora):
    """MLA's two forms agree: scores q_h.(W_uk c, r) = (W_uk^T q_n, q_r).(c, r), and
    the value W_uv c comes out of the softmax sum.  So masked MHA equals the MQA
    oracle run on absorbed queries, followed by the value up-projection."""
    T, N, H, k, Dc, Dr, Dn, Dvh = 9, 30, 3, 7, 32, 8, 16, 12
    q, kv, w_uk, w_uv = _mha_inputs(11, T, N, H, Dc, Dr, Dn, Dvh)
    idx = np.full((T, k), -1, np.int32)
    perm = synth.permutation(11, 5, N).numpy()
    for t in range(T):
        m = (t % k) + 1 if t != 4 else 0   # one query with an empty selection
        idx[t, :m] = perm[(3 * t + np.arange(m)) % N]
    scale = 0.17
    o, lse = ora.masked_mha_rows(q, kv, w_uk, w_uv, idx, scale, Dr=Dr)
    qn, qr = q[..., :Dn].numpy(), q[..., Dn:].numpy()
    q_abs = np.concatenate([np.einsum("hec,the->thc", w_uk.numpy(), qn), qr], axis=-1)
    oa, la = ora.sparse_mla_rows(np.ascontiguousarray(q_abs), kv.numpy(), idx, scale, Dv=Dc)
    ref = np.einsum("hec,thc->the", w_uv.numpy(), oa)
    np.testing.assert_allclose(o, ref, rtol=1e-11, atol=1e-13)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(la))
    fin = np.isfinite(la)
    np.testing.assert_allclose(lse[fin], la[fin], rtol=1e-12, atol=1e-12)
    assert np.all(o[4] == 0) and np.all(np.isneginf(lse[4]))


def test_masked_mha_full_selection_equals_dense_causal_mha(ora):
    """k >= L: the mask keeps every causal position, so the result is dense
    causal multi-head attention with per-head keys and values."""
    L, H, Dc, Dr, Dn, Dvh = 24, 2, 32, 8, 16, 12
    q, kv, w_uk, w_uv = _mha_inputs(12, L, L, H, Dc, Dr, Dn, Dvh)
    idx = np.full((L, 32), -1, np.int32)
    for t in range(L):
        idx[t, :t + 1] = np.arange(t + 1)
    scale = 1 / math.sqrt(Dn + Dr)
    o, lse = ora.masked_mha_rows(q, kv, w_uk, w_uv, idx, scale, Dr=Dr)
    K = torch.cat([torch.einsum("hec,sc->hse", w_uk, kv[:, :Dc]), kv[None, :, Dc:].expand(H, -1, -1)], -1)
    V = torch.einsum("hec,sc->hse", w_uv, kv[:, :Dc])
    qt = q.permute(1, 0, 2)
    mask = torch.tril(torch.ones(L, L, dtype=torch.bool))
    ro = torch.nn.functional.scaled_dot_product_attention(qt, K, V, attn_mask=mask, scale=scale)
    rl = torch.logsumexp(((qt @ K.transpose(1, 2)) * scale).masked_fill(~mask, -math.inf), -1)
    np.testing.assert_allclose(o, ro.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, rl.T.numpy(), rtol=1e-12, atol=1e-12)


def test_masked_mha_mask_order_and_padding_invariance(ora):
    T, N, H, k = 4, 40, 2, 16
    q, kv, w_uk, w_uv = _mha_inputs(13, T, N, H, dtype=torch.bfloat16)
    sel = synth.permutation(13, 6, N)[:T * 10].view(T, 10).to(torch.int32).numpy()
    pad = np.full((T, k), -1, np.int32)
    pad[:, 3:13] = sel
    a, la = ora.masked_mha_rows(q, kv, w_uk, w_uv, pad, 0.2, Dr=8)
    b, lb = ora.masked_mha_rows(q, kv, w_uk, w_uv, np.ascontiguousarray(sel[:, ::-1]), 0.2, Dr=8)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(la, lb, rtol=1e-14)


# ------------------------------------------------------------------ decode
def _small_decode(shuffled, seed=4, B=3, lo=70, hi=300, k=64):
    cfg = synth.DecodeConfig("t", B, lo, hi, 4, 32, 8, k, seed, shuffled)
    ctx = synth.decode_ctx(cfg)
    bt, nb = synth.decode_block_table(cfg, ctx)
    pools = synth.build_decode_pools(cfg, ctx, bt, nb)
    qside = synth.decode_queries(cfg)
    return cfg, ctx, bt, pools, qside


def test_decode_block_shuffle_invariance(ora):
    res = []
    for sh in (False, True):
        cfg, ctx, bt, (k8, ks, kv), (q8, qs, w, q) = _small_decode(sh)
        res.append(ora.decode(q8, qs, w, q, k8.view(-1, cfg.D_I), ks.view(-1), kv.view(-1, 576), bt, ctx,
                              cfg.k, cfg.sm_scale))
        if sh:
            assert not np.array_equal(bt.numpy(), _small_decode(False)[2].numpy())
    for a, b in zip(res[0], res[1]):
        assert np.array_equal(a, b)


def test_decode_equals_prefill_row_of_logical_sequence(ora):
    cfg, ctx, bt, (k8, ks, kv), (q8, qs, w, q) = _small_decode(True)
    idx, tau, o, lse = ora.decode(q8, qs, w, q, k8.view(-1, cfg.D_I), ks.view(-1), kv.view(-1, 576), bt,
                                  ctx, cfg.k, cfg.sm_scale)
    for b in range(cfg.B):
        c = int(ctx[b])
        kb, sb = synth.decode_seq_keys(cfg, b, c)
        lat = synth.decode_seq_latent(cfg, b, c)
        sc = ora.indexer_rows(q8[b:b + 1], kb, w[b:b + 1], np.array([c - 1], np.int32),
                              q_scale=qs[b:b + 1], k_scale=sb)
        i2, _, t2 = ora.topk_row(sc[0], cfg.k)
        assert np.array_equal(i2, idx[b]) and t2 == tau[b]
        o2, l2 = ora.sparse_mla_rows(q[b:b + 1], lat, i2[None], cfg.sm_scale)
        assert np.array_equal(o2[0], o[b]) and np.array_equal(l2[0], lse[b])


def test_decode_never_reads_page_tails(ora):
    cfg, ctx, bt, (k8, ks, kv), (q8, qs, w, q) = _small_decode(True)
    assert any(int(c) % 64 for c in ctx)
    a = ora.decode(q8, qs, w, q, k8.view(-1, cfg.D_I), ks.view(-1), kv.view(-1, 576), bt, ctx, cfg.k,
                   cfg.sm_scale)
    k8b, ksb, kvb = k8.clone(), ks.clone(), kv.clone()
    for b in range(cfg.B):
        c = int(ctx[b])
        last = int(bt[b, (c - 1) // 64])
        k8b[last, c % 64 or 64:] = 0x01
        ksb[last, c % 64 or 64:] = 7.0
        kvb[last, c % 64 or 64:] = -3.0
    b_ = ora.decode(q8, qs, w, q, k8b.view(-1, cfg.D_I), ksb.view(-1), kvb.view(-1, 576), bt, ctx, cfg.k,
                    cfg.sm_scale)
    for x, y in zip(a, b_):
        assert np.array_equal(x, y)


# ------------------------------------------------------------ cache append
def _append_case(shuffled):
    """Sequences of lengths ctx (one ends on a page boundary, so its next token
    opens a new page), a block table sized for one more token each, pools
    holding the first ctx tokens, and the logical token at position ctx."""
    cfg = synth.DecodeConfig("t", 4, 1, 1, 4, 32, 8, 64, 6, shuffled)
    ctx = torch.tensor([64, 130, 1, 255], dtype=torch.int64)
    bt, nb = synth.decode_block_table(cfg, ctx + 1)
    pools = synth.build_decode_pools(cfg, ctx, bt, nb)
    lat, k8, ks = [], [], []
    for b in range(cfg.B):
        c = int(ctx[b])
        kb, sb = synth.decode_seq_keys(cfg, b, c + 1)
        lat.append(synth.decode_seq_latent(cfg, b, c + 1)[c])
        k8.append(kb[c])
        ks.append(sb[c])
    return cfg, ctx, bt, nb, pools, (torch.stack(lat), torch.stack(k8), torch.stack(ks))


@pytest.mark.parametrize("shuffled", [False, True])
def test_cache_append_grows_the_logical_sequence(ora, shuffled):
    """Appending each sequence's token at position ctx to pools that hold ctx
    tokens gives, byte for byte, the pools that hold ctx + 1 tokens (the
    generator writes logical rows independently of the append)."""
    cfg, ctx, bt, nb, (k8, ks, kv), (lat, tk8, tks) = _append_case(shuffled)
    kvp, k8p, ksp = ora.paged_cache_append(lat, tk8, tks, ctx.to(torch.int32), bt, kv.view(-1, 576),
                                           k8.view(-1, cfg.D_I), ks.view(-1))
    ek8, eks, ekv = synth.build_decode_pools(cfg, ctx + 1, bt, nb)
    assert np.array_equal(k8p, ek8.view(-1, cfg.D_I).numpy())
    assert np.array_equal(ksp, eks.view(-1).numpy())
    assert np.array_equal(kvp, ekv.view(-1, 576).view(torch.int16).numpy().view(np.uint16))
    # and exactly one row per sequence changed
    changed = (kvp != kv.view(-1, 576).view(torch.int16).numpy().view(np.uint16)).any(axis=1)
    assert changed.sum() == cfg.B


def test_cache_append_skips_positions_outside_the_table(ora):
    cfg, ctx, bt, nb, (k8, ks, kv), (lat, tk8, tks) = _append_case(True)
    bt2 = bt.clone()
    bt2[3, :] = -1                                     # sequence 3: its page is unmapped
    pos = torch.tensor([-1, bt.shape[1] * 64, 5, 200], dtype=torch.int32)  # before, past the table, ok, unmapped
    kvp, k8p, ksp = ora.paged_cache_append(lat, tk8, tks, pos, bt2, kv.view(-1, 576), k8.view(-1, cfg.D_I),
                                           ks.view(-1))
    row = int(bt[2, 0]) * 64 + 5
    kv0 = kv.view(-1, 576).view(torch.int16).numpy().view(np.uint16)
    changed = np.nonzero((kvp != kv0).any(axis=1))[0]
    assert changed.tolist() == [row]
    assert np.array_equal(np.delete(k8p, row, 0), np.delete(k8.view(-1, cfg.D_I).numpy(), row, 0))
    assert ksp[row] == tks[2].item() and np.array_equal(np.delete(ksp, row), np.delete(ks.view(-1).numpy(), row))


def test_append_then_decode_equals_decode_of_longer_sequence(ora):
    cfg, ctx, bt, nb, (k8, ks, kv), (lat, tk8, tks) = _append_case(True)
    kvp, k8p, ksp = ora.paged_cache_append(lat, tk8, tks, ctx.to(torch.int32), bt, kv.view(-1, 576),
                                           k8.view(-1, cfg.D_I), ks.view(-1))
    q8, qs, w, q = synth.decode_queries(cfg)
    a = ora.decode(q8, qs, w, q, k8p, ksp, kvp, bt, ctx + 1, cfg.k, cfg.sm_scale)
    ek8, eks, ekv = synth.build_decode_pools(cfg, ctx + 1, bt, nb)
    b_ = ora.decode(q8, qs, w, q, ek8.view(-1, cfg.D_I), eks.view(-1), ekv.view(-1, 576), bt, ctx + 1, cfg.k,
                    cfg.sm_scale)
    for x, y in zip(a, b_):
        assert np.array_equal(x, y)
    # the appended token is a candidate of its own query (position ctx), selected when k covers it
    assert all(int(ctx[b]) in a[0][b] for b in range(cfg.B) if int(ctx[b]) + 1 <= cfg.k)


# ------------------------------------------------------------ page constants
def test_page_constants_fix_k_and_context():
    g = json.load(open(os.path.join(HERE, "golden", "pages_constants.json")))
    ctx = 128 * 1024
    assert round(g["warmup"]["steps"] * g["warmup"]["seqs_per_step"] * ctx / 1e9, 1) == g["warmup"]["tokens_billion"]
    assert round(g["sparse"]["steps"] * g["sparse"]["seqs_per_step"] * ctx / 1e9, 1) == g["sparse"]["tokens_billion"]
    for name in ("decode", "prefill16k", "prefill128k", "paged"):
        assert synth.CONFIGS[name].k == g["top_k"]
    assert synth.CONFIGS["prefill128k"].L == ctx
    assert synth.CONFIGS["paged"].ctx_hi == ctx


# ------------------------------------------------ indexer KL-alignment loss
def _kl_inputs(seed, T, N, H, D, k, q_std=1.0):
    q = synth.normal(seed, 1, (T, H, D), std=q_std).double()
    kv = synth.normal(seed, 2, (N, D), std=0.5).double()
    idx = np.full((T, k), -1, np.int32)
    for t in range(T):
        m = 2 + (3 * t) % (k - 1)
        idx[t, :m] = synth.permutation(seed, 10 + t, N)[:m].numpy()
    scores = synth.normal(seed, 3, (T, k), std=2.0).double().numpy()
    return q, kv, idx, scores


def _head_avg_attention(q, kv, sel, scale):
    """p over the entries sel of one query: per-head softmax (torch), averaged over heads."""
    z = scale * torch.einsum("hd,ad->ha", q, kv[torch.from_numpy(sel).long()])
    return torch.softmax(z, dim=1).mean(dim=0).numpy()


def test_indexer_kl_matches_scipy_relative_entropy(ora):
    """KL(p || pi) against scipy's relative entropy, with p from torch's softmax
    averaged over heads and pi from torch's softmax of the scores."""
    import scipy.stats
    T, N, H, D, k = 7, 40, 3, 12, 9
    q, kv, idx, sc = _kl_inputs(21, T, N, H, D, k)
    kl, mag = ora.indexer_kl_rows(q, kv, idx, sc, 0.3)
    for t in range(T):
        valid = idx[t] >= 0
        p = _head_avg_attention(q[t], kv, idx[t][valid], 0.3)
        pi = torch.softmax(torch.from_numpy(sc[t][valid]), dim=0).numpy()
        ref = scipy.stats.entropy(p, pi)
        assert abs(kl[t] - ref) <= 1e-12 * max(1.0, abs(ref))
        assert kl[t] >= 0.0 and mag[t] >= kl[t] - 1e-15


def test_indexer_kl_zero_when_scores_are_the_logits(ora):
    """One head whose logits are the index scores: p = pi, so the loss is 0."""
    T, N, D, k = 6, 30, 16, 8
    q, kv, idx, _ = _kl_inputs(22, T, N, 1, D, k)
    sc = np.zeros((T, k))
    for t in range(T):
        valid = idx[t] >= 0
        sc[t, valid] = (0.4 * (kv[torch.from_numpy(idx[t][valid]).long()] @ q[t, 0])).numpy()
        sc[t, ~valid] = np.nan  # ignored entries
    kl, mag = ora.indexer_kl_rows(q, kv, idx, sc, 0.4)
    assert np.all(np.abs(kl) < 1e-13) and np.all(mag < 1e-12)


def test_indexer_kl_two_entries_is_bernoulli_kl(ora):
    """Two entries and one head: KL of two Bernoulli distributions, closed form."""
    q, kv, _, _ = _kl_inputs(23, 1, 5, 1, 10, 4, q_std=2.0)
    idx = np.array([[3, -1, 1, -1]], np.int32)
    sc = np.array([[0.7, 5.0, -1.3, 9.0]])
    kl, _ = ora.indexer_kl_rows(q, kv, idx, sc, 0.5)
    z3, z1 = (0.5 * (kv[3] @ q[0, 0])).item(), (0.5 * (kv[1] @ q[0, 0])).item()
    p = 1.0 / (1.0 + math.exp(z1 - z3))
    pi = 1.0 / (1.0 + math.exp(-1.3 - 0.7))
    ref = p * math.log(p / pi) + (1 - p) * math.log((1 - p) / (1 - pi))
    assert abs(kl[0] - ref) <= 1e-13


def test_indexer_kl_uniform_indexer_is_log_m_minus_entropy(ora):
    """Equal index scores: KL(p || uniform) = log m - entropy(p)."""
    import scipy.stats
    T, N, H, D, k = 5, 50, 4, 8, 12
    q, kv, idx, _ = _kl_inputs(24, T, N, H, D, k, q_std=3.0)
    sc = np.full((T, k), 1.25)
    kl, _ = ora.indexer_kl_rows(q, kv, idx, sc, 0.2)
    for t in range(T):
        valid = idx[t] >= 0
        p = _head_avg_attention(q[t], kv, idx[t][valid], 0.2)
        ref = math.log(valid.sum()) - scipy.stats.entropy(p)
        assert abs(kl[t] - ref) <= 1e-12


def test_indexer_kl_invariances(ora):
    """Shifting every score by a constant, permuting the entries together with
    their scores, appending padding, and duplicating every head change nothing;
    an empty selection gives 0."""
    T, N, H, D, k = 6, 40, 2, 10, 7
    q, kv, idx, sc = _kl_inputs(25, T, N, H, D, k)
    kl, _ = ora.indexer_kl_rows(q, kv, idx, sc, 0.3)
    kl_shift, _ = ora.indexer_kl_rows(q, kv, idx, sc + 17.5, 0.3)
    np.testing.assert_allclose(kl_shift, kl, rtol=1e-11, atol=1e-13)
    perm = synth.permutation(25, 99, k).numpy()
    kl_perm, _ = ora.indexer_kl_rows(q, kv, idx[:, perm], sc[:, perm], 0.3)
    np.testing.assert_allclose(kl_perm, kl, rtol=1e-11, atol=1e-13)
    idx_pad = np.concatenate([idx, np.full((T, 5), -1, np.int32)], axis=1)
    sc_pad = np.concatenate([sc, np.full((T, 5), 1e9)], axis=1)
    kl_pad, _ = ora.indexer_kl_rows(q, kv, idx_pad, sc_pad, 0.3)
    np.testing.assert_allclose(kl_pad, kl, rtol=1e-13, atol=0)
    kl_dup, _ = ora.indexer_kl_rows(torch.cat([q, q], dim=1), kv, idx, sc, 0.3)
    np.testing.assert_allclose(kl_dup, kl, rtol=1e-11, atol=1e-13)
    kl_empty, mag_empty = ora.indexer_kl_rows(q[:1], kv, np.full((1, k), -1, np.int32), sc[:1], 0.3)
    assert kl_empty[0] == 0.0 and mag_empty[0] == 0.0
