"""Pins of the backward oracles (sparse MLA; the indexer's KL loss), on the CPU.

Each gradient is checked against something other than its own formula:
  * central finite differences through the oracle's forward functions
    (ora_sparse_mla_rows; ora_indexer_rows followed by ora_indexer_kl_rows),
  * torch autograd in fp64 on a plain gather / softmax / matmul formulation,
  * closed forms and invariants (zero upstream gradient, identical rows,
    score gradients that sum to zero per token, unselected rows).
"""
import numpy as np
import pytest
import torch

import synth


def _mla_case(seed=1, T=5, H=3, N=40, k=12, Dqk=24, Dv=16):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(T, H, Dqk))
    kv = rng.normal(size=(N, Dqk)) * 0.5
    dout = rng.normal(size=(T, H, Dv))
    idx = np.stack([rng.permutation(N - 1)[:k] for _ in range(T)]).astype(np.int32)  # row N-1 never selected
    idx[1, k // 2:] = -1          # ragged
    idx[2, :] = -1                # empty
    idx[3, 3] = idx[3, 0]         # one row listed twice in a selection
    idx[4, :4] = idx[0, :4]       # rows shared between queries
    return q, kv, dout, idx, 0.37


def _mla_loss(ora, q, kv, dout, idx, sm):
    o, _ = ora.sparse_mla_rows(q, kv, idx, sm, Dv=dout.shape[2])
    return float((o * dout).sum())


def test_mla_bwd_matches_finite_differences(ora):
    q, kv, dout, idx, sm = _mla_case()
    g = ora.sparse_mla_bwd(q, kv, idx, dout, sm, Dv=16)
    rng = np.random.default_rng(7)
    eps = 1e-6
    for _ in range(12):
        t, h, d = rng.integers(q.shape[0]), rng.integers(q.shape[1]), rng.integers(q.shape[2])
        qp, qm = q.copy(), q.copy()
        qp[t, h, d] += eps
        qm[t, h, d] -= eps
        fd = (_mla_loss(ora, qp, kv, dout, idx, sm) - _mla_loss(ora, qm, kv, dout, idx, sm)) / (2 * eps)
        assert abs(fd - g["dq"][t, h, d]) <= 1e-6 * max(1.0, abs(fd)), (t, h, d, fd, g["dq"][t, h, d])
    rows = np.unique(idx[idx >= 0])
    for r in list(rng.choice(rows, 6, replace=False)) + [int(idx[3, 0])]:
        for d in (0, 5, 15, 16, 23):     # value dims and logit-only dims
            kp, km = kv.copy(), kv.copy()
            kp[r, d] += eps
            km[r, d] -= eps
            fd = (_mla_loss(ora, q, kp, dout, idx, sm) - _mla_loss(ora, q, km, dout, idx, sm)) / (2 * eps)
            assert abs(fd - g["dkv"][r, d]) <= 1e-6 * max(1.0, abs(fd)), (r, d, fd, g["dkv"][r, d])
    assert np.all(g["dkv"][kv.shape[0] - 1] == 0)        # never selected
    assert np.all(g["dq"][2] == 0)                       # nothing selected


def test_mla_bwd_matches_torch_autograd(ora):
    q, kv, dout, idx, sm = _mla_case(seed=2)
    g = ora.sparse_mla_bwd(q, kv, idx, dout, sm, Dv=16)
    qt = torch.tensor(q, requires_grad=True)
    kvt = torch.tensor(kv, requires_grad=True)
    loss = torch.zeros((), dtype=torch.float64)
    for t in range(q.shape[0]):
        sel = torch.tensor(idx[t][idx[t] >= 0], dtype=torch.long)
        if sel.numel() == 0:
            continue
        c = kvt[sel]                                    # [m, Dqk]
        p = torch.softmax(sm * qt[t] @ c.T, dim=-1)      # [H, m]
        o = p @ c[:, :16]                                # [H, Dv]
        loss = loss + (o * torch.tensor(dout[t])).sum()
    loss.backward()
    np.testing.assert_allclose(g["dq"], qt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dkv"], kvt.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_mla_bwd_closed_forms(ora):
    q, kv, dout, idx, sm = _mla_case(seed=3)
    z = ora.sparse_mla_bwd(q, kv, idx, np.zeros_like(dout), sm, Dv=16)
    assert np.all(z["dq"] == 0) and np.all(z["dkv"] == 0)
    # every selected row identical: the softmax is uniform whatever q is, so dq = 0,
    # and each selected row's value gradient is sum over its selections of dout / m
    kv1 = np.tile(kv[:1], (kv.shape[0], 1))
    g = ora.sparse_mla_bwd(q, kv1, idx, dout, sm, Dv=16)
    np.testing.assert_allclose(g["dq"], 0, atol=1e-12)
    expect = np.zeros((kv.shape[0], 16))
    for t in range(q.shape[0]):
        sel = idx[t][idx[t] >= 0]
        for r in sel:
            expect[r] += dout[t].sum(axis=0) / len(sel)
    np.testing.assert_allclose(g["dkv"][:, :16], expect, rtol=1e-12, atol=1e-12)
    # and the logit-only dims of dkv: s * dz * q with dz = P (dP - D) = 0 for identical rows
    np.testing.assert_allclose(g["dkv"][:, 16:], 0, atol=1e-12)
    assert np.all(g["mag_dkv"] >= np.abs(g["dkv"]) - 1e-12) and np.all(g["mag_dq"] >= np.abs(g["dq"]) - 1e-12)


def _kl_case(seed=4, T=6, H=4, N=50, k=14, Dqk=20, H_I=3, D_I=8):
    rng = np.random.default_rng(seed)
    q_att = rng.normal(size=(T, H, Dqk))
    kv = rng.normal(size=(N, Dqk)) * 0.4
    q_idx = rng.normal(size=(T, H_I, D_I))
    k_idx = rng.normal(size=(N, D_I))
    w = rng.integers(-40, 41, size=(T, H_I)) / 64.0    # exact in fp32, so +-2^-8 is exact too
    idx = np.stack([np.sort(rng.permutation(N - 1)[:k]) for _ in range(T)]).astype(np.int32)
    idx[1, k - 5:] = -1
    idx[2, :] = -1
    idx[4, :5] = idx[0, :5]
    dkl = rng.uniform(0.5, 1.5, size=T)
    return q_att, kv, q_idx, k_idx, w, idx, dkl, 0.3


def _kl_loss(ora, q_att, kv, q_idx, k_idx, w, idx, dkl, sm):
    T = q_idx.shape[0]
    pos = np.full(T, k_idx.shape[0] - 1, np.int32)
    sc_full = ora.indexer_rows(q_idx, k_idx, w, pos)
    sc = np.take_along_axis(sc_full, np.maximum(idx, 0).astype(np.int64), axis=1)
    kl, _ = ora.indexer_kl_rows(q_att, kv, idx, sc, sm)
    return float((kl * dkl).sum())


def test_kl_bwd_matches_finite_differences(ora):
    q_att, kv, q_idx, k_idx, w, idx, dkl, sm = _kl_case()
    g = ora.indexer_kl_bwd(q_att, kv, q_idx, k_idx, w, idx, dkl, sm)
    rng = np.random.default_rng(9)
    eps = 1e-6
    for _ in range(10):
        t, j, d = rng.integers(q_idx.shape[0]), rng.integers(q_idx.shape[1]), rng.integers(q_idx.shape[2])
        qp, qm = q_idx.copy(), q_idx.copy()
        qp[t, j, d] += eps
        qm[t, j, d] -= eps
        fd = (_kl_loss(ora, q_att, kv, qp, k_idx, w, idx, dkl, sm) -
              _kl_loss(ora, q_att, kv, qm, k_idx, w, idx, dkl, sm)) / (2 * eps)
        assert abs(fd - g["dq"][t, j, d]) <= 1e-6 * max(1.0, abs(fd)), (t, j, d, fd, g["dq"][t, j, d])
    for r in list(np.unique(idx[idx >= 0])[:5]) + [int(idx[0, 0])]:
        for d in (0, 3, 7):
            kp, km = k_idx.copy(), k_idx.copy()
            kp[r, d] += eps
            km[r, d] -= eps
            fd = (_kl_loss(ora, q_att, kv, q_idx, kp, w, idx, dkl, sm) -
                  _kl_loss(ora, q_att, kv, q_idx, km, w, idx, dkl, sm)) / (2 * eps)
            assert abs(fd - g["dk"][r, d]) <= 1e-6 * max(1.0, abs(fd)), (r, d, fd, g["dk"][r, d])
    # w goes through the fp32 score path: steps of 2^-8 keep it exact; central differences
    # then carry an O(eps^2) truncation term
    h = 2.0 ** -8
    for t, j in ((0, 0), (3, 2), (4, 1)):
        wp, wm = w.copy(), w.copy()
        wp[t, j] += h
        wm[t, j] -= h
        fd = (_kl_loss(ora, q_att, kv, q_idx, k_idx, wp, idx, dkl, sm) -
              _kl_loss(ora, q_att, kv, q_idx, k_idx, wm, idx, dkl, sm)) / (2 * h)
        assert abs(fd - g["dw"][t, j]) <= 1e-3 * max(1.0, abs(fd)), (t, j, fd, g["dw"][t, j])
    assert np.all(g["dk"][k_idx.shape[0] - 1] == 0) and np.all(g["dq"][2] == 0) and np.all(g["dw"][2] == 0)


def test_kl_bwd_matches_torch_autograd(ora):
    q_att, kv, q_idx, k_idx, w, idx, dkl, sm = _kl_case(seed=5)
    g = ora.indexer_kl_bwd(q_att, kv, q_idx, k_idx, w, idx, dkl, sm)
    qt = torch.tensor(q_idx, requires_grad=True)
    kt = torch.tensor(k_idx, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    loss = torch.zeros((), dtype=torch.float64)
    score_grads = []
    for t in range(q_idx.shape[0]):
        sel = torch.tensor(idx[t][idx[t] >= 0], dtype=torch.long)
        if sel.numel() == 0:
            score_grads.append(None)
            continue
        with torch.no_grad():   # the target is detached
            p = torch.softmax(sm * torch.tensor(q_att[t]) @ torch.tensor(kv)[sel].T, dim=-1).mean(0)
        x = qt[t] @ kt[sel].T                          # [H_I, m]
        scores = (wt[t][:, None] * torch.relu(x)).sum(0)
        scores.retain_grad()
        kl = (p * (torch.log(p) - torch.log_softmax(scores, dim=0))).sum()
        loss = loss + dkl[t] * kl
        score_grads.append(scores)
    loss.backward()
    np.testing.assert_allclose(g["dq"], qt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dk"], kt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dw"], wt.grad.numpy(), rtol=1e-10, atol=1e-12)
    for t, s in enumerate(score_grads):
        if s is not None:
            valid = idx[t] >= 0
            np.testing.assert_allclose(g["g"][t][valid], s.grad.numpy(), rtol=1e-10, atol=1e-13)


def test_kl_bwd_score_gradient_sums_to_zero_and_vanishes_at_the_target(ora):
    q_att, kv, q_idx, k_idx, w, idx, dkl, sm = _kl_case(seed=6)
    g = ora.indexer_kl_bwd(q_att, kv, q_idx, k_idx, w, idx, dkl, sm)
    np.testing.assert_allclose(g["g"].sum(axis=1), 0, atol=1e-13)   # pi and p both sum to one
    assert np.all(g["g"][idx < 0] == 0)
    # one attention head whose logits equal the index scores: p = pi, so every gradient is zero.
    # With H_I = 1, w = 1 and non-negative keys and queries, I = x = q_idx . k_idx; the attention
    # reproduces it with q_att = q_idx / sm and kv = k_idx.
    rng = np.random.default_rng(11)
    T, N, D = 4, 30, 8
    qi = np.abs(rng.normal(size=(T, 1, D)))
    ki = np.abs(rng.normal(size=(N, D)))
    sel = np.stack([np.sort(rng.permutation(N)[:10]) for _ in range(T)]).astype(np.int32)
    z = ora.indexer_kl_bwd(qi / sm, ki, qi, ki, np.ones((T, 1)), sel, np.ones(T), sm)
    for key in ("g", "dw", "dq", "dk"):
        np.testing.assert_allclose(z[key], 0, atol=1e-12)


def test_kl_bwd_e4m3_equals_dequantised_f64(ora):
    """E4M3 payloads with scales give the gradients of the dequantised values."""
    cfg = synth.scaled_down(synth.CONFIGS["prefill16k"], L=40, k=16, H=4, H_I=64)
    q_i, k_i, w = synth.prefill_indexer_inputs(cfg)
    q8, qs = ora.quantize_rows(q_i.view(40, -1).numpy())
    k8, ks = ora.quantize_rows(k_i.numpy())
    q8 = q8.reshape(40, 64, 128)
    rng = np.random.default_rng(3)
    q_att = rng.normal(size=(40, 4, 24))
    kv = rng.normal(size=(40, 24)) * 0.3
    idx = np.stack([np.sort(rng.permutation(t + 1)[:16]) if t + 1 >= 16 else
                    np.concatenate([np.arange(t + 1), -np.ones(15 - t)]) for t in range(40)]).astype(np.int32)
    dkl = np.ones(40)
    a = ora.indexer_kl_bwd(q_att, kv, q8, k8, w.numpy().astype(np.float64), idx, dkl, 0.2, q_scale=qs, k_scale=ks)
    qd = ora.e4m3_decode(q8) * qs.astype(np.float64)[:, None, None]
    kd = ora.e4m3_decode(k8) * ks.astype(np.float64)[:, None]
    b = ora.indexer_kl_bwd(q_att, kv, qd, kd, w.numpy().astype(np.float64), idx, dkl, 0.2)
    for key in ("g", "dw", "dq", "dk"):
        np.testing.assert_allclose(a[key], b[key], rtol=1e-12, atol=1e-15)


def test_kl_bwd_is_the_composition_of_its_two_steps(ora):
    """ora_indexer_kl_bwd = index scores -> ora_indexer_kl_grad -> ora_indexer_bwd."""
    q_att, kv, q_idx, k_idx, w, idx, dkl, sm = _kl_case(seed=8)
    a = ora.indexer_kl_bwd(q_att, kv, q_idx, k_idx, w, idx, dkl, sm)
    pos = np.full(q_idx.shape[0], k_idx.shape[0] - 1, np.int32)
    sc = np.take_along_axis(ora.indexer_rows(q_idx, k_idx, w, pos), np.maximum(idx, 0).astype(np.int64), axis=1)
    g = ora.indexer_kl_grad(q_att, kv, idx, sc, dkl, sm)
    np.testing.assert_allclose(g, a["g"], rtol=1e-12, atol=1e-15)
    b = ora.indexer_bwd(q_idx, k_idx, w, idx, g)
    for key in ("dw", "dq", "dk"):
        np.testing.assert_allclose(b[key], a[key], rtol=1e-12, atol=1e-15)
