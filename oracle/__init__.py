"""fp64 CPU oracle for the DSA hot path (ctypes wrapper over dsa_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the GPU library or its binding.  It shares
no code with the GPU path; both sides draw their inputs from ``synth``.

Functions follow the plain definitions written out in dsa_oracle.c:
  * e4m3/bf16 codecs and per-row E4M3 quantisation,
  * indexer scores  I[t,s] = sum_j w[t,j] ReLU((qs q[t,j]) . (ks k[s]))  for s <= pos(t),
  * top-k under (score desc, position desc),
  * sparse MLA-MQA attention over the selected latent rows,
  * masked multi-head attention in MLA's multi-head form (short-prefill mode),
  * the indexer's KL-alignment loss per query token,
  * one paged decode query per sequence,
  * the paged cache append of one new token per sequence,
  * the backward of sparse MLA (dq, dkv) and of the indexer's KL loss
    (the score gradient, then dw, dq_I, dk_I).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, E4M3, F64 = 0, 1, 2, 3


def build(force: bool = False) -> str:
    """Compile dsa_oracle.c with gcc (OpenMP) into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                               "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, dbl = ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        L.ora_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.ora_e4m3_decode.restype = dbl
        L.ora_bf16_decode.argtypes = [ctypes.c_uint16]
        L.ora_bf16_decode.restype = dbl
        L.ora_e4m3_encode.argtypes = [ctypes.c_float]
        L.ora_e4m3_encode.restype = ctypes.c_uint8
        L.ora_quantize_rows.argtypes = [P, i64, i32, P, P]
        L.ora_indexer_rows.argtypes = [ctypes.c_int, P, P, P, P, P, P, i64, i64, i32, i32, P, i64, P]
        L.ora_topk_row.argtypes = [P, i64, i32, P, P]
        L.ora_topk_row.restype = i64
        L.ora_topk_rows.argtypes = [P, i64, P, i64, i32, P, P]
        L.ora_sparse_mla_rows.argtypes = [ctypes.c_int, P, P, P, i64, i32, i64, i32, i32, i32, dbl,
                                          P, i64, P, P]
        L.ora_masked_mha_rows.argtypes = [ctypes.c_int, P, P, P, P, P, i32, i32, i32, i32, i32, i32, dbl,
                                          P, i64, P, P]
        L.ora_indexer_kl_rows.argtypes = [ctypes.c_int, P, P, P, P, i32, i32, i32, dbl, P, i64, P, P]
        L.ora_decode.argtypes = [P, P, P, P, P, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, i32,
                                 dbl, P, i64, P, P, P, P]
        L.ora_paged_cache_append.argtypes = [P, P, P, P, i32, i32, i32, P, i32, i64, P, P, P]
        L.ora_sparse_mla_bwd.argtypes = [ctypes.c_int, P, P, P, P, i64, i32, i64, i32, i32, i32, dbl,
                                         P, P, P, P]
        L.ora_indexer_kl_bwd.argtypes = [ctypes.c_int, P, P, ctypes.c_int, P, P, P, P, P, P, P, i64, i64, i32,
                                         i32, i32, i32, i32, dbl, P, P, P, P, P, P, P, P, P, dbl]
        L.ora_indexer_kl_grad.argtypes = [ctypes.c_int, P, P, P, P, P, i64, i32, i32, i32, dbl, P]
        L.ora_indexer_bwd.argtypes = [ctypes.c_int, P, P, P, P, P, P, P, i64, i64, i32, i32, i32, P, P, P, P, P, P,
                                      P, P, dbl]
        _lib = L
    return _lib


def _np(x, dtype=None):
    """torch tensor or array -> contiguous numpy array (bf16 as raw uint16)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                x = x.view(torch.int16)
            x = x.numpy()
            if x.dtype == np.int16:
                x = x.view(np.uint16)
    except ImportError:
        pass
    x = np.ascontiguousarray(x)
    if dtype is not None and x.dtype != dtype:
        x = np.ascontiguousarray(x.astype(dtype))
    return x


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint8:
        return E4M3
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"unsupported dtype {a.dtype}")


# ---------------------------------------------------------------- codecs
def e4m3_decode(codes) -> np.ndarray:
    c = _np(codes, np.uint8)
    L = lib()
    return np.array([L.ora_e4m3_decode(int(v)) for v in c.ravel()], dtype=np.float64).reshape(c.shape)


def e4m3_encode(x) -> np.ndarray:
    a = _np(x, np.float32)
    L = lib()
    return np.array([L.ora_e4m3_encode(float(v)) for v in a.ravel()], dtype=np.uint8).reshape(a.shape)


def bf16_decode(bits) -> np.ndarray:
    b = _np(bits, np.uint16)
    L = lib()
    return np.array([L.ora_bf16_decode(int(v)) for v in b.ravel()], dtype=np.float64).reshape(b.shape)


def quantize_rows(x):
    """fp32 [..., cols] -> (E4M3 payload uint8 [..., cols], fp32 scale [...])."""
    a = _np(x, np.float32)
    cols = a.shape[-1]
    rows = a.size // cols
    x8 = np.empty(a.shape, dtype=np.uint8)
    sc = np.empty(a.shape[:-1], dtype=np.float32)
    lib().ora_quantize_rows(_p(a), rows, cols, _p(x8), _p(sc))
    return x8, sc


# ---------------------------------------------------------------- indexer
def indexer_rows(q, k, w, q_pos, rows=None, q_scale=None, k_scale=None, S=None):
    """Index scores for query rows ``rows`` (default all) -> float64 [n, S].

    q [T, H_I, D_I] and k [S, D_I] are either fp32 arrays, or E4M3 payloads
    (uint8) with fp32 q_scale [T] and k_scale [S].
    """
    q, k, w = _np(q), _np(k), _np(w, np.float32)
    dt = _dtype_code(q)
    assert _dtype_code(k) == dt
    T, H_I, D_I = q.shape
    S = k.shape[0] if S is None else S
    pos = _np(q_pos, np.int32)
    rows = np.arange(T, dtype=np.int64) if rows is None else _np(rows, np.int64)
    qs = _np(q_scale, np.float32) if q_scale is not None else np.ones(T, np.float32)
    ks = _np(k_scale, np.float32) if k_scale is not None else np.ones(k.shape[0], np.float32)
    out = np.empty((len(rows), S), dtype=np.float64)
    lib().ora_indexer_rows(dt, _p(q), _p(qs), _p(k), _p(ks), _p(w), _p(pos), T, S, H_I, D_I,
                           _p(rows), len(rows), _p(out))
    return out


# ------------------------------------------------------------------ top-k
def topk_row(scores, k):
    """-> (idx int32 [k] ascending then -1, K, tau)."""
    s = _np(scores, np.float64)
    idx = np.empty(k, dtype=np.int32)
    tau = ctypes.c_double()
    K = lib().ora_topk_row(_p(s), s.shape[0], k, _p(idx), ctypes.byref(tau))
    return idx, int(K), tau.value


def topk_rows(scores, n_valid, k):
    """scores [n, ld] float64, n_valid [n] -> (idx int32 [n, k], tau [n])."""
    s = _np(scores, np.float64)
    nv = _np(n_valid, np.int64)
    idx = np.empty((s.shape[0], k), dtype=np.int32)
    tau = np.empty(s.shape[0], dtype=np.float64)
    lib().ora_topk_rows(_p(s), s.shape[1], _p(nv), s.shape[0], k, _p(idx), _p(tau))
    return idx, tau


# ------------------------------------------------------------- sparse MLA
def sparse_mla_rows(q, kv, idx, sm_scale, rows=None, Dv=512):
    """q [T, H, Dqk], kv [N, Dqk] (fp32 or bf16), idx [T, k] -> (o [n,H,Dv], lse [n,H]) fp64."""
    q, kv, idx = _np(q), _np(kv), _np(idx, np.int32)
    dt = _dtype_code(q)
    assert _dtype_code(kv) == dt and dt in (F32, BF16, F64)
    T, H, Dqk = q.shape
    N = kv.shape[0]
    k = idx.shape[1]
    rows = np.arange(T, dtype=np.int64) if rows is None else _np(rows, np.int64)
    o = np.empty((len(rows), H, Dv), dtype=np.float64)
    lse = np.empty((len(rows), H), dtype=np.float64)
    lib().ora_sparse_mla_rows(dt, _p(q), _p(kv), _p(idx), T, H, N, k, Dqk, Dv, float(sm_scale),
                              _p(rows), len(rows), _p(o), _p(lse))
    return o, lse


def masked_mha_rows(q, kv, w_uk, w_uv, idx, sm_scale, rows=None, Dr=64):
    """Masked MHA in MLA's multi-head form.  q [T, H, Dn+Dr], kv [N, Dc+Dr],
    w_uk [H, Dn, Dc], w_uv [H, Dvh, Dc] (all fp32, bf16 or fp64, one dtype),
    idx [T, k] -> (o [n, H, Dvh], lse [n, H]) fp64."""
    q, kv, w_uk, w_uv, idx = _np(q), _np(kv), _np(w_uk), _np(w_uv), _np(idx, np.int32)
    dt = _dtype_code(q)
    assert all(_dtype_code(a) == dt for a in (kv, w_uk, w_uv)) and dt in (F32, BF16, F64)
    T, H, Dq = q.shape
    Hw, Dn, Dc = w_uk.shape
    Dvh = w_uv.shape[1]
    assert Hw == H and w_uv.shape == (H, Dvh, Dc) and Dn + Dr == Dq and kv.shape[1] == Dc + Dr
    k = idx.shape[1]
    rows = np.arange(T, dtype=np.int64) if rows is None else _np(rows, np.int64)
    o = np.empty((len(rows), H, Dvh), dtype=np.float64)
    lse = np.empty((len(rows), H), dtype=np.float64)
    lib().ora_masked_mha_rows(dt, _p(q), _p(kv), _p(w_uk), _p(w_uv), _p(idx), H, k, Dc, Dr, Dn, Dvh,
                              float(sm_scale), _p(rows), len(rows), _p(o), _p(lse))
    return o, lse


def indexer_kl_rows(q, kv, idx, scores, sm_scale, rows=None):
    """Per-token KL(p || pi) of the indexer against the head-averaged main
    attention over the valid entries of idx.  q [T, H, Dqk], kv [N, Dqk]
    (fp32, bf16 or fp64, one dtype), idx [T, k], scores [T, k] (index scores
    of the entries) -> (kl [n], mag [n]) fp64, mag = sum_a p_a |log p_a - log pi_a|."""
    q, kv, idx, sc = _np(q), _np(kv), _np(idx, np.int32), _np(scores, np.float64)
    dt = _dtype_code(q)
    assert _dtype_code(kv) == dt and dt in (F32, BF16, F64)
    T, H, Dqk = q.shape
    k = idx.shape[1]
    assert sc.shape == idx.shape and kv.shape[1] == Dqk
    rows = np.arange(T, dtype=np.int64) if rows is None else _np(rows, np.int64)
    kl = np.empty(len(rows), dtype=np.float64)
    mag = np.empty(len(rows), dtype=np.float64)
    lib().ora_indexer_kl_rows(dt, _p(q), _p(kv), _p(idx), _p(sc), H, k, Dqk, float(sm_scale), _p(rows), len(rows),
                              _p(kl), _p(mag))
    return kl, mag


# ------------------------------------------------------------------ decode
def decode(q8, qs, w, q, k8_pool, ks_pool, kv_pool, block_table, ctx, k, sm_scale, seqs=None,
           Dv=512):
    """Paged decode for sequences ``seqs`` -> (idx [n,k] logical, tau [n], o [n,H,Dv], lse [n,H])."""
    q8, qs, w, q = _np(q8, np.uint8), _np(qs, np.float32), _np(w, np.float32), _np(q)
    k8p, ksp, kvp = _np(k8_pool, np.uint8), _np(ks_pool, np.float32), _np(kv_pool)
    bt, ctx = _np(block_table, np.int32), _np(ctx, np.int32)
    assert q.dtype == np.uint16 and kvp.dtype == np.uint16
    B, H_I, D_I = q8.shape
    H, Dqk = q.shape[1], q.shape[2]
    seqs = np.arange(B, dtype=np.int64) if seqs is None else _np(seqs, np.int64)
    n = len(seqs)
    idx = np.empty((n, k), dtype=np.int32)
    tau = np.empty(n, dtype=np.float64)
    o = np.empty((n, H, Dv), dtype=np.float64)
    lse = np.empty((n, H), dtype=np.float64)
    lib().ora_decode(_p(q8), _p(qs), _p(w), _p(q), _p(k8p), _p(ksp), _p(kvp), _p(bt), bt.shape[1],
                     _p(ctx), B, H_I, D_I, H, k, Dqk, Dv, float(sm_scale), _p(seqs), n, _p(idx),
                     _p(tau), _p(o), _p(lse))
    return idx, tau, o, lse


def paged_cache_append(latent, k8, ks, pos, block_table, kv_pool, k8_pool, ks_pool):
    """Write token b (latent [B, Dqk] bf16, k8 [B, D_I] E4M3, ks [B] fp32) at
    logical position pos[b] of sequence b into copies of the pools (kv
    [n, Dqk] bf16 bits, k8 [n, D_I] u8, ks [n] f32; any leading shape that
    flattens to rows) -> the three updated pools (numpy)."""
    lat, k8, ks = _np(latent), _np(k8, np.uint8), _np(ks, np.float32)
    assert lat.dtype == np.uint16
    pos, bt = _np(pos, np.int32), _np(block_table, np.int32)
    kvp = np.array(_np(kv_pool), copy=True)
    k8p = np.array(_np(k8_pool, np.uint8), copy=True)
    ksp = np.array(_np(ks_pool, np.float32), copy=True)
    B, Dqk = lat.shape
    D_I = k8.shape[1]
    n_rows = ksp.size
    assert kvp.size == n_rows * Dqk and k8p.size == n_rows * D_I and bt.shape[0] == B
    lib().ora_paged_cache_append(_p(lat), _p(k8), _p(ks), _p(pos), B, D_I, Dqk, _p(bt), bt.shape[1], n_rows,
                                 _p(kvp), _p(k8p), _p(ksp))
    return kvp, k8p, ksp


# ------------------------------------------------------------------ backward
def sparse_mla_bwd(q, kv, idx, dout, sm_scale, Dv=512):
    """q [T,H,Dqk], kv [N,Dqk], dout [T,H,Dv] (one dtype: f32, bf16 or f64),
    idx [T,k] -> dict of fp64 arrays: dq [T,H,Dqk], dkv [N,Dqk], and the
    rounding magnitudes mag_dq, mag_dkv of the same shapes."""
    q, kv, idx, dout = _np(q), _np(kv), _np(idx, np.int32), _np(dout)
    dt = _dtype_code(q)
    assert _dtype_code(kv) == dt and _dtype_code(dout) == dt and dt in (F32, BF16, F64)
    T, H, Dqk = q.shape
    N = kv.shape[0]
    k = idx.shape[1]
    assert dout.shape == (T, H, Dv)
    dq = np.empty((T, H, Dqk)); mdq = np.empty((T, H, Dqk))
    dkv = np.empty((N, Dqk)); mdkv = np.empty((N, Dqk))
    lib().ora_sparse_mla_bwd(dt, _p(q), _p(kv), _p(idx), _p(dout), T, H, N, k, Dqk, Dv, float(sm_scale),
                             _p(dq), _p(dkv), _p(mdq), _p(mdkv))
    return {"dq": dq, "dkv": dkv, "mag_dq": mdq, "mag_dkv": mdkv}


def indexer_kl_grad(q_att, kv, idx, scores, dkl, sm_scale):
    """Gradient of sum_t dkl[t] KL_t with respect to the given index scores
    [T, k]: g = dkl (softmax(scores) - p) at the valid entries, 0 elsewhere."""
    q_att, kv = _np(q_att), _np(kv)
    at = _dtype_code(q_att)
    assert _dtype_code(kv) == at and at in (F32, BF16, F64)
    idx, sc, dkl = _np(idx, np.int32), _np(scores, np.float64), _np(dkl, np.float64)
    T, H, Dqk = q_att.shape
    k = idx.shape[1]
    g = np.empty((T, k))
    lib().ora_indexer_kl_grad(at, _p(q_att), _p(kv), _p(idx), _p(sc), _p(dkl), T, H, k, Dqk, float(sm_scale), _p(g))
    return g


def indexer_bwd(q_idx, k_idx, w, idx, g, q_scale=None, k_scale=None, kink_rel=None):
    """The indexer's gradients from a score gradient g [T, k] -> dict of fp64
    dw, dq, dk and mag_dw, mag_dq, mag_dk, amb_dq, amb_dk.  kink_rel: the
    relative accuracy of the evaluation being checked, which sets the width of
    the ambiguous band around the ReLU kink (default: an IEEE fp32 sum of D_I
    products, (D_I + 2) 2^-24)."""
    q_idx, k_idx = _np(q_idx), _np(k_idx)
    it = _dtype_code(q_idx)
    assert _dtype_code(k_idx) == it
    w, g, idx = _np(w, np.float64), _np(g, np.float64), _np(idx, np.int32)
    T, H_I, D_I = q_idx.shape
    N = k_idx.shape[0]
    k = idx.shape[1]
    qs = _np(q_scale, np.float32) if q_scale is not None else np.ones(T, np.float32)
    ks = _np(k_scale, np.float32) if k_scale is not None else np.ones(N, np.float32)
    out = {"dw": np.empty((T, H_I)), "dq": np.empty((T, H_I, D_I)), "dk": np.empty((N, D_I)),
           "mag_dw": np.empty((T, H_I)), "mag_dq": np.empty((T, H_I, D_I)), "mag_dk": np.empty((N, D_I)),
           "amb_dq": np.empty((T, H_I, D_I)), "amb_dk": np.empty((N, D_I))}
    lib().ora_indexer_bwd(it, _p(q_idx), _p(qs), _p(k_idx), _p(ks), _p(w), _p(idx), _p(g), T, N, H_I, D_I, k,
                          _p(out["dw"]), _p(out["dq"]), _p(out["dk"]), _p(out["mag_dw"]), _p(out["mag_dq"]),
                          _p(out["mag_dk"]), _p(out["amb_dq"]), _p(out["amb_dk"]), float(kink_rel or 0.0))
    return out


def indexer_kl_bwd(q_att, kv, q_idx, k_idx, w, idx, dkl, sm_scale, q_scale=None, k_scale=None, kink_rel=None):
    """Gradient of the per-token KL(p || pi) (weighted by dkl [T]) into the
    indexer.  q_att [T,H,Dqk], kv [N,Dqk] (f32, bf16 or f64); q_idx [T,H_I,D_I],
    k_idx [N,D_I] (E4M3 payloads with q_scale [T], k_scale [N], or f32/f64);
    w [T,H_I]; idx [T,k] rows of kv and k_idx.  -> dict of fp64 arrays
    g [T,k], dw [T,H_I], dq [T,H_I,D_I], dk [N,D_I], and mag_dw, mag_dq,
    mag_dk, amb_dq, amb_dk (see dsa_oracle.c); kink_rel as for indexer_bwd."""
    q_att, kv = _np(q_att), _np(kv)
    at = _dtype_code(q_att)
    assert _dtype_code(kv) == at and at in (F32, BF16, F64)
    q_idx, k_idx = _np(q_idx), _np(k_idx)
    it = _dtype_code(q_idx)
    assert _dtype_code(k_idx) == it
    w, dkl, idx = _np(w, np.float64), _np(dkl, np.float64), _np(idx, np.int32)
    T, H, Dqk = q_att.shape
    N = kv.shape[0]
    _, H_I, D_I = q_idx.shape
    k = idx.shape[1]
    assert k_idx.shape == (N, D_I) and w.shape == (T, H_I) and dkl.shape == (T,)
    qs = _np(q_scale, np.float32) if q_scale is not None else np.ones(T, np.float32)
    ks = _np(k_scale, np.float32) if k_scale is not None else np.ones(N, np.float32)
    out = {"g": np.empty((T, k)), "dw": np.empty((T, H_I)), "dq": np.empty((T, H_I, D_I)),
           "dk": np.empty((N, D_I)), "mag_dw": np.empty((T, H_I)), "mag_dq": np.empty((T, H_I, D_I)),
           "mag_dk": np.empty((N, D_I)), "amb_dq": np.empty((T, H_I, D_I)), "amb_dk": np.empty((N, D_I))}
    lib().ora_indexer_kl_bwd(at, _p(q_att), _p(kv), it, _p(q_idx), _p(qs), _p(k_idx), _p(ks), _p(w), _p(idx),
                             _p(dkl), T, N, H, H_I, D_I, k, Dqk, float(sm_scale), _p(out["g"]), _p(out["dw"]),
                             _p(out["dq"]), _p(out["dk"]), _p(out["mag_dw"]), _p(out["mag_dq"]), _p(out["mag_dk"]),
                             _p(out["amb_dq"]), _p(out["amb_dk"]), float(kink_rel or 0.0))
    return out
