"""Thin ctypes binding of libdsa (include/dsa.h), one function per C entry point.

Argument marshalling only: every step runs in the library's HIP kernels.
Tensors are torch device tensors (their data pointers are passed through);
work is enqueued on torch's current HIP stream unless ``stream`` is given.
A non-OK status raises DSAError carrying dsa_last_error().  There is no CPU
fallback: without a built libdsa.so, importing the library fails loudly.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = range(5)
DSA_F32, DSA_BF16, DSA_E4M3 = 0, 1, 2
STATUS_NAMES = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED", 3: "DSA_ERR_WORKSPACE",
                4: "DSA_ERR_HIP"}
EXPORTS = (
    "dsa_last_error", "dsa_version", "dsa_quantize_e4m3_per_token", "dsa_indexer_scores", "dsa_topk_select", "dsa_topk_workspace_bytes",
    "dsa_sparse_mla_workspace_bytes", "dsa_sparse_mla_fwd", "dsa_prefill_workspace_bytes", "dsa_prefill",
    "dsa_decode_workspace_bytes", "dsa_decode", "dsa_paged_cache_append", "dsa_prefill_select",
    "dsa_decode_indexer_scores", "dsa_sparse_mla_paged_fwd", "dsa_masked_mha_workspace_bytes",
    "dsa_masked_mha_prefill", "dsa_indexer_scores_at", "dsa_indexer_kl_fwd", "dsa_decode_static_scratch_bytes",
    "dsa_decode_noalloc", "dsa_indexer_kl_bwd", "dsa_indexer_bwd_workspace_bytes", "dsa_indexer_bwd",
    "dsa_sparse_mla_bwd_workspace_bytes", "dsa_sparse_mla_bwd", "dsa_sparse_mla_bwd_kl",
)


class DSAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_P = ctypes.c_void_p
_I32, _I64, _F32, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class PrefillArgs(ctypes.Structure):
    _fields_ = [("L", _I32), ("H_I", _I32), ("D_I", _I32), ("H", _I32), ("k", _I32),
                ("idx_dt", ctypes.c_int), ("q_idx", _P), ("q_scale", _P), ("k_idx", _P), ("k_scale", _P),
                ("w", _P), ("attn_dt", ctypes.c_int), ("q", _P), ("kv", _P), ("sm_scale", _F32),
                ("idx", _P), ("out", _P), ("lse", _P)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("B", _I32), ("H_I", _I32), ("D_I", _I32), ("H", _I32), ("k", _I32),
                ("q8", _P), ("q_scale", _P), ("w", _P), ("q", _P),
                ("k8_pool", _P), ("ks_pool", _P), ("kv_pool", _P), ("n_pool_rows", _I64),
                ("block_table", _P), ("max_blocks", _I32), ("ctx_len", _P), ("max_ctx", _I32),
                ("sm_scale", _F32), ("idx_out", _P), ("out", _P), ("lse", _P)]


_lib = None
F32_T, U8_T, I32_T = torch.float32, torch.uint8, torch.int32


def _check_fresh(L):
    """Refuse a library built from other sources than the ones beside it (a
    stale build would silently test old kernels).  Skipped when the sources
    are not present."""
    from . import build
    if not os.path.isdir(build.CSRC):
        return
    got = L.dsa_version().decode()
    want = build.source_hash()
    if not got.endswith("src=" + want):
        raise ImportError(f"libdsa.so is stale ({got}; sources are {want}); "
                          "rebuild with python -m sparse_attention_gemm_amd.build")


def load():
    """Load libdsa.so (built in-tree by sparse_attention_gemm_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libdsa.so not built ({LIB_PATH}); run python -m sparse_attention_gemm_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    L.dsa_last_error.restype = ctypes.c_char_p
    L.dsa_version.restype = ctypes.c_char_p
    _check_fresh(L)
    L.dsa_quantize_e4m3_per_token.argtypes = [_P, _I64, _I32, _P, _P, _P]
    L.dsa_indexer_scores.argtypes = [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, ctypes.c_int, _P, _I64, _P]
    L.dsa_topk_select.argtypes = [_P, _I64, _P, _I32, _I32, _P, _P, _SZ, _P]
    L.dsa_topk_workspace_bytes.argtypes = [_I32, _I64, _I32]
    L.dsa_topk_workspace_bytes.restype = _SZ
    L.dsa_sparse_mla_workspace_bytes.argtypes = [_I32, _I32, _I32]
    L.dsa_sparse_mla_workspace_bytes.restype = _SZ
    L.dsa_sparse_mla_fwd.argtypes = [_P, _P, ctypes.c_int, _P, _I32, _I32, _I64, _I32, _F32, _P, _P, _P, _SZ, _P]
    L.dsa_prefill_workspace_bytes.argtypes = [ctypes.POINTER(PrefillArgs)]
    L.dsa_prefill_workspace_bytes.restype = _SZ
    L.dsa_prefill.argtypes = [ctypes.POINTER(PrefillArgs), _P, _SZ, _P]
    L.dsa_decode_workspace_bytes.argtypes = [ctypes.POINTER(DecodeArgs)]
    L.dsa_decode_workspace_bytes.restype = _SZ
    L.dsa_decode.argtypes = [ctypes.POINTER(DecodeArgs), _P, _SZ, _P]
    L.dsa_decode_noalloc.argtypes = [ctypes.POINTER(DecodeArgs), _P]
    L.dsa_decode_static_scratch_bytes.argtypes = []
    L.dsa_decode_static_scratch_bytes.restype = _SZ
    L.dsa_paged_cache_append.argtypes = [_P, _P, _P, _P, _I32, _I32, _P, _I32, _P, _P, _P, _I64, _P]
    L.dsa_prefill_select.argtypes = [ctypes.POINTER(PrefillArgs), _P, _SZ, _P]
    L.dsa_decode_indexer_scores.argtypes = [ctypes.POINTER(DecodeArgs), _P, _I64, _P]
    L.dsa_sparse_mla_paged_fwd.argtypes = [_P, _P, _I64, _P, _I32, _P, _I32, _I32, _I32, _F32, _P, _P, _P, _SZ, _P]
    L.dsa_masked_mha_workspace_bytes.argtypes = [_I32, _I32]
    L.dsa_masked_mha_workspace_bytes.restype = _SZ
    L.dsa_masked_mha_prefill.argtypes = [_P, _P, _P, _P, _P, _I32, _I32, _I32, _F32, _P, _P, _P, _SZ, _P]
    L.dsa_indexer_scores_at.argtypes = [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P]
    L.dsa_indexer_kl_fwd.argtypes = [_P, _P, _P, _P, _P, _I32, _I32, _I64, _I32, _F32, _P, _P]
    L.dsa_indexer_kl_bwd.argtypes = [_P, _P, _P, _P, _P, _P, _I32, _I32, _I64, _I32, _F32, _P, _P]
    L.dsa_sparse_mla_bwd_workspace_bytes.argtypes = [_I32, _I32, _I64, _I32]
    L.dsa_sparse_mla_bwd_workspace_bytes.restype = _SZ
    L.dsa_sparse_mla_bwd.argtypes = [_P, _P, _P, _P, _P, _P, _I32, _I32, _I64, _I32, _F32, _P, _P, _P, _SZ, _P]
    L.dsa_sparse_mla_bwd_kl.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I64, _I32, _F32, _P, _P, _P, _P,
                                        _SZ, _P]
    L.dsa_indexer_bwd_workspace_bytes.argtypes = [_I32, _I32, _I32]
    L.dsa_indexer_bwd_workspace_bytes.restype = _SZ
    L.dsa_indexer_bwd.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _SZ, _P]
    for name in ("dsa_indexer_scores_at", "dsa_indexer_kl_fwd", "dsa_indexer_kl_bwd", "dsa_indexer_bwd", "dsa_sparse_mla_bwd", "dsa_sparse_mla_bwd_kl", "dsa_masked_mha_prefill", "dsa_quantize_e4m3_per_token", "dsa_indexer_scores", "dsa_topk_select", "dsa_sparse_mla_fwd",
                 "dsa_prefill", "dsa_decode", "dsa_decode_noalloc", "dsa_paged_cache_append", "dsa_prefill_select",
                 "dsa_decode_indexer_scores", "dsa_sparse_mla_paged_fwd"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _ptr(t, dtype=None, name="tensor"):
    """Device address of a torch tensor (ints pass through as raw addresses).
    The library reads tensors as dense, row-major device arrays: anything
    else is refused here, before its address reaches a kernel."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != DSA_OK:
        raise DSAError(status, load().dsa_last_error().decode())


def dsa_version() -> str:
    return load().dsa_version().decode()


def dsa_last_error() -> str:
    return load().dsa_last_error().decode()


def dsa_quantize_e4m3_per_token(x, x8, scale, rows=None, cols=None, stream=None):
    """x [rows, cols] fp32 -> x8 [rows, cols] uint8 (E4M3), scale [rows] fp32."""
    rows = x.numel() // x.shape[-1] if rows is None else rows
    cols = x.shape[-1] if cols is None else cols
    _check(load().dsa_quantize_e4m3_per_token(_ptr(x, F32_T, "x"), rows, cols, _ptr(x8, U8_T, "x8"),
                                              _ptr(scale, F32_T, "scale"), _stream(stream)))


def dsa_indexer_scores(q, q_scale, k, k_scale, w, q_pos, scores, dt, T=None, S=None, H_I=None, D_I=None,
                       ld_scores=None, stream=None):
    T = q.shape[0] if T is None else T
    S = k.shape[0] if S is None else S
    H_I = q.shape[1] if H_I is None else H_I
    D_I = q.shape[2] if D_I is None else D_I
    ld = scores.stride(0) if ld_scores is None else ld_scores
    qk_t = U8_T if dt == DSA_E4M3 else F32_T
    _check(load().dsa_indexer_scores(_ptr(q, qk_t, "q"), _ptr(q_scale, F32_T, "q_scale"), _ptr(k, qk_t, "k"),
                                     _ptr(k_scale, F32_T, "k_scale"), _ptr(w, F32_T, "w"), _ptr(q_pos, I32_T, "q_pos"),
                                     T, S, H_I, D_I, dt, _ptr(scores, F32_T, "scores"), ld, _stream(stream)))


def dsa_topk_select(scores, n_valid, k, idx, T=None, ld_scores=None, workspace=None, stream=None):
    T = scores.shape[0] if T is None else T
    ld = scores.stride(0) if ld_scores is None else ld_scores
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().dsa_topk_select(_ptr(scores, F32_T, "scores"), ld, _ptr(n_valid, I32_T, "n_valid"), T, k,
                                  _ptr(idx, I32_T, "idx"), _ptr(workspace, name="workspace"), ws_bytes,
                                  _stream(stream)))


def dsa_topk_workspace_bytes(T: int, ld_scores: int, k: int) -> int:
    return int(load().dsa_topk_workspace_bytes(T, ld_scores, k))


def dsa_sparse_mla_workspace_bytes(T: int, H: int, k: int) -> int:
    return int(load().dsa_sparse_mla_workspace_bytes(T, H, k))


def dsa_sparse_mla_fwd(q, kv, idx, sm_scale, out, lse=None, dt=None, workspace=None, N=None, stream=None):
    T, H = q.shape[0], q.shape[1]
    k = idx.shape[1]
    N = kv.shape[0] if N is None else N
    if dt is None:
        dt = DSA_BF16 if q.dtype == torch.bfloat16 else DSA_F32
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    at = torch.bfloat16 if dt == DSA_BF16 else torch.float32
    _check(load().dsa_sparse_mla_fwd(_ptr(q, at, "q"), _ptr(kv, at, "kv"), dt, _ptr(idx, I32_T, "idx"), T, H, N, k,
                                     float(sm_scale), _ptr(out, at, "out"), _ptr(lse, F32_T, "lse"),
                                     _ptr(workspace, name="workspace"), ws_bytes, _stream(stream)))


def dsa_masked_mha_workspace_bytes(L: int, H: int) -> int:
    return int(load().dsa_masked_mha_workspace_bytes(L, H))


def dsa_masked_mha_prefill(q, kv, w_uk, w_uv, idx, sm_scale, out, workspace, lse=None, stream=None):
    """q [L,H,192], kv [L,576], w_uk/w_uv [H,128,512] bf16, idx [L,k] -> out [L,H,128] bf16, lse [L,H]."""
    L, H = q.shape[0], q.shape[1]
    k = idx.shape[1]
    ws_bytes = workspace.numel() * workspace.element_size()
    bf = torch.bfloat16
    _check(load().dsa_masked_mha_prefill(_ptr(q, bf, "q"), _ptr(kv, bf, "kv"), _ptr(w_uk, bf, "w_uk"),
                                         _ptr(w_uv, bf, "w_uv"), _ptr(idx, I32_T, "idx"), L, H, k, float(sm_scale),
                                         _ptr(out, bf, "out"), _ptr(lse, F32_T, "lse"),
                                         _ptr(workspace, name="workspace"), ws_bytes, _stream(stream)))


def dsa_indexer_scores_at(q8, q_scale, k8, k_scale, w, idx, out, S=None, stream=None):
    """I[t, idx[t, a]] for E4M3 q8 [T, H_I, 128], k8 [S, 128] -> out [T, k] fp32."""
    T, H_I, D_I = q8.shape
    S = k8.shape[0] if S is None else S
    _check(load().dsa_indexer_scores_at(_ptr(q8, U8_T, "q8"), _ptr(q_scale, F32_T, "q_scale"), _ptr(k8, U8_T, "k8"),
                                        _ptr(k_scale, F32_T, "k_scale"), _ptr(w, F32_T, "w"), _ptr(idx, I32_T, "idx"),
                                        T, S, H_I, D_I, idx.shape[1], _ptr(out, F32_T, "out"), _stream(stream)))


def dsa_indexer_kl_fwd(q, kv, idx, idx_scores, lse, sm_scale, kl, N=None, stream=None):
    """Per-token KL(p || pi): q [T, H, 576], kv [N, 576] bf16, idx/idx_scores [T, k], lse [T, H] -> kl [T]."""
    T, H = q.shape[0], q.shape[1]
    N = kv.shape[0] if N is None else N
    bf = torch.bfloat16
    _check(load().dsa_indexer_kl_fwd(_ptr(q, bf, "q"), _ptr(kv, bf, "kv"), _ptr(idx, I32_T, "idx"),
                                     _ptr(idx_scores, F32_T, "idx_scores"), _ptr(lse, F32_T, "lse"), T, H, N,
                                     idx.shape[1], float(sm_scale), _ptr(kl, F32_T, "kl"), _stream(stream)))


def dsa_sparse_mla_bwd_workspace_bytes(T: int, H: int, N: int, k: int) -> int:
    return int(load().dsa_sparse_mla_bwd_workspace_bytes(T, H, N, k))


def dsa_sparse_mla_bwd(q, kv, idx, out, lse, dout, sm_scale, dq, dkv, workspace, N=None, stream=None):
    """dq [T, H, 576], dkv [N, 576] fp32 from the forward's out, lse and the upstream dout."""
    T, H = q.shape[0], q.shape[1]
    N = kv.shape[0] if N is None else N
    bf = torch.bfloat16
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().dsa_sparse_mla_bwd(_ptr(q, bf, "q"), _ptr(kv, bf, "kv"), _ptr(idx, I32_T, "idx"),
                                     _ptr(out, bf, "out"), _ptr(lse, F32_T, "lse"), _ptr(dout, bf, "dout"), T, H, N,
                                     idx.shape[1], float(sm_scale), _ptr(dq, F32_T, "dq"), _ptr(dkv, F32_T, "dkv"),
                                     _ptr(workspace, name="workspace"), ws_bytes, _stream(stream)))


def dsa_sparse_mla_bwd_kl(q, kv, idx, out, lse, dout, idx_scores, dkl, sm_scale, dq, dkv, grad, workspace, N=None,
                          stream=None):
    """dsa_sparse_mla_bwd's dq and dkv, and dsa_indexer_kl_bwd's score gradient grad [T, k] from the same P."""
    T, H = q.shape[0], q.shape[1]
    N = kv.shape[0] if N is None else N
    bf = torch.bfloat16
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().dsa_sparse_mla_bwd_kl(_ptr(q, bf, "q"), _ptr(kv, bf, "kv"), _ptr(idx, I32_T, "idx"),
                                        _ptr(out, bf, "out"), _ptr(lse, F32_T, "lse"), _ptr(dout, bf, "dout"),
                                        _ptr(idx_scores, F32_T, "idx_scores"), _ptr(dkl, F32_T, "dkl"), T, H, N,
                                        idx.shape[1], float(sm_scale), _ptr(dq, F32_T, "dq"), _ptr(dkv, F32_T, "dkv"),
                                        _ptr(grad, F32_T, "grad"), _ptr(workspace, name="workspace"), ws_bytes,
                                        _stream(stream)))


def dsa_indexer_kl_bwd(q, kv, idx, idx_scores, lse, dkl, sm_scale, grad, N=None, stream=None):
    """Score gradient of sum_t dkl[t] KL_t: grad [T, k] = dkl (pi - p) at the valid entries."""
    T, H = q.shape[0], q.shape[1]
    N = kv.shape[0] if N is None else N
    bf = torch.bfloat16
    _check(load().dsa_indexer_kl_bwd(_ptr(q, bf, "q"), _ptr(kv, bf, "kv"), _ptr(idx, I32_T, "idx"),
                                     _ptr(idx_scores, F32_T, "idx_scores"), _ptr(lse, F32_T, "lse"),
                                     _ptr(dkl, F32_T, "dkl"), T, H, N, idx.shape[1], float(sm_scale),
                                     _ptr(grad, F32_T, "grad"), _stream(stream)))


def dsa_indexer_bwd_workspace_bytes(T: int, S: int, k: int) -> int:
    return int(load().dsa_indexer_bwd_workspace_bytes(T, S, k))


def dsa_indexer_bwd(q8, q_scale, k8, k_scale, w, idx, grad, dw, dq, dk, workspace, S=None, stream=None):
    """dw [T, H_I], dq [T, H_I, D_I], dk [S, D_I] from the score gradient grad [T, k]."""
    T, H_I, D_I = q8.shape
    S = k8.shape[0] if S is None else S
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().dsa_indexer_bwd(_ptr(q8, U8_T, "q8"), _ptr(q_scale, F32_T, "q_scale"), _ptr(k8, U8_T, "k8"),
                                  _ptr(k_scale, F32_T, "k_scale"), _ptr(w, F32_T, "w"), _ptr(idx, I32_T, "idx"),
                                  _ptr(grad, F32_T, "grad"), T, S, H_I, D_I, idx.shape[1], _ptr(dw, F32_T, "dw"),
                                  _ptr(dq, F32_T, "dq"), _ptr(dk, F32_T, "dk"), _ptr(workspace, name="workspace"),
                                  ws_bytes, _stream(stream)))


def make_prefill_args(L, H_I, D_I, H, k, idx_dt, q_idx, q_scale, k_idx, k_scale, w, attn_dt, q, kv, sm_scale,
                      idx, out, lse=None) -> PrefillArgs:
    it = U8_T if idx_dt == DSA_E4M3 else F32_T
    at = torch.bfloat16 if attn_dt == DSA_BF16 else F32_T
    return PrefillArgs(L, H_I, D_I, H, k, idx_dt, _ptr(q_idx, it, "q_idx"), _ptr(q_scale, F32_T, "q_scale"),
                       _ptr(k_idx, it, "k_idx"), _ptr(k_scale, F32_T, "k_scale"), _ptr(w, F32_T, "w"), attn_dt,
                       _ptr(q, at, "q"), _ptr(kv, at, "kv"), float(sm_scale), _ptr(idx, I32_T, "idx"),
                       _ptr(out, at, "out"), _ptr(lse, F32_T, "lse"))


def dsa_prefill_workspace_bytes(args: PrefillArgs) -> int:
    return int(load().dsa_prefill_workspace_bytes(ctypes.byref(args)))


def dsa_prefill(args: PrefillArgs, workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().dsa_prefill(ctypes.byref(args), _ptr(workspace), ws_bytes, _stream(stream)))


def dsa_prefill_select(args: PrefillArgs, workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().dsa_prefill_select(ctypes.byref(args), _ptr(workspace), ws_bytes, _stream(stream)))


def make_decode_args(B, H_I, D_I, H, k, q8, q_scale, w, q, k8_pool, ks_pool, kv_pool, n_pool_rows, block_table,
                     max_blocks, ctx_len, max_ctx, sm_scale, out, lse=None, idx_out=None) -> DecodeArgs:
    bf = torch.bfloat16
    return DecodeArgs(B, H_I, D_I, H, k, _ptr(q8, U8_T, "q8"), _ptr(q_scale, F32_T, "q_scale"), _ptr(w, F32_T, "w"),
                      _ptr(q, bf, "q"), _ptr(k8_pool, U8_T, "k8_pool"), _ptr(ks_pool, F32_T, "ks_pool"),
                      _ptr(kv_pool, bf, "kv_pool"), n_pool_rows, _ptr(block_table, I32_T, "block_table"), max_blocks,
                      _ptr(ctx_len, I32_T, "ctx_len"), max_ctx, float(sm_scale), _ptr(idx_out, I32_T, "idx_out"),
                      _ptr(out, bf, "out"), _ptr(lse, F32_T, "lse"))


def dsa_decode_workspace_bytes(args: DecodeArgs) -> int:
    return int(load().dsa_decode_workspace_bytes(ctypes.byref(args)))


def dsa_decode(args: DecodeArgs, workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().dsa_decode(ctypes.byref(args), _ptr(workspace), ws_bytes, _stream(stream)))


def dsa_decode_static_scratch_bytes() -> int:
    return int(load().dsa_decode_static_scratch_bytes())


def dsa_decode_noalloc(args: DecodeArgs, stream=None):
    """dsa_decode with its workspace in the library's static device scratch."""
    _check(load().dsa_decode_noalloc(ctypes.byref(args), _stream(stream)))


def dsa_decode_indexer_scores(args: DecodeArgs, scores, ld_scores=None, stream=None):
    ld = scores.stride(0) if ld_scores is None else ld_scores
    _check(load().dsa_decode_indexer_scores(ctypes.byref(args), _ptr(scores), ld, _stream(stream)))


def dsa_sparse_mla_paged_fwd(q, kv_pool, block_table, idx, sm_scale, out, lse=None, workspace=None,
                             n_pool_rows=None, stream=None):
    T, H = q.shape[0], q.shape[1]
    k = idx.shape[1]
    n_pool_rows = kv_pool.numel() // 576 if n_pool_rows is None else n_pool_rows
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    bf = torch.bfloat16
    _check(load().dsa_sparse_mla_paged_fwd(_ptr(q, bf, "q"), _ptr(kv_pool, bf, "kv_pool"), n_pool_rows,
                                           _ptr(block_table, I32_T, "block_table"), block_table.shape[1],
                                           _ptr(idx, I32_T, "idx"), T, H, k, float(sm_scale), _ptr(out, bf, "out"),
                                           _ptr(lse, F32_T, "lse"), _ptr(workspace, name="workspace"), ws_bytes,
                                           _stream(stream)))


def dsa_paged_cache_append(latent, k8, ks, pos, block_table, kv_pool, k8_pool, ks_pool, B=None, D_I=None,
                           max_blocks=None, n_pool_rows=None, stream=None):
    B = latent.shape[0] if B is None else B
    D_I = k8.shape[-1] if D_I is None else D_I
    max_blocks = block_table.shape[1] if max_blocks is None else max_blocks
    n_pool_rows = kv_pool.numel() // 576 if n_pool_rows is None else n_pool_rows
    bf = torch.bfloat16
    _check(load().dsa_paged_cache_append(_ptr(latent, bf, "latent"), _ptr(k8, U8_T, "k8"), _ptr(ks, F32_T, "ks"),
                                         _ptr(pos, I32_T, "pos"), B, D_I, _ptr(block_table, I32_T, "block_table"),
                                         max_blocks, _ptr(kv_pool, bf, "kv_pool"), _ptr(k8_pool, U8_T, "k8_pool"),
                                         _ptr(ks_pool, F32_T, "ks_pool"), n_pool_rows, _stream(stream)))
