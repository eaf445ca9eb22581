"""The C ABI on the host, no GPU needed: the library loads, exports every
function include/dsa.h declares, and rejects bad arguments with the right
status before making any HIP call (nothing here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

FAKE = 0x1000  # a non-null pointer value; never dereferenced by failing validation


@pytest.fixture(scope="module")
def dsa():
    from sparse_attention_gemm_amd import build, dsa as d
    if not os.path.exists(d.LIB_PATH):
        build.build()
    d.load()
    return d


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("dsa_indexer_scores", "dsa_topk_select", "dsa_sparse_mla_fwd", "dsa_prefill", "dsa_decode",
              "dsa_quantize_e4m3_per_token", "dsa_paged_cache_append", "dsa_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(dsa):
    lib = ctypes.CDLL(dsa.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(_declared()) == set(dsa.EXPORTS)
    assert dsa.dsa_version().startswith("libdsa")


def _status(fn, *args):
    return fn(*args)


def test_quantize_validation(dsa):
    L = dsa.load()
    assert L.dsa_quantize_e4m3_per_token(FAKE, -1, 128, FAKE, FAKE, None) == dsa.DSA_ERR_INVALID_ARG
    assert L.dsa_quantize_e4m3_per_token(FAKE, 4, 0, FAKE, FAKE, None) == dsa.DSA_ERR_INVALID_ARG
    assert L.dsa_quantize_e4m3_per_token(None, 4, 128, FAKE, FAKE, None) == dsa.DSA_ERR_INVALID_ARG
    assert L.dsa_quantize_e4m3_per_token(FAKE, 4, 130, FAKE, FAKE, None) == dsa.DSA_ERR_UNSUPPORTED
    assert "multiple of 4" in dsa.dsa_last_error()
    # nothing to do is not an error (and launches nothing)
    assert L.dsa_quantize_e4m3_per_token(None, 0, 128, None, None, None) == dsa.DSA_OK


def test_indexer_validation(dsa):
    L = dsa.load()
    f = L.dsa_indexer_scores
    ok_args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 100, 64, 128, dsa.DSA_E4M3, FAKE, 100, None]
    bad = list(ok_args)
    bad[6] = -1
    assert f(*bad) == dsa.DSA_ERR_INVALID_ARG
    bad = list(ok_args)
    bad[12] = 50  # ld < S
    assert f(*bad) == dsa.DSA_ERR_INVALID_ARG
    bad = list(ok_args)
    bad[1] = None  # E4M3 without q scale
    assert f(*bad) == dsa.DSA_ERR_INVALID_ARG
    bad = list(ok_args)
    bad[9] = 96  # E4M3 widths are 64 or 128
    assert f(*bad) == dsa.DSA_ERR_UNSUPPORTED
    bad = list(ok_args)
    bad[8] = 65  # more than 64 E4M3 heads
    assert f(*bad) == dsa.DSA_ERR_UNSUPPORTED
    bad = list(ok_args)
    bad[10] = dsa.DSA_BF16
    assert f(*bad) == dsa.DSA_ERR_UNSUPPORTED
    bad = list(ok_args)
    bad[10], bad[8] = dsa.DSA_F32, 65
    assert f(*bad) == dsa.DSA_ERR_UNSUPPORTED
    bad = list(ok_args)
    bad[11] = None
    assert f(*bad) == dsa.DSA_ERR_INVALID_ARG
    empty = list(ok_args)
    empty[6] = 0
    assert f(*empty) == dsa.DSA_OK


def test_topk_validation(dsa):
    f = dsa.load().dsa_topk_select
    assert f(FAKE, 100, FAKE, 4, 0, FAKE, None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    assert f(FAKE, 100, FAKE, 4, 2049, FAKE, None, 0, None) == dsa.DSA_ERR_UNSUPPORTED
    assert f(FAKE, 100, None, 4, 16, FAKE, None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    assert f(FAKE, -1, FAKE, 4, 16, FAKE, None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    assert f(None, 100, None, 0, 16, None, None, 0, None) == dsa.DSA_OK


def test_sparse_mla_validation(dsa):
    L = dsa.load()
    f = L.dsa_sparse_mla_fwd
    base = [FAKE, FAKE, dsa.DSA_BF16, FAKE, 64, 128, 1000, 2048, 0.07, FAKE, FAKE, None, 0, None]
    b = list(base)
    b[5] = 20  # H not a multiple of 8 for bf16
    assert f(*b) == dsa.DSA_ERR_UNSUPPORTED
    b = list(base)
    b[7] = 4096
    assert f(*b) == dsa.DSA_ERR_UNSUPPORTED
    b = list(base)
    b[8] = -1.0
    assert f(*b) == dsa.DSA_ERR_INVALID_ARG
    b = list(base)
    b[8] = float("nan")
    assert f(*b) == dsa.DSA_ERR_INVALID_ARG
    b = list(base)
    b[2] = dsa.DSA_E4M3
    assert f(*b) == dsa.DSA_ERR_UNSUPPORTED
    b = list(base)
    b[11], b[12] = FAKE, 16  # a workspace smaller than required
    need = L.dsa_sparse_mla_workspace_bytes(64, 128, 2048)
    assert need > 16
    assert f(*b) == dsa.DSA_ERR_WORKSPACE
    assert L.dsa_sparse_mla_workspace_bytes(100000, 128, 2048) == 0  # enough queries: no split


def test_masked_mha_validation(dsa):
    L = dsa.load()
    f = L.dsa_masked_mha_prefill
    need = L.dsa_masked_mha_workspace_bytes(4096, 128)
    # K and V [L, H, 128] bf16 plus the L x L bit mask
    assert need >= 2 * 4096 * 128 * 128 * 2 + 4096 * 4096 // 8
    assert L.dsa_masked_mha_workspace_bytes(0, 128) == 0
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, 4096, 128, 2048, 0.07, FAKE, FAKE, FAKE, need, None]
    b = list(base)
    b[5] = -1
    assert f(*b) == dsa.DSA_ERR_INVALID_ARG
    b = list(base)
    b[5] = 65537
    assert f(*b) == dsa.DSA_ERR_UNSUPPORTED
    b = list(base)
    b[6] = 0
    assert f(*b) == dsa.DSA_ERR_INVALID_ARG
    b = list(base)
    b[7] = 0
    assert f(*b) == dsa.DSA_ERR_INVALID_ARG
    b = list(base)
    b[8] = float("nan")
    assert f(*b) == dsa.DSA_ERR_INVALID_ARG
    b = list(base)
    b[2] = None  # w_uk
    assert f(*b) == dsa.DSA_ERR_INVALID_ARG
    b = list(base)
    b[11] = None  # the workspace is required
    assert f(*b) == dsa.DSA_ERR_INVALID_ARG
    b = list(base)
    b[12] = need - 1
    assert f(*b) == dsa.DSA_ERR_WORKSPACE
    b = list(base)
    b[5] = 0  # nothing to do
    assert f(*b) == dsa.DSA_OK


def test_indexer_kl_validation(dsa):
    L = dsa.load()
    f = L.dsa_indexer_kl_fwd
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, 64, 128, 5000, 2048, 0.07, FAKE, None]
    b = list(base)
    b[6] = 48  # H not in {16, 32, 64, 128}
    assert f(*b) == dsa.DSA_ERR_UNSUPPORTED
    b = list(base)
    b[8] = 2049
    assert f(*b) == dsa.DSA_ERR_UNSUPPORTED
    b = list(base)
    b[3] = None  # scores
    assert f(*b) == dsa.DSA_ERR_INVALID_ARG
    b = list(base)
    b[9] = 0.0
    assert f(*b) == dsa.DSA_ERR_INVALID_ARG
    b = list(base)
    b[5] = 0
    assert f(*b) == dsa.DSA_OK
    g = L.dsa_indexer_scores_at
    gb = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 5000, 64, 128, 2048, FAKE, None]
    b = list(gb)
    b[8] = 16
    assert g(*b) == dsa.DSA_ERR_UNSUPPORTED
    b = list(gb)
    b[7] = 0
    assert g(*b) == dsa.DSA_ERR_INVALID_ARG
    b = list(gb)
    b[11] = None
    assert g(*b) == dsa.DSA_ERR_INVALID_ARG


def test_sparse_mla_bwd_kl_validation(dsa):
    """The fused backward refuses what dsa_sparse_mla_bwd refuses, and a missing
    score or gradient pointer, before any device work."""
    L = dsa.load()
    f = L.dsa_sparse_mla_bwd_kl
    T, H, N, k = 6, 128, 5000, 2048
    need = dsa.dsa_sparse_mla_bwd_workspace_bytes(T, H, N, k)
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, T, H, N, k, 0.07, FAKE, FAKE, FAKE, FAKE, need, None]
    for i in (6, 7, 15):  # idx_scores, dkl, grad_scores
        b = list(base)
        b[i] = None
        assert f(*b) == dsa.DSA_ERR_INVALID_ARG, i
    b = list(base)
    b[9] = 48  # H not a multiple of 32
    assert f(*b) == dsa.DSA_ERR_UNSUPPORTED
    b = list(base)
    b[11] = 2049
    assert f(*b) == dsa.DSA_ERR_UNSUPPORTED
    b = list(base)
    b[17] = need - 1
    assert f(*b) == dsa.DSA_ERR_WORKSPACE
    b = list(base)
    b[8] = 0
    assert f(*b) == dsa.DSA_OK


def test_prefill_validation(dsa):
    L = dsa.load()
    a = dsa.make_prefill_args(1000, 64, 128, 128, 2048, dsa.DSA_E4M3, FAKE, FAKE, FAKE, FAKE, FAKE, dsa.DSA_BF16,
                              FAKE, FAKE, 0.07, FAKE, FAKE, FAKE)
    assert L.dsa_prefill(None, None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    a.H_I = 80
    assert L.dsa_prefill(ctypes.byref(a), None, 0, None) == dsa.DSA_ERR_UNSUPPORTED
    # other E4M3 shapes are accepted (unfused, L x L scores in the workspace): the missing workspace is the error
    a.H_I, a.D_I = 4, 64
    assert L.dsa_prefill(ctypes.byref(a), None, 0, None) == dsa.DSA_ERR_WORKSPACE
    assert L.dsa_prefill_workspace_bytes(ctypes.byref(a)) >= 1000 * 1000 * 4
    a.L = 20000  # ... but only while L x L fits
    assert L.dsa_prefill(ctypes.byref(a), None, 0, None) == dsa.DSA_ERR_UNSUPPORTED
    a.L, a.H_I, a.D_I = 1000, 64, 128
    a.k = 0
    assert L.dsa_prefill(ctypes.byref(a), None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    a.k = 2048
    a.q_scale = None
    assert L.dsa_prefill(ctypes.byref(a), None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    a.q_scale = FAKE
    a.H = 12  # not a multiple of 8
    assert L.dsa_prefill(ctypes.byref(a), None, 0, None) == dsa.DSA_ERR_UNSUPPORTED
    a.H = 128
    a.idx_dt = dsa.DSA_F32
    a.q_scale = a.k_scale = None
    need = dsa.dsa_prefill_workspace_bytes(a)
    assert need >= 1000 * 1000 * 4
    assert L.dsa_prefill(ctypes.byref(a), None, 0, None) == dsa.DSA_ERR_WORKSPACE
    assert L.dsa_prefill(ctypes.byref(a), FAKE, need - 1, None) == dsa.DSA_ERR_WORKSPACE
    a.L = 20000
    assert L.dsa_prefill(ctypes.byref(a), FAKE, 1 << 40, None) == dsa.DSA_ERR_UNSUPPORTED


def test_decode_validation(dsa):
    L = dsa.load()
    a = dsa.make_decode_args(4, 64, 128, 128, 2048, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64 * 100, FAKE, 100,
                             FAKE, 6400, 0.07, FAKE, FAKE, None)
    need = dsa.dsa_decode_workspace_bytes(a)
    assert need >= 4 * 6400 * 4 + 4 * 2048 * 4
    assert L.dsa_decode(ctypes.byref(a), None, 0, None) == dsa.DSA_ERR_WORKSPACE
    a.max_blocks = 50
    assert L.dsa_decode(ctypes.byref(a), FAKE, need, None) == dsa.DSA_ERR_INVALID_ARG
    a.max_blocks = 100
    a.n_pool_rows = 6401
    assert L.dsa_decode(ctypes.byref(a), FAKE, need, None) == dsa.DSA_ERR_INVALID_ARG
    a.n_pool_rows = 6400
    a.H = 124  # not a multiple of 8
    assert L.dsa_decode(ctypes.byref(a), FAKE, need, None) == dsa.DSA_ERR_UNSUPPORTED
    a.H = 128
    a.ctx_len = None
    assert L.dsa_decode(ctypes.byref(a), FAKE, need, None) == dsa.DSA_ERR_INVALID_ARG


def test_cache_append_validation(dsa):
    f = dsa.load().dsa_paged_cache_append
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 128, FAKE, 10, FAKE, FAKE, FAKE, 100, None) == dsa.DSA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 120, FAKE, 10, FAKE, FAKE, FAKE, 640, None) == dsa.DSA_ERR_UNSUPPORTED
    # the decode reads the key pool at a 128-byte stride: other key widths are refused
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 64, FAKE, 10, FAKE, FAKE, FAKE, 640, None) == dsa.DSA_ERR_UNSUPPORTED
    assert "D_I = 128" in dsa.dsa_last_error()
    assert f(FAKE, None, FAKE, FAKE, 4, 128, FAKE, 10, FAKE, FAKE, FAKE, 640, None) == dsa.DSA_ERR_INVALID_ARG
    assert f(None, None, None, None, 0, 128, None, 10, None, None, None, 640, None) == dsa.DSA_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import importlib
    from sparse_attention_gemm_amd import dsa as d
    monkeypatch.setattr(d, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(d, "_lib", None)
    with pytest.raises(ImportError):
        d.load()
    importlib.reload(d)


def test_binding_refuses_host_strided_and_mistyped_tensors(dsa):
    """The binding passes raw addresses to the library, so it checks each
    tensor first: host memory, a strided view or the wrong dtype raises before
    the library is called."""
    import torch
    host = torch.zeros((4, 8), dtype=torch.float32)
    with pytest.raises(ValueError, match="device tensor"):
        dsa.dsa_topk_select(host, host[:, 0].to(torch.int32), 4, torch.zeros((4, 4), dtype=torch.int32))
    with pytest.raises(ValueError, match="device tensor"):
        dsa.make_decode_args(1, 64, 128, 16, 4, host.to(torch.uint8), None, None, None, None, None, None, 64, None,
                             1, None, 1, 0.1, None)
    # the dtype and layout checks, exercised on the checker itself (no device here)
    class Fake:
        is_cuda = True

        def __init__(self, dtype, contiguous=True):
            self.dtype, self._c = dtype, contiguous

        def is_contiguous(self):
            return self._c

        def data_ptr(self):
            return 0x1000
    assert dsa._ptr(Fake(torch.float32), torch.float32) == 0x1000
    with pytest.raises(TypeError, match="must be"):
        dsa._ptr(Fake(torch.float16), torch.bfloat16, "q")
    with pytest.raises(ValueError, match="contiguous"):
        dsa._ptr(Fake(torch.float32, contiguous=False), torch.float32)


def test_binding_refuses_a_stale_library(dsa, monkeypatch):
    """A library stamped with other sources' hash is refused on load."""
    from sparse_attention_gemm_amd import build
    L = dsa.load()
    dsa._check_fresh(L)  # the built library matches its sources
    monkeypatch.setattr(build, "source_hash", lambda: "0123456789abcdef")
    with pytest.raises(ImportError, match="stale"):
        dsa._check_fresh(L)


def test_noalloc_decode_refuses_oversized_request(dsa):
    """dsa_decode_noalloc checks the request's workspace against its static
    scratch before touching the device: B = 1024 sequences at context 131072
    is refused with DSA_ERR_UNSUPPORTED (nothing here reaches HIP)."""
    L = dsa.load()
    a = L.dsa_decode_noalloc.argtypes[0]._type_()  # the struct class this library object was bound with
    a.B, a.H_I, a.D_I, a.H, a.k = 1024, 64, 128, 128, 2048
    for f in ("q8", "q_scale", "w", "q", "k8_pool", "ks_pool", "kv_pool", "block_table", "ctx_len", "out"):
        setattr(a, f, FAKE)
    a.n_pool_rows, a.max_blocks, a.max_ctx, a.sm_scale = 64, 2048, 131072, 0.07
    assert L.dsa_decode_workspace_bytes(ctypes.byref(a)) > L.dsa_decode_static_scratch_bytes() == 128 << 20
    assert L.dsa_decode_noalloc(ctypes.byref(a), None) == dsa.DSA_ERR_UNSUPPORTED
    assert "static scratch" in dsa.dsa_last_error()
    a.B = -1
    assert L.dsa_decode_noalloc(ctypes.byref(a), None) == dsa.DSA_ERR_INVALID_ARG
