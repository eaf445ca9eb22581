"""How the gfx950 E4M3 MFMA adds up its products.

The full-size indexer forms each head's dot product <q8[t,j], k8[s]> of 128
E4M3 products with one 16x16x128 MFMA.  Every product is exact, but the matrix
core does not add the 128 of them as a chain of IEEE fp32 additions: on random
operands its fp32 result differs from the exact sum by up to about 2^-12 of
the sum of the products' magnitudes, where a sequential fp32 sum stays within
127 x 2^-24 of it.  The indexer's score tolerance (the fp32 floor of the score
check) holds at full size only because the 64 heads' errors average out; the
other E4M3 shapes are summed with fp32 fused multiply-adds instead.  These
tests pin the property with a bound twice the largest error measured, and
print the measured figures.
"""
import ctypes

import numpy as np
import pytest
import torch

import synth
from tests.parity import FP8_MFMA_SUM_REL

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N = 2048  # trials of one 16x16x128 MFMA: 524288 dot products


def _lib():
    from sparse_attention_gemm_amd import build
    lib = ctypes.CDLL(build.PEAKS_LIB)
    lib.dsa_peak_fp8_mfma_dot.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_void_p]
    lib.dsa_peak_fp8_mfma_dot.restype = ctypes.c_int
    return lib


def _finite_codes(seed, tid):
    """Uniform E4M3 codes with the two NaN codes (0x7F, 0xFF) moved one step down."""
    c = synth.randint(seed, tid, (N * 16, 128), 0, 255).numpy().astype(np.uint8)
    c[(c & 0x7F) == 0x7F] -= 1
    return c


def _operands(ora, kind):
    if kind == "indexer_rows":  # per-token quantised Gaussian rows, as the indexer's q_I and k_I
        a, _ = ora.quantize_rows(synth.normal(21, synth.T_QI, (N * 16, 128)).numpy())
        b, _ = ora.quantize_rows(synth.normal(21, synth.T_KI, (N * 16, 128)).numpy())
    else:  # every finite code: products from 2^-18 to 448^2
        a, b = _finite_codes(22, 1), _finite_codes(22, 2)
        if kind == "upper_half_zero":  # the layout of a 64-dim head zero-padded to 128
            a[:, 64:] = 0
            b[:, 64:] = 0
    return a.reshape(N, 16, 128), b.reshape(N, 16, 128)


@pytest.mark.parametrize("kind", ["indexer_rows", "any_finite", "upper_half_zero"])
def test_fp8_mfma_sum_error_bound(ora, kind):
    print(f"[case] E4M3 16x16x128 MFMA sums, operands {kind}", flush=True)
    a8, b8 = _operands(ora, kind)
    d = torch.empty((N, 16, 16), dtype=torch.float32, device=DEV)
    da, db = torch.from_numpy(a8).to(DEV), torch.from_numpy(b8).to(DEV)
    assert _lib().dsa_peak_fp8_mfma_dot(da.data_ptr(), db.data_ptr(), d.data_ptr(), N, None) == 0
    torch.cuda.synchronize()
    got = d.cpu().double().numpy()
    # exact sums: every product has at most 8 significant bits and lies in
    # [2^-18, 2^17.7], so float64 adds 128 of them without rounding
    a, b = ora.e4m3_decode(a8), ora.e4m3_decode(b8)
    exact = np.einsum("tik,tjk->tij", a, b)
    mag = np.einsum("tik,tjk->tij", np.abs(a), np.abs(b))
    nz = mag > 0
    units = np.abs(got - exact)[nz] / (2.0 ** -24 * mag[nz])
    print(f"[mfma] {kind}: |error| / (2^-24 sum|products|): max {units.max():.1f}, mean {units.mean():.2f}, "
          f"exact {np.mean(units == 0):.1%} (a sequential fp32 sum stays within 127)", flush=True)
    assert np.all(got[~nz] == 0.0)
    assert units.max() <= FP8_MFMA_SUM_REL * 2.0 ** 24, "the MFMA sums moved beyond their stated accuracy"
