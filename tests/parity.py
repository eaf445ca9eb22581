"""Comparison rules between the GPU path and the fp64 oracle.

Tolerances (stated once, used by every parity test):
  * index scores: |gpu - ora| <= max(1e-3 |ora|, (D_I + H_I + 2) u C), with
    u = 2^-24 and C = sum_j |w_j| sum_d |q_jd k_d| (scales included): plain
    1e-3 relative error, floored at the a-priori rounding bound of any fp32
    evaluation of the score (a dot product of D_I terms per head, a sum over
    H_I heads, and the two scale products).  The floor decides only where
    the score is small next to C, i.e. where the heads' terms cancel or a
    dot product sits near the ReLU kink; no fp32 evaluation can promise a
    relative error there.  check_scores reports the worst error/bound ratio
    and the worst plain relative error.
  * top-k sets: identical, except that a position may differ between the two
    sets only if its oracle score is within 1e-4 * max(1, |tau|) of the
    oracle's k-th score tau.  Counts, range, uniqueness and ascending order
    are checked exactly.
  * attention: bf16 max|do| <= 2e-2 and <= 1e-2 * max|o_ora|, |dlse| <= 1e-3;
    fp32 max|do| <= 1e-4 and <= 1e-5 * max|o_ora|, |dlse| <= 1e-5.
    Attention is always checked with the GPU's own selection fed to the
    oracle, since a legal tie swap changes the output.
  * masked MHA (MLA's multi-head form): the attention bounds above, with
    lse_slack added to the lse bound: each up-projected key is held in fp16
    once (unit roundoff 2^-11), which moves a logit by at most
    2^-11 sm_scale sum_e |q_e K_e|; the slack is twice that (fp32
    accumulation order on top), maximised over the row's selected keys.
"""
import numpy as np

SCORE_RTOL = 1e-3
TIE_RTOL = 1e-4
# Accuracy of one E4M3 16x16x128 MFMA dot product: its fp32 result lies within
# this fraction of the sum of the 128 products' magnitudes of the exact sum
# (twice the largest error measured; test_gpu_fp8_mfma_sums.py pins it).
FP8_MFMA_SUM_REL = 2.0 ** -11


def abs_payload(x):
    """|x| for fp32 arrays, or the E4M3 payload with its sign bit cleared."""
    x = np.asarray(x)
    return (x & 0x7F).astype(np.uint8) if x.dtype == np.uint8 else np.abs(x)


def oracle_score_bounds(ora, q, k, w, pos, rows=None, q_scale=None, k_scale=None):
    """(scores, scores with |w|, |q|, |k|) from the oracle: the second is C,
    the magnitude that bounds the rounding of any fp32 evaluation."""
    w = np.asarray(w)
    o = ora.indexer_rows(q, k, w, pos, rows=rows, q_scale=q_scale, k_scale=k_scale)
    m = ora.indexer_rows(abs_payload(q), abs_payload(k), np.abs(w), pos, rows=rows, q_scale=q_scale,
                         k_scale=k_scale)
    return o, m


def check_scores(gpu, ora, ora_mag, n_terms, label=""):
    """ora_mag: oracle score with |w|, |q|, |k| (C); n_terms = D_I + H_I.
    Returns (worst err/bound, worst err/|ora| over the entries the relative
    term decides, fraction of entries the floor decides)."""
    gpu = np.asarray(gpu, np.float64)
    fin = np.isfinite(ora)
    assert np.array_equal(np.isfinite(gpu), fin), f"{label}: -inf pattern differs"
    assert np.all(gpu[~fin] == -np.inf)
    err = np.abs(gpu[fin] - ora[fin])
    rel = SCORE_RTOL * np.abs(ora[fin])
    floor = (n_terms + 2) * 2.0 ** -24 * ora_mag[fin]
    bound = np.maximum(rel, floor)
    bad = err > bound
    assert not bad.any(), (f"{label}: {bad.sum()} scores out of tolerance; worst err {err.max():.3e}, "
                           f"bound there {bound[np.argmax(err)]:.3e}")
    if not err.size:
        return 0.0, 0.0, 0.0
    ratio = float((err / np.maximum(bound, 1e-300)).max())
    by_rel = rel >= floor
    worst_rel = float((err[by_rel] / np.abs(ora[fin][by_rel])).max()) if by_rel.any() else 0.0
    print(f"[scores] {label}: worst err/bound {ratio:.3g}, worst relative error {worst_rel:.3g} "
          f"(relative term decides {by_rel.mean():.1%} of {err.size} entries)", flush=True)
    return ratio, worst_rel, float(1.0 - by_rel.mean())


def check_topk_row(gpu_idx, ora_scores_row, n, k, label=""):
    """gpu_idx: int array [k]; ora_scores_row: fp64 scores of positions 0..n-1."""
    K = min(k, n)
    g = np.asarray(gpu_idx)
    assert np.all(g[K:] == -1), f"{label}: padding"
    sel = g[:K]
    assert np.all(sel >= 0) and np.all(sel < n), f"{label}: out of range"
    assert np.all(np.diff(sel) > 0), f"{label}: not strictly ascending"
    if K == n:
        assert np.array_equal(sel, np.arange(n))
        return 0
    s = ora_scores_row[:n]
    order = np.lexsort((-np.arange(n), -s))  # score desc, then position desc
    ref = np.sort(order[:K])
    tau = s[order[K - 1]]
    diff = np.setxor1d(sel, ref)
    if diff.size:
        tol = TIE_RTOL * max(1.0, abs(tau))
        far = np.abs(s[diff] - tau) > tol
        assert not far.any(), (f"{label}: {far.sum()} selection differences beyond the tie band "
                               f"(tau={tau}, worst |s-tau|={np.abs(s[diff] - tau).max():.3e})")
    return int(diff.size)


def check_attention(o_gpu, lse_gpu, o_ora, lse_ora, dtype, label="", lse_slack=0.0):
    o_gpu = np.asarray(o_gpu, np.float64)
    lse_gpu = np.asarray(lse_gpu, np.float64)
    d = np.abs(o_gpu - o_ora).max() if o_ora.size else 0.0
    omax = np.abs(o_ora).max() if o_ora.size else 0.0
    if dtype == "bf16":
        abs_tol, rel_tol, lse_tol = 2e-2, 1e-2, 1e-3
    else:
        abs_tol, rel_tol, lse_tol = 1e-4, 1e-5, 1e-5
    assert d <= abs_tol, f"{label}: max|do| {d:.3e} > {abs_tol}"
    assert d <= rel_tol * omax + 1e-30, f"{label}: max|do| {d:.3e} > {rel_tol} * max|o| ({omax:.3e})"
    fin = np.isfinite(lse_ora)
    assert np.array_equal(np.isfinite(lse_gpu), fin), f"{label}: lse -inf pattern"
    if fin.any():
        slack = np.broadcast_to(np.asarray(lse_slack, np.float64), lse_ora.shape)[fin]
        dl = np.abs(lse_gpu[fin] - lse_ora[fin])
        bad = dl > lse_tol + slack
        assert not bad.any(), (f"{label}: {bad.sum()} lse out of tolerance; worst |dlse| {dl.max():.3e} "
                               f"(bound {lse_tol} + slack up to {slack.max() if slack.size else 0:.3e})")
    return d, omax
