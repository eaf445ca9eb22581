"""The comparison rules of tests/parity.py, checked on the CPU.

Each rule is exercised on values whose outcome is known: a result inside the
stated bound passes, a planted error just outside it fails.  The planted
errors sit in the values handed to the checker, never in the GPU path.
"""
import numpy as np
import pytest

from tests.parity import SCORE_RTOL, TIE_RTOL, check_attention, check_scores, check_topk_row

U = 2.0 ** -24


def _scores(n=4000, seed=0):
    rng = np.random.default_rng(seed)
    ora = rng.normal(size=n) * 50.0
    mag = np.abs(ora) * 30.0 + 1.0   # C, the score of |w|, |q|, |k|: always >= |score|
    return ora, mag


def test_scores_pass_within_relative_bound():
    ora, mag = _scores()
    gpu = ora * (1 + 0.9 * SCORE_RTOL)
    ratio, worst_rel, _ = check_scores(gpu, ora, mag, 192, "inside")
    assert ratio <= 1.0 and worst_rel <= SCORE_RTOL


def test_scores_fail_past_relative_bound():
    ora, mag = _scores()
    gpu = ora.copy()
    big = np.argmax(np.abs(ora))
    gpu[big] *= 1 + 1.5 * SCORE_RTOL      # a large score off by 1.5e-3 relative
    with pytest.raises(AssertionError, match="out of tolerance"):
        check_scores(gpu, ora, mag, 192, "planted")


def test_scores_floor_covers_fp32_rounding_only():
    """A cancelling score (|score| << C) may be off by the fp32 floor, not more."""
    ora = np.array([1e-6, 0.0, -2e-7, 5.0])
    mag = np.array([1e3, 1e3, 1e3, 10.0])
    floor = 194 * U * mag
    check_scores(ora + 0.99 * floor, ora, mag, 192, "floor")
    gpu = ora.copy()
    gpu[0] += 1.01 * floor[0]
    with pytest.raises(AssertionError):
        check_scores(gpu, ora, mag, 192, "past floor")


def test_scores_inf_pattern_must_match():
    ora = np.array([1.0, -np.inf, 2.0])
    mag = np.array([2.0, 0.0, 3.0])
    check_scores(np.array([1.0, -np.inf, 2.0]), ora, mag, 192)
    with pytest.raises(AssertionError, match="-inf pattern"):
        check_scores(np.array([1.0, 0.0, 2.0]), ora, mag, 192)


def _row(n=300, seed=1):
    rng = np.random.default_rng(seed)
    return rng.normal(size=n)


def test_topk_exact_selection_passes_and_padding_is_checked():
    s = _row()
    k = 40
    ref = np.sort(np.lexsort((-np.arange(s.size), -s))[:k]).astype(np.int32)
    assert check_topk_row(ref, s, s.size, k) == 0
    # a row shorter than k: every position, ascending, then -1
    assert check_topk_row(np.concatenate([np.arange(30), [-1] * 10]).astype(np.int32), s, 30, k) == 0
    with pytest.raises(AssertionError, match="padding"):
        check_topk_row(np.concatenate([np.arange(30), [-1] * 9, [5]]).astype(np.int32), s, 30, k)
    with pytest.raises(AssertionError):   # a valid row of length n > k may not be padded early
        check_topk_row(np.concatenate([ref[:35], [-1] * 5]).astype(np.int32), s, s.size, k)
    with pytest.raises(AssertionError, match="ascending"):
        check_topk_row(ref[::-1].copy(), s, s.size, k)
    bad = ref.copy()
    bad[-1] = s.size          # out of range
    with pytest.raises(AssertionError):
        check_topk_row(np.sort(bad), s, s.size, k)


def test_topk_swap_allowed_only_inside_tie_band():
    s = _row()
    k = 40
    order = np.lexsort((-np.arange(s.size), -s))
    kth, next_ = order[k - 1], order[k]
    tau = s[kth]
    # put the (k+1)-th candidate within the tie band of tau: swapping it in is legal
    s2 = s.copy()
    s2[next_] = tau - 0.5 * TIE_RTOL * max(1.0, abs(tau))
    sel = np.sort(np.concatenate([order[:k - 1], [next_]])).astype(np.int32)
    assert check_topk_row(sel, s2, s.size, k) == 2
    # the same swap with a gap larger than the band is a failure
    s3 = s.copy()
    s3[next_] = tau - 3.0 * TIE_RTOL * max(1.0, abs(tau))
    with pytest.raises(AssertionError, match="tie band"):
        check_topk_row(sel, s3, s.size, k)


def test_topk_tie_rule_prefers_larger_position():
    s = np.zeros(10)
    # all tied: the k most recent positions are the unique answer, any other set is out of range of the rule
    assert check_topk_row(np.arange(6, 10, dtype=np.int32), s, 10, 4) == 0
    # a different tied set differs only by ties, which the band allows
    assert check_topk_row(np.array([0, 7, 8, 9], np.int32), s, 10, 4) == 2


def test_attention_bounds():
    rng = np.random.default_rng(3)
    o = rng.normal(size=(2, 4, 8)) * 0.5
    lse = rng.normal(size=(2, 4))
    check_attention(o + 0.9e-2 * np.abs(o).max(), lse + 0.9e-3, o, lse, "bf16")
    with pytest.raises(AssertionError, match="max"):
        check_attention(o + 1.1e-2 * np.abs(o).max(), lse, o, lse, "bf16")
    with pytest.raises(AssertionError, match="lse"):
        check_attention(o, lse + 1.1e-3, o, lse, "bf16")
    check_attention(o + 0.9e-5 * np.abs(o).max(), lse + 0.9e-5, o, lse, "f32")
    with pytest.raises(AssertionError):
        check_attention(o + 2e-5 * np.abs(o).max(), lse, o, lse, "f32")
    # an empty selection: -inf lse on both sides, o = 0
    lse2 = lse.copy()
    lse2[0, 1] = -np.inf
    check_attention(o, lse2, o, lse2, "bf16")
    with pytest.raises(AssertionError, match="-inf pattern"):
        check_attention(o, lse, o, lse2, "bf16")
