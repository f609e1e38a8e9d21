"""The GPU-vs-oracle checker on hand-made rows (CPU): it accepts the exact
result and swaps of pages whose oracle scores lie within the tolerance, and
rejects everything else -- swaps beyond the tolerance, a NaN page in place of
a number or the reverse, another NaN page, a broken contract, and GPU scores
whose NaN pattern differs from the oracle's."""

import numpy as np
import pytest

from tests import checker


def _row(ids, L):
    o = np.full(16, -1, dtype=np.int32)
    o[:len(ids)] = ids
    o[15] = L
    return o[None, None, :]


def _case():
    # 5 history pages: scores 10, 7, 7 + 5e-4 (within 1e-4 x 10), NaN, 1
    s = np.array([10.0, 7.0, 7.0005, np.nan, 1.0])
    L = np.array([5])
    ref = _row([0, 2, 1, 4, 3], 5)
    return s, L, ref


def test_exact_and_near_tie_swap_pass():
    s, L, ref = _case()
    assert checker.compare(ref, ref, [[s]], L) == 1.0
    swapped = _row([0, 1, 2, 4, 3], 5)
    assert checker.compare(swapped, ref, [[s]], L) == 0.0


def test_swap_beyond_tolerance_fails():
    s, L, ref = _case()
    with pytest.raises(AssertionError):
        checker.compare(_row([2, 0, 1, 4, 3], 5), ref, [[s]], L)


def test_nan_pick_must_match():
    s, L, ref = _case()
    with pytest.raises(AssertionError):       # NaN page ranked above a number
        checker.compare(_row([0, 2, 1, 3, 4], 5), ref, [[s]], L)
    s2 = np.array([10.0, 7.0, np.nan, np.nan, 1.0])
    ref2 = _row([0, 1, 4, 2, 3], 5)
    assert checker.compare(ref2, ref2, [[s2]], L) == 1.0
    with pytest.raises(AssertionError):       # the NaN pages out of id order
        checker.compare(_row([0, 1, 4, 3, 2], 5), ref2, [[s2]], L)


def test_contract_violations_fail():
    s, L, ref = _case()
    with pytest.raises(AssertionError):       # wrong local page
        bad = ref.copy()
        bad[0, 0, 15] = 4
        checker.compare(bad, ref, [[s]], L)
    with pytest.raises(AssertionError):       # repeated id
        checker.compare(_row([0, 0, 1, 4, 3], 5), ref, [[s]], L)
    with pytest.raises(AssertionError):       # id past the history
        checker.compare(_row([0, 2, 1, 4, 5], 5), ref, [[s]], L)
    with pytest.raises(AssertionError):       # padding row not all -1
        checker.compare(_row([], 0), np.full((1, 1, 16), -1), [[np.zeros(0)]], np.array([-1]))


def test_gpu_scores_nan_pattern_and_tolerance():
    s, L, ref = _case()
    good = s.astype(np.float32).astype(np.float64)[None, None, :]
    checker.compare(ref, ref, [[s]], L, gpu_scores=good)
    bad = good.copy()
    bad[0, 0, 3] = 5.0                         # a number where the oracle has NaN
    with pytest.raises(AssertionError):
        checker.compare(ref, ref, [[s]], L, gpu_scores=bad)
    bad = good.copy()
    bad[0, 0, 1] = 7.01                        # beyond 1e-4 x 10
    with pytest.raises(AssertionError):
        checker.compare(ref, ref, [[s]], L, gpu_scores=bad)
