"""Pins of the general forced-block selection of the oracle (``oracle.forced``,
the vllm "indexer_flashinfer" page, ``forward`` / ``build``): exhaustive brute
force over subsets on tiny rows, the special cases the clamps produce, the
default configuration against the 16-slot selection, and the output's form
(ascending ids, ``-1`` tail)."""

import itertools

import numpy as np
import pytest

import oracle


def _brute(scores, L, topk, init_blocks, local_blocks, max_k_tiles, local_score=None):
    """Every subset of the row's valid pages of the right size that holds the
    forced pages; the winner's non-forced part is the best when its members
    are listed best first (score descending, NaN last, lower id first on a
    tie) and compared entry by entry.  The local page, when it competes,
    carries ``local_score``."""
    if L < 0:
        return [-1] * topk
    nvp = L + 1
    if nvp <= topk:
        return list(range(nvp)) + [-1] * (topk - nvp)
    fb = min(init_blocks, max_k_tiles, topk)          # the page's clamps
    fe = min(local_blocks, topk - fb)
    forced = set(range(fb)) | set(range(nvp - fe, nvp))
    rest = [j for j in range(nvp) if j not in forced]
    full = list(scores[:L]) + [local_score]

    def rank(j):
        s = full[j]
        return (1, 0.0, j) if np.isnan(s) else (0, -s, j)
    best = None
    for sub in itertools.combinations(rest, topk - len(forced)):
        key = sorted(rank(j) for j in sub)
        if best is None or key < best[0]:
            best = (key, sub)
    return sorted(forced | set(best[1]))


def test_bruteforce_tiny_rows():
    rng = np.random.default_rng(5)
    for _ in range(600):
        L = int(rng.integers(-1, 10))
        topk = int(rng.integers(1, 7))
        init = int(rng.integers(0, 5))
        local = int(rng.integers(1, 4))
        mkt = int(rng.integers(0, 12))
        # few distinct values, so ties are common; some NaN
        s = rng.integers(0, 4, size=max(L, 0)).astype(np.float64)
        if L > 0 and rng.random() < 0.2:
            s[rng.integers(0, L)] = np.nan
        got = oracle.select_forced_row(s, L, topk, init, local, mkt)
        want = _brute(s, L, topk, init, local, mkt)
        assert list(got) == want, (s, L, topk, init, local, mkt, got, want)


def test_bruteforce_tiny_rows_local_page_competing():
    """No trailing window (local_blocks = 0, or init_blocks >= topk): the
    local page competes on its causal-prefix score; topk beyond 16 too."""
    rng = np.random.default_rng(15)
    for _ in range(600):
        L = int(rng.integers(-1, 11))
        topk = int(rng.integers(1, 8))
        init = int(rng.integers(0, 5))
        local = int(rng.integers(0, 3))
        mkt = int(rng.integers(0, 12))
        s = rng.integers(0, 4, size=max(L, 0)).astype(np.float64)
        if L > 0 and rng.random() < 0.2:
            s[rng.integers(0, L)] = np.nan
        ls = float(rng.integers(0, 4)) if rng.random() > 0.1 else np.nan
        got = oracle.select_forced_row(s, L, topk, init, local, mkt, local_score=ls)
        want = _brute(s, L, topk, init, local, mkt, local_score=ls)
        assert list(got) == want, (s, L, topk, init, local, mkt, ls, got, want)
    # a large topk over a long row: the forced windows and the best pages
    s = rng.standard_normal(300)
    got = oracle.select_forced_row(s, 300, 64, 3, 0, 10 ** 6, local_score=10.0)
    order = [j for j in np.argsort(-s, kind="stable") if j >= 3][:60]
    assert list(got) == sorted([0, 1, 2, 300] + order)


def test_local_page_competes_special_cases():
    s = np.array([5.0, 1.0, 4.0, 2.0, 3.0, 0.0, 6.0, 7.0])      # history 0..7, L = 8
    # a high local score takes a slot, a low one does not
    assert list(oracle.select_forced_row(s, 8, 4, 0, 0, 9, local_score=6.5)) == [0, 6, 7, 8]
    assert list(oracle.select_forced_row(s, 8, 4, 0, 0, 9, local_score=0.5)) == [0, 2, 6, 7]
    # a tie with a history page at the last slot goes to the lower id (page 6)
    assert list(oracle.select_forced_row(s, 8, 2, 0, 0, 9, local_score=6.0)) == [6, 7]
    assert list(oracle.select_forced_row(s, 8, 3, 0, 0, 9, local_score=6.0)) == [6, 7, 8]
    # NaN ranks last
    assert list(oracle.select_forced_row(s, 8, 4, 1, 0, 9, local_score=np.nan)) == [0, 2, 6, 7]
    # init_blocks >= topk leaves no trailing window either: leading pages only
    assert list(oracle.select_forced_row(s, 8, 4, 9, 1, 9, local_score=None)) == [0, 1, 2, 3]
    # the local score is demanded exactly when the local page competes
    with pytest.raises(ValueError):
        oracle.select_forced_row(s, 8, 4, 0, 0, 9)
    assert list(oracle.select_forced_row(s[:3], 3, 4, 0, 0, 9)) == [0, 1, 2, 3]


def test_default_configuration_selects_the_sixteen_slot_set():
    rng = np.random.default_rng(6)
    for _ in range(200):
        L = int(rng.integers(0, 60))
        s = rng.standard_normal(L)
        a = oracle.select_forced_row(s, L, 16, 0, 1, 10 ** 6)
        b = oracle.select_row(s, L)
        assert set(a[a >= 0]) == set(b[b >= 0])


def test_special_cases():
    s = np.array([5.0, 1.0, 4.0, 2.0, 3.0, 0.0, 6.0, 7.0])      # pages 0..7, L = 8
    # a padding row
    assert list(oracle.select_forced_row(s, -1, 4, 1, 1, 9)) == [-1] * 4
    # at most topk valid pages: all of them, ascending
    assert list(oracle.select_forced_row(s[:3], 3, 4, 0, 1, 9)) == [0, 1, 2, 3]
    # init_blocks >= topk: the leading pages only (no score is consulted)
    assert list(oracle.select_forced_row(s, 8, 4, 7, 1, 9)) == [0, 1, 2, 3]
    # max_k_tiles = 0 removes the leading window: the 3 best history pages
    # (7, 6, 0) and the local page
    assert list(oracle.select_forced_row(s, 8, 4, 3, 1, 0)) == [0, 6, 7, 8]
    # with max_k_tiles = 2 the leading window is pages 0, 1
    assert list(oracle.select_forced_row(s, 8, 4, 3, 1, 2)) == [0, 1, 7, 8]
    # a wide local window is clamped to topk - force_begin
    assert list(oracle.select_forced_row(s, 8, 4, 1, 9, 9)) == [0, 6, 7, 8]
    # the worked row: forced {0} and {8}; best two of pages 1..7 are 7 and 6
    assert list(oracle.select_forced_row(s, 8, 4, 1, 1, 9)) == [0, 6, 7, 8]
    assert list(oracle.select_forced_row(s, 8, 5, 1, 1, 9)) == [0, 2, 6, 7, 8]
    assert list(oracle.select_forced_row(s, 8, 5, 0, 2, 9)) == [0, 2, 6, 7, 8]


def test_output_form():
    rng = np.random.default_rng(7)
    for _ in range(300):
        L = int(rng.integers(-1, 40))
        topk = int(rng.integers(1, 17))
        init = int(rng.integers(0, 6))
        out = oracle.select_forced_row(rng.standard_normal(max(L, 0)), L, topk, init,
                                       int(rng.integers(1, 4)), 64)
        ids = out[out >= 0]
        assert np.all(out[len(ids):] == -1)                 # -1 only as a tail
        assert np.all(np.diff(ids) > 0)                     # ascending, distinct
        assert len(ids) == (0 if L < 0 else min(topk, L + 1))
        if L >= 0:
            assert ids.max() <= L
            if min(init, 64) < topk:                        # a trailing window exists
                assert L in ids


def test_rejects_unserved_configurations():
    with pytest.raises(ValueError):
        oracle.select_forced_row(np.zeros(4), 4, 4, 0, -1, 9)
    with pytest.raises(ValueError):
        oracle.select_forced_row(np.zeros(4), 4, 0, 0, 1, 9)
