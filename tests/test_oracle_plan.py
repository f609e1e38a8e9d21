"""Pins of the oracle's prefill chunking (CPU only)."""

import numpy as np

import oracle
from oracle import plan as P


def test_max_gather_pages_closed_form():
    # ceil(max(65536, 4 * 32768) / 128) = 1024
    assert oracle.max_gather_pages(65536, 32768) == 1024
    assert oracle.max_gather_pages(1000, 1) == 8           # ceil(1000/128)
    assert oracle.max_gather_pages(128, 32) == 1


def _brute_chunks(h, budget):
    """Every split into consecutive non-empty groups, keeping the one a greedy
    left-to-right packer must produce: each group is as long as possible."""
    out = []
    i = 0
    while i < len(h):
        best = i + 1
        for j in range(i + 1, len(h) + 1):
            if j == i + 1 or sum(h[i:j]) <= budget:
                best = j
            else:
                break
        out.append((i, best, sum(h[i:best])))
        i = best
    return out


def test_chunks_against_bruteforce_and_properties():
    rng = np.random.default_rng(0)
    for _ in range(200):
        n = int(rng.integers(1, 12))
        seq = rng.integers(1, 3000, size=n)
        budget = int(rng.integers(0, 40))
        h = [max((int(s) - 1) // 128, 0) for s in seq]
        ch = oracle.prefill_chunks(seq, budget)
        assert ch == _brute_chunks(h, budget)
        assert ch[0][0] == 0 and ch[-1][1] == n
        for (a, b, tot), nxt in zip(ch, ch[1:] + [None]):
            assert b > a
            assert tot == sum(h[a:b])
            assert tot <= budget or b == a + 1
            if nxt is not None:
                assert tot + h[b] > budget


def test_chunks_extremes():
    seq = [129, 1000, 5000, 1]
    assert oracle.prefill_chunks(seq, 10 ** 9) == [(0, 4, 1 + 7 + 39 + 0)]
    assert [c[:2] for c in oracle.prefill_chunks(seq, 0)] == [(0, 1), (1, 2), (2, 3), (3, 4)]
    assert [c[:2] for c in oracle.prefill_chunks(seq, 39)] == [(0, 2), (2, 4)]
    assert list(P.history_pages([0, 1, 128, 129, 256, 257])) == [0, 0, 0, 1, 1, 2]
