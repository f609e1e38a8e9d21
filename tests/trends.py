"""Monotone-score workloads: constructed K and Q whose page scores are exact
and strictly increasing (or decreasing) in the logical page id.

Every query row is all ones (E4M3 0x38 = 1.0), so a page's score is the sum of
its dequantized K values.  Token 0 of page j is a vector of E2M1 grid values
whose 32-dim blocks each contain a 4.0 (so every E8M0 scale is exactly 1 and
every value is stored exactly) summing to 16 + 0.5 * m(j); every other token
is zero.  With m(j) = j the scores rise with j (every page is a record of
the running top-15); with m(j) = J - j they fall.
"""

import numpy as np

import workloads as W

E4M3_ONE = 0x38


def token_with_sum(total):
    """128 values on the E2M1 grid (scale 1) with block maxima 4.0 and the
    given sum (a multiple of 0.5, 16 <= total <= 500)."""
    assert total >= 16 and (total * 2) == int(total * 2) and total <= 500
    k = np.zeros(128, dtype=np.float32)
    k[[0, 32, 64, 96]] = 4.0
    rest = total - 16.0
    free = [d for d in range(128) if d % 32 != 0]
    i = 0
    while rest >= 4.0:
        k[free[i]] = 4.0
        rest -= 4.0
        i += 1
    # 0 <= rest < 4 in steps of 0.5: at most two grid values
    for v in (3.0, 2.0, 1.5, 1.0, 0.5):
        if rest >= v:
            k[free[i]] = v
            rest -= v
            i += 1
    assert rest == 0.0
    return k


def make_trend(name, seed, direction):
    """The workload `name` with constructed K and Q; direction +1: scores
    rise with the page id, -1: they fall."""
    w = W.make_workload(name, seed)
    w.q_codes = np.full_like(w.q_codes, E4M3_ONE)

    def k_rows(r):
        n = int(w.seq_lens[r])
        k = np.zeros((n, 128), dtype=np.float32)
        pages = (n + 127) // 128
        for j in range(pages):
            m = j if direction > 0 else pages - 1 - j
            k[j * 128] = token_with_sum(16.0 + 0.5 * m)
        return k

    w.k_rows = k_rows
    return w
