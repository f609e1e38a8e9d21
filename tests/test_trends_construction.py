"""The monotone-score construction, checked with the oracle on the CPU: the
stored pages decode to exactly the intended scores."""

import numpy as np

import oracle
import workloads as W
from tests.trends import make_trend, token_with_sum


def test_token_sums_are_exact_after_mxfp4():
    for total in [16.0, 16.5, 19.5, 20.0, 23.5, 100.0, 499.5, 500.0]:
        k = token_with_sum(total)
        pages = np.zeros((1, 8704), dtype=np.uint8)
        oracle.write_pages(pages, np.array([0]), k[None, :])
        dec = oracle.decode_pages(pages)[0, 0]
        assert np.array_equal(dec, k.astype(np.float64))
        assert dec.sum() == total


def test_trend_scores_are_monotone():
    for direction in (1, -1):
        w = make_trend("trend_decode", 0, direction)
        pool = W.host_pool(w, oracle.write_pages)
        _, scores, L = oracle.oracle_decode(w.q_codes[:w.n_decode_rows], pool,
                                            w.block_table[:w.Rd], w.dec_seq_lens, w.query_len)
        s = np.asarray(scores[0][0])           # row 0, head 0: pages 0..L-1
        d = np.diff(s)
        assert (d > 0).all() if direction > 0 else (d < 0).all()
