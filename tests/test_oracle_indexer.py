"""Pins of the oracle's page scores and 16-slot selection (CPU only).

Each test checks the oracle against something other than itself: a hand-worked
example, exact rational brute force, a heap selection, closed forms (one-hot
queries, zero queries, identical pages) and invariants of the method.
"""

import numpy as np
import torch
import pytest

import oracle
import workloads as W
from tests import pins


def _hand_pool(ex):
    num = ex["num_blocks"]
    pool = np.zeros((num, 128, 68), dtype=np.uint8)
    pool[:, :, 64:] = 127
    bt = ex["block_table_logical_to_physical"]
    for tk in ex["tokens"]:
        phys = bt[tk["page"]]
        t, d = tk["token"], tk["dim"]
        b = d // 2
        if d % 2 == 0:
            pool[phys, t, b] = (pool[phys, t, b] & 0xF0) | tk["code"]
        else:
            pool[phys, t, b] = (pool[phys, t, b] & 0x0F) | (tk["code"] << 4)
        pool[phys, t, 64 + d // 32] = tk["scale_byte"]
    return pool.reshape(num, 8704), np.array([bt], dtype=np.int32)


def test_hand_worked_example():
    ex = pins.hand_example()
    pool, bt = _hand_pool(ex)
    H = len(ex["q_onehot_dims_per_head"])
    q = np.zeros((1, H, 128), dtype=np.uint8)
    for h, d in enumerate(ex["q_onehot_dims_per_head"]):
        q[0, h, d] = 0x38                      # E4M3 1.0
    out, scores, L = oracle.oracle_decode(q, pool, bt, np.array([ex["seq_len"]]),
                                          ex["query_len"])
    assert out[0].tolist() == ex["expected"]
    for h in range(H):
        assert scores[0][h].tolist() == ex["expected_scores"][h]


def _random_case(rng, n_pages, dup=True):
    """Random page bytes (scale bytes 120..134, no NaN), with duplicated pages
    to create exact ties."""
    pool = rng.integers(0, 256, size=(n_pages, 128, 68), dtype=np.uint8)
    pool[:, :, 64:] = rng.integers(120, 135, size=(n_pages, 128, 4))
    if dup and n_pages >= 4:
        pool[1] = pool[3]                      # an exact tie between pages
    return pool.reshape(n_pages, 8704)


def _random_q(rng, shape):
    q = rng.integers(0, 256, size=shape, dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x38              # no NaN codes
    return q


def test_exact_bruteforce_decode():
    rng = np.random.default_rng(1)
    pool = _random_case(rng, 7)
    seq_lens = np.array([3 * 128 + 5, 2, 6 * 128 + 1], dtype=np.int32)  # one padding row
    ql, H = 3, 2
    bt = np.array([[4, 1, 3, 0, 6, 6, 6, 6], [5, 6, 6, 6, 6, 6, 6, 6],
                   [2, 1, 3, 0, 4, 5, 6, 6]], dtype=np.int32)
    q = _random_q(rng, (len(seq_lens) * ql, H, 128))
    scale = 0.375
    out, scores, L = oracle.oracle_decode(q, pool, bt, seq_lens, ql, scale)
    # the q_len rows of a request are its last q_len token positions
    req = [r for r in range(len(seq_lens)) for _ in range(ql)]
    pos = [p for s in seq_lens for p in range(int(s) - ql, int(s))]
    ex_out, ex_sc = pins.Exact().run(q, pool, bt, req, pos, scale)
    assert np.array_equal(out, ex_out)
    for (row, h), s in ex_sc.items():
        assert scores[row][h].tolist() == [float(x) for x in s]
    pins.check_invariants(out, L)


def test_exact_bruteforce_decode_bf16_queries():
    """bfloat16 index-Q (the other dtype of the vllm "indexer_mxfp4" page's
    scorers): the oracle against exact rationals from torch's bf16 cast."""
    rng = np.random.default_rng(11)
    pool = _random_case(rng, 5)
    seq_lens = np.array([2 * 128 + 9, 4 * 128 + 1], dtype=np.int32)
    ql, H = 2, 2
    bt = np.array([[3, 0, 4, 4, 4], [1, 2, 0, 3, 4]], dtype=np.int32)
    qf = rng.standard_normal((len(seq_lens) * ql, H, 128)).astype(np.float32) * 3.0
    q = torch.from_numpy(qf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    out, scores, L = oracle.oracle_decode(q, pool, bt, seq_lens, ql, 0.5, q_dtype="bf16")
    req = [r for r in range(len(seq_lens)) for _ in range(ql)]
    pos = [p for s in seq_lens for p in range(int(s) - ql, int(s))]
    ex_out, ex_sc = pins.Exact().run(q, pool, bt, req, pos, 0.5, q_dtype="bf16")
    assert np.array_equal(out, ex_out)
    for (row, h), s in ex_sc.items():
        assert scores[row][h].tolist() == [float(x) for x in s]
    pins.check_invariants(out, L)


def test_exact_bruteforce_prefill():
    rng = np.random.default_rng(2)
    pool = _random_case(rng, 6)
    ctx = np.array([250, 0], dtype=np.int32)
    new = np.array([270, 3], dtype=np.int32)
    cu = np.array([0, 270, 273], dtype=np.int32)
    bt = np.array([[5, 3, 1, 0, 2, 4], [4, 0, 0, 0, 0, 0]], dtype=np.int32)
    H = 1
    q = _random_q(rng, (273, H, 128))
    # exact run on a sample of rows spanning page boundaries
    sample = np.array([0, 5, 6, 133, 134, 261, 262, 269, 270, 272])
    out, scores, L = oracle.oracle_prefill(q, pool, bt, cu, ctx + new, ctx, 1.0)
    # chunk rows follow the request's context tokens
    req = np.array([0] * 270 + [1] * 3)
    pos = np.array(list(range(250, 250 + 270)) + [0, 1, 2])
    ex_out, ex_sc = pins.Exact().run(q[sample], pool, bt, req[sample], pos[sample], 1)
    assert np.array_equal(out[sample], ex_out)
    pins.check_invariants(out, L)


def test_onehot_query_reads_single_dims():
    """q = e_d gives s_j = max_t k_t[d], read straight from the bytes."""
    rng = np.random.default_rng(4)
    pool = _random_case(rng, 3, dup=False)
    ex = pins.Exact()
    for d in [0, 1, 31, 32, 63, 64, 100, 127]:
        q = np.zeros((1, 1, 128), dtype=np.uint8)
        q[0, 0, d] = 0x38
        seq = np.array([3 * 128 + 1], dtype=np.int32)
        bt = np.array([[2, 0, 1, 1]], dtype=np.int32)
        _, scores, _ = oracle.oracle_decode(q, pool, bt, seq, 1)
        for j, phys in enumerate([2, 0, 1]):
            want = max(float(ex.token(pool[phys], t)[d]) for t in range(128))
            assert scores[0][0][j] == want, (d, j)


def test_zero_query_gives_ascending_ids():
    w = W.make_workload("decode_batch_small", 0)
    pool = W.host_pool(w, oracle.write_pages)
    q = np.zeros_like(w.q_codes)
    out, _, L = oracle.oracle_decode(q, pool, w.block_table, w.dec_seq_lens, w.query_len)
    for t in range(out.shape[0]):
        n = min(15, int(L[t]))
        assert out[t, 0, :n].tolist() == list(range(n))


def test_identical_pages_tie_to_lower_id():
    rng = np.random.default_rng(9)
    page = _random_case(rng, 1, dup=False)
    pool = np.repeat(page, 20, axis=0)
    q = _random_q(rng, (1, 1, 128))
    out, _, _ = oracle.oracle_decode(q, pool, np.array([np.arange(20)[::-1]], dtype=np.int32),
                                     np.array([20 * 128], dtype=np.int32), 1)
    assert out[0, 0].tolist() == list(range(15)) + [19]


def test_nan_scores_rank_last():
    s = np.array([1.0, np.nan, 3.0, np.nan, -np.inf])
    assert oracle.select_row(s, 5).tolist()[:5] == [2, 0, 4, 1, 3]


def test_nan_token_makes_page_nan_and_ranks_last():
    """OCP MX v1.0: E8M0 byte 0xFF is NaN and makes every value of its 32-dim
    block NaN; a dot product with a NaN term is NaN whatever query element
    meets it (0 x NaN is NaN in IEEE 754); the page max propagates it and NaN
    pages rank after every number, among themselves by lower id."""
    rng = np.random.default_rng(21)
    clean = _random_case(rng, 12, dup=False).reshape(12, 128, 68)
    pool = clean.copy()
    pool[5, 17, 64] = 0xFF          # block 0 of a token of physical page 5
    pool[8, 100, 67] = 0xFF         # block 3 of a token of physical page 8
    bt = np.array([np.arange(12)[::-1]], dtype=np.int32)      # logical j -> physical 11-j
    q = np.zeros((1, 1, 128), dtype=np.uint8)
    q[0, 0, 40] = 0x38               # one-hot on dim 40 (block 1): NaN blocks meet zeros
    seq = np.array([11 * 128 + 3], dtype=np.int32)            # history 0..10
    out, scores, L = oracle.oracle_decode(q, pool.reshape(12, 8704), bt, seq, 1)
    nan_logical = {11 - 5, 11 - 8}
    s = scores[0][0]
    assert set(np.nonzero(np.isnan(s))[0].tolist()) == nan_logical
    _, ex = pins.Exact().run(q, clean.reshape(12, 8704), bt, [0], [int(seq[0]) - 1], 1.0)
    finite = sorted((j for j in range(11) if j not in nan_logical),
                    key=lambda j: (-ex[(0, 0)][j], j))
    assert out[0, 0].tolist() == finite + sorted(nan_logical) + [-1] * 4 + [11]


def test_nan_query_element_makes_every_page_nan():
    """An E4M3 NaN byte (0x7F / 0xFF) in the query makes every dot product,
    hence every page score, NaN: all pages tie and go in id order."""
    rng = np.random.default_rng(22)
    pool = _random_case(rng, 30, dup=False)
    bt = np.array([np.arange(30)], dtype=np.int32)
    for code in (0x7F, 0xFF):
        q = _random_q(rng, (1, 1, 128))
        q[0, 0, 77] = code
        out, scores, _ = oracle.oracle_decode(q, pool, bt, np.array([25 * 128 + 1]), 1)
        assert np.all(np.isnan(scores[0][0]))
        assert out[0, 0].tolist() == list(range(15)) + [25]


def test_rows_past_max_pages_are_refused():
    """A row whose history needs block-table column max_pages or later is
    refused (all 16 slots -1, L = -1); a row whose history ends exactly at
    max_pages columns is served as without the bound."""
    w = W.make_workload("edge_short", 0)
    pool = W.host_pool(w, oracle.write_pages)
    base, _, Lb = oracle.oracle_decode(w.q_codes, pool, w.block_table, w.dec_seq_lens,
                                       w.query_len)
    mp = 2
    out, _, L = oracle.oracle_decode(w.q_codes, pool, w.block_table, w.dec_seq_lens,
                                     w.query_len, max_pages=mp)
    _, pos = oracle.rows_decode(w.dec_seq_lens, w.query_len)
    for t in range(len(pos)):
        if pos[t] >= 0 and pos[t] // 128 > mp:
            assert L[t] == -1 and np.all(out[t] == -1), t
        else:
            assert L[t] == Lb[t] and np.array_equal(out[t], base[t]), t
    assert (L == -1).sum() > (Lb == -1).sum() and (Lb == mp).any()


def test_local_page_scores_exact_bruteforce():
    """Causal local-page scores against exact rationals over tokens
    0 .. p % 128 of the row's own page (FlashInfer page, forward: causal)."""
    rng = np.random.default_rng(31)
    pool = _random_case(rng, 5, dup=False)
    bt = np.array([[3, 1, 4, 0, 2], [2, 0, 1, 3, 4]], dtype=np.int32)
    positions = [0, 1, 127, 128, 200, 255, 300, 511, 522]
    req = [i % 2 for i in range(len(positions))]
    q = _random_q(rng, (len(positions), 2, 128))
    got = oracle.oracle_local_scores(q, pool, bt, req, positions, scale=0.5)
    ex = pins.Exact()
    for t, p in enumerate(positions):
        page = pool[bt[req[t]][p // 128]]
        for h in range(2):
            qv = [ex.e4m3[int(c)] for c in q[t, h]]
            assert got[t, h] == float(0.5 * ex.page_score(page, qv, p % 128 + 1)), (t, h)
    # rows without a readable local page
    nan = oracle.oracle_local_scores(q[:2], pool, bt, [0, 1], [-1, 4 * 128 + 5], max_pages=4)
    assert np.all(np.isnan(nan))


def test_local_page_scores_causal_boundary():
    """A one-hot query reads one dim: of tokens ..., k-1, k, k+1 holding 2, 4
    and 6 (k = p % 128), the score is 4: the row's own token counts, the next
    one does not."""
    for k in (0, 1, 77, 126):
        page = np.zeros((1, 128, 68), dtype=np.uint8)
        page[0, :, 64:] = 127                     # scale 1
        if k > 0:
            page[0, k - 1, 5] = 0x04              # dim 10 (low nibble of byte 5): 2.0
        page[0, k, 5] = 0x06                      # 4.0
        page[0, k + 1, 5] = 0x07                  # 6.0
        q = np.zeros((1, 1, 128), dtype=np.uint8)
        q[0, 0, 10] = 0x38                        # 1.0 on dim 10
        bt = np.array([[0, 0, 0, 0]], dtype=np.int32)
        got = oracle.oracle_local_scores(q, page.reshape(1, 8704), bt, [0], [3 * 128 + k])
        assert got[0, 0] == 4.0, (k, got)


def test_heap_selection_agrees():
    rng = np.random.default_rng(12)
    for L in [0, 1, 7, 15, 16, 40, 300]:
        s = rng.integers(-5, 5, size=L).astype(np.float64)   # many ties
        assert oracle.select_row(s, L).tolist() == pins.heap_select(list(s), L)


@pytest.mark.parametrize("name", ["tiny_decode", "decode_batch_small", "multi_token_small",
                                  "edge_short", "edge_wide", "edge_heads5"])
def test_decode_invariants(name):
    w = W.make_workload(name, 0)
    pool = W.host_pool(w, oracle.write_pages)
    out, _, L = oracle.oracle_decode(w.q_codes, pool, w.block_table, w.dec_seq_lens, w.query_len)
    pins.check_invariants(out, L)
    req, pos = oracle.rows_decode(w.dec_seq_lens, w.query_len)
    assert np.array_equal(L, np.where(pos >= 0, pos // 128, -1))


@pytest.mark.parametrize("name", ["ragged_prefill_small", "edge_prefill"])
def test_prefill_invariants(name):
    w = W.make_workload(name, 0)
    pool = W.host_pool(w, oracle.write_pages)
    out, _, L = oracle.oracle_prefill(w.q_codes, pool, w.block_table, w.cu_seqlens_q,
                                      w.seq_lens, w.pre_ctx)
    pins.check_invariants(out, L)


def test_positive_scale_leaves_selection_unchanged():
    w = W.make_workload("multi_token_small", 1)
    pool = W.host_pool(w, oracle.write_pages)
    base, _, _ = oracle.oracle_decode(w.q_codes, pool, w.block_table, w.dec_seq_lens, w.query_len)
    for scale in [2.0, 0.5, 2.0 ** -20, 0.7, 3.3]:
        o, _, _ = oracle.oracle_decode(w.q_codes, pool, w.block_table, w.dec_seq_lens,
                                       w.query_len, scale)
        assert np.array_equal(o, base), scale


def test_doubling_query_codes_leaves_selection_unchanged():
    """Adding one to the E4M3 exponent field doubles every normal q value
    exactly; the selection must not move."""
    w = W.make_workload("decode_batch_small", 2)
    pool = W.host_pool(w, oracle.write_pages)
    q = w.q_codes.copy()
    e = (q >> 3) & 0xF
    ok = (e >= 1) & (e <= 13)
    q2 = q.copy()
    q2[ok] = q[ok] + 8
    q[~ok] = 0
    q2[~ok] = 0
    a, _, _ = oracle.oracle_decode(q, pool, w.block_table, w.dec_seq_lens, w.query_len)
    b, sb, _ = oracle.oracle_decode(q2, pool, w.block_table, w.dec_seq_lens, w.query_len)
    assert np.array_equal(a, b)


def test_physical_placement_does_not_matter():
    w = W.make_workload("mixed_small", 0)
    pool = W.host_pool(w, oracle.write_pages)
    out1, _, _ = oracle.oracle_decode(w.q_codes[:w.n_decode_rows], pool, w.block_table[:w.Rd],
                                      w.dec_seq_lens, w.query_len)
    perm = np.random.default_rng(99).permutation(w.num_blocks)
    pool2 = np.empty_like(pool)
    pool2[perm] = pool
    bt2 = perm[w.block_table].astype(np.int32)
    out2, _, _ = oracle.oracle_decode(w.q_codes[:w.n_decode_rows], pool2, bt2[:w.Rd],
                                      w.dec_seq_lens, w.query_len)
    assert np.array_equal(out1, out2)


def test_heads_are_independent():
    w = W.make_workload("ragged_prefill_small", 0)
    pool = W.host_pool(w, oracle.write_pages)
    out, _, _ = oracle.oracle_prefill(w.q_codes, pool, w.block_table, w.cu_seqlens_q,
                                      w.seq_lens, w.pre_ctx)
    for h in range(w.H):
        o1, _, _ = oracle.oracle_prefill(w.q_codes[:, h:h + 1], pool, w.block_table,
                                         w.cu_seqlens_q, w.seq_lens, w.pre_ctx)
        assert np.array_equal(o1[:, 0], out[:, h])


def test_prefill_row_equals_decode_row_at_same_position():
    w = W.make_workload("ragged_prefill_small", 3)
    pool = W.host_pool(w, oracle.write_pages)
    out, _, _ = oracle.oracle_prefill(w.q_codes, pool, w.block_table, w.cu_seqlens_q,
                                      w.seq_lens, w.pre_ctx)
    req, pos = oracle.rows_prefill(w.cu_seqlens_q, w.pre_ctx)
    for t in [0, 17, 128, 299, 300, 555, 899]:
        r = int(req[t])
        d, _, _ = oracle.oracle_decode(w.q_codes[t:t + 1], pool, w.block_table[r:r + 1],
                                       np.array([pos[t] + 1], dtype=np.int32), 1)
        assert np.array_equal(d[0], out[t])
        # a multi-query decode row at the same position agrees too
        d4, _, _ = oracle.oracle_decode(np.repeat(w.q_codes[t:t + 1], 4, axis=0), pool,
                                        w.block_table[r:r + 1],
                                        np.array([pos[t] + 4], dtype=np.int32), 4)
        assert np.array_equal(d4[0], out[t]) or pos[t] < 3


def test_planted_pages_dominate():
    w = W.make_workload("multi_token_small", 0)
    pool = W.host_pool(w, oracle.write_pages)
    out, _, L = oracle.oracle_decode(w.q_codes, pool, w.block_table, w.dec_seq_lens, w.query_len)
    hits = total = 0
    for r in range(w.Rd):
        planted = set(w.planted_pages(r).tolist())
        for i in range(w.query_len):
            row = r * w.query_len + i
            n = min(15, int(L[row]))
            top = set(out[row, 0, :min(n, len(planted))].tolist())
            hits += len(top & planted)
            total += min(n, len(planted))
    assert hits >= 0.9 * total
