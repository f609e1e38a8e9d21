"""The general selection on the GPU, through the C ABI: a score call with
scores_out, mi_idx_score_local (each row's own page over its causal prefix)
and mi_idx_select_topk, against the oracle's select_forced_row on the
oracle's page scores and local-page scores -- topk up to 64, leading and
trailing windows with the flashinfer page's clamps, and local_blocks = 0,
where the local page competes."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import checker
from tests.gpu_common import lib, oracle_rows_parallel, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

# (topk, init_blocks, local_blocks)
CONFIGS = [(16, 0, 1), (24, 0, 1), (32, 2, 1), (64, 0, 0), (8, 1, 0), (20, 3, 2), (1, 0, 0),
           (40, 0, 0), (16, 0, 0), (5, 9, 0), (33, 1, 3)]


def _device_rows(w, dw):
    """Decode then prefill: (q, block table, local-score call kwargs, rows)."""
    parts = []
    if w.Rd:
        parts.append((dw.q_dec, dw.bt_dec, dict(seq_lens=dw.sl_dec, query_len=w.query_len)))
    if w.Rp:
        parts.append((dw.q_pre, dw.bt_pre, dict(cu_seqlens_q=dw.cu, context_lens=dw.ctx)))
    return parts


def _local_scores(w, dw, max_pages):
    m = lib()
    outs = [m.mi_idx_score_local(q, dw.pool, bt, max_pages, **kw) for q, bt, kw in
            _device_rows(w, dw)]
    torch.cuda.synchronize()
    return torch.cat(outs)


def _oracle_local(w, pool):
    parts = []
    if w.Rd:
        req, pos = oracle.rows_decode(w.dec_seq_lens, w.query_len)
        parts.append(oracle.oracle_local_scores(w.q_codes[:w.n_decode_rows], pool,
                                                w.block_table[:w.Rd], req, pos,
                                                q_dtype=w.q_dtype, max_pages=w.width))
    if w.Rp:
        req, pos = oracle.rows_prefill(w.cu_seqlens_q, w.pre_ctx)
        parts.append(oracle.oracle_local_scores(w.q_codes[w.n_decode_rows:], pool,
                                                w.block_table[w.Rd:], req, pos,
                                                q_dtype=w.q_dtype, max_pages=w.width))
    return np.concatenate(parts)


@pytest.mark.parametrize("name", ["mixed_small", "edge_wide", "edge_prefill", "multi_token_small",
                                  "edge_short", "prefill_h1_small", "edge_heads5"])
def test_general_selection_parity(name):
    print(f"[gpu-test] general selection {name}", flush=True)
    m = lib()
    w = W.make_workload(name, 0)
    out, sd, sp, dw, _ = run_gpu(w, scores=True)
    ref, scores, L, pool = run_oracle(w)
    gs = torch.from_numpy(np.concatenate([x for x in (sd, sp) if x is not None and len(x)])).cuda()
    loc = _local_scores(w, dw, w.width)
    loc_o = _oracle_local(w, pool)
    loc_g = loc.cpu().numpy().astype(np.float64)
    # local scores: NaN exactly where the oracle has none, else within the
    # row's tolerance (1e-4 x the largest |score| of its history and local page)
    assert np.array_equal(np.isnan(loc_g), np.isnan(loc_o))
    for t in range(w.T):
        for h in range(w.H):
            if np.isnan(loc_o[t, h]):
                continue
            base = np.abs(np.append(scores[t][h], loc_o[t, h]))
            assert abs(loc_g[t, h] - loc_o[t, h]) <= checker.REL_TOL * base.max(), (t, h)
    full = [[np.append(scores[t][h], loc_o[t, h]) if L[t] >= 0 else np.zeros(0)
             for h in range(w.H)] for t in range(w.T)]
    mkt = int(-(-int(np.max(w.seq_lens)) // 128))
    for topk, init, local in CONFIGS:
        for max_k_tiles in (mkt, 1):
            g = m.mi_idx_select_topk(dw.out, gs, topk, init, local, max_k_tiles,
                                     local_scores=loc)
            torch.cuda.synchronize()
            g = g.cpu().numpy()
            o = [[oracle.select_forced_row(scores[t][h] if L[t] > 0 else np.zeros(0), int(L[t]),
                                           topk, init, local, max_k_tiles,
                                           local_score=loc_o[t, h])
                  for h in range(w.H)] for t in range(w.T)]
            frac = checker.compare_forced(g, o, full, L, topk, init, local, max_k_tiles)
            print(f"[gpu-test] {name} topk={topk} init={init} local={local} "
                  f"max_k_tiles={max_k_tiles}: exact {frac:.4f}", flush=True)
            if topk <= 16 and local >= 1:
                # the fast path from the ranked rows gives the same selection
                f = m.mi_idx_select_forced(dw.out, topk, init, local, max_k_tiles)
                torch.cuda.synchronize()
                assert np.array_equal(f.cpu().numpy(), g)


def test_general_selection_bf16_and_nan():
    """bfloat16 queries, NaN tokens on the local pages, topk 64 and 8."""
    print("[gpu-test] general selection bf16 + NaN", flush=True)
    m = lib()
    w = W.make_workload("mixed_small", 2, q_dtype="bf16")
    out, sd, sp, dw, _ = run_gpu(w, scores=True)
    pool = W.host_pool(w, oracle.write_pages).reshape(w.num_blocks, 128, 68)
    # a NaN scale in token 0 of every request's last page (a local page of
    # its last rows; token 0 is in every causal prefix)
    dev = dw.pool.view(w.num_blocks, 128, 68)
    for r in range(len(w.seq_lens)):
        last = int(w.block_table[r, (int(w.seq_lens[r]) - 1) // 128])
        pool[last, 0, 65] = 0xFF
        dev[last, 0, 65] = 0xFF
    torch.cuda.synchronize()
    pool = pool.reshape(w.num_blocks, 8704)
    ref, scores, L, _ = run_oracle(w, pool=pool)
    gs = torch.from_numpy(np.concatenate([sd, sp])).cuda()
    loc = _local_scores(w, dw, w.width)
    loc_o = _oracle_local(w, pool)
    assert np.isnan(loc_o).sum() > 0
    assert np.array_equal(np.isnan(loc.cpu().numpy()), np.isnan(loc_o))
    full = [[np.append(scores[t][h], loc_o[t, h]) if L[t] >= 0 else np.zeros(0)
             for h in range(w.H)] for t in range(w.T)]
    for topk, init, local in ((64, 0, 0), (8, 0, 0), (24, 2, 1)):
        g = m.mi_idx_select_topk(dw.out, gs, topk, init, local, 10 ** 6, local_scores=loc)
        torch.cuda.synchronize()
        o = [[oracle.select_forced_row(scores[t][h] if L[t] > 0 else np.zeros(0), int(L[t]),
                                       topk, init, local, 10 ** 6, local_score=loc_o[t, h])
              for h in range(w.H)] for t in range(w.T)]
        checker.compare_forced(g.cpu().numpy(), o, full, L, topk, init, local, 10 ** 6)


def test_general_selection_argument_errors_and_empty():
    m = lib()
    w = W.make_workload("tiny_decode", 0)
    out, sd, _, dw, _ = run_gpu(w, scores=True)
    gs = torch.from_numpy(sd).cuda()
    with pytest.raises(m.MiIdxError):        # the local page competes: local scores needed
        m.mi_idx_select_topk(dw.out, gs, 8, 0, 0, 100)
    with pytest.raises(m.MiIdxError):
        m.mi_idx_select_topk(dw.out, gs, 0, 0, 1, 100)
    with pytest.raises(m.MiIdxError):
        m.mi_idx_select_topk(dw.out, gs, m.MAX_TOPK + 1, 0, 1, 100)
    # no local scores needed when the leading window fills topk
    m.mi_idx_select_topk(dw.out, gs, 8, 9, 0, 100)
    empty = torch.empty((0, 1, 16), dtype=torch.int32, device="cuda")
    assert m.mi_idx_select_topk(empty, torch.empty((0, 1, 5), device="cuda"), 8, 0, 1,
                                10).shape == (0, 1, 8)


def _direct_rows(rng, n, stride):
    """n synthetic (row, head) rows: local pages L (slot 15 of ranked) from
    -1 (padding) through stride, and float32 scores of four kinds -- normal,
    three values only (ties everywhere), a fifth NaN, and signed zeros among
    tiny numbers."""
    L = rng.integers(0, stride + 1, size=n).astype(np.int32)
    L[:6] = [-1, 0, 1, 63, 64, stride]
    s = rng.normal(3.0, 1.0, size=(n, stride))
    s[1::4] = rng.integers(0, 3, size=s[1::4].shape)
    nan = rng.random(size=(n, stride)) < 0.2
    s[2::4] = np.where(nan[2::4], np.nan, s[2::4])
    s[3::4] = rng.choice(np.array([0.0, -0.0, 1e-30, -1e-30]), size=s[3::4].shape)
    loc = rng.normal(3.0, 1.0, size=n)
    loc[1::4] = rng.integers(0, 3, size=loc[1::4].shape)
    loc[2::8] = np.nan
    ranked = np.full((n, 16), -1, dtype=np.int32)
    ranked[:, 15] = L
    return ranked, s.astype(np.float32), loc.astype(np.float32)


@pytest.mark.parametrize("stride", [300, 900, 2100, 5000])
def test_select_topk_direct_rows(stride):
    """mi_idx_select_topk alone, on synthetic rows whose candidates span every
    register size of the selection (up to 512, 1024, 2048) and rows of more
    than 2048 candidates (read again at every radix pass), with ties, NaN and
    signed zeros: the same ids as the oracle's select_forced_row, exactly."""
    print(f"[gpu-test] direct selection stride={stride}", flush=True)
    m = lib()
    rng = np.random.default_rng(stride)
    ranked, s, loc = _direct_rows(rng, 64, stride)
    dr, ds, dl = (torch.from_numpy(x).cuda() for x in (ranked, s, loc))
    for topk, init, local, mkt in ((64, 0, 0, 10 ** 6), (1, 0, 0, 10 ** 6), (300, 2, 0, 10 ** 6),
                                   (1024, 0, 1, 10 ** 6), (17, 3, 2, 5), (700, 0, 0, 40),
                                   (16, 1, 0, 10 ** 6)):
        g = m.mi_idx_select_topk(dr, ds, topk, init, local, mkt, local_scores=dl)
        torch.cuda.synchronize()
        g = g.cpu().numpy()
        for i in range(len(ranked)):
            Li = int(ranked[i, 15])
            o = oracle.select_forced_row(s[i, :max(Li, 0)].astype(np.float64), Li, topk, init,
                                         local, mkt, local_score=float(loc[i]))
            assert np.array_equal(g[i], o), (stride, topk, init, local, mkt, i, Li)


@pytest.mark.slow
def test_full_size_general_selection():
    """The mixed step at full size (16 448 rows, 4 heads, 57 768 + 2 174 history
    pages) through the general path as the benchmark times it: a score call
    writing every page score, the local scores, and topk 64 with
    local_blocks = 0.  Against the oracle on every 4th decode request and a
    whole row tile of each prefill request: local scores within the
    tolerance, selections rank by rank."""
    print("[gpu-test] full-size general selection", flush=True)
    m = lib()
    w = W.make_workload("mixed_step", 0)
    out, sd, sp, dw, _ = run_gpu(w, scores=True)
    gs = torch.from_numpy(np.concatenate([sd, sp])).cuda()
    del sd, sp
    loc = _local_scores(w, dw, w.width)
    mkt = int(-(-int(np.max(w.seq_lens)) // 128))
    topk = 64
    g = m.mi_idx_select_topk(dw.out, gs, topk, 0, 0, mkt, local_scores=loc)
    torch.cuda.synchronize()
    g, loc_g = g.cpu().numpy(), loc.cpu().numpy().astype(np.float64)
    del gs
    M = 256 // w.H
    jobs = [(r, np.arange(w.query_len)) for r in range(0, w.Rd, 4)]
    jobs.append((w.Rd, np.arange(8192 - M, 8192)))
    jobs.append((w.Rd + 1, np.arange(64 * M, 65 * M)))
    print(f"[gpu-test] oracle on {sum(len(x) for _, x in jobs)} rows", flush=True)
    compared = 0
    for T, _, sc, L, lo in oracle_rows_parallel(w, jobs, local=True):
        for i, t in enumerate(T):
            for h in range(w.H):
                if np.isnan(lo[i, h]):
                    assert np.isnan(loc_g[t, h])
                    continue
                base = np.abs(np.append(sc[i][h], lo[i, h])).max()
                assert abs(loc_g[t, h] - lo[i, h]) <= checker.REL_TOL * base, (t, h)
        o = [[oracle.select_forced_row(sc[i][h], int(L[i]), topk, 0, 0, mkt,
                                       local_score=lo[i, h]) for h in range(w.H)]
             for i in range(len(T))]
        full = [[np.append(sc[i][h], lo[i, h]) for h in range(w.H)] for i in range(len(T))]
        checker.compare_forced(g[T], o, full, L, topk, 0, 0, mkt)
        compared += len(T)
    print(f"[gpu-test] full-size general selection: {compared} rows x {w.H} heads match",
          flush=True)
