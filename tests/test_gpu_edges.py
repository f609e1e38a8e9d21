"""GPU parity on edge inputs: NaN page tokens and NaN query elements (E4M3
and bfloat16), identical pages that tie on a non-zero score, and rows whose
history runs past the block-table columns the caller vouches for.

Readings (the oracle's): a token whose q.k is NaN makes its page's score NaN
and NaN pages rank after every number, by lower id among themselves; a row
whose local page lies past max_pages columns is refused (all 16 slots -1)
and flagged by error bit 2.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import checker, pins
from tests.gpu_common import (decode_error_bits, lib, prefill_error_bits, run_gpu,
                              run_oracle)
from workloads.device import DeviceWorkload

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(f"[gpu-test] {msg}", flush=True)


def _nan_case(q_dtype, seed):
    """mixed_small with E8M0 0xFF bytes in one token of several pages of every
    request (scale blocks 0..3 in turn) and NaN query elements in a few
    (row, head) pairs.  Returns the workload, its device copy and the host
    pool the oracle reads."""
    w = W.make_workload("mixed_small", seed, q_dtype=q_dtype)
    rng = np.random.default_rng([seed, 77])
    nan_q = {}
    for t in rng.choice(w.T, size=6, replace=False):
        h = int(rng.integers(w.H))
        d = int(rng.integers(128))
        nan_q[(int(t), h)] = d
        w.q_codes[t, h, d] = 0x7F if q_dtype == "e4m3" else 0x7FC0
    dw = DeviceWorkload(w, lib().mi_idx_insert_mxfp4)
    pool = W.host_pool(w, oracle.write_pages).reshape(w.num_blocks, 128, 68)
    dev = dw.pool.view(w.num_blocks, 128, 68)
    marks = []
    for r in range(len(w.seq_lens)):
        hist = max((int(w.seq_lens[r]) - 1) // 128, 0)
        if hist == 0:
            continue
        for i, j in enumerate(rng.choice(hist, size=min(4, hist), replace=False)):
            phys = int(w.block_table[r, j])
            tok = int(rng.integers(128))
            pool[phys, tok, 64 + i % 4] = 0xFF
            dev[phys, tok, 64 + i % 4] = 0xFF
            marks.append((r, int(j)))
    torch.cuda.synchronize()
    return w, dw, pool.reshape(w.num_blocks, 8704), marks, nan_q


@pytest.mark.parametrize("q_dtype", ["e4m3", "bf16"])
def test_nan_tokens_and_nan_queries(q_dtype):
    _banner(f"NaN tokens and queries ({q_dtype})")
    w, dw, pool, marks, nan_q = _nan_case(q_dtype, 11)
    out, sd, sp, _, _ = run_gpu(w, dw=dw, scores=True)
    ref, scores, L, _ = run_oracle(w, pool=pool)
    # the construction reaches the case: NaN pages inside the oracle's
    # selections, and rows whose every page is NaN
    nan_picked = sum(np.isnan(scores[t][h][ref[t, h, :min(15, int(L[t]))]]).any()
                     for t in range(w.T) for h in range(w.H) if L[t] > 0)
    assert nan_picked > 0
    for (t, h) in nan_q:
        if L[t] > 0:
            assert np.all(np.isnan(scores[t][h]))
    gs = np.concatenate([sd, sp])
    frac = checker.compare(out, ref, scores, L, gpu_scores=gs)
    _banner(f"NaN case {q_dtype}: exact fraction {frac:.4f}, {len(marks)} NaN pages, "
            f"{nan_picked} selections holding one")
    pins.check_invariants(out, L)


def _tie_rows(out, a, b, rows):
    """For every (row, head) holding both pages a < b, a comes first."""
    n = 0
    for t in rows:
        for h in range(out.shape[1]):
            ids = out[t, h, :15].tolist()
            if a in ids and b in ids:
                assert ids.index(a) < ids.index(b), (t, h, ids)
                n += 1
    return n


def test_identical_pages_tie_to_lower_id_decode_and_prefill():
    """Two logical pages that map to one physical page score identically
    (and non-zero): the lower logical id ranks first.  Decode: each
    request's first planted page (a clear winner) is mapped again at a
    later logical page.  Prefill: each request's most often top-ranked page
    is mapped again at the next logical page."""
    _banner("identical pages tie")
    w = W.make_workload("multi_token_small", 2)
    pairs = {}
    for r in range(w.Rd):
        pl = w.planted_pages(r)
        hist = max((int(w.seq_lens[r]) - 1) // 128, 0)
        if len(pl) == 0 or hist < 3:
            continue
        a = int(pl[0])
        b = next(j for j in range(hist - 1, -1, -1) if j != a and j not in set(pl.tolist()))
        w.block_table[r, b] = w.block_table[r, a]
        pairs[r] = (min(a, b), max(a, b))
    out, _, _, _, _ = run_gpu(w)
    ref, scores, L, _ = run_oracle(w)
    checker.compare(out, ref, scores, L)
    n = sum(_tie_rows(out, a, b, range(r * w.query_len, (r + 1) * w.query_len))
            for r, (a, b) in pairs.items())
    assert n >= len(pairs)

    wp = W.make_workload("ragged_prefill_small", 4)
    ref0, _, _, _ = run_oracle(wp)
    ppairs = {}
    for r in range(wp.Rp):
        sl = wp.request_slice(r)
        top = ref0[sl, :, 0].ravel()
        top = top[top >= 0]
        a = int(np.bincount(top).argmax())
        hist = max((int(wp.seq_lens[r]) - 1) // 128, 0)
        if a + 1 >= hist:
            continue
        wp.block_table[r, a + 1] = wp.block_table[r, a]
        ppairs[r] = (a, a + 1)
    out, _, _, _, _ = run_gpu(wp)
    ref, scores, L, _ = run_oracle(wp)
    checker.compare(out, ref, scores, L)
    n = sum(_tie_rows(out, a, b, range(wp.request_slice(r).start, wp.request_slice(r).stop))
            for r, (a, b) in ppairs.items())
    assert n > 0


@pytest.mark.parametrize("name,mp", [("mixed_small", 20), ("edge_short", 2),
                                     ("ragged_prefill_small", 10)])
def test_rows_past_max_pages_are_refused(name, mp):
    """Rows whose history runs past max_pages block-table columns are refused
    (all 16 slots -1), the others are served as usual; error bit 2 of the
    decode workspace / prefill plan reports it, and a run with a wide enough
    bound leaves both error words clear."""
    _banner(f"refused rows {name} max_pages {mp}")
    w = W.make_workload(name, 5)
    out, _, _, dw, step = run_gpu(w, max_pages=mp)
    ref, scores, L, _ = run_oracle(w, max_pages=mp)
    checker.compare(out, ref, scores, L)
    req_d, pos_d = oracle.rows_decode(w.dec_seq_lens, w.query_len) if w.Rd else ([], [])
    refused_d = any(p >= 0 and p // 128 > mp for p in pos_d)
    if w.Rp:
        _, pos_p = oracle.rows_prefill(w.cu_seqlens_q, w.pre_ctx)
        refused_p = bool(np.any(pos_p // 128 > mp))
    else:
        refused_p = False
    assert refused_d or refused_p
    if w.Rd:
        assert bool(decode_error_bits(step) & 4) == refused_d
    if w.Rp:
        assert bool(prefill_error_bits(step) & 4) == refused_p
    _, _, _, _, step2 = run_gpu(w, dw=dw)
    if w.Rd:
        assert decode_error_bits(step2) == 0
    if w.Rp:
        assert prefill_error_bits(step2) == 0
