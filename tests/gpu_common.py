"""Helpers of the GPU tests: run a workload through the library and through
the oracle."""

import multiprocessing
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import torch

import oracle
import workloads as W
from workloads.device import DeviceWorkload


def lib():
    import sparse_attention_block_mxfp4_amd as m
    return m


def run_gpu(w, dw=None, scale=1.0, budget=None, seq_lens_host_ub=None, scores=False,
            max_pages=None, layers=1):
    """Plan + score the workload's decode and prefill rows; returns
    (out [T,H,16] numpy, decode scores, prefill scores, DeviceWorkload)."""
    m = lib()
    from sparse_attention_block_mxfp4_amd.step import IndexerStep
    if dw is None:
        dw = DeviceWorkload(w, m.mi_idx_insert_mxfp4)
    mp = w.width if max_pages is None else max_pages
    step = IndexerStep(w.H, mp, max_decode_reqs=w.Rd, query_len=max(w.query_len, 1),
                       max_prefill_reqs=w.Rp, max_prefill_rows=w.n_prefill_rows)
    sl_pre_host = w.seq_lens[w.Rd:] if seq_lens_host_ub is None else seq_lens_host_ub
    step.plan(dw.sl_dec if w.Rd else None, w.cu_seqlens_q if w.Rp else None,
              sl_pre_host if w.Rp else None,
              gather_budget_pages=(w.budget or 0) if budget is None else budget)
    dw.out.fill_(-7)
    sd = sp = None
    if scores:
        sd = torch.full((w.n_decode_rows, w.H, mp), float("nan"), device=dw.device)
        sp = torch.full((w.n_prefill_rows, w.H, mp), float("nan"), device=dw.device)
    for _ in range(layers):
        if w.Rd:
            step.decode(dw.q_dec, dw.pool, dw.bt_dec, dw.sl_dec, dw.out[:dw.nd], scale=scale,
                        scores_out=sd)
        if w.Rp:
            step.prefill(dw.q_pre, dw.pool, dw.bt_pre, dw.cu, dw.sl_pre, dw.ctx, dw.out[dw.nd:],
                         scale=scale, scores_out=sp)
    torch.cuda.synchronize()
    out = dw.out.cpu().numpy()
    return (out, None if sd is None else sd.cpu().numpy(),
            None if sp is None else sp.cpu().numpy(), dw, step)


def run_oracle(w, pool=None, scale=1.0, max_pages=None):
    """Oracle outputs of the whole workload (small workloads only)."""
    if pool is None:
        pool = W.host_pool(w, oracle.write_pages)
    outs, scs, Ls = [], [], []
    if w.Rd:
        o, s, L = oracle.oracle_decode(w.q_codes[:w.n_decode_rows], pool, w.block_table[:w.Rd],
                                       w.dec_seq_lens, w.query_len, scale, q_dtype=w.q_dtype,
                                       max_pages=max_pages)
        outs.append(o), scs.extend(s), Ls.append(L)
    if w.Rp:
        o, s, L = oracle.oracle_prefill(w.q_codes[w.n_decode_rows:], pool, w.block_table[w.Rd:],
                                        w.cu_seqlens_q, w.seq_lens[w.Rd:], w.pre_ctx, scale,
                                        q_dtype=w.q_dtype, max_pages=max_pages)
        outs.append(o), scs.extend(s), Ls.append(L)
    return np.concatenate(outs), scs, np.concatenate(Ls), pool


def oracle_request_rows(w, r, rows_in_req, scale=1.0, local=False):
    """Oracle outputs of selected rows of request r, from that request's own
    pages (encoded by the oracle from the generator's K rows).  With
    ``local``, also each row's local-page score ([n, H], over the causal
    prefix of its own page, NaN for a padding row)."""
    k = w.k_rows(r)
    npages = int(w.n_pages[r])
    pages = w.poisoned_pool()[:npages].copy()
    slots = np.arange(k.shape[0], dtype=np.int64)          # logical placement
    oracle.write_pages(pages, slots, k)
    rows_in_req = np.asarray(rows_in_req)
    if r < w.Rd:
        T0 = r * w.query_len
        pos = int(w.seq_lens[r]) - w.query_len + rows_in_req
    else:
        p = r - w.Rd
        T0 = w.n_decode_rows + int(w.cu_seqlens_q[p])
        pos = int(w.pre_ctx[p]) + rows_in_req
    q = oracle.q_values(w.q_codes[T0 + rows_in_req], w.q_dtype)
    hist = int(max(pos.max() // 128, 0)) if pos.max() >= 0 else 0
    kp = oracle.decode_pages(pages[:hist])
    out, sc, L = oracle.index_rows(q, pos, kp, scale)
    scores = [sc[i, :, :max(int(L[i]), 0)] for i in range(len(rows_in_req))]
    if not local:
        return T0 + rows_in_req, out, scores, L
    loc = np.full((len(rows_in_req), w.H), np.nan)
    for i, p in enumerate(pos):
        if p >= 0:
            kpage = oracle.decode_pages(pages[int(p) // 128:int(p) // 128 + 1])[0]
            loc[i] = scale * oracle.local_page_scores(q[i], kpage, int(p))
    return T0 + rows_in_req, out, scores, L, loc


def _one_thread_blas():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def oracle_rows_parallel(w, jobs, workers=None, local=False):
    """oracle_request_rows(w, r, rows) for every (r, rows) in ``jobs``, on CPU
    worker processes (fresh interpreters started by spawn: they import only
    numpy, the oracle and the generators, never touch the GPU and run one
    BLAS thread each).  Returns the results in job order."""
    if workers is None:
        workers = min(12, len(os.sched_getaffinity(0)), max(len(jobs), 1))
    ctx = multiprocessing.get_context("spawn")
    with ProcessPoolExecutor(max_workers=workers, mp_context=ctx,
                             initializer=_one_thread_blas) as ex:
        futs = [ex.submit(oracle_request_rows, w, r, np.asarray(rows), 1.0, local)
                for r, rows in jobs]
        return [f.result() for f in futs]


def split_tiles(step):
    """(request, first row, row count) of every tile the last prefill plan of
    ``step`` split into page ranges, read from the pinned staging copy of the
    plan (header word 6 = split tiles, word 7 = their word offset, 8 words
    each)."""
    k = (step._plans - 1) % len(step.pre_staging)
    st = step.pre_staging[k].numpy().view(np.int32)
    n, off = int(st[6]), int(st[7])
    return [tuple(int(x) for x in st[off + 8 * i:off + 8 * i + 3]) for i in range(n)]


def decode_error_bits(step):
    """Error word of the decode workspace (bit 0: invalid page id skipped,
    bit 1: plan overflow, bit 2: rows refused past max_pages)."""
    return int(step.dec_ws[:4].view(torch.int32).item())


def prefill_error_bits(step):
    """Error word of the prefill plan (int32 word 9; bit 0: invalid page id
    skipped, bit 2: rows refused past max_pages)."""
    return int(step.pre_plan[36:40].view(torch.int32).item())
