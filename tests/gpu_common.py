"""Helpers of the GPU tests: run a workload through the library and through
the oracle."""

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


def run_oracle(w, pool=None, scale=1.0):
    """Oracle outputs of the whole workload (small workloads only)."""
    if pool is None:
        pool = W.host_pool(w, oracle.write_pages)
    outs, scs, Ls = [], [], []
    if w.Rd:
        o, s, L = oracle.oracle_decode(w.q_codes[:w.n_decode_rows], pool, w.block_table[:w.Rd],
                                       w.dec_seq_lens, w.query_len, scale, q_dtype=w.q_dtype)
        outs.append(o), scs.extend(s), Ls.append(L)
    if w.Rp:
        o, s, L = oracle.oracle_prefill(w.q_codes[w.n_decode_rows:], pool, w.block_table[w.Rd:],
                                        w.cu_seqlens_q, w.seq_lens[w.Rd:], w.pre_ctx, scale,
                                        q_dtype=w.q_dtype)
        outs.append(o), scs.extend(s), Ls.append(L)
    return np.concatenate(outs), scs, np.concatenate(Ls), pool


def oracle_request_rows(w, r, rows_in_req, scale=1.0):
    """Oracle outputs of selected rows of request r, from that request's own
    pages (encoded by the oracle from the generator's K rows)."""
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
    return T0 + rows_in_req, out, scores, L
