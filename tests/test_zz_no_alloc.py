"""The allocation-free decode entry point, mi_idx_decode_noalloc, through the
C ABI: its output must equal that of mi_idx_plan_decode +
mi_idx_score_topk_decode on caller buffers (the same kernels), and meet the
oracle's bar, on consecutive calls whose inputs shrink (the static scratch
keeps the previous call's contents, which must not leak into the next)."""

import numpy as np
import pytest
import torch

import workloads as W
from tests import checker
from tests.gpu_common import lib, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


def _noalloc(w, dw, scores=False):
    m = lib()
    out = torch.full((w.n_decode_rows, w.H, 16), -7, dtype=torch.int32, device=dw.device)
    sc = None
    if scores:
        sc = torch.full((w.n_decode_rows, w.H, w.width), float("nan"), device=dw.device)
    m.mi_idx_decode_noalloc(dw.q_dec, dw.pool, dw.bt_dec, dw.sl_dec, w.query_len, w.width, out,
                            scores_out=sc)
    torch.cuda.synchronize()
    return out.cpu().numpy(), None if sc is None else sc.cpu().numpy()


def test_noalloc_matches_plan_and_score_on_shrinking_calls():
    # largest first: 4 requests x 8 queries x 8 heads (64 columns), then
    # 10 requests x 4 queries, then 2 requests x 1 query
    for name in ("edge_wide", "multi_token_small", "tiny_decode"):
        print(f"[gpu-test] noalloc {name}", flush=True)
        w = W.make_workload(name, 0)
        ref_gpu, sd, _, dw, _ = run_gpu(w, scores=True)
        got, gs = _noalloc(w, dw, scores=True)
        nd = w.n_decode_rows
        assert np.array_equal(got, ref_gpu[:nd]), name
        ref, scores, L, _ = run_oracle(w)
        checker.compare(got, ref[:nd], scores[:nd], L[:nd], gpu_scores=gs)
        # the scores of every history page equal the caller-buffer path's
        written = ~np.isnan(sd[:nd])
        assert np.array_equal(~np.isnan(gs), written)
        assert np.array_equal(gs[written], sd[:nd][written])


def test_noalloc_repeat_and_stream():
    """Two calls in a row on one input give the same result, also on a side
    stream."""
    w = W.make_workload("decode_batch_small", 3)
    ref_gpu, _, _, dw, _ = run_gpu(w)
    a, _ = _noalloc(w, dw)
    s = torch.cuda.Stream()
    m = lib()
    out = torch.full((w.n_decode_rows, w.H, 16), -7, dtype=torch.int32, device=dw.device)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        m.mi_idx_decode_noalloc(dw.q_dec, dw.pool, dw.bt_dec, dw.sl_dec, w.query_len, w.width,
                                out)
    torch.cuda.synchronize()
    assert np.array_equal(a, ref_gpu[:w.n_decode_rows])
    assert np.array_equal(out.cpu().numpy(), a)
