"""The general forced-block selection on the GPU (``mi_idx_select_forced``,
through the C ABI) against the oracle's ``select_forced_row`` computed from
the oracle's own page scores: leading / trailing windows with the flashinfer
page's clamps, topk 1..16, ascending ids, -1 tail."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import checker
from tests.gpu_common import lib, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

# (topk, init_blocks, local_blocks)
CONFIGS = [(16, 0, 1), (16, 2, 1), (16, 1, 3), (12, 4, 2), (8, 0, 1), (8, 3, 2), (4, 1, 1),
           (1, 0, 1), (3, 5, 1), (16, 40, 1), (5, 0, 9)]


@pytest.mark.parametrize("name", ["mixed_small", "edge_wide", "edge_prefill",
                                  "multi_token_small", "edge_short"])
def test_forced_selection_parity(name):
    print(f"[gpu-test] forced selection {name}", flush=True)
    m = lib()
    w = W.make_workload(name, 0)
    out, _, _, dw, _ = run_gpu(w)
    _, scores, L, _ = run_oracle(w)
    mkt = int(-(-int(np.max(w.seq_lens)) // 128))
    for topk, init, local in CONFIGS:
        for max_k_tiles in (mkt, 1):
            g = m.mi_idx_select_forced(dw.out, topk, init, local, max_k_tiles)
            torch.cuda.synchronize()
            g = g.cpu().numpy()
            o = [[oracle.select_forced_row(scores[t][h] if L[t] > 0 else np.zeros(0), int(L[t]),
                                           topk, init, local, max_k_tiles)
                  for h in range(w.H)] for t in range(w.T)]
            frac = checker.compare_forced(g, o, scores, L, topk, init, local, max_k_tiles)
            print(f"[gpu-test] {name} topk={topk} init={init} local={local} "
                  f"max_k_tiles={max_k_tiles}: exact {frac:.4f}", flush=True)


def test_forced_selection_in_place_and_empty():
    print("[gpu-test] forced selection in place", flush=True)
    m = lib()
    w = W.make_workload("mixed_small", 1)
    out, _, _, dw, _ = run_gpu(w)
    want = m.mi_idx_select_forced(dw.out, 16, 2, 2, 100).cpu().numpy()
    r = dw.out.clone()
    m.mi_idx_select_forced(r, 16, 2, 2, 100, out=r)          # the allowed in-place call
    torch.cuda.synchronize()
    assert np.array_equal(r.cpu().numpy(), want)
    empty = torch.empty((0, 4, 16), dtype=torch.int32, device="cuda")
    assert m.mi_idx_select_forced(empty, 8, 0, 1, 10).shape == (0, 4, 8)
