"""Decode phase captured in a HIP graph and replayed across steps.

The decode plan is built on the device into persistent buffers, the score
grid is fixed by the plan's capacity, and no call records a memset, so one
capture of (plan, score) serves every later step: only the contents of the
persistent seq_lens / block-table / query buffers change between replays.
Each replay is checked against an eager run of the same step and against
the oracle (the vllm "indexer_nvfp4" page's builder keeps persistent decode
buffers for exactly this kind of capture)."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import checker
from tests.gpu_common import lib
from workloads.device import DeviceWorkload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["decode_batch_small", "multi_token_small", "edge_wide"])
def test_decode_graph_replays_follow_changing_seq_lens(name):
    print(f"[gpu-test] graph replay {name}", flush=True)
    m = lib()
    from sparse_attention_block_mxfp4_amd.step import IndexerStep
    w = W.make_workload(name, 5)
    dw = DeviceWorkload(w, m.mi_idx_insert_mxfp4)
    host_pool = W.host_pool(w, oracle.write_pages)
    step = IndexerStep(w.H, w.width, max_decode_reqs=w.Rd, query_len=w.query_len)
    sl = dw.sl_dec.clone()                       # persistent seq_lens buffer
    out_graph = torch.full_like(dw.out[:dw.nd], -7)
    out_eager = torch.full_like(dw.out[:dw.nd], -7)
    torch.cuda.synchronize()

    # warm up on a side stream, as torch's capture recipe asks
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step.plan(sl)
        step.decode(dw.q_dec, dw.pool, dw.bt_dec, sl, out_graph)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.plan(sl)
        step.decode(dw.q_dec, dw.pool, dw.bt_dec, sl, out_graph)

    rng = np.random.default_rng([5, 77])
    full = w.dec_seq_lens.astype(np.int64)
    for rep in range(4):
        # shorter histories of the same requests (the pool already holds them)
        new_sl = (rng.random(w.Rd) * (full + 1)).astype(np.int32)
        if rep == 0:
            new_sl = full.astype(np.int32)
        sl.copy_(torch.from_numpy(new_sl))
        out_graph.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out_graph.cpu().numpy()
        # eager run of the same step, between replays
        out_eager.fill_(-7)
        step.plan(sl)
        step.decode(dw.q_dec, dw.pool, dw.bt_dec, sl, out_eager)
        torch.cuda.synchronize()
        assert np.array_equal(got, out_eager.cpu().numpy()), f"replay {rep} != eager"
        ref, scores, L = oracle.oracle_decode(w.q_codes[:w.n_decode_rows], host_pool,
                                              w.block_table[:w.Rd], new_sl, w.query_len)
        checker.compare(got, ref, scores, L)
