"""bfloat16 index-Q through the GPU path (the vllm "indexer_mxfp4" page's
scorers take bf16 or E4M3 queries).  The pages' values are converted exactly
to bf16 and scored on the bf16 MFMA; the oracle decodes the same bf16 bit
patterns exactly (fp64)."""

import numpy as np
import pytest

import oracle
import workloads as W
from tests import checker, pins
from tests.gpu_common import oracle_request_rows, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

SMALL_BF16 = ["tiny_decode", "decode_batch_small", "multi_token_small", "ragged_prefill_small",
              "mixed_small", "edge_short", "edge_wide", "edge_prefill", "edge_heads5",
              "prefill_h1_small", "prefill_h8_small", "prefill_many_tiles",
              "prefill_split_small"]


@pytest.mark.parametrize("name", SMALL_BF16)
def test_bf16_small_workload_parity(name):
    print(f"[gpu-test] bf16 {name}", flush=True)
    w = W.make_workload(name, 4, q_dtype="bf16")
    out, _, _, _, _ = run_gpu(w)
    ref, scores, L, _ = run_oracle(w)
    checker.compare(out, ref, scores, L)


def test_bf16_scores_out_match_the_oracle():
    print("[gpu-test] bf16 scores_out", flush=True)
    w = W.make_workload("mixed_small", 6, q_dtype="bf16")
    out, sd, sp, _, _ = run_gpu(w, scores=True, scale=0.7)
    ref, scores, L, _ = run_oracle(w, scale=0.7)
    gs = np.concatenate([sd, sp]) if sd is not None and sp is not None else (sd if sp is None else sp)
    checker.compare(out, ref, scores, L, gpu_scores=gs)


@pytest.mark.slow
def test_bf16_full_size_mixed_step_sampled():
    w = W.make_workload("mixed_step", 0, q_dtype="bf16")
    print(f"[gpu-test] bf16 full-size mixed_step T={w.T}", flush=True)
    out, _, _, _, _ = run_gpu(w)
    req, pos = oracle.rows_decode(w.dec_seq_lens, w.query_len)
    _, pp = oracle.rows_prefill(w.cu_seqlens_q, w.pre_ctx)
    L = np.concatenate([np.where(pos >= 0, pos // 128, -1), pp // 128])
    pins.check_invariants(out, L)
    for r in (0, w.Rd - 1, w.Rd, len(w.seq_lens) - 1):
        nrows = w.query_len if r < w.Rd else int(w.pre_new[r - w.Rd])
        sel = np.unique(np.concatenate([[0, nrows - 1], np.arange(nrows)[::max(nrows // 5, 1)]]))
        T, o, sc, Lr = oracle_request_rows(w, r, sel)
        checker.compare(out[T], o, sc, Lr)
