"""Host logic of bench.py, without a GPU: the one-GPU refusal, the algorithmic
work it divides by (against an independent count from the oracle's row
positions), the comment-insensitive source digest that keys the counter
traffic, and the timing event's refusal without a device."""

import os
import subprocess
import sys

import numpy as np

import bench
import oracle
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_work_counts():
    for name in ("mixed_small", "edge_prefill", "multi_token_small"):
        w = W.make_workload(name, 0)
        alg = bench.algorithmic(w)
        # decode: every history page of every request once (page + its
        # block-table entry), plus each row's query and output per head
        hist = [max((int(s) - 1) // 128, 0) for s in w.dec_seq_lens]
        want = sum(hist) * (8704 + 4) + w.n_decode_rows * w.H * (128 + 64)
        assert alg["dec_bytes"] == want and alg["dec_pages"] == sum(hist)
        # prefill: 2*128*128 flops per (row, head, history page), the rows'
        # positions from the oracle
        if w.Rp:
            _, pos = oracle.rows_prefill(w.cu_seqlens_q, w.pre_ctx)
            assert alg["pre_flops"] == int(np.sum(pos // 128)) * w.H * 2 * 128 * 128
        else:
            assert alg["pre_flops"] == 0


def test_code_digest_ignores_comments_only():
    code = "int f(int x) {\n  return x + 1;  // one more\n}\n"
    d = bench.code_digest(code)
    assert bench.code_digest("/* a note */ int f(int x)\n{ return x + 1; }") == d
    assert bench.code_digest(code.replace("+ 1", "+ 2")) != d
    assert bench.source_digest("prefill.hip") != bench.source_digest("decode.hip")


def test_measured_traffic_sums_kernels_and_checks_digest(tmp_path, monkeypatch):
    csrc = tmp_path / "sparse_attention_block_mxfp4_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("__global__ void a() {}\n")
    (csrc / "common.h").write_text("#pragma once\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d = bench.source_digest("k.hip")
    (tmp_path / "profiles" / "mixed_step_kernels.txt").write_text(
        "kernel fetch_bytes write_bytes source_digest\n"
        f"ka 1000 24 {d}\nkb 300 7 {d}\nkc 5 5 0000000000000000\n")
    assert bench.measured_traffic(("ka",), "k.hip") == 1024
    assert bench.measured_traffic(("ka", "kb"), "k.hip") == 1331
    # a kernel without a line, or with a stale digest, gives no figure
    assert bench.measured_traffic(("ka", "kz"), "k.hip") is None
    assert bench.measured_traffic(("kc",), "k.hip") is None
    # the summary of another workload is not used
    assert bench.measured_traffic(("ka",), "k.hip", "ragged_prefill") is None
    (tmp_path / "profiles" / "ragged_prefill_kernels.txt").write_text(f"ka 7 1 {d}\n")
    assert bench.measured_traffic(("ka",), "k.hip", "ragged_prefill") == 8
    # a code change makes every line stale; a comment does not
    (csrc / "k.hip").write_text("// note\n__global__ void a() {}\n")
    assert bench.measured_traffic(("ka",), "k.hip") == 1024
    (csrc / "k.hip").write_text("__global__ void a() { int x; }\n")
    assert bench.measured_traffic(("ka",), "k.hip") is None


def test_auto_pool_copies_defeat_the_infinity_cache():
    mb = 1 << 20
    assert bench.auto_pool_copies(522 * mb) == 2          # mixed step
    assert bench.auto_pool_copies(856 * mb) == 2          # multi-token decode
    n = bench.auto_pool_copies(89 * mb)                   # decode batch
    assert n == 7 and (n - 1) * 89 * mb >= 2 * 256 * mb
    assert bench.auto_pool_copies(200 * 1024) == 16       # tiny pools: capped


def test_timing_event_needs_a_device():
    """Without a GPU the fence-free timing event refuses with an error (no
    HIP runtime in the process, or no device behind it), never a crash."""
    import pytest
    with pytest.raises(RuntimeError):
        bench.TimingEvent()


def test_cpu_baseline_extrapolates_by_work():
    """The oracle's sample and its extrapolation: a decode-only workload small
    enough to be sampled whole is not extrapolated (the estimate is the
    sample's time), and a prefill-only one whose requests differ in length
    is extrapolated by history pages and (row, page) pairs: between the
    sample scaled by the smaller and by the larger of the two ratios."""
    w = W.make_workload("decode_batch_small", 0)
    cb = bench.cpu_baseline(w, budget_s=60.0)
    assert cb["kind"] == "oracle" and cb["cores"] == len(os.sched_getaffinity(0))
    assert f"decode requests 0..{w.Rd - 1} of {w.Rd}" in cb["sample"]
    assert abs(cb["step_seconds_est"] - cb["sample_seconds"]) <= 1e-3
    assert abs(w.T / cb["value"] - cb["step_seconds_est"]) <= 1e-3
    w = W.make_workload("ragged_prefill_small", 0)
    cb = bench.cpu_baseline(w, budget_s=60.0)
    assert f"rows 0..{int(w.pre_new[0]) - 1} of {int(w.pre_new[0])}" in cb["sample"]
    hist = [(int(c) + int(q) - 1) // 128 for c, q in zip(w.pre_ctx, w.pre_new)]
    pairs = [int(np.sum((int(c) + np.arange(int(q))) // 128 + 1))
             for c, q in zip(w.pre_ctx, w.pre_new)]
    ratios = (sum(hist) / hist[0], sum(pairs) / pairs[0])
    assert len(set(pairs)) > 1                  # the requests differ in work
    est, sample = cb["step_seconds_est"], cb["sample_seconds"]
    assert sample * min(ratios) - 1e-3 <= est <= sample * max(ratios) + 1e-3
