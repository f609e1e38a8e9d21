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
