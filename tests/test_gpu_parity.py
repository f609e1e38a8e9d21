"""GPU parity: the HIP path against the oracle, through the C ABI.

Small workloads (several tiles, ragged tails, edge cases) are compared row by
row in full; the full-size workloads are run in the benchmark's launch
configuration and compared on sampled rows, plus the contract invariants on
every row.  Insert parity is bit-exact on the page bytes.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import checker, pins
from tests.gpu_common import (decode_error_bits, lib, oracle_rows_parallel, prefill_error_bits,
                              run_gpu, run_oracle, split_tiles)
from workloads.device import DeviceWorkload

pytestmark = pytest.mark.gpu

SMALL = ["tiny_decode", "decode_batch_small", "multi_token_small", "ragged_prefill_small",
         "mixed_small", "edge_short", "edge_wide", "edge_prefill", "edge_prefill_empty",
         "edge_heads5",
         "prefill_h1_small", "prefill_h8_small", "prefill_many_tiles", "prefill_split_small"]


def _banner(msg):
    print(f"[gpu-test] {msg}", flush=True)


@pytest.mark.parametrize("name", SMALL)
def test_insert_is_byte_exact(name):
    _banner(f"insert {name}")
    w = W.make_workload(name, 0)
    dw = DeviceWorkload(w, lib().mi_idx_insert_mxfp4)
    torch.cuda.synchronize()
    ref = W.host_pool(w, oracle.write_pages)
    got = dw.host_pool()
    assert np.array_equal(got, ref)


def test_insert_bf16_and_strided_rows_byte_exact():
    _banner("insert bf16/strided")
    m = lib()
    rng = np.random.default_rng(5)
    n = 1000
    k = rng.standard_normal((n, 160)).astype(np.float32)
    k[:20] *= 1e-38                    # tiny blocks
    k[20:40] = 0.0                     # zero blocks
    k[40:60] *= 1e4
    kb = torch.from_numpy(k).to(torch.bfloat16)
    slots = rng.permutation(16 * 128)[:n].astype(np.int64)
    slots[::97] = -1                   # skipped rows
    for kt, kh in ((torch.from_numpy(k), k), (kb, kb.float().numpy())):
        pool = torch.zeros((16, 8704), dtype=torch.uint8, device="cuda")
        m.mi_idx_insert_mxfp4(kt.cuda(), torch.from_numpy(slots).cuda(), pool)
        ref = np.zeros((16, 8704), dtype=np.uint8)
        oracle.write_pages(ref, slots, kh[:, :128])
        torch.cuda.synchronize()
        assert np.array_equal(pool.cpu().numpy(), ref)


@pytest.mark.parametrize("name", SMALL)
def test_small_workload_parity(name):
    _banner(f"parity {name}")
    w = W.make_workload(name, 0)
    out, sd, sp, dw, _ = run_gpu(w, scores=True)
    ref, scores, L, _ = run_oracle(w)
    gs = np.concatenate([x for x in (sd, sp) if x is not None and x.shape[0] > 0])
    frac = checker.compare(out, ref, scores, L, gpu_scores=gs)
    print(f"[gpu-test] {name}: exact fraction {frac:.4f}", flush=True)
    pins.check_invariants(out, L)


@pytest.mark.parametrize("seed", [1, 2])
def test_small_workload_parity_other_seeds(seed):
    for name in ["multi_token_small", "mixed_small"]:
        _banner(f"parity {name} seed {seed}")
        w = W.make_workload(name, seed)
        out, _, _, _, _ = run_gpu(w)
        ref, scores, L, _ = run_oracle(w)
        checker.compare(out, ref, scores, L)


def test_scale_and_repeat_invariance():
    _banner("scale invariance")
    w = W.make_workload("mixed_small", 3)
    a, _, _, dw, _ = run_gpu(w)
    for scale in (2.0, 0.125, 0.7):
        b, _, _, _, _ = run_gpu(w, dw=dw, scale=scale)
        assert np.array_equal(a, b), scale
    # several layers scored on one plan
    c, _, _, _, _ = run_gpu(w, dw=dw, layers=3)
    assert np.array_equal(a, c)


def test_physical_permutation_invariance():
    _banner("permutation invariance")
    w = W.make_workload("mixed_small", 4)
    a, _, _, dw, _ = run_gpu(w)
    perm = torch.from_numpy(np.random.default_rng(8).permutation(w.num_blocks)).cuda()
    pool2 = torch.empty_like(dw.pool)
    pool2[perm] = dw.pool
    dw.pools[0] = pool2
    dw.pool = pool2
    bt2 = perm[dw.block_table.long()].int()
    dw.block_table = bt2
    dw.bt_dec = bt2[:w.Rd]
    dw.bt_pre = bt2[w.Rd:]
    b, _, _, _, _ = run_gpu(w, dw=dw)
    assert np.array_equal(a, b)


def test_prefill_plan_upper_bounds_and_budget_do_not_matter():
    _banner("prefill plan bounds")
    w = W.make_workload("ragged_prefill_small", 5)
    a, _, _, dw, _ = run_gpu(w)
    b, _, _, _, _ = run_gpu(w, dw=dw, seq_lens_host_ub=w.seq_lens[w.Rd:] + 1000)
    c, _, _, _, _ = run_gpu(w, dw=dw, budget=1)
    d, _, _, _, _ = run_gpu(w, dw=dw, budget=0)
    assert np.array_equal(a, b) and np.array_equal(a, c) and np.array_equal(a, d)


def test_prefill_work_lists_repeat_and_upper_bounds():
    """Multi-piece work lists with split tiles: one plan scored three times
    (each call rewrites the workspace's partial lists before the merge reads
    them) and a plan from upper-bound lengths (more splits; pieces past a
    tile's device pages walk nothing) give the first result, which matches
    the oracle."""
    _banner("prefill work lists: repeat, upper bounds")
    w = W.make_workload("prefill_split_small", 1)
    a, _, _, dw, step = run_gpu(w)
    sh = step.pre_launch
    assert sh.num_merges > 0 and sh.num_pieces > sh.num_lists
    b, _, _, _, _ = run_gpu(w, dw=dw, layers=3)
    c, _, _, _, step_c = run_gpu(w, dw=dw, seq_lens_host_ub=w.seq_lens[w.Rd:] + 3000)
    assert step_c.pre_launch.num_merges > 0
    assert np.array_equal(a, b) and np.array_equal(a, c)
    ref, scores, L, _ = run_oracle(w)
    checker.compare(a, ref, scores, L)


def test_back_to_back_steps_through_the_staging_ring():
    """Forty steps enqueued back to back with no host synchronisation (the
    prefill plans cycle through the pinned staging ring and its guard
    events; budgets alternate, so consecutive plans differ), each into an
    output buffer of its own: every step gives the first step's result, which
    matches the oracle."""
    _banner("back-to-back steps, staging ring")
    m = lib()
    from sparse_attention_block_mxfp4_amd.step import IndexerStep
    w = W.make_workload("mixed_small", 3)
    dw = DeviceWorkload(w, m.mi_idx_insert_mxfp4)
    step = IndexerStep(w.H, w.width, max_decode_reqs=w.Rd, query_len=max(w.query_len, 1),
                       max_prefill_reqs=w.Rp, max_prefill_rows=w.n_prefill_rows)
    outs = []
    for i in range(40):
        step.plan(dw.sl_dec, w.cu_seqlens_q, w.seq_lens[w.Rd:],
                  gather_budget_pages=(0, 1, 7)[i % 3])
        o = torch.full_like(dw.out, -7)
        step.decode(dw.q_dec, dw.pool, dw.bt_dec, dw.sl_dec, o[:dw.nd])
        step.prefill(dw.q_pre, dw.pool, dw.bt_pre, dw.cu, dw.sl_pre, dw.ctx, o[dw.nd:])
        outs.append(o)
    torch.cuda.synchronize()
    first = outs[0].cpu().numpy()
    ref, scores, L, _ = run_oracle(w)
    checker.compare(first, ref, scores, L)
    for i, o in enumerate(outs[1:], 1):
        assert np.array_equal(o.cpu().numpy(), first), i


def test_decode_replan_in_place():
    """Persistent plan/workspace re-planned with new lengths give the same
    result as a fresh allocation."""
    _banner("decode replan")
    m = lib()
    from sparse_attention_block_mxfp4_amd.step import IndexerStep
    w1 = W.make_workload("decode_batch_small", 6)
    w2 = W.make_workload("decode_batch_small", 7)
    width = max(w1.width, w2.width)
    step = IndexerStep(1, width, max_decode_reqs=16, query_len=1)
    for w in (w1, w2, w1):
        dw = DeviceWorkload(w, m.mi_idx_insert_mxfp4)
        bt = torch.full((w.Rd, width), int(w.spare[0]), dtype=torch.int32, device="cuda")
        bt[:, :w.width] = dw.bt_dec
        step.plan(dw.sl_dec)
        step.decode(dw.q_dec, dw.pool, bt, dw.sl_dec, dw.out)
        torch.cuda.synchronize()
        got = dw.out.cpu().numpy()
        ref, scores, L, _ = run_oracle(w)
        checker.compare(got, ref, scores, L)


def test_zero_queries():
    """All-zero queries: every page scores 0, so ids go in ascending order
    (identical non-zero pages are tested in test_gpu_edges.py)."""
    _banner("zero queries")
    w = W.make_workload("decode_batch_small", 8)
    w.q_codes = np.zeros_like(w.q_codes)
    out, _, _, _, _ = run_gpu(w)
    _, _, L, _ = run_oracle(w)
    for t in range(out.shape[0]):
        n = min(15, int(L[t]))
        assert out[t, 0, :n].tolist() == list(range(n))


def test_poisoned_block_table_tail_and_spare_pages_are_never_read():
    """Block-table columns past each request's pages point at a poison page
    and the pool's spare pages are poison: reading any of them would put a
    poison page (score ~2^116) into the selection."""
    _banner("poison")
    w = W.make_workload("edge_short", 9)
    out, _, _, dw, step = run_gpu(w)
    ref, scores, L, _ = run_oracle(w)
    checker.compare(out, ref, scores, L)
    # error word of the decode workspace: no invalid page id, no overflow
    assert decode_error_bits(step) == 0


def test_invalid_page_ids_inside_a_history_are_skipped():
    """Block-table entries outside [0, num_blocks) inside a history are never
    dereferenced: the page is skipped (as if its score were NaN, which the
    oracle ranks last) and the decode workspace's error bit 0 is set.  Every
    row here has at least 20 history pages, so a skipped page never has to
    fill a slot."""
    _banner("invalid page ids")
    w = W.make_workload("mixed_small", 3)
    m = lib()
    dw = DeviceWorkload(w, m.mi_idx_insert_mxfp4)
    ref, scores, L, _ = run_oracle(w)
    bad_ids = {1: -3, 5: w.num_blocks + 7, 17: -(1 << 30)}
    bt = dw.block_table.cpu().numpy()
    for r in range(len(w.seq_lens)):
        for j, v in bad_ids.items():
            bt[r, j] = v
    dw.block_table.copy_(torch.from_numpy(bt))
    out, _, _, _, step = run_gpu(w, dw=dw)
    # expected: the oracle's scores with the bad pages as NaN
    scores_mod = []
    ref_mod = np.array(ref)
    for t in range(out.shape[0]):
        assert int(L[t]) >= 20
        row = []
        for h in range(w.H):
            s = np.array(scores[t][h], dtype=np.float64)
            s[list(bad_ids)] = np.nan
            row.append(s)
            ref_mod[t, h] = oracle.select_row(s, int(L[t]))
        scores_mod.append(row)
    finite = [[np.where(np.isnan(s), -np.inf, s) for s in row] for row in scores_mod]
    checker.compare(out, ref_mod, finite, L)
    for t in range(out.shape[0]):
        assert not set(bad_ids) & set(out[t, :, :15].ravel().tolist())
    assert decode_error_bits(step) & 1 == 1
    assert prefill_error_bits(step) & 1 == 1


def _full_size(name, pick, seed=0, q_dtype="e4m3"):
    """Run a full-size workload in the benchmark's launch configuration; check
    the contract invariants on every row, and compare the rows ``pick(w,
    step)`` names -- a list of (request, rows of the request) -- with the
    oracle, computed on CPU worker processes."""
    w = W.make_workload(name, seed, q_dtype=q_dtype)
    _banner(f"full-size {name} seed {seed} {q_dtype}: T={w.T} pages={w.num_blocks}")
    out, _, _, dw, step = run_gpu(w)
    Ls = []
    if w.Rd:
        _, pos = oracle.rows_decode(w.dec_seq_lens, w.query_len)
        Ls.append(np.where(pos >= 0, pos // 128, -1))
    if w.Rp:
        _, pp = oracle.rows_prefill(w.cu_seqlens_q, w.pre_ctx)
        Ls.append(pp // 128)
    L = np.concatenate(Ls)
    pins.check_invariants(out, L)
    jobs = pick(w, step)
    _banner(f"full-size {name}: oracle on {sum(len(r) for _, r in jobs)} rows of "
            f"{len(jobs)} requests")
    compared = 0
    for T, o, sc, Lr in oracle_rows_parallel(w, jobs):
        checker.compare(out[T], o, sc, Lr)
        compared += len(T)
    _banner(f"full-size {name}: {compared} rows x {w.H} heads match the oracle")
    return w, out


def _decode_requests(rs):
    return lambda w, step: [(r, np.arange(w.query_len)) for r in rs]


def _prefill_tile(w, r, tile):
    """Rows of one whole row tile (256 / H rows) of prefill request r."""
    M = 256 // w.H
    n = int(w.pre_new[r - w.Rd])
    return np.arange(tile * M, min(n, (tile + 1) * M))


@pytest.mark.slow
def test_full_size_tiny_decode():
    w = W.make_workload("tiny_decode", 0)
    out, sd, _, _, _ = run_gpu(w, scores=True)
    ref, scores, L, _ = run_oracle(w)
    checker.compare(out, ref, scores, L, gpu_scores=sd)


@pytest.mark.slow
def test_full_size_decode_batch():
    """Every row of the 64-request decode batch."""
    _full_size("decode_batch", _decode_requests(range(64)))


@pytest.mark.slow
@pytest.mark.parametrize("seed", [0, 1])
def test_full_size_multi_token_decode(seed):
    """Every 8th request (16 of 128), all four query rows."""
    w, out = _full_size("multi_token_decode", _decode_requests(range(seed, 128, 8)), seed)
    hits = total = 0
    for r in range(w.Rd):
        planted = set(w.planted_pages(r).tolist())
        for i in range(w.query_len):
            top = set(out[r * w.query_len + i, 0, :min(15, len(planted))].tolist())
            hits += len(top & planted)
            total += min(15, len(planted))
    assert hits >= 0.9 * total


@pytest.mark.slow
@pytest.mark.parametrize("seed,q_dtype", [(0, "e4m3"), (1, "e4m3"), (2, "e4m3"), (0, "bf16")])
def test_full_size_ragged_prefill(seed, q_dtype):
    """Every request: its last whole row tile (the longest histories) and one
    row of each of its tiles the plan split into page ranges.  Three seeds:
    their context lengths give plans of 64, 128 and 101 split tiles; seed 0
    also with a bf16 index-Q (the bf16 scorer's work-list path)."""
    def pick(w, step):
        splits = split_tiles(step)
        assert splits, "the ragged batch is expected to split tiles"
        jobs = []
        for r in range(w.Rd, len(w.seq_lens)):
            n = int(w.pre_new[r - w.Rd])
            rows = set(_prefill_tile(w, r, (n - 1) // (256 // w.H)).tolist())
            rows |= {row0 + nrows // 2 for (rq, row0, nrows) in splits if rq == r - w.Rd}
            jobs.append((r, np.array(sorted(rows))))
        return jobs
    _full_size("ragged_prefill", pick, seed, q_dtype)


@pytest.mark.slow
@pytest.mark.parametrize("seed", [0, 1])
def test_full_size_mixed_step(seed):
    """Every 4th decode request (8 of 32), both rows; a whole row tile of
    each prefill request (the last of the first, a middle one of the
    second; other tiles and requests for seed 1)."""
    def pick(w, step):
        jobs = [(r, np.arange(w.query_len)) for r in range(seed, w.Rd, 4)]
        jobs.append((w.Rd, _prefill_tile(w, w.Rd, 8192 // 64 - 1 - 7 * seed)))
        jobs.append((w.Rd + 1, _prefill_tile(w, w.Rd + 1, 64 + 13 * seed)))
        return jobs
    _full_size("mixed_step", pick, seed)
