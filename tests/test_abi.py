"""The C ABI without a GPU: the library loads, exports every entry point that
include/mi_idx.h declares, and rejects bad arguments on the host (status +
reason, nothing launched).  The prefill plan's host logic is checked against
the oracle's chunking through the pinned-staging bytes it writes before its
single copy (which has no device to go to here)."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    # the indexer's ABI (the probe header is checked on its own below)
    txt = open(os.path.join(ROOT, "include", "mi_idx.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(mi_idx_[a-z_0-9]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def m():
    import sparse_attention_block_mxfp4_amd as m
    return m


def test_probe_library_exports_its_header(m):
    """libmi_idx_probe.so (the benchmark's HBM read and MFMA ceiling probes)
    exports what include/mi_idx_probe.h declares, and its argument checks
    refuse before any launch."""
    txt = open(os.path.join(ROOT, "include", "mi_idx_probe.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    names = sorted(set(re.findall(r"\b(mi_idx_probe_[a-z_0-9]+)\s*\(", txt)))
    assert names == ["mi_idx_probe_device", "mi_idx_probe_mfma", "mi_idx_probe_read_pages",
                     "mi_idx_probe_read_stream"]
    raw = ctypes.CDLL(os.path.join(ROOT, "sparse_attention_block_mxfp4_amd", "libmi_idx_probe.so"))
    for n in names:
        assert hasattr(raw, n), n
    ci, cu, vp, i64 = ctypes.c_int, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int64
    raw.mi_idx_probe_mfma.argtypes = [ci, ci, ci, ci, cu, cu, vp, i64, vp, vp]
    raw.mi_idx_probe_device.argtypes = [vp, vp, vp]
    fake = 1 << 20                      # never dereferenced: refused before any call
    for kind, fold, iters, bpc, sink, clocks in ((2, 0, 1, 1, fake, fake), (0, 2, 1, 1, fake, fake),
                                                 (0, 0, 0, 1, fake, fake), (0, 0, 1, 9, fake, fake),
                                                 (0, 0, 1, 1, None, fake), (1, 1, 1, 1, fake, None),
                                                 (0, 0, 1, 1, fake, fake + 4)):
        assert raw.mi_idx_probe_mfma(kind, fold, iters, bpc, 0, 0, sink, 1 << 20, clocks,
                                     None) == 1
    assert raw.mi_idx_probe_device(None, None, None) == 1


def test_library_exports_every_declared_symbol(m):
    names = _declared()
    assert len(names) == 18
    raw = ctypes.CDLL(m.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_version_and_reason(m):
    assert "gfx950" in m.mi_idx_version()
    r = m.mi_idx_unsupported_reason(topk_blocks=8)
    assert r is not None and "topk_blocks=16" in r
    assert "score_type" in m.mi_idx_unsupported_reason(score_type="sum")
    assert "heads" in m.mi_idx_unsupported_reason(num_heads=9)
    assert "8 decode queries" in m.mi_idx_unsupported_reason(max_query_len=9)
    # a valid config on a machine without a gfx950 device
    r = m.mi_idx_unsupported_reason()
    assert r is None or "device" in r or "gfx950" in r


def test_sizes(m):
    assert m.mi_idx_decode_plan_bytes(64) == 64 + (64 + 2048) * 16
    assert m.mi_idx_decode_workspace_bytes(64, 1, 1) == 256 + 512 + (64 + 2048) * 16 * 8
    assert m.mi_idx_decode_workspace_bytes(0, 0, 1) == 0
    # header, 512 work lists, tiles + 512 pieces, 512 split tiles
    tiles = 32768 // 64 + 8 + 1
    assert m.mi_idx_prefill_plan_bytes(8, 32768, 4) == 4 * (16 + 4 * 512 + 8 * (tiles + 512)
                                                            + 8 * 512)
    assert m.mi_idx_prefill_plan_bytes(1, 10, 9) == 0
    assert m.mi_idx_prefill_workspace_bytes() == 1024 * 256 * 16 * 8


def test_decode_plan_capacity(m):
    """Work items of a decode plan: one per request plus the 2048 the scorer
    holds at once; 64 header bytes + 16 bytes per item make the plan."""
    for R in (0, 1, 64, 1000):
        cap = m.mi_idx_decode_plan_capacity(R, 2048, 2, 4)
        assert cap == R + 2048
        assert m.mi_idx_decode_plan_bytes(R) == 64 + 16 * cap
    assert m.mi_idx_decode_plan_capacity(-1, 10, 1, 1) == 0
    assert m.mi_idx_decode_plan_capacity(4, -1, 1, 1) == 0
    assert m.mi_idx_decode_plan_capacity(4, 10, 0, 1) == 0
    assert m.mi_idx_decode_plan_capacity(4, 10, 9, 1) == 0
    assert m.mi_idx_decode_plan_capacity(4, 10, 1, 9) == 0


def test_decode_noalloc_argument_errors(m):
    """The allocation-free decode call rejects what the caller-buffer calls
    reject, and inputs whose plan + workspace exceed its static scratch,
    before touching any device memory."""
    L = m.lib
    buf = _fake().ctypes.data

    def call(R=4, ql=2, H=2, mp=16, sc=1.0, qd=0, q=buf, out=buf, bts=16, nb=10):
        return L.mi_idx_decode_noalloc(q, qd, buf, nb, buf, bts, buf, R, ql, H, mp, sc, out,
                                       None, None)
    assert call(ql=9) == m.EUNSUPPORTED
    assert call(H=0) == m.EUNSUPPORTED
    assert call(R=-1) == m.EINVAL
    assert call(mp=-1) == m.EINVAL
    assert call(sc=0.0) == m.EINVAL
    assert call(qd=3) == m.EINVAL
    assert call(q=None) == m.EINVAL
    assert call(out=buf + 4) == m.EINVAL
    assert call(bts=8) == m.EINVAL
    assert call(nb=0) == m.EINVAL
    # plan (rounded to 256) + workspace against the 32 MiB scratch
    need = lambda R, ql, H: (-(-m.mi_idx_decode_plan_bytes(R) // 256) * 256  # noqa: E731
                             + m.mi_idx_decode_workspace_bytes(R, ql, H))
    assert need(512, 8, 8) <= m.NOALLOC_SCRATCH_BYTES
    big = next(R for R in range(512, 1 << 16, 64) if need(R, 8, 8) > m.NOALLOC_SCRATCH_BYTES)
    assert call(R=big, ql=8, H=8) == m.ECAPACITY
    assert b"scratch" in L.mi_idx_last_error()
    assert call(R=0) == m.OK


def _fake(n=1 << 20):
    # host memory standing in for device buffers: every call below must be
    # rejected before anything touches it
    return np.zeros(n, dtype=np.uint8)


def test_decode_argument_errors(m):
    L = m.lib
    plan, ws = _fake(), _fake(1 << 24)
    P, W = plan.ctypes.data, ws.ctypes.data
    pb, wb = m.mi_idx_decode_plan_bytes(4), m.mi_idx_decode_workspace_bytes(4, 2, 2)
    buf = _fake().ctypes.data
    ok = dict(q=buf, qd=0, pages=buf, nb=10, bt=buf, bts=16, sl=buf, R=4, ql=2, H=2, mp=16,
              sc=1.0, P=P, pb=pb, W=W, wb=wb, out=buf)

    def call(**kw):
        a = dict(ok, **kw)
        return L.mi_idx_score_topk_decode(a["q"], a["qd"], a["pages"], a["nb"], a["bt"], a["bts"],
                                          a["sl"],
                                          a["R"], a["ql"], a["H"], a["mp"], a["sc"], a["P"],
                                          a["pb"], a["W"], a["wb"], a["out"], None, None)
    assert call(ql=9) == m.EUNSUPPORTED
    assert call(ql=0) == m.EUNSUPPORTED
    assert call(H=9) == m.EUNSUPPORTED
    assert call(sc=0.0) == m.EINVAL
    assert call(sc=float("nan")) == m.EINVAL
    assert call(sc=float("inf")) == m.EINVAL
    assert call(pb=pb - 1) == m.ECAPACITY
    assert call(wb=wb - 1) == m.ECAPACITY
    assert call(q=None) == m.EINVAL
    assert call(out=None) == m.EINVAL
    assert call(bts=8) == m.EINVAL
    assert call(nb=0) == m.EINVAL
    assert call(q=buf + 4) == m.EINVAL          # misaligned
    assert call(qd=2) == m.EINVAL               # neither E4M3 nor bf16
    assert call(qd=-1) == m.EINVAL
    assert b"scale" in L.mi_idx_last_error() or True
    assert call(R=0) == m.OK                    # nothing to do, nothing launched
    assert L.mi_idx_plan_decode(buf, 4, 9, 2, 16, P, pb, W, wb, None) == m.EUNSUPPORTED
    assert L.mi_idx_plan_decode(buf, 4, 2, 9, 16, P, pb, W, wb, None) == m.EUNSUPPORTED
    assert L.mi_idx_plan_decode(buf, 5, 2, 2, 16, P, pb, W, wb, None) == m.ECAPACITY
    assert L.mi_idx_plan_decode(buf, 4, 2, 4, 16, P, pb, W, wb, None) == m.ECAPACITY
    assert L.mi_idx_plan_decode(None, 4, 2, 2, 16, P, pb, W, wb, None) == m.EINVAL
    assert L.mi_idx_plan_decode(buf, 4, 2, 2, -1, P, pb, W, wb, None) == m.EINVAL
    assert len(L.mi_idx_last_error()) > 0


def test_insert_argument_errors(m):
    L = m.lib
    buf = _fake().ctypes.data
    assert L.mi_idx_insert_mxfp4(buf, 2, 128, buf, 4, buf, 4, None) == m.EINVAL
    assert L.mi_idx_insert_mxfp4(buf, 0, 100, buf, 4, buf, 4, None) == m.EINVAL
    assert L.mi_idx_insert_mxfp4(None, 0, 128, buf, 4, buf, 4, None) == m.EINVAL
    assert L.mi_idx_insert_mxfp4(buf, 0, 128, buf, -1, buf, 4, None) == m.EINVAL
    assert L.mi_idx_insert_mxfp4(buf, 0, 128, buf, 0, buf, 4, None) == m.OK
    assert L.mi_idx_insert_mxfp4(buf, 0, 128, buf, 4, buf, 0, None) == m.EINVAL
    assert L.mi_idx_insert_mxfp4(buf + 4, 0, 128, buf, 4, buf, 4, None) == m.EINVAL


def test_norm_rope_insert_argument_errors(m):
    L = m.lib
    buf = _fake(1 << 16)
    B = buf.ctypes.data
    B = B + (-B) % 16

    def call(k=B, kd=0, stride=128, w=B, eps=1e-6, pos=B, rd=64, base=10000.0, style=0,
             slots=B, n=4, pages=B, nb=4):
        return L.mi_idx_norm_rope_insert_mxfp4(k, kd, stride, w, eps, pos, rd, base, style,
                                               slots, n, pages, nb, None)
    assert call(rd=12) == m.EUNSUPPORTED                 # not a multiple of 8
    assert call(rd=136) == m.EUNSUPPORTED
    assert call(style=2) == m.EINVAL
    assert call(base=0.0) == m.EINVAL
    assert call(base=float("inf")) == m.EINVAL
    assert call(eps=-1.0) == m.EINVAL
    assert call(eps=float("nan")) == m.EINVAL
    assert call(pos=None) == m.EINVAL                    # rotation needs positions
    assert call(w=B + 4) == m.EINVAL                     # misaligned weights
    assert call(kd=3) == m.EINVAL
    assert call(stride=100) == m.EINVAL
    assert call(n=-1) == m.EINVAL
    assert call(nb=0) == m.EINVAL
    assert call(n=0) == m.OK
    assert call(n=0, rd=0, pos=None, w=None) == m.OK     # a plain insert of nothing


def test_select_forced_argument_errors(m):
    L = m.lib
    buf = _fake(1 << 16)
    B = buf.ctypes.data
    B = B + (-B) % 16                                   # 16-byte aligned
    O = B + 4096

    def call(ranked=B, n=4, topk=8, init=0, local=1, mkt=10, out=O):
        return L.mi_idx_select_forced(ranked, n, topk, init, local, mkt, out, None)
    assert call(topk=0) == m.EUNSUPPORTED
    assert call(topk=17) == m.EUNSUPPORTED
    assert call(local=0) == m.EUNSUPPORTED               # the local page is never scored
    assert call(init=-1) == m.EINVAL
    assert call(mkt=-1) == m.EINVAL
    assert call(n=-1) == m.EINVAL
    assert call(ranked=None) == m.EINVAL
    assert call(out=None) == m.EINVAL
    assert call(ranked=B + 4) == m.EINVAL                # misaligned rows
    assert call(out=B + 32) == m.EINVAL                  # overlaps the input
    assert call(out=B, topk=8) == m.EINVAL               # in place needs topk 16
    assert call(n=0) == m.OK                             # nothing to do, nothing launched
    assert b"select_forced" in L.mi_idx_last_error() or True


def test_prefill_argument_errors(m):
    L = m.lib
    buf = _fake().ctypes.data
    pb = m.mi_idx_prefill_plan_bytes(2, 100, 1)
    wb = m.mi_idx_prefill_workspace_bytes()
    launch = m.PrefillLaunch(2, 3, 1, 1)
    args = [buf, 0, buf, 10, buf, 16, buf, buf, buf, 2, 100, 1, 16, 1.0, buf, pb,
            ctypes.addressof(launch), buf, wb, buf, None, None]

    def call(i=None, v=None, shape=(2, 3, 1, 1)):
        launch.num_lists, launch.num_pieces, launch.num_merges, launch.num_chunks = shape
        a = list(args)
        if i is not None:
            a[i] = v
        return L.mi_idx_score_topk_prefill(*a)
    assert call(11, 9) == m.EUNSUPPORTED
    assert call(13, -1.0) == m.EINVAL
    assert call(0, None) == m.EINVAL
    assert call(16, None) == m.EINVAL            # no launch shape
    assert call(shape=(10 ** 6, 10 ** 6, 0, 1)) == m.ECAPACITY
    assert call(shape=(2, 3, 10 ** 6, 1)) == m.ECAPACITY   # more split tiles than work lists
    assert call(shape=(2, 3, -1, 1)) == m.EINVAL
    assert call(shape=(3, 2, 0, 1)) == m.EINVAL  # fewer pieces than work lists
    assert call(17, None) == m.EINVAL            # split tiles need the workspace
    assert call(17, buf + 4) == m.EINVAL         # misaligned workspace
    assert call(18, wb - 1) == m.ECAPACITY
    assert call(5, 8) == m.EINVAL
    assert call(1, 5) == m.EINVAL               # unknown q dtype
    assert call(shape=(0, 0, 0, 0)) == m.OK
    cu = np.array([0, 5, 3], dtype=np.int32)
    sl = np.array([10, 10], dtype=np.int32)
    out = m.PrefillLaunch()
    st = _fake()

    def plan(nbytes=pb, shape=ctypes.byref(out)):
        return L.mi_idx_plan_prefill(cu.ctypes.data, sl.ctypes.data, 2, 1, 0, st.ctypes.data, buf,
                                     nbytes, shape, None)
    assert plan() == m.EINVAL
    cu = np.array([0, 5, 30], dtype=np.int32)
    assert plan() == m.EINVAL
    cu = np.array([0, 5, 8], dtype=np.int32)
    assert plan(nbytes=16) == m.ECAPACITY
    assert plan(shape=None) == m.EINVAL


def _plan_host(m, cu, sl, H, budget):
    """Run the host plan; return the staging words it wrote and its outputs."""
    R = len(sl)
    pb = m.mi_idx_prefill_plan_bytes(R, int(cu[-1]), H)
    st = _fake(pb)
    out = m.PrefillLaunch()
    status = m.lib.mi_idx_plan_prefill(cu.ctypes.data, sl.ctypes.data, R, H, budget,
                                       st.ctypes.data, 256, pb, ctypes.byref(out), None)
    # no device here: the single copy fails after the staging is written
    assert status in (m.OK, m.EHIP)
    words = st.view(np.int32)
    assert out.num_pieces == words[4]
    return words, out.num_lists, out.num_chunks, out.num_merges


# The planner's cost of a piece's set-up, in pages (its lists balance pages +
# this per piece).
PIECE_COST = 24


def _check_plan(words, n_lists, n_chunks, n_merges, cu, sl, H, budget):
    """Every row in exactly one tile of M rows; each tile's pieces split its
    pages [0, pages) into consecutive ranges, with slots consecutive in page
    order and one merge record when split; work lists hold consecutive
    pieces and come in request order of their first piece; the chunk count
    is the pages' greedy rule.  Returns the list costs (pages + PIECE_COST
    per piece)."""
    qn = np.diff(cu)
    M = 256 // H
    assert words[0] == n_lists and words[1] == M and words[2] == H and words[3] == n_chunks
    n_pieces, poff, n_split, soff, n_slots = (int(x) for x in words[4:9])
    assert n_split == n_merges
    assert 1 <= n_lists <= 256 or (n_lists == 0 and n_pieces == 0)
    lists = words[16:16 + 4 * n_lists].reshape(-1, 4)
    assert poff == 16 + 4 * n_lists and soff == poff + 8 * n_pieces
    # the lists, in piece order, cover the pieces once, consecutively
    nxt = 0
    for first, cnt, _, _ in sorted(lists.tolist()):
        assert first == nxt and cnt >= 1
        nxt += cnt
    assert nxt == n_pieces
    pieces = words[poff:poff + 8 * n_pieces].reshape(-1, 8)
    splits = words[soff:soff + 8 * n_split].reshape(-1, 8)
    want_chunks = oracle.prefill_chunks(sl, budget if budget > 0 else 10 ** 12)
    assert n_chunks == len(want_chunks)
    cover = [np.zeros(q, dtype=int) for q in qn]
    ranges = {}
    for r, row0, nr, pa, pe, slot, _, _ in pieces:
        assert 0 < nr <= M and row0 % M == 0
        ranges.setdefault((r, row0, nr), []).append((pa, pe, slot))
    for (r, row0, nr), rs in ranges.items():
        rs.sort()
        cover[r][row0:row0 + nr] += 1
        pages = max((sl[r] - qn[r] + row0 + nr - 1) // 128, 0)
        assert rs[0][0] == 0 and rs[-1][1] == pages
        for (a0, b0, _), (a1, _, _) in zip(rs, rs[1:]):
            assert b0 == a1 and a0 < b0
        slots = [x[2] for x in rs]
        if len(rs) == 1:
            assert slots == [-1]
        else:
            assert slots == list(range(slots[0], slots[0] + len(rs)))
            match = [s for s in splits if tuple(s[:3]) == (r, row0, nr)]
            assert len(match) == 1 and match[0][3] == slots[0] and match[0][4] == len(rs)
    assert all(np.all(c == 1) for c in cover)
    assert len(splits) == sum(1 for rs in ranges.values() if len(rs) > 1)
    assert n_slots == sum(len(rs) for rs in ranges.values() if len(rs) > 1)
    # lists in piece order start with requests in order (the placement puts
    # a request's lists on neighbouring workgroups of one XCD)
    firsts = [int(pieces[f][0]) for f, _, _, _ in sorted(lists.tolist())]
    assert firsts == sorted(firsts)
    return [int(sum(p[4] - p[3] + PIECE_COST for p in pieces[f:f + c])) for f, c, _, _ in lists]


@pytest.mark.parametrize("H", [1, 3, 4, 8])
def test_prefill_host_plan_matches_oracle_chunking(m, H):
    rng = np.random.default_rng(H)
    for trial in range(20):
        R = int(rng.integers(1, 9))
        qn = rng.integers(0, 700, size=R).astype(np.int32)
        ctx = rng.integers(0, 9000, size=R).astype(np.int32)
        sl = ctx + qn
        sl = np.maximum(sl, 1).astype(np.int32)
        cu = np.concatenate([[0], np.cumsum(qn)]).astype(np.int32)
        budget = int(rng.integers(0, 60))
        words, n, ch, mg = _plan_host(m, cu, sl, H, budget)
        _check_plan(words, n, ch, mg, cu, sl, H, budget)


@pytest.mark.parametrize("seed", [0, 1, 2, 5, 6])
def test_prefill_work_lists_balance_ragged_rows(m, seed):
    """Ragged prefill shapes (8 requests x 4096 rows over 0..61440 context
    tokens, 4 heads): at most 256 lists (one per CU without a device), none
    costing more than 1.10 x the balanced share (the longest-first filling
    with rebalancing lands within 8 % on seeds 0..7)."""
    rng = np.random.default_rng(seed)
    qn = np.full(8, 4096, dtype=np.int32)
    ctx = rng.integers(0, 61441, size=8).astype(np.int32)
    sl = (ctx + qn).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(qn)]).astype(np.int32)
    words, n, ch, mg = _plan_host(m, cu, sl, 4, 1024)
    costs = _check_plan(words, n, ch, mg, cu, sl, 4, 1024)
    M = 64
    tile_cost = [max((c + r0 + M - 1) // 128, 0) + PIECE_COST for c in ctx
                 for r0 in range(0, 4096, M)]
    share = sum(tile_cost) / 256
    assert n <= 256 and max(costs) <= 1.10 * share
    assert mg > 0                       # the longest tiles exceed the share and are split


def test_prefill_equal_tiles_stay_whole(m):
    """Two requests of 8192 rows over 131072-token contexts (tiles within 5 %
    of each other): one whole tile per list, nothing to merge."""
    qn = np.full(2, 8192, dtype=np.int32)
    sl = (131072 + qn).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(qn)]).astype(np.int32)
    words, n, ch, mg = _plan_host(m, cu, sl, 4, 0)
    _check_plan(words, n, ch, mg, cu, sl, 4, 0)
    assert n == 256 and mg == 0


def test_prefill_plan_adversarial_shapes(m):
    """Host planning on shapes far from the workloads (the ones the heap
    rebalancing and the offset arithmetic see least): thousands of tiny
    requests, one request of many more tiles than work lists, contexts near a
    billion tokens, empty requests between others and an all-empty batch."""
    rng = np.random.default_rng(44)
    cases = []
    qn = rng.integers(0, 6, size=2000).astype(np.int32)
    cases.append((qn, rng.integers(0, 10 ** 6, size=2000).astype(np.int32), 1, 0))
    cases.append((np.array([200000, 3, 0, 7], dtype=np.int32),
                  np.array([0, 50, 10 ** 5, 1], dtype=np.int32), 1, 0))
    cases.append((np.array([1, 300, 1], dtype=np.int32),
                  np.array([10 ** 9, 5000, 3], dtype=np.int32), 4, 64))
    cases.append((np.array([0, 0, 0], dtype=np.int32), np.array([5, 0, 9], dtype=np.int32), 2, 0))
    cases.append((np.array([8192] * 16, dtype=np.int32),
                  np.array([131072] * 8 + [0] * 8, dtype=np.int32), 8, 100))
    for qn, ctx, H, budget in cases:
        sl = np.maximum(ctx + qn, 1).astype(np.int32)
        cu = np.concatenate([[0], np.cumsum(qn)]).astype(np.int32)
        words, n, ch, mg = _plan_host(m, cu, sl, H, budget)
        if cu[-1] == 0:
            assert n == 0 and words[4] == 0
            continue
        _check_plan(words, n, ch, mg, cu, sl, H, budget)


def test_general_selection_argument_errors(m):
    """mi_idx_score_local / mi_idx_select_topk reject bad arguments on the
    host (nothing launched)."""
    L = m.lib
    buf = _fake().ctypes.data

    def local(**kw):
        a = dict(q=buf, qd=0, pages=buf, nb=10, bt=buf, bts=16, sl=buf, cu=None, ctx=None, R=4,
                 ql=2, T=8, H=2, mp=16, sc=1.0, out=buf)
        a.update(kw)
        return L.mi_idx_score_local(a["q"], a["qd"], a["pages"], a["nb"], a["bt"], a["bts"],
                                    a["sl"], a["cu"], a["ctx"], a["R"], a["ql"], a["T"], a["H"],
                                    a["mp"], a["sc"], a["out"], None)
    assert local(H=9) == m.EUNSUPPORTED
    assert local(qd=2) == m.EINVAL
    assert local(sc=0.0) == m.EINVAL
    assert local(ql=9) == m.EUNSUPPORTED
    assert local(T=7) == m.EINVAL                      # decode rows = num_reqs * query_len
    assert local(cu=buf, ctx=None) == m.EINVAL         # prefill rows need context_lens
    assert local(q=None) == m.EINVAL
    assert local(nb=0) == m.EINVAL
    assert local(bts=8) == m.EINVAL
    assert local(R=0, T=0) == m.OK

    def sel(**kw):
        a = dict(s=buf, st=16, loc=buf, rk=buf, n=4, topk=8, init=0, local=1, mkt=10, out=buf)
        a.update(kw)
        return L.mi_idx_select_topk(a["s"], a["st"], a["loc"], a["rk"], a["n"], a["topk"],
                                    a["init"], a["local"], a["mkt"], a["out"], None)
    assert sel(topk=0) == m.EUNSUPPORTED
    assert sel(topk=m.MAX_TOPK + 1) == m.EUNSUPPORTED
    assert sel(init=-1) == m.EINVAL
    assert sel(local=-1) == m.EINVAL
    assert sel(n=-1) == m.EINVAL
    assert sel(s=None) == m.EINVAL
    assert sel(st=0) == m.EINVAL
    assert sel(local=0, loc=None) == m.EINVAL          # the local page competes
    assert sel(n=0) == m.OK
