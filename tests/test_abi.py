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
    txt = open(os.path.join(ROOT, "include", "mi_idx.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(mi_idx_[a-z_0-9]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def m():
    import sparse_attention_block_mxfp4_amd as m
    return m


def test_library_exports_every_declared_symbol(m):
    names = _declared()
    assert len(names) == 13
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
    assert m.mi_idx_prefill_plan_bytes(8, 32768, 4) == 64 + (32768 // 64 + 8 + 1) * 16
    assert m.mi_idx_prefill_plan_bytes(1, 10, 9) == 0


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
    args = [buf, 0, buf, 10, buf, 16, buf, buf, buf, 2, 100, 1, 16, 1.0, buf, pb, 2, buf, None,
            None]

    def call(i=None, v=None):
        a = list(args)
        if i is not None:
            a[i] = v
        return L.mi_idx_score_topk_prefill(*a)
    assert call(11, 9) == m.EUNSUPPORTED
    assert call(13, -1.0) == m.EINVAL
    assert call(0, None) == m.EINVAL
    assert call(16, 10 ** 6) == m.ECAPACITY
    assert call(5, 8) == m.EINVAL
    assert call(1, 5) == m.EINVAL               # unknown q dtype
    assert call(16, 0) == m.OK
    cu = np.array([0, 5, 3], dtype=np.int32)
    sl = np.array([10, 10], dtype=np.int32)
    tiles, ch = ctypes.c_int(), ctypes.c_int()
    st = _fake()
    assert L.mi_idx_plan_prefill(cu.ctypes.data, sl.ctypes.data, 2, 1, 0, st.ctypes.data, buf,
                                 pb, ctypes.byref(ch), ctypes.byref(tiles), None) == m.EINVAL
    cu = np.array([0, 5, 30], dtype=np.int32)
    assert L.mi_idx_plan_prefill(cu.ctypes.data, sl.ctypes.data, 2, 1, 0, st.ctypes.data, buf,
                                 pb, ctypes.byref(ch), ctypes.byref(tiles), None) == m.EINVAL
    cu = np.array([0, 5, 8], dtype=np.int32)
    assert L.mi_idx_plan_prefill(cu.ctypes.data, sl.ctypes.data, 2, 1, 0, st.ctypes.data, buf,
                                 16, ctypes.byref(ch), ctypes.byref(tiles), None) == m.ECAPACITY


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
        pb = m.mi_idx_prefill_plan_bytes(R, int(cu[-1]), H)
        st = _fake(pb)
        tiles, ch = ctypes.c_int(), ctypes.c_int()
        status = m.lib.mi_idx_plan_prefill(cu.ctypes.data, sl.ctypes.data, R, H, budget,
                                           st.ctypes.data, 256, pb, ctypes.byref(ch),
                                           ctypes.byref(tiles), None)
        # no device here: the single copy fails after the staging is written
        assert status in (m.OK, m.EHIP)
        words = st.view(np.int32)
        n = words[0]
        assert n == tiles.value
        M = 256 // H
        assert words[1] == M and words[2] == H
        want_chunks = oracle.prefill_chunks(sl, budget if budget > 0 else 10 ** 12)
        assert words[3] == len(want_chunks) == ch.value
        t = words[16:16 + 4 * n].reshape(n, 4)
        chunk_of = np.zeros(R, dtype=int)
        for c, (a, b, _) in enumerate(want_chunks):
            chunk_of[a:b] = c
        # tiles cover every row exactly once, in row tiles of M
        cover = [np.zeros(q, dtype=int) for q in qn]
        for r, row0, nr, pages in t:
            assert 0 < nr <= M and row0 % M == 0
            cover[r][row0:row0 + nr] += 1
            assert pages == max((sl[r] - qn[r] + row0 + nr - 1) // 128, 0)
        assert all(np.all(c == 1) for c in cover)
        # chunks are launched in order (the tile order inside a chunk is a
        # placement choice and is not part of the contract)
        ch_seq = [chunk_of[r] for r, _, _, _ in t]
        assert ch_seq == sorted(ch_seq)
