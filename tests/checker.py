"""GPU-vs-oracle comparison of [T, H, 16] outputs.

Per (row, head), with L the row's local page (-1 for a padding row):
* a padding row is -1 in all 16 slots on both sides;
* slot 15 is L; slots n..14 are -1 with n = min(15, L);
* the GPU's ids in slots 0..n-1 are distinct and in [0, L);
* rank by rank, the oracle scores of the GPU's pick and of the oracle's pick
  differ by at most tol = 1e-4 * max |oracle score| over the row's history
  pages (so only pages whose scores are within that tolerance may swap,
  in order or across the 15th place); ties of exactly equal score must keep
  the lower id, which this allows as a zero-difference swap only if the
  GPU's pick is also a valid tie;
* NaN scores (pages with a NaN token) take no tolerance: the tolerance base is
  the largest finite |score|, and at every rank the GPU's pick must be NaN
  exactly when the oracle's is, and then the same page (NaN pages rank last,
  by id).
Returns the fraction of (row, head) outputs that match bit-exactly.
"""

import numpy as np

REL_TOL = 1e-4


def _tol(s, rel_tol):
    f = np.abs(s[np.isfinite(s)])
    return rel_tol * (f.max() if f.size else 0.0)


def _rank_gaps(ids_g, ids_o, s, tol):
    """Per rank: whether the GPU's pick is acceptable against the oracle's."""
    sg, so = s[ids_g], s[ids_o]
    ng, no = np.isnan(sg), np.isnan(so)
    ok = np.where(ng | no, ng & no & (ids_g == ids_o), True)
    finite = ~(ng | no)
    with np.errstate(invalid="ignore"):
        diff = np.where(finite, np.abs(sg - so), 0.0)
    # +inf / -inf picks must be the same value (their difference is NaN)
    ok &= np.where(finite, (diff <= tol) | (sg == so), True)
    return ok, sg - so


def compare(gpu, ora, scores, L, rows=None, rel_tol=REL_TOL, gpu_scores=None):
    gpu = np.asarray(gpu)
    ora = np.asarray(ora)
    rows = range(gpu.shape[0]) if rows is None else rows
    exact = total = 0
    for t in rows:
        for h in range(gpu.shape[1]):
            g = gpu[t, h]
            o = ora[t, h]
            total += 1
            Lt = int(L[t])
            if Lt < 0:
                assert np.all(g == -1), f"row {t} head {h}: padding row not all -1: {g}"
                exact += 1
                continue
            assert g[15] == Lt, f"row {t} head {h}: local slot {g[15]} != {Lt}"
            n = min(15, Lt)
            assert np.all(g[n:15] == -1), f"row {t} head {h}: bad padding {g}"
            ids = g[:n]
            assert np.all((ids >= 0) & (ids < Lt)), f"row {t} head {h}: id outside [0,{Lt}): {g}"
            assert len(set(ids.tolist())) == n, f"row {t} head {h}: repeated id {g}"
            if np.array_equal(g, o):
                exact += 1
            else:
                s = np.asarray(scores[t][h], dtype=np.float64)
                tol = _tol(s, rel_tol)
                ok, gap = _rank_gaps(ids, o[:n], s, tol)
                assert ok.all(), (
                    f"row {t} head {h}: gpu {g[:n]} vs oracle {o[:n]}; score gaps "
                    f"{gap[~ok]} exceed tol {tol} (or NaN picks differ)")
            if gpu_scores is not None and Lt > 0:
                s = np.asarray(scores[t][h], dtype=np.float64)
                tol = _tol(s, rel_tol)
                gs = np.asarray(gpu_scores[t, h, :Lt], dtype=np.float64)
                assert np.array_equal(np.isnan(gs), np.isnan(s)), (
                    f"row {t} head {h}: NaN scores at {np.nonzero(np.isnan(gs))[0]} vs "
                    f"oracle {np.nonzero(np.isnan(s))[0]}")
                fin = ~np.isnan(s)
                with np.errstate(invalid="ignore"):
                    diff = np.where(gs[fin] == s[fin], 0.0, np.abs(gs[fin] - s[fin]))
                assert np.all(diff <= tol), (
                    f"row {t} head {h}: score error {diff.max()} > tol {tol}")
    return exact / max(total, 1)


def compare_forced(gpu, ora, scores, L, topk, init_blocks, local_blocks, max_k_tiles,
                   rel_tol=REL_TOL):
    """GPU-vs-oracle comparison of the general forced selection ([T, H, topk],
    ascending ids, -1 tail).  Per (row, head): the form (ascending, distinct,
    -1 only as a tail, ids in 0..L), the forced windows exactly, and the pages
    taken between them rank by rank in oracle score within tol (as in
    ``compare``).  Returns the bit-exact fraction."""
    gpu = np.asarray(gpu)
    exact = total = 0
    for t in range(gpu.shape[0]):
        Lt = int(L[t])
        for h in range(gpu.shape[1]):
            g = gpu[t, h]
            o = np.asarray(ora[t][h])
            total += 1
            if Lt < 0:
                assert np.all(g == -1), f"row {t} head {h}: padding row not all -1: {g}"
                exact += 1
                continue
            nvp = Lt + 1
            ids = g[g >= 0]
            assert len(ids) == min(topk, nvp), f"row {t} head {h}: {g}"
            assert np.all(g[len(ids):] == -1) and np.all(np.diff(ids) > 0), f"row {t} {h}: {g}"
            assert ids.max() <= Lt, f"row {t} head {h}: id past the local page: {g}"
            if np.array_equal(g, o):
                exact += 1
                continue
            assert nvp > topk, f"row {t} head {h}: a short row must list all pages: {g}"
            fb = min(init_blocks, max_k_tiles, topk)
            fe = min(local_blocks, topk - fb)
            forced = set(range(fb)) | set(range(nvp - fe, nvp))
            assert forced <= set(ids.tolist()), f"row {t} head {h}: forced pages missing: {g}"
            gm = np.array(sorted(set(ids.tolist()) - forced))
            om = np.array(sorted(set(o[o >= 0].tolist()) - forced))
            assert len(gm) == len(om)
            s = np.asarray(scores[t][h], dtype=np.float64)
            tol = _tol(s, rel_tol)
            # the chosen pages in selection order (score desc, NaN last, id asc)
            key = lambda j: (np.isnan(s[j]), -s[j] if not np.isnan(s[j]) else 0.0, j)  # noqa: E731
            ok, gap = _rank_gaps(np.array(sorted(gm, key=key), dtype=np.int64),
                                 np.array(sorted(om, key=key), dtype=np.int64), s, tol)
            assert ok.all(), (f"row {t} head {h}: gpu {g} vs oracle {o}; score gaps "
                              f"{gap[~ok]} exceed tol {tol} (or NaN picks differ)")
    return exact / max(total, 1)


_E2M1_BOUNDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def compare_encoded(records, y, rel=1e-5):
    """GPU-written MXFP4 token records [n, 68] against the exact (fp64) rows
    y [n, 128] they encode.  Each block's scale byte must equal the oracle
    encoder's, unless the block's amax is within ``rel`` of a power of two
    (where the GPU's fp32 arithmetic may land on either side); each code must
    equal the oracle's, unless the scaled value |y| / 2^X is within ``rel`` of
    a rounding boundary between the two codes (same sign, adjacent
    magnitudes) or both are zero.  Returns the bit-exact fraction of
    records."""
    import oracle
    rec = np.asarray(records, dtype=np.uint8).reshape(-1, 68)
    y = np.asarray(y, dtype=np.float64)
    codes_o, sb_o = oracle.mxfp4_encode_rows(y)
    cb = rec[:, :64].astype(np.int64)
    codes_g = np.empty((rec.shape[0], 128), dtype=np.int64)
    codes_g[:, 0::2] = cb & 0xF
    codes_g[:, 1::2] = cb >> 4
    sb_g = rec[:, 64:68].astype(np.int64)
    exact = 0
    for r in range(rec.shape[0]):
        row_exact = True
        for b in range(4):
            blk = slice(32 * b, 32 * b + 32)
            amax = np.abs(y[r, blk]).max()
            if sb_g[r, b] != sb_o[r, b]:
                row_exact = False
                m = amax / 2.0 ** np.round(np.log2(amax)) if amax > 0 else 0.0
                assert amax > 0 and abs(m - 1.0) <= rel, (
                    f"row {r} block {b}: scale {sb_g[r, b]} vs {sb_o[r, b]}, amax {amax}")
                continue
            X = int(sb_o[r, b]) - 127
            x = np.abs(y[r, blk]) / 2.0 ** X
            for d in np.nonzero(codes_g[r, blk] != codes_o[r, blk])[0]:
                row_exact = False
                cg, co = int(codes_g[r, 32 * b + d]), int(codes_o[r, 32 * b + d])
                if (cg & 7) == 0 and (co & 7) == 0:
                    continue                                  # +0 / -0
                assert (cg & 8) == (co & 8) and abs((cg & 7) - (co & 7)) == 1, (
                    f"row {r} dim {32 * b + d}: code {cg} vs {co}, value {y[r, 32 * b + d]}")
                bound = _E2M1_BOUNDS[min(cg & 7, co & 7)]
                assert abs(x[d] - bound) <= rel * bound, (
                    f"row {r} dim {32 * b + d}: code {cg} vs {co} away from a boundary "
                    f"(scaled {x[d]})")
        exact += row_exact
    return exact / max(rec.shape[0], 1)
